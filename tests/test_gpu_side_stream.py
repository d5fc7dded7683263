"""A chunk of a layer with a shared expert runs the shared expert on the
library's side stream, beside the routing kernels, and joins the caller's
stream before the combine.  The results must be those of the same kernels on
the caller's stream alone (the timed entry point never forks), bit for bit,
also for calls chained without synchronisation, where each call reads the
previous one's output, and for the residual form; on the c3 layer (Q4_0
experts, Q8_0 shared expert) and on a Q8_0 layer with a Q4_1 shared
expert."""
import numpy as np
import pytest

from synth import workloads as W

from .gpu_common import moe_layer, require_gpu, say

pytestmark = pytest.mark.gpu

# Q8_0 experts with a Q4_1 shared expert (other kernels on both streams)
_SIDE = W.MoESpec("side_q8_sh_q41", 54, 1536, 512, 16, 2, "gelu_tanh", "q8_0", (1e-3, 1e-2), 0.05, None, (1,),
                  shared_F=1536, shared_fmt="q4_1", shared_d_range=(1e-3, 2e-2))
_side_layer = {}
LAYERS = ["c3", "side_q8_sh_q41"]


def _layer(name):
    if name == "c3":
        return W.spec("c3"), moe_layer("c3")
    if name not in _side_layer:
        from synth.device import device_moe
        _side_layer[name] = device_moe(_SIDE)
    return _SIDE, _side_layer[name]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _one_stream(md, layer, x, y, idx, gates, ws):
    """The same forward with every launch on the caller's stream."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()  # torch creates the HIP event at its first record
    b.record()
    md.moe_layer_forward_timed(layer, x, "shared", a, b, y=y, idx=idx, gates=gates, workspace=ws)


@pytest.mark.parametrize("name", LAYERS)
@pytest.mark.parametrize("T", [17, 33, 128])
def test_side_stream_gives_the_same_bits(name, T):
    import moe_decode_amd as md
    import torch
    say(f"[side] {name} T={T}")
    sp, layer = _layer(name)
    x = torch.from_numpy(W.moe_x(sp, T)).cuda()
    ws = torch.empty(md.moe_workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    y1, y2 = (torch.empty(T, sp.H, device="cuda") for _ in range(2))
    i1, i2 = (torch.empty(T, sp.k, dtype=torch.int32, device="cuda") for _ in range(2))
    g1, g2 = (torch.empty(T, sp.k, device="cuda") for _ in range(2))
    md.moe_layer_forward(layer, x, y=y1, idx=i1, gates=g1, workspace=ws)
    _one_stream(md, layer, x, y2, i2, g2, ws)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(g1, g2)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("name", LAYERS)
def test_chained_calls_without_synchronisation(name):
    """Four calls, each on the previous output (through a tanh on the same
    stream, which keeps the values in range), enqueued back to back on one
    stream reusing one workspace, against the same chain on one stream."""
    import moe_decode_amd as md
    import torch
    T, n = 128, 4
    say(f"[side] {name} chain of {n} x T={T}")
    sp, layer = _layer(name)
    x0 = torch.from_numpy(W.moe_x(sp, T)).cuda() * 0.25
    ws = torch.empty(md.moe_workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, device="cuda")
    outs = []
    for forked in (True, False):
        xs, ys = [x0], []
        for i in range(n):
            y = torch.empty(T, sp.H, device="cuda")
            if forked:
                md.moe_layer_forward(layer, xs[i], y=y, idx=idx, gates=gates, workspace=ws)
            else:
                _one_stream(md, layer, xs[i], y, idx, gates, ws)
            ys.append(y)
            xs.append(torch.tanh(y))
        torch.cuda.synchronize()
        outs.append(torch.stack(ys))
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("name", LAYERS)
def test_residual_form_on_the_side_stream(name):
    """residual + layer(x) with the residual being y itself, against the
    layer on one stream followed by the add."""
    import moe_decode_amd as md
    import torch
    T = 128
    say(f"[side] {name} residual T={T}")
    sp, layer = _layer(name)
    x = torch.from_numpy(W.moe_x(sp, T)).cuda()
    ws = torch.empty(md.moe_workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, device="cuda")
    r = torch.from_numpy(np.random.default_rng(5).standard_normal((T, sp.H)).astype(np.float32)).cuda()
    y = r.clone()
    md.moe_layer_forward(layer, x, y=y, idx=idx, gates=gates, workspace=ws, residual=y)
    y_ref = torch.empty(T, sp.H, device="cuda")
    _one_stream(md, layer, x, y_ref, idx, gates, ws)
    out = torch.empty_like(y_ref)
    md.add(r, y_ref, out=out)
    torch.cuda.synchronize()
    assert torch.equal(y, out)


@pytest.mark.parametrize("name", LAYERS)
def test_graph_capture_takes_the_side_stream_in(name):
    """A chunk forward captured in a HIP graph from a torch stream (the side
    stream joins the capture through the fork event and leaves it through
    the join), replayed three times with eager forwards of other inputs in
    between: every replay gives the eager result for its input, bit for bit."""
    import moe_decode_amd as md
    import torch
    T = 128
    say(f"[side] {name} graph capture T={T}")
    sp, layer = _layer(name)
    x = torch.from_numpy(W.moe_x(sp, T)).cuda()
    x_other = torch.tanh(x * 3.0)
    ws = torch.empty(md.moe_workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws)
    y = torch.empty(T, sp.H, device="cuda")
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, device="cuda")
    y_ref = torch.empty_like(y)
    md.moe_layer_forward(layer, x, y=y_ref, workspace=ws_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            md.moe_layer_forward(layer, x, y=y, idx=idx, gates=gates, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    y_other = torch.empty_like(y)
    for rep in range(3):
        y.fill_(float("nan"))
        g.replay()
        md.moe_layer_forward(layer, x_other, y=y_other, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}"
    del g
