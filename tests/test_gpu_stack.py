"""Stacked layers: the residual add (exact fp32), a stack of MoE layers run
eagerly and checked layer by layer against the oracle, and the same stack
captured in a HIP graph and replayed several times with eager work between
the replays, every replay bit-identical to the eager run."""
from dataclasses import replace

import numpy as np
import pytest

from synth import workloads as W

from .gpu_common import assert_within, oracle_moe, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _specs(n):
    base = W.spec("c0")
    return [replace(base, key=f"c0_layer{l}", variant=50 + l) for l in range(n)]


_layers = {}


def _device_layers(specs):
    from synth.device import device_moe
    out = []
    for sp in specs:
        if sp.key not in _layers:
            _layers[sp.key] = device_moe(sp)
        out.append(_layers[sp.key])
    return out


def test_add_is_exact():
    import moe_decode_amd as md
    import torch
    rng = np.random.default_rng(5)
    for n in (1, 3, 4, 1000, 6144 * 3 + 2):
        a = rng.standard_normal(n).astype(np.float32)
        b = rng.standard_normal(n).astype(np.float32)
        y = md.add(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), a + b), n



def test_read_probe_reads_everything():
    """The bandwidth probe covers whole tiles, a ragged tail and grids larger
    and smaller than the tile count; it writes only on a key match."""
    import moe_decode_amd as md
    import torch
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    for nbytes in (16, 16 * 1000, 1 << 20, (1 << 20) + 48):
        src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        for wg in (0, 1, 3):
            md.hbm_read_probe(src, sink, key=1, workgroups=wg)
            torch.cuda.synchronize()
            assert sink[0].item() == 7, (nbytes, wg)
        # every lane's xor of zeroed memory is 0: key 0 must be stored
        md.hbm_read_probe(src, sink, key=0)
        torch.cuda.synchronize()
        assert sink[0].item() == 0, nbytes
        sink.fill_(7)
    # one word set to 5 in the first, a middle and the last whole-tile chunk:
    # only the lane that reads that chunk holds 5, and it stores key 5
    src = torch.zeros((1 << 20) + 48, dtype=torch.uint8, device="cuda")
    for chunk in (0, 30000, 65535):
        src.zero_()
        src[chunk * 16 + 4] = 5
        sink.fill_(7)
        md.hbm_read_probe(src, sink, key=5, workgroups=3)
        torch.cuda.synchronize()
        assert sink[0].item() == 5, chunk

@pytest.mark.parametrize("T", [1, 3])
def test_stack_eager_matches_oracle(orc_mt, T):
    import moe_decode_amd as md
    import torch
    specs = _specs(3)
    layers = _device_layers(specs)
    cur = torch.from_numpy(W.moe_x(specs[0], T)).cuda()
    for sp, layer in zip(specs, layers):
        x_np = cur.cpu().numpy()
        idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
        gates = torch.empty(T, sp.k, dtype=torch.float32, device="cuda")
        y = md.moe_layer_forward(layer, cur, idx=idx, gates=gates)
        nxt = md.add(cur, y)
        torch.cuda.synchronize()
        y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x_np)
        assert np.array_equal(idx.cpu().numpy(), i_ref)
        assert np.max(np.abs(gates.cpu().numpy() - g_ref)) <= 1e-6
        ratio = assert_within(y.cpu().numpy(), y_ref, S, f"{sp.key} T={T}")
        assert np.array_equal(nxt.cpu().numpy(), x_np + y.cpu().numpy())
        say(f"[stack] {sp.key} T={T} max err/S {ratio:.2e}")
        cur = nxt


@pytest.mark.parametrize("T", [1, 3])
def test_stack_graph_replays_match_eager(T):
    import moe_decode_amd as md
    import torch
    specs = _specs(3)
    layers = _device_layers(specs)
    x = torch.from_numpy(W.moe_x(specs[0], T)).cuda()
    wss = [torch.empty(md.moe_workspace_size(l, T), dtype=torch.uint8, device="cuda") for l in layers]
    ys = [torch.empty(T, specs[0].H, device="cuda") for _ in layers]
    curs = [x] + [torch.empty(T, specs[0].H, device="cuda") for _ in layers]

    def run():
        # layer l: curs[l+1] = curs[l] + layer(curs[l]) (the residual joins the
        # layer's last kernel); the last layer adds with md_add instead
        for l, layer in enumerate(layers):
            if l + 1 < len(layers):
                md.moe_layer_forward(layer, curs[l], y=curs[l + 1], workspace=wss[l], residual=curs[l])
            else:
                md.moe_layer_forward(layer, curs[l], y=ys[l], workspace=wss[l])
                md.add(curs[l], ys[l], out=curs[l + 1])

    run()
    torch.cuda.synchronize()
    eager = [c.clone() for c in curs[1:]]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for c in curs[1:] + ys:
            c.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, (c, e) in enumerate(zip(curs[1:], eager)):
            assert torch.equal(c, e), f"replay {rep}, layer {l}"
    say(f"[stack] graph of {len(layers)} layers, T={T}: 4 replays equal the eager run")


@pytest.mark.parametrize("key,T", [("c0", 1), ("c0", 2), ("c3", 1), ("c3", 33), ("c4_i4", 12), ("q4_sh", 3)])
def test_residual_forward_equals_forward_then_add(key, T):
    """y = residual + layer(x) from the residual entry point equals the layer
    followed by md_add, bit for bit, on every path (one-token kernels without
    and with a shared expert, the merged routed + shared launches, the grouped
    GEMMs with and without a shared expert), with the residual a separate
    buffer and with the residual being y itself."""
    import moe_decode_amd as md
    import torch
    from .gpu_common import moe_layer
    if key == "q4_sh":
        from .test_gpu_moe import _RAGGED
        from synth.device import device_moe
        sp = _RAGGED["q4_e24_k2_sh"]
        layer = device_moe(sp)
    else:
        sp = W.spec(key)
        layer = moe_layer(key)
    x = torch.from_numpy(W.moe_x(sp, T)).cuda()
    r = torch.from_numpy(np.random.default_rng([7, T]).standard_normal((T, sp.H)).astype(np.float32)).cuda()
    y0 = md.moe_layer_forward(layer, x)
    want = md.add(r, y0)
    got = md.moe_layer_forward(layer, x, residual=r)
    inplace = r.clone()
    md.moe_layer_forward(layer, x, y=inplace, residual=inplace)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert torch.equal(inplace, want)
