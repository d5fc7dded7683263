"""md_moe_layer_stage_relaunch (the measurement aid that re-enqueues one
stage of an earlier call): relaunching every stage in order after a call,
or the last stage alone over a cleared output, gives the call's results
bit for bit, on the one-token path (with and without the merged shared
expert) and on the grouped-GEMM path."""
import numpy as np
import pytest

from synth import workloads as W

from .gpu_common import moe_layer, require_gpu, say

pytestmark = pytest.mark.gpu

STAGES = ("shared", "router", "select", "gateup", "down", "combine")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("key,T", [("c0", 1), ("c3", 1), ("c3", 4), ("c4_i4", 1), ("c4_i4", 33), ("c3", 128),
                                   ("c4_i2", 9)])
def test_relaunched_stages_give_the_same_results(key, T):
    import moe_decode_amd as md
    import torch
    sp = W.spec(key)
    layer = moe_layer(key)
    x = torch.from_numpy(W.moe_x(sp, T)).cuda()
    ws = torch.empty(md.moe_workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, sp.H, device="cuda")
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, device="cuda")
    md.moe_layer_forward(layer, x, y=y, idx=idx, gates=gates, workspace=ws)
    torch.cuda.synchronize()
    y0, i0, g0 = y.clone(), idx.clone(), gates.clone()
    say(f"[relaunch] {key} T={T}")
    # the last stage alone over a cleared output
    last = "down" if T <= 8 or (key == "c3" and T <= 16) else "combine"
    y.fill_(float("nan"))
    md.moe_layer_stage_relaunch(layer, x, last, y, ws, idx=idx, gates=gates)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    # every stage in order, outputs cleared first
    y.fill_(float("nan"))
    idx.fill_(-1)
    gates.fill_(float("nan"))
    for st in STAGES:
        md.moe_layer_stage_relaunch(layer, x, st, y, ws, idx=idx, gates=gates)
    torch.cuda.synchronize()
    assert torch.equal(idx, i0) and torch.equal(gates, g0) and torch.equal(y, y0)


def test_relaunch_rejects_a_bad_stage():
    import moe_decode_amd as md
    import torch
    sp = W.spec("c0")
    layer = moe_layer("c0")
    x = torch.from_numpy(W.moe_x(sp, 1)).cuda()
    ws = torch.empty(md.moe_workspace_size(layer, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty(1, sp.H, device="cuda")
    with pytest.raises(md.MDError) as ei:
        md.moe_layer_stage_relaunch(layer, x, 9, y, ws)
    assert ei.value.name == "MD_ERR_INVALID_ARG"
