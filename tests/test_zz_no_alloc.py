"""md_moe_layer_forward_noalloc (the layer forward on the library's built-in
scratch) against md_moe_layer_forward with a caller workspace, through the C
ABI: two calls in a row, the second with fewer tokens, each bit-identical to
the workspace call (same kernels, same arithmetic), and the oracle's bound."""
import numpy as np
import pytest

from synth import workloads as W

from .gpu_common import assert_within, moe_layer, oracle_moe, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _outputs(sp, T):
    import torch
    return (torch.full((T, sp.H), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((T, sp.k), -1, dtype=torch.int32, device="cuda"),
            torch.full((T, sp.k), float("nan"), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("key,T1,T2", [("c4_i4", 128, 1), ("c3", 16, 3), ("c0", 2, 1), ("c4_i8", 8, 4)])
def test_noalloc_equals_workspace_call(orc_mt, key, T1, T2):
    import moe_decode_amd as md
    import torch
    sp = W.spec(key)
    layer = moe_layer(key)
    for T in (T1, T2):
        say(f"[noalloc] {key} T={T}")
        x = torch.from_numpy(W.moe_x(sp, T)).cuda()
        y0, i0, g0 = _outputs(sp, T)
        md.moe_layer_forward(layer, x, y=y0, idx=i0, gates=g0)
        y1, i1, g1 = _outputs(sp, T)
        md.moe_layer_forward_noalloc(layer, x, y1, idx=i1, gates=g1)
        torch.cuda.synchronize()
        assert torch.equal(i1, i0) and torch.equal(g1, g0) and torch.equal(y1, y0)
        if T <= 16:
            y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x.cpu().numpy())
            assert np.array_equal(i1.cpu().numpy(), i_ref)
            assert_within(y1.cpu().numpy(), y_ref, S, f"{key} T={T} noalloc")


def test_noalloc_rejects_more_than_its_scratch():
    """128 tokens of a 256-expert layer of hidden size 16384 would need more
    than the 64 MiB built in: MD_ERR_UNSUPPORTED, nothing written."""
    import moe_decode_amd as md
    import torch
    sp = W.spec("c4_i4")
    base = moe_layer("c4_i4")
    big = md.MoELayer(16384, 16384, 256, 8, sp.act, base.gate, base.up, base.down, base.Wr, None)
    x = torch.zeros(128, 16384, dtype=torch.float32, device="cuda")
    y = torch.full((128, 16384), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(md.MDError) as ei:
        md.moe_layer_forward_noalloc(big, x, y)
    assert ei.value.name == "MD_ERR_UNSUPPORTED"
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
