"""GPU checks of the experts-for-a-given-routing entry point and of the
host-memory expert tier: outputs bit-identical to the resident layer (the
same kernels on the same weights, only the expert addresses differ), the
cache's hits and misses equal to the policy model, and every slot holding
its expert's bytes."""
import numpy as np
import pytest

from synth import workloads as W

from .gpu_common import require_gpu, say
from .test_tier_cpu import PolicyModel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_res = {}


def _resident(key):
    from synth.device import device_moe
    if key not in _res:
        _res[key] = device_moe(W.spec(key))
    return _res[key]


def _forward(layer, x):
    import moe_decode_amd as md
    import torch
    T = x.shape[0]
    idx = torch.empty(T, layer.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, layer.k, dtype=torch.float32, device="cuda")
    y = md.moe_layer_forward(layer, x, idx=idx, gates=gates)
    return y, idx, gates


@pytest.mark.parametrize("key,T", [("c0", 1), ("c0", 3), ("c0", 33), ("c4_i4", 1), ("c4_i2", 4),
                                   ("c4_q41", 1), ("c4_q41", 33)])
def test_experts_forward_equals_layer(key, T):
    import moe_decode_amd as md
    import torch
    say(f"[tier] experts forward {key} T={T}")
    layer = _resident(key)
    sp = W.spec(key)
    x = torch.from_numpy(W.moe_x(sp, T)).cuda()
    y, idx, gates = _forward(layer, x)
    y2 = md.moe_experts_forward(layer, x, idx, gates)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_experts_forward_clamps_the_routing():
    import moe_decode_amd as md
    import torch
    layer = _resident("c0")
    sp = W.spec("c0")
    x = torch.from_numpy(W.moe_x(sp, 2)).cuda()
    gates = torch.tensor([[0.75, 0.25], [0.5, 0.5]], dtype=torch.float32, device="cuda")
    wild = torch.tensor([[-3, 2], [5, 40]], dtype=torch.int32, device="cuda")
    tame = torch.tensor([[0, 2], [5, 7]], dtype=torch.int32, device="cuda")
    y1 = md.moe_experts_forward(layer, x, wild, gates)
    y2 = md.moe_experts_forward(layer, x, tame, gates)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def _tier(key, S, overlap=True):
    import moe_decode_amd as md
    from synth.device import host_moe
    return md.ExpertTier(host_moe(W.spec(key)), S, overlap=overlap)


def _slots_hold_their_experts(tier):
    host, slots, c = tier.host, tier.slots, tier.cache
    for part in ("gate", "up", "down"):
        hm, sm = getattr(host, part), getattr(slots, part)
        per = hm.q.numel() // host.E
        sq = sm.q.cpu()
        for s, e in enumerate(c.expert_in_slot.tolist()):
            if e < 0:
                continue
            assert np.array_equal(sq[s * per:(s + 1) * per].numpy(), hm.q[e * per:(e + 1) * per].numpy()), (part, s)
            if hm.row_scale is not None:
                r = hm.rows
                assert np.array_equal(sm.row_scale[s * r:(s + 1) * r].cpu().numpy(),
                                      hm.row_scale[e * r:(e + 1) * r].numpy())


def test_tier_decode_sequence_c0():
    import torch
    say("[tier] c0 S=4 decode sequence")
    layer = _resident("c0")
    sp = W.spec("c0")
    tier = _tier("c0", 4)
    model = PolicyModel(sp.E, 4)
    xs = np.random.default_rng([0, 901]).standard_normal((40, 1, sp.H)).astype(np.float32)
    for i in range(40):
        x = torch.from_numpy(xs[i]).cuda()
        y, idx, gates = _forward(layer, x)
        idx2 = torch.empty_like(idx)
        gates2 = torch.empty_like(gates)
        y2 = tier.forward(x, idx=idx2, gates=gates2)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2) and torch.equal(gates, gates2), i
        assert torch.equal(y, y2), i
        model.plan(idx.cpu().numpy().reshape(-1))
        assert (tier.cache.hits, tier.cache.misses) == (model.hits, model.misses), i
    assert tier.cache.misses > 4 and tier.cache.hits > 0
    _slots_hold_their_experts(tier)


def test_tier_chunk_c0():
    import torch
    layer = _resident("c0")
    sp = W.spec("c0")
    tier = _tier("c0", 8)
    for T in (33, 5, 128):
        x = torch.from_numpy(W.moe_x(sp, T)).cuda()
        y, _, _ = _forward(layer, x)
        y2 = tier.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), T
    _slots_hold_their_experts(tier)


def test_tier_decode_c4_int4():
    import torch
    say("[tier] c4_i4 S=16")
    layer = _resident("c4_i4")
    sp = W.spec("c4_i4")
    tier = _tier("c4_i4", 16)
    rng = np.random.default_rng([4, 902])
    for i, T in enumerate((1, 1, 1, 2, 1, 1)):
        x = torch.from_numpy(rng.standard_normal((T, sp.H)).astype(np.float32)).cuda()
        y, _, _ = _forward(layer, x)
        y2 = tier.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), i
    _slots_hold_their_experts(tier)


@pytest.mark.parametrize("overlap", [True, False])
def test_tier_with_shared_expert_c3(orc_mt, overlap):
    """The 128-expert layer with its shared expert: misses load on a stream of
    their own while the shared expert runs (or on the one stream); outputs
    within the tolerance of the oracle, and the two orders bit-identical."""
    import torch
    from .gpu_common import assert_within, oracle_moe
    say(f"[tier] c3 S=32 overlap={overlap}")
    sp = W.spec("c3")
    tier = _tier("c3", 32, overlap=overlap)
    rng = np.random.default_rng([3, 903])
    outs = []
    for i, T in enumerate((1, 1, 2, 1, 3, 1)):
        x = rng.standard_normal((T, sp.H)).astype(np.float32)
        y = tier.forward(torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        y_ref, _, _, S = oracle_moe(orc_mt, sp, x)
        assert_within(y.cpu().numpy(), y_ref, S, f"c3 tier step {i}")
        outs.append(y.cpu().numpy())
    assert tier.cache.misses > 0
    _slots_hold_their_experts(tier)
    _c3_outs.setdefault("runs", []).append(outs)
    if len(_c3_outs["runs"]) == 2:
        a, b = _c3_outs["runs"]
        assert all(np.array_equal(u, v) for u, v in zip(a, b))


_c3_outs = {}
