"""GPU parity of the router and the MoE layer against the oracle: expert
indices bit-exact, gates within 1e-6, outputs within 1e-4*S + 1e-6, at the
workloads' full sizes (decode, batch decode, 128-token chunks), plus the
exact-tie rule through the GPU route path and invariants."""
import numpy as np
import pytest

from synth import workloads as W

from .gpu_common import assert_within, moe_layer, oracle_moe, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _route_gpu(x, Wr, b, k, E):
    import moe_decode_amd as md
    import torch
    T = x.shape[0]
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx, gates = md.moe_route_topk(_t(x), _t(Wr), None if b is None else _t(b), k, logits=logits)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gates.cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("key,T", [("c0", 1), ("c3", 1), ("c3", 128), ("c4_i4", 1), ("c4_i4", 4), ("c4_i4", 128)])
def test_route_matches_oracle(orc_mt, key, T):
    sp = W.spec(key)
    Wr, b = W.moe_router(sp)
    x = W.moe_x(sp, T)
    i_ref, g_ref, l_ref, margin = orc_mt.route_topk(x, Wr, b, sp.k)
    i_gpu, g_gpu, l_gpu = _route_gpu(x, Wr, b, sp.k, sp.E)
    assert np.array_equal(l_gpu, l_ref), "logits differ"
    mism = np.argwhere(i_gpu != i_ref)
    assert mism.size == 0, f"idx mismatch at {mism[:5].tolist()}, margins {margin[mism[:5, 0]].tolist()}"
    assert np.max(np.abs(g_gpu - g_ref)) <= 1e-6


def _one_hot_route(logits_wanted, k, H=256):
    l = np.asarray(logits_wanted, dtype=np.float32)
    Wr = np.zeros((l.shape[0], H), dtype=np.float32)
    Wr[:, 0] = l
    x = np.zeros((1, H), dtype=np.float32)
    x[0, 0] = 1.0
    return x, Wr


@pytest.mark.parametrize("case", ["all_equal", "boundary_tie", "inner_ties", "signed_zero", "k_equals_E"])
def test_route_ties_through_gpu(orc, case):
    E, k = 64, 8
    if case == "all_equal":
        l = [0.5] * E
    elif case == "boundary_tie":
        l = list(np.linspace(-1, 1, E))
        l[10] = l[50] = 5.0
        for e in range(20, 26):
            l[e] = 3.0
        l[40] = l[33] = 3.0                 # 8 values of 3.0 compete for 6 slots
    elif case == "inner_ties":
        l = [0.25 * (e % 5) for e in range(E)]
    elif case == "signed_zero":
        l = [-1.0] * E
        for e in (3, 7, 9, 11):
            l[e] = -0.0
        for e in (4, 8, 12, 60):
            l[e] = 0.0
    else:
        E = k = 8
        l = [1.0, -2.0, 1.0, 0.0, -0.0, 3.0, 1.0, 3.0]
    x, Wr = _one_hot_route(l, k)
    i_ref, g_ref, _, _ = orc.route_topk(x, Wr, None, k)
    i_gpu, g_gpu, _ = _route_gpu(x, Wr, None, k, len(l))
    assert np.array_equal(i_gpu, i_ref), (i_gpu, i_ref)
    assert np.max(np.abs(g_gpu - g_ref)) <= 1e-6


def _moe_gpu(key, x):
    import moe_decode_amd as md
    import torch
    sp = W.spec(key)
    layer = moe_layer(key)
    T = x.shape[0]
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, dtype=torch.float32, device="cuda")
    y = md.moe_layer_forward(layer, _t(x), idx=idx, gates=gates)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), gates.cpu().numpy()


@pytest.mark.parametrize("key,T", [("c0", 1), ("c3", 1), ("c4_i4", 1), ("c4_i4", 4), ("c4_i8", 1), ("c4_i8", 4),
                                   ("c3", 128),
                                   # verify-sized batches: small layers stay on the one-token kernels up to
                                   # 16 tokens, the large ones group by expert above 8
                                   ("c0", 16), ("c3", 12), ("c3", 16), ("c4_i4", 12),
                                   # packed int2 experts: one token, a batch, a verify batch
                                   ("c4_i2", 1), ("c4_i2", 4), ("c4_i2", 12),
                                   # Q4_1 block experts
                                   ("c4_q41", 1), ("c4_q41", 4), ("c4_q41", 12)])
def test_moe_layer_matches_oracle(orc_mt, key, T):
    sp = W.spec(key)
    x = W.moe_x(sp, T)
    say(f"[moe] {key} T={T}")
    y, idx, gates = _moe_gpu(key, x)
    y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x)
    assert np.array_equal(idx, i_ref)
    assert np.max(np.abs(gates - g_ref)) <= 1e-6
    ratio = assert_within(y, y_ref, S, f"{key} T={T}")
    say(f"[moe] {key} T={T} max err/S {ratio:.2e}")


@pytest.mark.timeout(900)  # the oracle's 128 tokens of the 256-expert layer take minutes on a few cores
@pytest.mark.parametrize("key", ["c4_i4", "c4_i8", "c4_i2", "c4_q41"])
def test_moe_prefill_chunk_full(orc_mt, key):
    """128-token chunk at full size: routing and output of every token
    against the oracle."""
    sp = W.spec(key)
    x = W.moe_x(sp, 128)
    say(f"[moe] {key} T=128")
    y, idx, gates = _moe_gpu(key, x)
    y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x)
    assert np.array_equal(idx, i_ref)
    assert np.max(np.abs(gates - g_ref)) <= 1e-6
    ratio = assert_within(y, y_ref, S, f"{key} T=128")
    say(f"[moe] {key} T=128 max err/S {ratio:.2e}")


def test_prefill_equals_token_by_token():
    sp = W.spec("c3")
    x = W.moe_x(sp, 128)[:16]
    y, idx, _ = _moe_gpu("c3", x)
    for t in (0, 5, 15):
        yt, it, _ = _moe_gpu("c3", x[t:t + 1])
        assert np.array_equal(it[0], idx[t])
        assert np.max(np.abs(yt[0] - y[t])) <= 1e-5 * np.max(np.abs(y[t])) + 1e-6


def test_moe_deterministic():
    sp = W.spec("c3")
    x = W.moe_x(sp, 128)[:8]
    a = _moe_gpu("c3", x)
    b = _moe_gpu("c3", x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_single_expert_gate_one_is_its_ffn():
    """k = 1: the layer output is that expert's FFN (gate exactly 1)."""
    import moe_decode_amd as md
    import torch
    sp = W.spec("c0")
    base = moe_layer("c0")
    layer = md.MoELayer(sp.H, sp.F, sp.E, 1, sp.act, base.gate, base.up, base.down, base.Wr, base.bias)
    x = W.moe_x(sp, 4)
    idx = torch.empty(4, 1, dtype=torch.int32, device="cuda")
    gates = torch.empty(4, 1, dtype=torch.float32, device="cuda")
    y = md.moe_layer_forward(layer, _t(x), idx=idx, gates=gates)
    torch.cuda.synchronize()
    assert torch.all(gates == 1.0)
    for t in range(4):
        e = int(idx[t, 0])
        ffn = md.FFN(sp.act, base.gate.expert(e), base.up.expert(e), base.down.expert(e))
        yf = md.ffn_forward(ffn, _t(x[t:t + 1]))
        torch.cuda.synchronize()
        assert torch.equal(yf[0], y[t])


@pytest.mark.parametrize("key,T", [("c0", 1), ("c3", 1), ("c3", 8), ("c4_i4", 1), ("c4_i4", 4), ("c4_i8", 1)])
def test_moe_few_tokens_repeatable(orc_mt, key, T):
    """The few-token layer against the oracle, called twice: the second call
    (same buffers, same inputs) gives the same bits, indices and gates."""
    sp = W.spec(key)
    x = W.moe_x(sp, T)
    say(f"[moe repeat] {key} T={T}")
    y, idx, gates = _moe_gpu(key, x)
    y2, id2, g2 = _moe_gpu(key, x)
    y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x)
    assert np.array_equal(idx, i_ref) and np.array_equal(id2, i_ref)
    assert np.array_equal(gates, g2) and np.array_equal(y, y2)
    assert np.max(np.abs(gates - g_ref)) <= 1e-6
    assert_within(y, y_ref, S, f"{key} T={T}")


@pytest.mark.parametrize("key", ["c4_i4", "c4_i8", "c3"])
def test_moe_decode_activation_outliers(orc_mt, key):
    """Activations with a few channels 200x larger than the rest (as trained
    models have): the one-token kernels scale their integer digit planes per
    weight chunk's group of activations, so a group holding an outlier
    resolves its other values relative to it; outputs stay within the bound."""
    sp = W.spec(key)
    x = W.moe_x(sp, 2).copy()
    rng = np.random.default_rng([sp.index, 4242])
    ch = rng.choice(sp.H, size=max(4, sp.H // 200), replace=False)
    x[:, ch] *= 200.0
    say(f"[moe outliers] {key}: {len(ch)} channels x200")
    y, idx, gates = _moe_gpu(key, x)
    y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x)
    assert np.array_equal(idx, i_ref)
    assert np.max(np.abs(gates - g_ref)) <= 1e-6
    ratio = assert_within(y, y_ref, S, f"{key} outliers")
    say(f"[moe outliers] {key} max err/S {ratio:.2e}")


def _tie_logits(E):
    """Four logit vectors with exact ties placed across the four experts each
    lane of the selecting wave holds (e, e + 64, e + 128, e + 192)."""
    hi = E - 1
    boundary = np.linspace(-1, 1, E).astype(np.float32)
    boundary[[10, E - 28]] = 5.0
    boundary[[70, 71, 72, E // 2 + 4, E // 2 + 5, E // 2 + 6, hi, 40]] = 3.0   # 8 values for 6 slots
    equal = np.full(E, 0.5, dtype=np.float32)
    zeros = np.full(E, -1.0, dtype=np.float32)
    zeros[[3, 65, E // 2 + 2, hi - 1]] = -0.0
    zeros[[4, 66, E // 2 + 3, hi]] = 0.0
    e = np.arange(E)
    inner = np.where(e >= E - 70, 0.25 * (e % 5), -1.0).astype(np.float32)   # ties straddle e = 64j
    return [boundary, equal, zeros, inner]


@pytest.mark.parametrize("key", ["c4_i4", "c3"])
def test_layer_ties_through_decode(orc_mt, key):
    """Exact logit ties through the layer's own decode path (the selection
    inside the gate/up kernel), against the oracle: 4 tokens, each with one
    tie pattern.  c4: the logits come from one router column per token;
    c3: a zero router and the pattern in the bias (one pattern per call)."""
    import moe_decode_amd as md
    import torch
    sp = W.spec(key)
    base = moe_layer(key)
    cases = _tie_logits(sp.E)
    x = W.moe_x(sp, 4).copy()
    calls = []
    if sp.bias_std is None:
        Wr = np.zeros((sp.E, sp.H), dtype=np.float32)
        for t in range(4):
            Wr[:, t] = cases[t]
        x[:, :4] = np.eye(4, dtype=np.float32)
        calls.append((Wr, None, x))
    else:
        for c in cases:
            calls.append((np.zeros((sp.E, sp.H), dtype=np.float32), c, x[:1]))
    for Wr, b, xt in calls:
        T = xt.shape[0]
        layer = md.MoELayer(sp.H, sp.F, sp.E, sp.k, sp.act, base.gate, base.up, base.down, _t(Wr),
                            None if b is None else _t(b), base.shared)
        idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
        gates = torch.empty(T, sp.k, dtype=torch.float32, device="cuda")
        y = md.moe_layer_forward(layer, _t(xt), idx=idx, gates=gates)
        torch.cuda.synchronize()
        i_ref, g_ref, _, _ = orc_mt.route_topk(xt, Wr, b, sp.k)
        say(f"[moe ties] {key} T={T}: {i_ref.tolist()}")
        assert np.array_equal(idx.cpu().numpy(), i_ref), (idx.cpu().numpy(), i_ref)
        assert np.max(np.abs(gates.cpu().numpy() - g_ref)) <= 1e-6
        experts = {int(e): W.moe_expert(sp, int(e)) for e in np.unique(i_ref)}
        y_ref, _, _, S = orc_mt.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, experts, W.moe_shared(sp), xt)
        assert_within(y.cpu().numpy(), y_ref, S, f"{key} ties")


# Layers of unusual shape: widths that are odd multiples of 256, expert counts
# that are not multiples of 64, k = 2, 3, 5, a shared expert outside the merged
# family, and an int4 layer whose FFN width the one-token kernels do not take
# (so every token count goes to the grouped GEMMs).
_RAGGED = {
    "q8_e40_k3": W.MoESpec("q8_e40_k3", 41, 1280, 768, 40, 3, "silu", "q8_0", (1e-3, 1e-2), 0.05, 0.5, (1,)),
    "i4_e72_k5": W.MoESpec("i4_e72_k5", 42, 768, 1280, 72, 5, "gelu_tanh", "i4_row", (1e-3, 1e-2), 0.05, None, (1,)),
    "q4_e24_k2_sh": W.MoESpec("q4_e24_k2_sh", 43, 1536, 512, 24, 2, "gelu_tanh", "q4_0", (1e-3, 2e-2), 0.05, None,
                              (1,), shared_F=768, shared_fmt="q8_0", shared_d_range=(1e-3, 1e-2)),
    # the widest hidden size the library takes (16384)
    "q8_h16384": W.MoESpec("q8_h16384", 44, 16384, 256, 8, 2, "gelu_tanh", "q8_0", (1e-3, 1e-2), 0.05, None, (1,)),
    "i4_h16384": W.MoESpec("i4_h16384", 45, 16384, 512, 16, 4, "silu", "i4_row", (1e-3, 1e-2), 0.05, 0.5, (1,)),
    # packed int2: the one-token kernels (hidden 2560: 8-lane groups, 5 slices;
    # FFN 1536: 3 chunks a lane), a layer only the grouped GEMMs take (FFN 1280),
    # the widest hidden size, and an int2 shared expert beside Q8_0 experts
    "i2_e72_k5": W.MoESpec("i2_e72_k5", 46, 2560, 1536, 72, 5, "gelu_tanh", "i2_row", (1e-3, 1e-2), 0.05, None,
                           (1,)),
    "i2_e24_k3": W.MoESpec("i2_e24_k3", 47, 768, 1280, 24, 3, "silu", "i2_row", (1e-3, 1e-2), 0.05, 0.5, (1,)),
    "i2_h16384": W.MoESpec("i2_h16384", 48, 16384, 512, 16, 4, "silu", "i2_row", (1e-3, 1e-2), 0.05, None, (1,)),
    "q8_e16_sh_i2": W.MoESpec("q8_e16_sh_i2", 49, 1536, 512, 16, 2, "gelu_tanh", "q8_0", (1e-3, 1e-2), 0.05, None,
                              (1,), shared_F=1536, shared_fmt="i2_row", shared_d_range=(1e-3, 1e-2)),
    # Q4_1 experts (w = d n + m): a biased router with k = 3, a Q4_1 shared
    # expert beside Q4_1 experts, and one beside Q8_0 experts
    "q41_e40_k3": W.MoESpec("q41_e40_k3", 50, 1280, 768, 40, 3, "silu", "q4_1", (1e-3, 2e-2), 0.05, 0.5, (1,)),
    "q41_e24_k2_sh": W.MoESpec("q41_e24_k2_sh", 51, 1536, 512, 24, 2, "gelu_tanh", "q4_1", (1e-3, 2e-2), 0.05,
                               None, (1,), shared_F=768, shared_fmt="q4_1", shared_d_range=(1e-3, 2e-2)),
    "q8_e16_sh_q41": W.MoESpec("q8_e16_sh_q41", 52, 1536, 512, 16, 2, "gelu_tanh", "q8_0", (1e-3, 1e-2), 0.05,
                               None, (1,), shared_F=1536, shared_fmt="q4_1", shared_d_range=(1e-3, 2e-2)),
}
_ragged_layers = {}


@pytest.mark.parametrize("name", sorted(_RAGGED))
@pytest.mark.parametrize("T", [1, 3, 9, 33])
def test_moe_ragged_shapes(orc_mt, name, T):
    import moe_decode_amd as md
    import torch
    from synth.device import device_moe
    sp = _RAGGED[name]
    if name not in _ragged_layers:
        _ragged_layers[name] = device_moe(sp)
    layer = _ragged_layers[name]
    x = W.moe_x(sp, T)
    say(f"[moe ragged] {name} T={T}")
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, dtype=torch.float32, device="cuda")
    y = md.moe_layer_forward(layer, _t(x), idx=idx, gates=gates)
    torch.cuda.synchronize()
    y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x)
    assert np.array_equal(idx.cpu().numpy(), i_ref)
    assert np.max(np.abs(gates.cpu().numpy() - g_ref)) <= 1e-6
    ratio = assert_within(y.cpu().numpy(), y_ref, S, f"{name} T={T}")
    say(f"[moe ragged] {name} T={T} max err/S {ratio:.2e}")


@pytest.mark.parametrize("name", ["q41_e40_k3", "q41_e24_k2_sh"])
def test_moe_q4_1_chunk(orc_mt, name):
    """A 128-token chunk of Q4_1 layers (grouped GEMMs over several 16-token
    tiles per expert), against the oracle."""
    test_moe_ragged_shapes(orc_mt, name, 128)
