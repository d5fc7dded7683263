"""Pins of the oracle's gated FFN and whole MoE layer: a float64 composition
of library routines (numpy matmul, lexsort, torch's GELU/SiLU) on weights
built here from integer codes, special cases (k = 1, zero experts), and
invariants (relabelling, token independence, thread count)."""
import numpy as np
import pytest
import torch

from synth import formats as F
from synth import workloads as Wk


def _rand_q8(rng, rows, K, zero=False):
    d = rng.uniform(1e-3, 1e-2, (rows, K // 32)).astype(np.float16)
    if zero:
        d[:] = 0
    q = rng.integers(-127, 128, (rows, K))
    return F.pack_q8_0(d, q), np.repeat(d.astype(np.float64), 32, axis=1) * q


def _act(name, z):
    t = torch.from_numpy(z)
    if name == "gelu_tanh":
        return torch.nn.functional.gelu(t, approximate="tanh").numpy()
    return torch.nn.functional.silu(t).numpy()


def _ffn_ref(Wg, Wu, Wd, act, x):
    a = x @ Wg.T
    u = x @ Wu.T
    h = _act(act, a) * u
    return h @ Wd.T, np.abs(h) @ np.abs(Wd.T)


@pytest.mark.parametrize("act", ["gelu_tanh", "silu"])
def test_ffn_matches_library_composition(orc, act):
    rng = np.random.default_rng(21)
    H, Fd, T = 64, 96, 3
    (mg, Wg), (mu, Wu), (md, Wd) = _rand_q8(rng, Fd, H), _rand_q8(rng, Fd, H), _rand_q8(rng, H, Fd)
    x = rng.standard_normal((T, H)).astype(np.float32)
    y, S = orc.ffn(mg, mu, md, act, x)
    ref, Sref = _ffn_ref(Wg, Wu, Wd, act, x.astype(np.float64))
    assert np.allclose(S, Sref, rtol=1e-10)
    assert np.all(np.abs(y - ref) <= 1e-10 * S + np.abs(ref) * 2.0 ** -24)


def test_activation_limits(orc):
    # identity gate/up/down (one-hot rows, d = 1): y_i = act(x_i) * x_i
    H = 32
    d = np.full((H, 1), np.float16(1.0))
    eye = F.pack_q8_0(d, np.eye(H, dtype=np.int64))
    x = np.zeros((1, H), dtype=np.float32)
    x[0, :4] = [0.0, 12.0, -12.0, 1.0]
    y, _ = orc.ffn(eye, eye, eye, "gelu_tanh", x)
    assert y[0, 0] == 0.0
    assert y[0, 1] == np.float32(144.0)              # gelu(12) == 12 to double precision
    assert abs(y[0, 2]) < 1e-30                        # gelu(-12) ~ 0
    # gelu(1) = 0.5 * (1 + tanh(sqrt(2/pi) * 1.044715)) = 0.8411919906...
    assert abs(y[0, 3] - 0.8411919906082768) < 1e-7
    y, _ = orc.ffn(eye, eye, eye, "silu", x)
    assert y[0, 0] == 0.0 and abs(y[0, 3] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-7


def _tiny_layer(rng, H=64, Fd=64, E=6, shared=False, zero_experts=()):
    experts, dense = {}, {}
    for e in range(E):
        z = e in zero_experts
        (mg, Wg), (mu, Wu), (md, Wd) = _rand_q8(rng, Fd, H, z), _rand_q8(rng, Fd, H, z), _rand_q8(rng, H, Fd, z)
        experts[e] = {"gate": mg, "up": mu, "down": md}
        dense[e] = (Wg, Wu, Wd)
    sh = shd = None
    if shared:
        (mg, Wg), (mu, Wu), (md, Wd) = _rand_q8(rng, 128, H), _rand_q8(rng, 128, H), _rand_q8(rng, H, 128)
        sh = {"gate": mg, "up": mu, "down": md}
        shd = (Wg, Wu, Wd)
    Wr = rng.normal(0, 0.05, (E, H)).astype(np.float32)
    bias = rng.normal(0, 1, E).astype(np.float32)
    return experts, dense, sh, shd, Wr, bias


@pytest.mark.parametrize("shared", [False, True])
def test_layer_matches_library_composition(orc, shared):
    rng = np.random.default_rng(22)
    H, Fd, E, k, T = 64, 64, 6, 2, 5
    experts, dense, sh, shd, Wr, bias = _tiny_layer(rng, H, Fd, E, shared)
    x = rng.standard_normal((T, H)).astype(np.float32)
    y, idx, gates, S = orc.moe_forward(H, Fd, E, k, "gelu_tanh", Wr, bias, experts, sh, x)
    xd = x.astype(np.float64)
    logits = (xd @ Wr.T.astype(np.float64) + bias).astype(np.float32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))[:k]
        assert list(idx[t]) == list(order)
        sel = logits[t][order].astype(np.float64)
        g = np.exp(sel - sel.max())
        g /= g.sum()
        assert np.allclose(gates[t], g, rtol=1e-7, atol=1e-8)
        ref = np.zeros(H)
        Sref = np.zeros(H)
        for j, e in enumerate(order):
            o, s = _ffn_ref(*dense[e], "gelu_tanh", xd[t:t + 1])
            ref += float(gates[t, j]) * o[0]
            Sref += float(gates[t, j]) * s[0]
        if shared:
            o, s = _ffn_ref(*shd, "gelu_tanh", xd[t:t + 1])
            ref += o[0]
            Sref += s[0]
        assert np.allclose(S[t], Sref, rtol=1e-10)
        assert np.all(np.abs(y[t] - ref) <= 1e-10 * S[t] + np.abs(ref) * 2.0 ** -24)


def test_k1_equals_the_plain_expert_chain(orc):
    rng = np.random.default_rng(23)
    H, Fd, E = 64, 64, 6
    experts, _, _, _, Wr, bias = _tiny_layer(rng, H, Fd, E)
    x = rng.standard_normal((4, H)).astype(np.float32)
    y, idx, gates, S = orc.moe_forward(H, Fd, E, 1, "gelu_tanh", Wr, bias, experts, None, x)
    assert np.all(gates == 1.0)
    for t in range(4):
        e = int(idx[t, 0])
        yf, Sf = orc.ffn(experts[e]["gate"], experts[e]["up"], experts[e]["down"], "gelu_tanh", x[t:t + 1])
        assert np.array_equal(y[t], yf[0]) and np.array_equal(S[t], Sf[0])


def test_zero_experts_leave_only_the_shared_branch(orc):
    rng = np.random.default_rng(24)
    H, Fd, E = 64, 64, 4
    experts, _, sh, _, Wr, bias = _tiny_layer(rng, H, Fd, E, True, zero_experts=range(E))
    x = rng.standard_normal((3, H)).astype(np.float32)
    y, _, _, _ = orc.moe_forward(H, Fd, E, 2, "gelu_tanh", Wr, bias, experts, sh, x)
    ys, _ = orc.ffn(sh["gate"], sh["up"], sh["down"], "gelu_tanh", x)
    assert np.array_equal(y, ys)


def test_relabelling_experts_permutes_idx_only(orc):
    rng = np.random.default_rng(25)
    H, Fd, E, k = 64, 64, 6, 3
    experts, _, _, _, Wr, bias = _tiny_layer(rng, H, Fd, E)
    x = rng.standard_normal((4, H)).astype(np.float32)
    y, idx, gates, _ = orc.moe_forward(H, Fd, E, k, "gelu_tanh", Wr, bias, experts, None, x)
    perm = rng.permutation(E)                     # new label of old expert e is perm[e]
    inv = np.argsort(perm)
    experts2 = {int(perm[e]): experts[e] for e in range(E)}
    y2, idx2, gates2, _ = orc.moe_forward(H, Fd, E, k, "gelu_tanh", Wr[inv], bias[inv], experts2, None, x)
    assert np.array_equal(idx2, perm[idx])
    assert np.array_equal(gates2, gates) and np.array_equal(y2, y)


def test_tokens_are_independent(orc):
    sp = Wk.spec("c0")
    Wr, b = Wk.moe_router(sp)
    x = Wk.moe_x(sp, 1)
    x4 = np.concatenate([x, -x, 2 * x, 0.5 * x])
    experts = {e: Wk.moe_expert(sp, e) for e in range(sp.E)}
    y, idx, gates, S = orc.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, experts, None, x4)
    for t in range(4):
        yt, it, gt, St = orc.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, experts, None, x4[t:t + 1])
        assert np.array_equal(yt[0], y[t]) and np.array_equal(it[0], idx[t]) and np.array_equal(St[0], S[t])


def test_missing_expert_is_an_error(orc):
    import oracle
    sp = Wk.spec("c0")
    Wr, b = Wk.moe_router(sp)
    x = Wk.moe_x(sp, 1)
    with pytest.raises(oracle.OracleError):
        orc.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, {}, None, x)


def test_threads_bitwise_layer(orc, orc_mt):
    sp = Wk.spec("c0")
    Wr, b = Wk.moe_router(sp)
    x = np.concatenate([Wk.moe_x(sp, 1), Wk.moe_x(sp, 4)])
    experts = {e: Wk.moe_expert(sp, e) for e in range(sp.E)}
    r1 = orc.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, experts, None, x)
    r2 = orc_mt.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, experts, None, x)
    for a, c in zip(r1, r2):
        assert np.array_equal(a, c)
