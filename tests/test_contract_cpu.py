"""The accuracy contract of the integer paths, checked on the CPU with a model
of their activation rounding (tests/digit_model.py).

The library's one-token kernels round each group of activations to 2^-22 of
the group's largest magnitude, and its int8 matrix-core chunks round each
activation row to 2^-30 of the row's largest magnitude.  Per contraction
y = sum_c w_c x_c the error is therefore at most

    one-token kernels:  2^-22 * A + (fp32 combines),  A = sum_g max_g|x| * sum_{c in g} |w_c|
    int8 chunks:        2^-30 * max|x| * sum_c |w_c| + (fp32 combines)

and the tolerance 1e-4 * sum|w x| + 1e-6 follows when A <= 400 * sum|w x|
(one-token) or max|x| * sum|w| <= 1e5 * sum|w x| (int8 chunks).  These
tests pin the model to hand-computed roundings, check the bounds on inputs
of any spread, show that an input outside the precondition does break the
tolerance (so the precondition is a real term of the contract), and measure
how far inside it the workloads' inputs sit."""
import numpy as np
import pytest

import oracle
from synth import workloads as W

from . import digit_model as dm


def test_group_rounding_by_hand():
    """A group of 32 with one 1.0 and 31 values 4195 * 2^-22: the group's
    exponent is 1 (1.0 = 0.5 * 2^1), so s = 21 and each small value is
    2097.5 units of 2^-21, which rounds (ties to even) to 2098: an error of
    exactly 2^-22 per value."""
    small = np.float32(4195 * 2.0 ** -22)
    x = np.full(32, small, dtype=np.float32)
    x[5] = 1.0
    xr = dm.round_groups(x, 32)
    assert xr[5] == 1.0
    assert np.all(np.delete(xr, 5) == 4196 * 2.0 ** -22)
    # codes +7 everywhere except 0 on the 1.0: relative error 1/4195 of S
    w = np.full((1, 32), 7.0)
    w[0, 5] = 0.0
    exact = float((w @ x.astype(np.float64))[0])
    err = abs(float((w @ xr)[0]) - exact)
    assert err == 7 * 31 * 2.0 ** -22
    assert err / exact == pytest.approx(1 / 4195, rel=1e-12)
    assert err / exact > 1e-4                                   # outside the tolerance
    A = dm.group_spread(w, x, 32)[0]
    assert A == 7 * 31                                          # one group, max 1.0
    assert A / exact == pytest.approx(2.0 ** 22 / 4195, rel=1e-12)   # ~1000 > 400


def test_row_rounding_by_hand():
    """A row whose largest value is 3.0 (exponent 2): the grid is 2^(2-30);
    a value of 5.5 grid units rounds to 6 (ties to even), 6.5 to 6."""
    u = 2.0 ** -28
    x = np.array([[3.0, 5.5 * u, 6.5 * u, -5.5 * u, 0.0, 1.0]], dtype=np.float32)
    xr = dm.round_rows(x)
    assert xr[0, 0] == 3.0 and xr[0, 5] == 1.0 and xr[0, 4] == 0.0
    assert xr[0, 1] == 6 * u and xr[0, 2] == 6 * u and xr[0, 3] == -6 * u


def test_group_exponent_matches_frexp():
    for m, e in [(1.0, 1), (0.5, 0), (0.9999, 0), (2.0, 2), (3.0, 2), (0.0, 0), (2.0 ** -130, -129)]:
        assert dm.group_exponent(m) == e, m


@pytest.mark.parametrize("nv", [16, 32, 64])
@pytest.mark.parametrize("spread", [1.0, 1e2, 1e4, 1e8])
def test_group_bound_any_spread(nv, spread):
    """|model - exact| <= 2^-22 * A for any input: groups whose values span
    up to 8 decades, weights with many zero codes."""
    rng = np.random.default_rng([nv, int(np.log10(spread))])
    K, R = 1024, 64
    x = (rng.standard_normal(K) * spread ** rng.random(K)).astype(np.float32)
    x[rng.random(K) < 0.1] = 0.0
    w = rng.integers(-8, 8, size=(R, K)).astype(np.float64) * rng.uniform(1e-3, 1e-2, size=(R, 1))
    exact = w @ x.astype(np.float64)
    err = np.abs(w @ dm.round_groups(x, nv) - exact)
    A = dm.group_spread(w, x, nv)
    assert np.all(err <= 2.0 ** -22 * A * (1 + 1e-12))


@pytest.mark.parametrize("spread", [1.0, 1e3, 1e6])
def test_row_bound_any_spread(spread):
    rng = np.random.default_rng([7, int(np.log10(spread))])
    K, R = 2048, 64
    x = (rng.standard_normal((1, K)) * spread ** rng.random(K)).astype(np.float32)
    w = rng.integers(-8, 8, size=(R, K)).astype(np.float64)
    exact = w @ x[0].astype(np.float64)
    err = np.abs(w @ dm.round_rows(x)[0] - exact)
    assert np.all(err <= 2.0 ** -30 * dm.row_spread(w, x[0]) * (1 + 1e-12))


def test_row_precondition_is_needed():
    """A row with one 1.0 on zero weights and the rest at 10.5 units of its
    2^-30 grid: each rounds to 10 (ties to even), 1/21 of its value."""
    K = 256
    u = 2.0 ** -30
    x = np.full((1, K), 10.5 * u, dtype=np.float32)
    x[0, 0] = 0.75                                   # exponent 0: grid 2^-30
    w = np.ones((1, K))
    w[0, 0] = 0.0
    exact = float((w @ x[0].astype(np.float64))[0])
    err = abs(float((w @ dm.round_rows(x)[0])[0]) - exact)
    assert err / exact == pytest.approx(1 / 21, rel=1e-9)
    assert dm.row_spread(w, x[0])[0] / exact > 1e5


def _decoded_rows(orc, m, rows):
    return np.stack([orc.decode_row(m.fmt, m.data[r], 1.0 if m.scales is None else m.scales[r], m.cols)
                     for r in rows])


@pytest.mark.parametrize("key", ["c4_i4", "c3", "c0"])
def test_workloads_inside_the_precondition(key):
    """The workloads' activations sit far inside the precondition: for the
    gate rows of expert 0 against the token's x, and for the down rows
    against h = act(gate x) * (up x), the ratios A / sum|w x| stay below 40
    (bound 400) and max|x| sum|w| / sum|w x| below 1e3 (bound 1e5)."""
    orc = oracle.Oracle()
    sp = W.spec(key)
    nv = {"q8_0": 16, "i8_row": 16, "i2_row": 64}.get(sp.fmt, 32)
    ex = W.moe_expert(sp, 0)
    rows = np.arange(0, sp.F, max(1, sp.F // 128))
    Wg = _decoded_rows(orc, ex["gate"], range(sp.F))
    Wu = _decoded_rows(orc, ex["up"], range(sp.F))
    dn = np.arange(0, sp.H, max(1, sp.H // 128))
    Wd = _decoded_rows(orc, ex["down"], dn)
    for x in W.moe_x(sp, 4):
        x64 = x.astype(np.float64)
        S = np.abs(Wg[rows]) @ np.abs(x64)
        assert np.max(dm.group_spread(Wg[rows], x, nv) / S) < 40
        assert np.max(dm.row_spread(Wg[rows], x) / S) < 1e3
        h = (dm.gelu_tanh(Wg @ x64) * (Wu @ x64)).astype(np.float32)
        Sd = np.abs(Wd) @ np.abs(h.astype(np.float64))
        assert np.max(dm.group_spread(Wd, h, nv) / Sd) < 40
        assert np.max(dm.row_spread(Wd, h) / Sd) < 1e3
