"""A numpy model of how the library's integer paths round their activations
(test infrastructure).

The oracle stays the exact definition of the layer; this module models the
one rounding that the library's integer arithmetic adds, so that tests can
state and check the library's accuracy contract:

* one-token kernels (up to 8 tokens, 16 on small layers): the activations a
  16-byte weight chunk multiplies (a group of ``nv`` consecutive values: 32
  for Q4_0 / Q4_1 / packed int4, 16 for Q8_0 / int8, 64 for packed int2) are
  scaled by 2^s, s = 22 - e (e the binary exponent of the group's largest
  magnitude m, m = f * 2^e with f in [0.5, 1); s at most 120), and rounded to
  the nearest integer, ties to even;
* grouped GEMMs on the int8 matrix cores (chunks of the per-row formats):
  each activation row is scaled by 2^(30 - E), E the binary exponent of the
  row's largest magnitude, and rounded the same way.

Everything else in those paths is exact integer arithmetic or fp32 rounding
of the final combines.  The bounds below follow from the rounding: a value
moves by at most half a unit of its grid, 2^(-s-1) <= 2^-22 * m per value for
the groups and 2^(E-31) <= 2^-30 * max|row| for the rows.
"""
import numpy as np


def group_exponent(m):
    """e with m = f * 2^e, f in [0.5, 1) (0 for m == 0), as C's frexp."""
    return np.frexp(np.asarray(m, dtype=np.float64))[1].astype(np.int64)


def round_groups(x, nv, bits=22, cap=120):
    """x (..., K) rounded as the one-token kernels' digit planes hold it."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    shp = x.shape
    g = x.reshape(-1, nv)
    s = np.minimum(bits - group_exponent(np.abs(g).max(axis=1)), cap)
    X = np.rint(np.ldexp(g, s[:, None]))
    return np.ldexp(X, -s[:, None]).reshape(shp)


def round_rows(x, bits=30):
    """x (R, K) rounded as the int8 matrix-core path's activation digits hold it."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    E = group_exponent(np.abs(x).max(axis=-1))
    X = np.rint(np.ldexp(x, (bits - E)[..., None]))
    return np.ldexp(X, (E - bits)[..., None])


def group_spread(w, x, nv):
    """A[r] = sum over groups g of max_{c in g} |x_c| * sum_{c in g} |w[r, c]|
    (the weight of the one-token paths' rounding term)."""
    w = np.abs(np.asarray(w, dtype=np.float64))
    m = np.abs(np.asarray(x, dtype=np.float64)).reshape(-1, nv).max(axis=1)
    return (w.reshape(w.shape[0], -1, nv).sum(axis=2) * m[None, :]).sum(axis=1)


def row_spread(w, x):
    """max|x| * sum_c |w[r, c]| (the weight of the row path's rounding term)."""
    return np.abs(np.asarray(x, dtype=np.float64)).max() * np.abs(np.asarray(w, dtype=np.float64)).sum(axis=1)


def gelu_tanh(z):
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def silu(z):
    return z / (1.0 + np.exp(-z))


def ffn_one_token(Wg, Wu, Wd, x, nv, act="gelu_tanh"):
    """The dense gated FFN of one token with the one-token kernels' roundings
    of x and of h, every contraction exact (float64): what the kernels compute
    up to fp32 rounding of their combines."""
    f = gelu_tanh if act == "gelu_tanh" else silu
    xr = round_groups(x, nv)
    h = f(Wg @ xr) * (Wu @ xr)
    return Wd @ round_groups(h.astype(np.float32), nv)
