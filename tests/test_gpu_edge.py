"""Edge cases on the GPU, against the oracle: every row count 1..64, the codes
and scales at the ends of each format's range (int8 code -128, fp16 scales of
0, -0, the smallest subnormal and negative values, Q4_1 minima of 0 and far
larger than the scale), guard canaries around every output buffer, a
128-token chunk whose tokens all choose one expert, and 128-token chunks
checked token by token against one-token calls."""
import numpy as np
import pytest

from synth import formats as F
from synth import workloads as W

from .gpu_common import assert_within, moe_layer, oracle_moe, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# fp16 bit patterns: +0, -0, the smallest subnormal (2^-24), a negative
# subnormal, negative normals, the largest finite (65504)
_SPECIAL_D = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0xBC00, 0xA11F, 0x7BFF], dtype=np.uint16)


def _special_matrix(rng, fmt, rows, cols):
    """Random codes over the format's whole range with scales drawn from the
    special values about a quarter of the time (the rest ~U[1e-3, 2e-2],
    either sign); int8 codes include -128."""
    nb = cols // 32
    if fmt in ("q8_0", "q4_0", "q4_1"):
        d = rng.uniform(1e-3, 2e-2, (rows, nb)) * rng.choice([-1.0, 1.0], (rows, nb))
        d = d.astype(np.float16).view(np.uint16)
        pick = rng.random((rows, nb)) < 0.25
        d[pick] = rng.choice(_SPECIAL_D[:-1], size=int(pick.sum()))   # 65504 only in the GEMV case below
        if fmt == "q8_0":
            q = rng.integers(-128, 128, (rows, cols))
            q[:, ::7] = -128
            return F.pack_q8_0(d, q)
        if fmt == "q4_0":
            return F.pack_q4_0(d, rng.integers(0, 16, (rows, cols)))
        # Q4_1: minima of 0, of either sign up to 100x the scale, and the
        # special patterns
        dd = d.view(np.float16).astype(np.float64)
        m = dd * rng.choice([0.0, -8.0, 3.0, 100.0, -100.0], (rows, nb))
        m = m.astype(np.float16).view(np.uint16)
        pm = rng.random((rows, nb)) < 0.1
        m[pm] = rng.choice(_SPECIAL_D[:-1], size=int(pm.sum()))
        return F.pack_q4_1(d, m, rng.integers(0, 16, (rows, cols)))
    s = rng.uniform(1e-3, 1e-2, rows) * rng.choice([-1.0, 1.0], rows)
    s[rng.random(rows) < 0.2] = 0.0
    s = s.astype(np.float32)
    if fmt == "i8_row":
        q = rng.integers(-128, 128, (rows, cols))
        q[:, ::5] = -128
        return F.pack_i8_row(s, q)
    if fmt == "i2_row":
        return F.pack_i2_row(s, rng.integers(-2, 2, (rows, cols)))
    return F.pack_i4_row(s, rng.integers(-8, 8, (rows, cols)))


def _upload(m):
    from moe_decode_amd.upload import upload_matrix
    return upload_matrix(m)


def _gemv(dev, x):
    import moe_decode_amd as md
    import torch
    y = md.qgemv(dev, _t(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("batch", [1, 4, 8])
def test_qgemv_every_row_count(orc_mt, fmt, batch):
    """Rows 1..64 at 256 columns (prefixes of one 64-row matrix), each its
    own call, against the oracle."""
    import moe_decode_amd as md
    rng = np.random.default_rng([101, F.FORMATS.index(fmt), batch])
    m = _special_matrix(rng, fmt, 64, 256)
    x = rng.standard_normal((batch, 256)).astype(np.float32)
    y_ref, S = orc_mt.qgemv(m, x)
    dev = _upload(m)
    say(f"[edge rows] {fmt} batch {batch}")
    for r in range(1, 65):
        view = md.DevQMatrix(dev.type, r, 256, dev.q, dev.row_scale)
        assert_within(_gemv(view, x), y_ref[:, :r], S[:, :r], f"{fmt} rows {r} batch {batch}")


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_qgemv_special_codes_and_scales(orc_mt, fmt):
    """Codes at the ends of the range and special fp16 scales (including
    65504 for the block formats) at two shapes, batches 1, 4 and 8."""
    rng = np.random.default_rng([102, F.FORMATS.index(fmt)])
    for rows, cols in ((96, 1024), (1000, 2304)):
        m = _special_matrix(rng, fmt, rows, cols)
        if fmt in ("q8_0", "q4_0", "q4_1"):   # one block scaled by the largest fp16
            off = 0
            m.data[3, off:off + 2] = np.frombuffer(np.uint16(0x7BFF).tobytes(), np.uint8)
        dev = _upload(m)
        for batch in (1, 4, 8):
            x = rng.standard_normal((batch, cols)).astype(np.float32)
            y_ref, S = orc_mt.qgemv(m, x)
            assert_within(_gemv(dev, x), y_ref, S, f"{fmt} {rows}x{cols} b{batch} special")


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("T", [1, 3, 33])
def test_ffn_special_codes_and_scales(orc_mt, fmt, T):
    """A dense gated FFN whose three matrices carry the special codes and
    scales: one-token kernels (1, 3 tokens) and grouped GEMMs (33)."""
    import moe_decode_amd as md
    import torch
    rng = np.random.default_rng([103, F.FORMATS.index(fmt), T])
    H, Fw = 768, 512
    g, u, d = (_special_matrix(rng, fmt, Fw, H), _special_matrix(rng, fmt, Fw, H), _special_matrix(rng, fmt, H, Fw))
    x = rng.standard_normal((T, H)).astype(np.float32)
    ffn = md.FFN("gelu_tanh", _upload(g), _upload(u), _upload(d))
    y = md.ffn_forward(ffn, _t(x))
    torch.cuda.synchronize()
    y_ref, S = orc_mt.ffn(g, u, d, "gelu_tanh", x)
    say(f"[edge ffn] {fmt} T={T}")
    assert_within(y.cpu().numpy(), y_ref, S, f"ffn {fmt} T={T}")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_1"])
@pytest.mark.parametrize("T", [17, 48, 100, 128])
def test_ffn_dense_chunk_token_counts(orc_mt, fmt, T):
    """A dense FFN over 17..128 tokens on the block formats (the grouped
    GEMM in dense mode: one launch tile per 16 tokens, the last one ragged),
    on matrices with special codes and scales and one token 300 times the
    others, every token against the oracle."""
    import moe_decode_amd as md
    import torch
    rng = np.random.default_rng([104, ("q8_0", "q4_0", "q4_1").index(fmt), T])
    H, Fw = 1024, 768
    g, u, d = (_special_matrix(rng, fmt, Fw, H), _special_matrix(rng, fmt, Fw, H), _special_matrix(rng, fmt, H, Fw))
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[T // 2] *= 300.0   # one token far larger than the others
    ffn = md.FFN("silu", _upload(g), _upload(u), _upload(d))
    y = md.ffn_forward(ffn, _t(x))
    torch.cuda.synchronize()
    y_ref, S = orc_mt.ffn(g, u, d, "silu", x)
    say(f"[edge dense chunk] {fmt} T={T}")
    assert_within(y.cpu().numpy(), y_ref, S, f"dense chunk {fmt} T={T}")


# ---- canaries ---------------------------------------------------------------

_GUARD = 256  # elements (1 KiB) of guard on each side


def _guarded(n, dtype, fill):
    import torch
    buf = torch.empty(n + 2 * _GUARD, dtype=dtype, device="cuda")
    buf.view(torch.int32).fill_(fill)
    return buf, buf[_GUARD:_GUARD + n]


def _guards_intact(buf, fill):
    import torch
    torch.cuda.synchronize()
    g = buf.view(torch.int32)
    return bool(torch.all(g[:_GUARD] == fill)) and bool(torch.all(g[-_GUARD:] == fill))


@pytest.mark.parametrize("key,T", [("c0", 1), ("c3", 1), ("c3", 4), ("c4_i4", 1), ("c4_i4", 8), ("c3", 128),
                                   ("c4_i8", 33)])
def test_layer_outputs_stay_inside_their_buffers(orc_mt, key, T):
    """y, idx and gates placed between guard regions filled with a pattern:
    the layer writes every element of its outputs (checked against the
    oracle) and nothing around them."""
    import moe_decode_amd as md
    sp = W.spec(key)
    layer = moe_layer(key)
    x = W.moe_x(sp, T)
    pat = 0x7FC0DEAD  # a NaN pattern for the fp32 buffers
    ybuf, y = _guarded(T * sp.H, __import__("torch").float32, pat)
    ibuf, idx = _guarded(T * sp.k, __import__("torch").int32, pat)
    gbuf, gates = _guarded(T * sp.k, __import__("torch").float32, pat)
    say(f"[canary] {key} T={T}")
    md.moe_layer_forward(layer, _t(x), y=y.view(T, sp.H), idx=idx.view(T, sp.k), gates=gates.view(T, sp.k))
    assert _guards_intact(ybuf, pat) and _guards_intact(ibuf, pat) and _guards_intact(gbuf, pat)
    y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x)
    assert np.array_equal(idx.view(T, sp.k).cpu().numpy(), i_ref)
    assert np.max(np.abs(gates.view(T, sp.k).cpu().numpy() - g_ref)) <= 1e-6
    assert_within(y.view(T, sp.H).cpu().numpy(), y_ref, S, f"{key} T={T} canary")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "i4_row", "i2_row"])
@pytest.mark.parametrize("batch", [1, 8])
def test_qgemv_output_stays_inside_its_buffer(orc_mt, fmt, batch):
    import moe_decode_amd as md
    import torch
    rng = np.random.default_rng([104, batch])
    rows, cols = 1000, 2048
    m = _special_matrix(rng, fmt, rows, cols)
    x = rng.standard_normal((batch, cols)).astype(np.float32)
    pat = 0x7FC0BEEF
    ybuf, y = _guarded(batch * rows, torch.float32, pat)
    md.qgemv(_upload(m), _t(x), y=y.view(batch, rows))
    assert _guards_intact(ybuf, pat)
    y_ref, S = orc_mt.qgemv(m, x)
    assert_within(y.view(batch, rows).cpu().numpy(), y_ref, S, f"{fmt} b{batch} canary")


# ---- routing extremes and chunk = token-by-token ------------------------------

@pytest.mark.parametrize("key", ["c3", "c4_i4"])
def test_chunk_with_one_expert_for_every_token(orc_mt, key):
    """A bias of +1000 on one expert: all 128 tokens choose it first (its
    16-token tiles run eight times over the same expert), the other slots
    follow the router; every token checked against the oracle."""
    import moe_decode_amd as md
    import torch
    sp = W.spec(key)
    base = moe_layer(key)
    Wr, b = W.moe_router(sp)
    hot = 17 if key == "c3" else 200
    b2 = np.zeros(sp.E, np.float32) if b is None else b.copy()
    b2[hot] += 1000.0
    layer = md.MoELayer(sp.H, sp.F, sp.E, sp.k, sp.act, base.gate, base.up, base.down, base.Wr, _t(b2), base.shared)
    T = 128
    x = W.moe_x(sp, T)
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, dtype=torch.float32, device="cuda")
    say(f"[hot expert] {key}")
    y = md.moe_layer_forward(layer, _t(x), idx=idx, gates=gates)
    torch.cuda.synchronize()
    i_ref, g_ref, _, _ = orc_mt.route_topk(x, Wr, b2, sp.k)
    assert np.all(i_ref[:, 0] == hot)
    assert np.array_equal(idx.cpu().numpy(), i_ref)
    assert np.max(np.abs(gates.cpu().numpy() - g_ref)) <= 1e-6
    experts = {int(e): W.moe_expert(sp, int(e)) for e in np.unique(i_ref)}
    y_ref, _, _, S = orc_mt.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b2, experts, W.moe_shared(sp), x)
    assert_within(y.cpu().numpy(), y_ref, S, f"{key} hot expert")


def test_c3_chunk_equals_128_decode_calls(orc_mt):
    """The 128-token chunk (grouped GEMMs) and 128 one-token calls give the
    same expert indices and gates for every token, and both meet the bound
    against the oracle on every token."""
    import moe_decode_amd as md
    import torch
    sp = W.spec("c3")
    layer = moe_layer("c3")
    x = W.moe_x(sp, 128)
    y_c, i_c, g_c = (a.cpu().numpy() for a in _layer(md, layer, sp, x))
    y_1 = np.empty_like(y_c)
    i_1 = np.empty_like(i_c)
    g_1 = np.empty_like(g_c)
    for t in range(128):
        yt, it, gt = _layer(md, layer, sp, x[t:t + 1])
        y_1[t], i_1[t], g_1[t] = yt.cpu().numpy()[0], it.cpu().numpy()[0], gt.cpu().numpy()[0]
    torch.cuda.synchronize()
    assert np.array_equal(i_c, i_1)
    assert np.array_equal(g_c, g_1)
    y_ref, i_ref, g_ref, S = oracle_moe(orc_mt, sp, x)
    assert np.array_equal(i_c, i_ref)
    assert_within(y_c, y_ref, S, "c3 chunk")
    assert_within(y_1, y_ref, S, "c3 one token at a time")


def _layer(md, layer, sp, x):
    import torch
    T = x.shape[0]
    idx = torch.empty(T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, dtype=torch.float32, device="cuda")
    y = md.moe_layer_forward(layer, _t(x), idx=idx, gates=gates)
    return y, idx, gates
