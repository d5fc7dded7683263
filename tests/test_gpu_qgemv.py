"""GPU parity of md_qgemv against the oracle: every format, ragged and
multi-tile shapes, batches 1..8, fp32 and bf16 activations, the dense
workloads at full size, and closed forms that must hold bitwise."""
import numpy as np
import pytest

from synth import formats as F
from synth import workloads as W

from .gpu_common import assert_within, dense_matrix, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _random_qmatrix(rng, fmt, rows, cols):
    if fmt == "q8_0":
        return F.pack_q8_0(rng.uniform(1e-3, 1e-2, (rows, cols // 32)).astype(np.float16),
                           rng.integers(-127, 128, (rows, cols)))
    if fmt == "q4_0":
        return F.pack_q4_0(rng.uniform(1e-3, 2e-2, (rows, cols // 32)).astype(np.float16),
                           rng.integers(0, 16, (rows, cols)))
    if fmt == "q4_1":
        d = rng.uniform(1e-3, 2e-2, (rows, cols // 32)).astype(np.float16)
        mn = (-d.astype(np.float64) * rng.uniform(6.0, 10.0, (rows, cols // 32))).astype(np.float16)
        return F.pack_q4_1(d, mn, rng.integers(0, 16, (rows, cols)))
    s = rng.uniform(1e-3, 1e-2, rows).astype(np.float32)
    if fmt == "i8_row":
        return F.pack_i8_row(s, rng.integers(-127, 128, (rows, cols)))
    if fmt == "i2_row":
        return F.pack_i2_row(s, rng.integers(-2, 2, (rows, cols)))
    assert fmt == "i4_row"
    return F.pack_i4_row(s, rng.integers(-8, 8, (rows, cols)))


def _run(m, x_np):
    import moe_decode_amd as md
    from moe_decode_amd.upload import upload_matrix
    from synth.device import x_tensor
    import torch
    W_d = upload_matrix(m)
    y = md.qgemv(W_d, x_tensor(x_np))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("rows,cols", [(7, 256), (33, 512), (300, 768), (129, 2048), (64, 5632)])
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_qgemv_random(orc_mt, fmt, rows, cols, batch):
    say(f"[qgemv] {fmt} {rows}x{cols} batch {batch}")
    rng = np.random.default_rng([F.FORMATS.index(fmt), rows, cols, batch])
    m = _random_qmatrix(rng, fmt, rows, cols)
    x = rng.standard_normal((batch, cols)).astype(np.float32)
    y_ref, S = orc_mt.qgemv(m, x)
    assert_within(_run(m, x), y_ref, S, f"{fmt} {rows}x{cols} b{batch}")


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("batch", [1, 8])
def test_qgemv_bf16(orc_mt, fmt, batch):
    rng = np.random.default_rng([9, F.FORMATS.index(fmt), batch])
    m = _random_qmatrix(rng, fmt, 96, 1024)
    xb = F.f32_to_bf16_bits(rng.standard_normal((batch, 1024)))
    y_ref, S = orc_mt.qgemv(m, xb, "bf16")
    assert_within(_run(m, xb), y_ref, S, f"bf16 {fmt}")


@pytest.mark.parametrize("name", ["gate", "up", "down", "q", "o", "k", "v"])
def test_dense_q8_0_llama_shapes(orc_mt, name):
    import moe_decode_amd as md
    import torch
    from synth.device import x_tensor
    sp = W.spec("c1")
    say(f"[c1] {name}")
    m = W.dense_matrix(sp, name)
    x = W.dense_x(sp, m.cols, 1)
    y_ref, S = orc_mt.qgemv(m, x)
    y = md.qgemv(dense_matrix("c1", name), x_tensor(x))
    torch.cuda.synchronize()
    assert_within(y.cpu().numpy(), y_ref, S, f"c1 {name}")


def test_dense_swiglu_ffn(orc_mt):
    import moe_decode_amd as md
    import torch
    sp = W.spec("c1")
    g, u, d = (W.dense_matrix(sp, n) for n in ("gate", "up", "down"))
    x = W.dense_x(sp, 2048, 1)
    y_ref, S = orc_mt.ffn(g, u, d, "silu", x)
    ffn = md.FFN("silu", dense_matrix("c1", "gate"), dense_matrix("c1", "up"), dense_matrix("c1", "down"))
    y = md.ffn_forward(ffn, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert_within(y.cpu().numpy(), y_ref, S, "c1 SwiGLU FFN")


@pytest.mark.parametrize("name", ["w_10240x2560", "w_2560x10240"])
@pytest.mark.parametrize("batch", [1, 8])
def test_dense_q4_0_bf16(orc_mt, name, batch):
    import moe_decode_amd as md
    import torch
    from synth.device import x_tensor
    sp = W.spec("c2")
    say(f"[c2] {name} batch {batch}")
    m = W.dense_matrix(sp, name)
    x = W.dense_x(sp, m.cols, batch)
    y_ref, S = orc_mt.qgemv(m, x, "bf16")
    y = md.qgemv(dense_matrix("c2", name), x_tensor(x))
    torch.cuda.synchronize()
    assert_within(y.cpu().numpy(), y_ref, S, f"c2 {name} b{batch}")


@pytest.mark.parametrize("key,name,batch", [("q41", "w_10240x2560", 1), ("q41", "w_10240x2560", 8),
                                            ("q41", "w_2560x10240", 1), ("q41", "w_2560x10240", 8),
                                            ("i2", "gate_2048x6144", 1), ("i2", "gate_2048x6144", 4),
                                            ("i2", "down_6144x2048", 1), ("i2", "down_6144x2048", 4)])
def test_dense_more_codecs(orc_mt, key, name, batch):
    """The Q4_1 and packed-int2 dense workloads at full size."""
    import moe_decode_amd as md
    import torch
    from synth.device import x_tensor
    sp = W.spec(key)
    say(f"[{key}] {name} batch {batch}")
    m = W.dense_matrix(sp, name)
    x = W.dense_x(sp, m.cols, batch)
    y_ref, S = orc_mt.qgemv(m, x, sp.x_dtype)
    y = md.qgemv(dense_matrix(key, name), x_tensor(x))
    torch.cuda.synchronize()
    assert_within(y.cpu().numpy(), y_ref, S, f"{key} {name} b{batch}")


def test_q4_0_code_eight_is_exact_zero():
    rng = np.random.default_rng(31)
    m = F.pack_q4_0(rng.uniform(1e-3, 2e-2, (70, 16)).astype(np.float16), np.full((70, 512), 8))
    y = _run(m, rng.standard_normal((2, 512)).astype(np.float32))
    assert np.all(y == 0.0)


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_one_hot_x_is_bitwise_one_weight(orc, fmt):
    rng = np.random.default_rng([32, F.FORMATS.index(fmt)])
    m = _random_qmatrix(rng, fmt, 40, 512)
    for c in (0, 31, 300, 511):
        x = np.zeros((1, 512), dtype=np.float32)
        x[0, c] = 1.0
        y_ref, _ = orc.qgemv(m, x)
        assert np.array_equal(_run(m, x), y_ref), (fmt, c)


def _split_matrix():
    """A short, wide matrix (64 x 5632 Q8_0) that md_qgemv splits over K."""
    import moe_decode_amd as md
    from moe_decode_amd.upload import upload_matrix
    m = upload_matrix(_random_qmatrix(np.random.default_rng(77), "q8_0", 64, 5632))
    assert md.qgemv_workspace_size(m, 1) > 0, "expected the split-K path"
    return m


def test_deterministic_repeat():
    import moe_decode_amd as md
    import torch
    from synth.device import x_tensor
    sp = W.spec("c1")
    for m in (dense_matrix("c1", "k"), _split_matrix()):
        x = x_tensor(W.dense_x(sp, m.cols, 1))
        a = md.qgemv(m, x)
        b = md.qgemv(m, x)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("T", [9, 32, 128])
def test_dense_swiglu_ffn_chunk(orc_mt, T):
    """A chunk of tokens through the dense FFN (grouped GEMM on the matrix cores)."""
    import moe_decode_amd as md
    import torch
    sp = W.spec("c1")
    g, u, d = (W.dense_matrix(sp, n) for n in ("gate", "up", "down"))
    x = np.concatenate([W.dense_x(sp, 2048, 1, salt=s) for s in range(T)])
    y_ref, S = orc_mt.ffn(g, u, d, "silu", x)
    ffn = md.FFN("silu", dense_matrix("c1", "gate"), dense_matrix("c1", "up"), dense_matrix("c1", "down"))
    y = md.ffn_forward(ffn, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert_within(y.cpu().numpy(), y_ref, S, f"c1 SwiGLU FFN T={T}")


def test_qgemv_graph_replays_match_eager():
    """qgemv calls captured in a HIP graph (the plain kernel and the split-K
    kernel with its reduce), replayed several times with eager work and
    synchronisations in between: every replay equals the eager result."""
    import moe_decode_amd as md
    import torch
    from synth.device import x_tensor
    sp = W.spec("c1")
    mats = [dense_matrix("c1", "gate"), _split_matrix()]
    xs = [x_tensor(W.dense_x(sp, m.cols, 1, salt=3)) for m in mats]
    wss = [torch.empty(max(md.qgemv_workspace_size(m, 1), 1), dtype=torch.uint8, device="cuda") for m in mats]
    eager = [md.qgemv(m, x, workspace=w).clone() for m, x, w in zip(mats, xs, wss)]
    ys = [torch.zeros_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for m, x, y, w in zip(mats, xs, ys, wss):
                md.qgemv(m, x, y=y, workspace=w)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y, e), f"replay {rep}"


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("batch", [1, 8])
def test_qgemv_widest_rows(orc_mt, fmt, batch):
    """The widest rows the library takes (16384 columns)."""
    rng = np.random.default_rng([31, F.FORMATS.index(fmt), batch])
    m = _random_qmatrix(rng, fmt, 48, 16384)
    x = rng.standard_normal((batch, 16384)).astype(np.float32)
    y_ref, S = orc_mt.qgemv(m, x)
    assert_within(_run(m, x), y_ref, S, f"{fmt} 48x16384 b{batch}")


@pytest.mark.parametrize("fmt", ["q4_0", "i8_row", "q4_1", "i2_row"])
def test_qgemv_most_rows(orc_mt, fmt):
    """The most rows the library takes (65536); every 97th row is compared."""
    rng = np.random.default_rng([32, F.FORMATS.index(fmt)])
    m = _random_qmatrix(rng, fmt, 65536, 256)
    x = rng.standard_normal((2, 256)).astype(np.float32)
    y = _run(m, x)
    rows = np.arange(0, 65536, 97)
    sub = F.QMatrix(fmt=m.fmt, rows=len(rows), cols=m.cols, data=np.ascontiguousarray(m.data[rows]),
                    scales=None if m.scales is None else np.ascontiguousarray(m.scales[rows]))
    y_ref, S = orc_mt.qgemv(sub, x)
    assert_within(y[:, rows], y_ref, S, f"{fmt} 65536x256 sampled rows")
