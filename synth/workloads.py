"""The synthetic workloads and their seeded generators.

Every tensor is drawn from its own numpy PCG64 stream seeded with
``[workload index, tensor tag, expert, variant]`` (``numpy.random.default_rng``
of that list), so any single expert can be regenerated on its own and both the
oracle and the GPU path see the same bytes.  Inside one tensor the scales are
drawn first, then the quantized codes.

Workloads (shapes and value ranges of the pages' models; the weights are
random, not trained):

``c0``     tiny MoE layer: hidden 256, 8 experts, top-2, expert FFN 512, GeGLU,
           Q8_0 experts, fp32 router ~N(0, 0.05), one token.
``c1``     dense Q8_0 decode GEMVs of a 1.1B-Llama-shaped block (the TinyLlama
           Q8_0 row of the Camelid README): gate/up 5632x2048, down 2048x5632,
           q/o 2048x2048, k/v 256x2048, SwiGLU FFN, batch 1.
``c2``     dense Q4_0 GEMVs 10240x2560 and 2560x10240, bf16 activations,
           batch 1 and 8 (the Q4_0 projection GEMVs of the Gemma 4 QAT rows).
``c3``     128 experts, top-8, hidden 2048, expert FFN 768 in Q4_0, dense
           shared expert (FFN 2048, Q8_0), router with a per-expert bias
           ~N(0, 1); one token and a 128-token chunk (the 26B-A4B block of the
           TurboFieldfare summary, "memory and expert streaming").
``c4_i4``  256 experts, top-8, hidden 6144, expert FFN 2048, packed int4 with
           a per-row fp32 scale (about 18.9 MB per expert, the colibri
           summary's expert size); 1, 4 and 128 tokens.
``c4_i8``  the same layer with int8 per-row weights.
``c4_i2``  the same layer with packed int2 per-row weights (the colibri
           summary's third expert format); its own router seed (variant 2).
``c4_q41`` the same layer with Q4_1 block experts (d ~ the Q4_0 range, block
           minimum m = -d * U[6, 10]); its own router seed (variant 3).
``q41``    dense Q4_1 GEMVs at the ``c2`` shapes and activations (bf16), batch
           1 and 8; block minimum m = -d * U[6, 10] (rounded to fp16).
``i2``     dense packed-int2 per-row GEMVs at the ``c4`` expert shapes
           (2048x6144 and 6144x2048), fp32 activations, batch 1 and 4.
"""

from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .formats import QMatrix, ROW_FORMATS, pack_q8_0, pack_i8_row, row_bytes, f32_to_bf16_bits

# tensor tags (part of every seed)
TAG_ROUTER, TAG_BIAS, TAG_GATE, TAG_UP, TAG_DOWN = 1, 2, 3, 4, 5
TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN, TAG_X = 6, 7, 8, 9
TAG_DENSE0 = 20

Q8_D = (1e-3, 1e-2)
Q4_D = (1e-3, 2e-2)
ROW_S = (1e-3, 1e-2)


@dataclass(frozen=True)
class MoESpec:
    key: str
    index: int                  # workload index (first seed word)
    H: int
    F: int
    E: int
    k: int
    act: str                    # "gelu_tanh" or "silu"
    fmt: str                    # expert weight format
    d_range: Tuple[float, float]
    router_std: float
    bias_std: Optional[float]
    tokens: Tuple[int, ...]     # token counts to run
    variant: int = 0            # fourth seed word (c4 int4 vs int8)
    shared_F: int = 0           # 0: no shared expert
    shared_fmt: Optional[str] = None
    shared_d_range: Optional[Tuple[float, float]] = None

    @property
    def kind(self):
        return "moe"

    def expert_bytes(self) -> int:
        from .formats import matrix_bytes
        return (2 * matrix_bytes(self.fmt, self.F, self.H)
                + matrix_bytes(self.fmt, self.H, self.F))

    def router_bytes(self) -> int:
        return 4 * self.E * self.H + (4 * self.E if self.bias_std is not None else 0)

    def shared_bytes(self) -> int:
        from .formats import matrix_bytes
        if not self.shared_F:
            return 0
        return (2 * matrix_bytes(self.shared_fmt, self.shared_F, self.H)
                + matrix_bytes(self.shared_fmt, self.H, self.shared_F))


@dataclass(frozen=True)
class DenseSpec:
    key: str
    index: int
    fmt: str
    d_range: Tuple[float, float]
    matrices: Tuple[Tuple[str, int, int], ...]     # (name, rows, cols)
    x_dtype: str                                    # "f32" or "bf16"
    batches: Tuple[int, ...]
    ffn: Optional[Tuple[str, str, str, str]] = None  # (gate, up, down, act)

    @property
    def kind(self):
        return "dense"

    def shape(self, name):
        for n, r, c in self.matrices:
            if n == name:
                return r, c
        raise KeyError(name)


SPECS: Dict[str, object] = {
    "c0": MoESpec("c0", 0, H=256, F=512, E=8, k=2, act="gelu_tanh", fmt="q8_0",
                  d_range=Q8_D, router_std=0.05, bias_std=None, tokens=(1,)),
    "c1": DenseSpec("c1", 1, "q8_0", Q8_D,
                    (("gate", 5632, 2048), ("up", 5632, 2048), ("down", 2048, 5632),
                     ("q", 2048, 2048), ("o", 2048, 2048), ("k", 256, 2048), ("v", 256, 2048)),
                    x_dtype="f32", batches=(1,), ffn=("gate", "up", "down", "silu")),
    "c2": DenseSpec("c2", 2, "q4_0", Q4_D,
                    (("w_10240x2560", 10240, 2560), ("w_2560x10240", 2560, 10240)),
                    x_dtype="bf16", batches=(1, 8)),
    "c3": MoESpec("c3", 3, H=2048, F=768, E=128, k=8, act="gelu_tanh", fmt="q4_0",
                  d_range=Q4_D, router_std=0.05, bias_std=1.0, tokens=(1, 128),
                  shared_F=2048, shared_fmt="q8_0", shared_d_range=Q8_D),
    "c4_i4": MoESpec("c4_i4", 4, H=6144, F=2048, E=256, k=8, act="gelu_tanh", fmt="i4_row",
                     d_range=ROW_S, router_std=0.05, bias_std=None, tokens=(1, 4, 128), variant=0),
    "c4_i8": MoESpec("c4_i8", 4, H=6144, F=2048, E=256, k=8, act="gelu_tanh", fmt="i8_row",
                     d_range=ROW_S, router_std=0.05, bias_std=None, tokens=(1, 4, 128), variant=1),
    # the 256-expert layer once more with packed int2 per-row experts
    "c4_i2": MoESpec("c4_i2", 4, H=6144, F=2048, E=256, k=8, act="gelu_tanh", fmt="i2_row",
                     d_range=ROW_S, router_std=0.05, bias_std=None, tokens=(1, 4, 128), variant=2),
    # and with Q4_1 block experts (23.6 MB per expert)
    "c4_q41": MoESpec("c4_q41", 4, H=6144, F=2048, E=256, k=8, act="gelu_tanh", fmt="q4_1",
                      d_range=Q4_D, router_std=0.05, bias_std=None, tokens=(1, 4, 128), variant=3),
    # the two further codecs, on dense GEMVs: Q4_1 at the Q4_0 workload's
    # shapes, packed int2 per-row at the 256-expert layer's expert shapes
    "q41": DenseSpec("q41", 5, "q4_1", Q4_D,
                     (("w_10240x2560", 10240, 2560), ("w_2560x10240", 2560, 10240)),
                     x_dtype="bf16", batches=(1, 8)),
    "i2": DenseSpec("i2", 6, "i2_row", ROW_S,
                    (("gate_2048x6144", 2048, 6144), ("down_6144x2048", 6144, 2048)),
                    x_dtype="f32", batches=(1, 4)),
}


def spec(key: str):
    return SPECS[key]


def _rng(index, tag, a=0, b=0):
    return np.random.default_rng([index, tag, a, b])


def _uniform_bytes(rng, n):
    """n independent uniform bytes (raw 64-bit PCG64 outputs, little-endian)."""
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n].copy()


def _int8_symmetric(rng, n):
    """n independent int8 values uniform on [-127, 127]: uniform bytes with
    every 0x80 (-128) redrawn until none is left (rejection sampling)."""
    b = _uniform_bytes(rng, n)
    bad = np.flatnonzero(b == 0x80)
    while bad.size:
        b[bad] = _uniform_bytes(rng, bad.size)
        bad = bad[b[bad] == 0x80]
    return b.view(np.int8)


def _gen_qmatrix(fmt, rows, cols, rng, d_range) -> QMatrix:
    lo, hi = d_range
    if fmt == "q8_0":
        d = rng.uniform(lo, hi, (rows, cols // 32)).astype(np.float16)
        q = _int8_symmetric(rng, rows * cols).reshape(rows, cols)
        return pack_q8_0(d, q)
    if fmt == "q4_0":
        nb = cols // 32
        d = rng.uniform(lo, hi, (rows, nb)).astype(np.float16).view(np.uint16)
        # a uniform random byte is two independent uniform nibbles 0..15
        qs = _uniform_bytes(rng, rows * nb * 16).reshape(rows, nb, 16)
        out = np.empty((rows, nb, 18), dtype=np.uint8)
        out[:, :, 0] = (d & 0xFF).astype(np.uint8)
        out[:, :, 1] = (d >> 8).astype(np.uint8)
        out[:, :, 2:] = qs
        return QMatrix("q4_0", rows, cols, out.reshape(rows, nb * 18))
    if fmt == "i8_row":
        s = rng.uniform(lo, hi, rows).astype(np.float32)
        q = _int8_symmetric(rng, rows * cols).reshape(rows, cols)
        return pack_i8_row(s, q)
    if fmt == "i4_row":
        s = rng.uniform(lo, hi, rows).astype(np.float32)
        # two independent uniform signed nibbles per byte == a uniform byte
        data = _uniform_bytes(rng, rows * cols // 2).reshape(rows, cols // 2)
        return QMatrix("i4_row", rows, cols, data, s)
    if fmt == "q4_1":
        nb = cols // 32
        d = rng.uniform(lo, hi, (rows, nb)).astype(np.float16)
        # the block minimum sits 6..10 steps below zero, so values span both signs
        m = (-d.astype(np.float64) * rng.uniform(6.0, 10.0, (rows, nb))).astype(np.float16)
        qs = _uniform_bytes(rng, rows * nb * 16).reshape(rows, nb, 16)
        d, m = d.view(np.uint16), m.view(np.uint16)
        out = np.empty((rows, nb, 20), dtype=np.uint8)
        out[:, :, 0] = (d & 0xFF).astype(np.uint8)
        out[:, :, 1] = (d >> 8).astype(np.uint8)
        out[:, :, 2] = (m & 0xFF).astype(np.uint8)
        out[:, :, 3] = (m >> 8).astype(np.uint8)
        out[:, :, 4:] = qs
        return QMatrix("q4_1", rows, cols, out.reshape(rows, nb * 20))
    if fmt == "i2_row":
        s = rng.uniform(lo, hi, rows).astype(np.float32)
        # four independent uniform 2-bit codes per byte == a uniform byte
        data = _uniform_bytes(rng, rows * cols // 4).reshape(rows, cols // 4)
        return QMatrix("i2_row", rows, cols, data, s)
    raise ValueError(fmt)


# ---------------------------------------------------------------- MoE layers

def moe_router(sp: MoESpec):
    """Router weights W_r (E x H fp32) and the per-expert bias (or None)."""
    W = _rng(sp.index, TAG_ROUTER, 0, sp.variant).normal(0.0, sp.router_std, (sp.E, sp.H))
    W = W.astype(np.float32)
    b = None
    if sp.bias_std is not None:
        b = _rng(sp.index, TAG_BIAS, 0, sp.variant).normal(0.0, sp.bias_std, sp.E).astype(np.float32)
    return W, b


def moe_expert(sp: MoESpec, e: int) -> Dict[str, QMatrix]:
    """Expert e's gate (F x H), up (F x H) and down (H x F) matrices."""
    if not 0 <= e < sp.E:
        raise IndexError(e)
    return {
        "gate": _gen_qmatrix(sp.fmt, sp.F, sp.H, _rng(sp.index, TAG_GATE, e, sp.variant), sp.d_range),
        "up": _gen_qmatrix(sp.fmt, sp.F, sp.H, _rng(sp.index, TAG_UP, e, sp.variant), sp.d_range),
        "down": _gen_qmatrix(sp.fmt, sp.H, sp.F, _rng(sp.index, TAG_DOWN, e, sp.variant), sp.d_range),
    }


def moe_expert_part(sp: MoESpec, e: int, part: str) -> QMatrix:
    tag = {"gate": TAG_GATE, "up": TAG_UP, "down": TAG_DOWN}[part]
    rows, cols = (sp.H, sp.F) if part == "down" else (sp.F, sp.H)
    return _gen_qmatrix(sp.fmt, rows, cols, _rng(sp.index, tag, e, sp.variant), sp.d_range)


def moe_expert_stack(sp: MoESpec, part: str, experts: Optional[Sequence[int]] = None,
                     out: Optional[np.ndarray] = None, out_scales: Optional[np.ndarray] = None):
    """One part ("gate", "up" or "down") of several experts stacked expert-major:
    returns (data uint8 [n, rows, row_bytes], scales float32 [n, rows] or None)."""
    experts = range(sp.E) if experts is None else experts
    rows, cols = (sp.H, sp.F) if part == "down" else (sp.F, sp.H)
    rb = row_bytes(sp.fmt, cols)
    n = len(experts)
    if out is None:
        out = np.empty((n, rows, rb), dtype=np.uint8)
    per_row = sp.fmt in ROW_FORMATS
    if per_row and out_scales is None:
        out_scales = np.empty((n, rows), dtype=np.float32)
    for i, e in enumerate(experts):
        m = moe_expert_part(sp, e, part)
        out[i] = m.data
        if per_row:
            out_scales[i] = m.scales
    return out, (out_scales if per_row else None)


def moe_shared(sp: MoESpec) -> Optional[Dict[str, QMatrix]]:
    """The dense shared expert's gate/up (F_s x H) and down (H x F_s), or None."""
    if not sp.shared_F:
        return None
    Fs, fmt, dr = sp.shared_F, sp.shared_fmt, sp.shared_d_range
    return {
        "gate": _gen_qmatrix(fmt, Fs, sp.H, _rng(sp.index, TAG_SH_GATE, 0, sp.variant), dr),
        "up": _gen_qmatrix(fmt, Fs, sp.H, _rng(sp.index, TAG_SH_UP, 0, sp.variant), dr),
        "down": _gen_qmatrix(fmt, sp.H, Fs, _rng(sp.index, TAG_SH_DOWN, 0, sp.variant), dr),
    }


def moe_x(sp: MoESpec, T: int) -> np.ndarray:
    """T tokens of layer input, fp32 ~N(0, 1), shape (T, H)."""
    return _rng(sp.index, TAG_X, T, sp.variant).standard_normal((T, sp.H)).astype(np.float32)


# ---------------------------------------------------------------- dense GEMVs

def dense_matrix(sp: DenseSpec, name: str) -> QMatrix:
    names = [m[0] for m in sp.matrices]
    rows, cols = sp.shape(name)
    return _gen_qmatrix(sp.fmt, rows, cols, _rng(sp.index, TAG_DENSE0 + names.index(name)), sp.d_range)


def dense_x(sp: DenseSpec, cols: int, batch: int, salt: int = 0) -> np.ndarray:
    """Activations for a dense GEMV: (batch, cols) fp32, or bf16 bit patterns
    (uint16) when the workload's activations are bf16."""
    x = _rng(sp.index, TAG_X, cols * 16 + batch, salt).standard_normal((batch, cols)).astype(np.float32)
    if sp.x_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x
