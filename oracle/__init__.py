"""ctypes front end of the plain CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the GPU library and its binding never do.

Matrices are passed as any object with ``fmt``, ``rows``, ``cols``, ``data``
(uint8, canonical layout) and ``scales`` (float32 per row, or None).
"""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MD_SANITIZE=1: the AddressSanitizer + UndefinedBehaviorSanitizer build
# (build(sanitize=True); the process must preload the clang ASan runtime)
SANITIZE = os.environ.get("MD_SANITIZE") == "1"
LIB = os.path.join(HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
SRC = os.path.join(HERE, "oracle.c")
CLANG = "/opt/rocm/llvm/bin/clang"

FMT = {"q8_0": 1, "q4_0": 2, "i8_row": 3, "i4_row": 4, "q4_1": 5, "i2_row": 6}
ACT = {"gelu_tanh": 0, "silu": 1}
XT = {"f32": 0, "bf16": 1}
ERR = {0: "ok", 1: "invalid argument", 2: "non-finite logit", 3: "selected expert not supplied"}


def build(force=True, sanitize=False):
    """Compile the oracle with gcc: plain C, no fast-math, no FMA contraction.
    sanitize: a single-threaded AddressSanitizer + UndefinedBehaviorSanitizer
    build with clang (liboracle_san.so; any undefined behaviour aborts)."""
    lib = os.path.join(HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    if not force and os.path.exists(lib):
        return lib
    tmp = lib + ".tmp"
    if sanitize:
        cmd = [CLANG, "-O1", "-g", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-shared-libsan", "-Wall", "-Wno-unknown-pragmas", "-o", tmp, SRC, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, lib)
    return lib


class _QMat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Moe(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("F", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("act", ctypes.c_int32),
                ("Wr", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("has_shared", ctypes.c_int32),
                ("sh_gate", _QMat), ("sh_up", _QMat), ("sh_down", _QMat)]


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data


class Oracle:
    def __init__(self, threads=1):
        if not os.path.exists(LIB):
            build()
        self.lib = ctypes.CDLL(LIB)
        L = self.lib
        for name in ("or_qgemv", "or_route_topk", "or_ffn", "or_moe_forward", "or_decode_row"):
            getattr(L, name).restype = ctypes.c_int
        L.or_set_threads.argtypes = [ctypes.c_int]
        L.or_set_threads.restype = ctypes.c_int
        L.or_row_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.or_row_bytes.restype = ctypes.c_int
        L.or_decode_row.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        L.or_qgemv.argtypes = [ctypes.POINTER(_QMat), ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_void_p, ctypes.c_void_p]
        L.or_route_topk.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.or_ffn.argtypes = [ctypes.POINTER(_QMat)] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                                          ctypes.c_void_p, ctypes.c_void_p]
        L.or_moe_forward.argtypes = [ctypes.POINTER(_Moe), ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        self.threads = L.or_set_threads(threads)

    def set_threads(self, n):
        self.threads = self.lib.or_set_threads(int(n))
        return self.threads

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise OracleError(ERR.get(rc, f"error {rc}"))

    def row_bytes(self, fmt, cols):
        return self.lib.or_row_bytes(FMT[fmt], cols)

    # -- marshalling ---------------------------------------------------------
    def _qmat(self, m, keep):
        if m is None:
            return _QMat(0, 0, 0, None, None)
        data = np.ascontiguousarray(m.data, dtype=np.uint8)
        keep.append(data)
        sc = None
        if m.scales is not None:
            sc = np.ascontiguousarray(m.scales, dtype=np.float32)
            keep.append(sc)
        return _QMat(FMT[m.fmt], m.rows, m.cols, _ptr(data), _ptr(sc))

    # -- entry points --------------------------------------------------------
    def decode_row(self, fmt, row, scale, cols):
        row = np.ascontiguousarray(np.frombuffer(bytes(row), dtype=np.uint8) if isinstance(row, (bytes, bytearray))
                                   else row, dtype=np.uint8)
        w = np.empty(cols, dtype=np.float64)
        self._check(self.lib.or_decode_row(FMT[fmt], _ptr(row), float(scale), cols, _ptr(w)))
        return w

    def qgemv(self, m, x, xtype="f32"):
        """y (B x rows, fp32) and S (B x rows, float64) for x (B x cols)."""
        keep = []
        qm = self._qmat(m, keep)
        x = np.ascontiguousarray(x, dtype=np.float32 if xtype == "f32" else np.uint16)
        if x.ndim == 1:
            x = x[None, :]
        B = x.shape[0]
        if x.shape[1] != m.cols:
            raise ValueError("x has the wrong number of columns")
        y = np.empty((B, m.rows), dtype=np.float32)
        S = np.empty((B, m.rows), dtype=np.float64)
        self._check(self.lib.or_qgemv(ctypes.byref(qm), XT[xtype], _ptr(x), B, _ptr(y), _ptr(S)))
        return y, S

    def route_topk(self, x, Wr, bias, k):
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim == 1:
            x = x[None, :]
        Wr = np.ascontiguousarray(Wr, dtype=np.float32)
        E, H = Wr.shape
        T = x.shape[0]
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        idx = np.empty((T, k), dtype=np.int32)
        gates = np.empty((T, k), dtype=np.float32)
        logits = np.empty((T, E), dtype=np.float32)
        margin = np.empty(T, dtype=np.float32)
        self._check(self.lib.or_route_topk(_ptr(x), T, H, _ptr(Wr), _ptr(b), E, k, _ptr(idx), _ptr(gates),
                                           _ptr(logits), _ptr(margin)))
        return idx, gates, logits, margin

    def ffn(self, gate, up, down, act, x):
        keep = []
        g, u, d = (self._qmat(m, keep) for m in (gate, up, down))
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim == 1:
            x = x[None, :]
        T = x.shape[0]
        y = np.empty((T, down.rows), dtype=np.float32)
        S = np.empty((T, down.rows), dtype=np.float64)
        self._check(self.lib.or_ffn(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), ACT[act], _ptr(x), T,
                                    _ptr(y), _ptr(S)))
        return y, S

    def moe_forward(self, H, F, E, k, act, Wr, bias, experts, shared, x):
        """experts: dict e -> {"gate","up","down"} matrices (only the experts the
        tokens select need to be present); shared: dict or None.
        Returns y (T x H fp32), idx (T x k), gates (T x k), S (T x H float64)."""
        keep = []
        arrs = {}
        for part in ("gate", "up", "down"):
            arr = (_QMat * E)()
            for e in range(E):
                if e in experts:
                    arr[e] = self._qmat(experts[e][part], keep)
                else:
                    arr[e] = _QMat(0, 0, 0, None, None)
            arrs[part] = arr
        Wr = np.ascontiguousarray(Wr, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        L = _Moe()
        L.H, L.F, L.E, L.k, L.act = H, F, E, k, ACT[act]
        L.Wr, L.bias = _ptr(Wr), _ptr(b)
        L.gate = ctypes.cast(arrs["gate"], ctypes.c_void_p)
        L.up = ctypes.cast(arrs["up"], ctypes.c_void_p)
        L.down = ctypes.cast(arrs["down"], ctypes.c_void_p)
        L.has_shared = 1 if shared else 0
        if shared:
            L.sh_gate = self._qmat(shared["gate"], keep)
            L.sh_up = self._qmat(shared["up"], keep)
            L.sh_down = self._qmat(shared["down"], keep)
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim == 1:
            x = x[None, :]
        T = x.shape[0]
        y = np.empty((T, H), dtype=np.float32)
        idx = np.empty((T, k), dtype=np.int32)
        gates = np.empty((T, k), dtype=np.float32)
        S = np.empty((T, H), dtype=np.float64)
        self._check(self.lib.or_moe_forward(ctypes.byref(L), _ptr(x), T, _ptr(y), _ptr(idx), _ptr(gates), _ptr(S)))
        return y, idx, gates, S
