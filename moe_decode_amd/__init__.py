"""Python binding of libmoe_decode (ctypes; argument marshalling only).

Every computation runs in the HIP library.  PyTorch supplies device memory
and the current stream; this module only packs descriptors, allocates
workspaces with torch, and turns error codes into exceptions.  There is no
fallback: if the library is missing, importing the binding's functions raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(HERE, "libmoe_decode.so")

Q8_0, Q4_0, I8_ROW, I4_ROW, Q4_1, I2_ROW = 1, 2, 3, 4, 5, 6
TYPES = {"q8_0": Q8_0, "q4_0": Q4_0, "i8_row": I8_ROW, "i4_row": I4_ROW, "q4_1": Q4_1, "i2_row": I2_ROW}
ROW_TYPES = (I8_ROW, I4_ROW, I2_ROW)
ACTS = {"gelu_tanh": 0, "silu": 1}
X_F32, X_BF16 = 0, 1

STATUS = {0: "MD_OK", 1: "MD_ERR_INVALID_ARG", 2: "MD_ERR_SHAPE", 3: "MD_ERR_UNSUPPORTED",
          4: "MD_ERR_ALIGNMENT", 5: "MD_ERR_WORKSPACE", 6: "MD_ERR_HIP"}

EXPORTS = ("md_abi_version", "md_status_string", "md_last_error_detail", "md_row_bytes", "md_prepare_layout",
           "md_qgemv_workspace_size", "md_qgemv", "md_route_workspace_size", "md_moe_route_topk",
           "md_ffn_workspace_size", "md_ffn_forward", "md_moe_workspace_size", "md_moe_layer_forward",
           "md_moe_layer_forward_timed", "md_moe_layer_forward_residual", "md_add",
           "md_hbm_read_probe", "md_moe_experts_forward", "md_expert_cache_reset", "md_expert_cache_plan",
           "md_expert_cache_fill", "md_moe_cached_workspace_size", "md_moe_cached_forward",
           "md_moe_layer_forward_noalloc", "md_moe_layer_stage_relaunch")
STAGES = {"shared": 0, "router": 1, "select": 2, "gateup": 3, "down": 4, "combine": 5}


class MDError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class QMatrixDesc(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("row_scale", ctypes.c_void_p)]


class FFNDesc(ctypes.Structure):
    _fields_ = [("act", ctypes.c_int32), ("gate", QMatrixDesc), ("up", QMatrixDesc), ("down", QMatrixDesc)]


class MoELayerDesc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("F", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("act", ctypes.c_int32), ("type", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p), ("down_scale", ctypes.c_void_p),
                ("W_r", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("has_shared", ctypes.c_int32), ("shared", FFNDesc)]


_lib = None


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise ImportError(f"{LIBPATH} is missing: build it with `python -m moe_decode_amd.build`")
        # torch first: its HIP runtime is then the one the library binds to
        # (two runtimes in one process would each see the device as busy)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIBPATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        psz = ctypes.POINTER(ctypes.c_size_t)
        sig = {
            "md_abi_version": (i32, []),
            "md_status_string": (ctypes.c_char_p, [i32]),
            "md_last_error_detail": (ctypes.c_char_p, []),
            "md_row_bytes": (ctypes.c_int64, [i32, i32]),
            "md_prepare_layout": (i32, [i32, i32, i32, i32, vp, vp, vp]),
            "md_qgemv_workspace_size": (i32, [vp, i32, psz]),
            "md_qgemv": (i32, [vp, vp, i32, i32, vp, vp, sz, vp]),
            "md_route_workspace_size": (i32, [i32, i32, i32, i32, psz]),
            "md_moe_route_topk": (i32, [vp, i32, i32, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]),
            "md_ffn_workspace_size": (i32, [vp, i32, psz]),
            "md_ffn_forward": (i32, [vp, vp, i32, vp, vp, sz, vp]),
            "md_moe_workspace_size": (i32, [vp, i32, psz]),
            "md_moe_layer_forward": (i32, [vp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "md_moe_layer_forward_timed": (i32, [vp, vp, i32, vp, vp, vp, vp, sz, vp, i32, vp, vp]),
            "md_moe_layer_forward_residual": (i32, [vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "md_add": (i32, [vp, vp, vp, ctypes.c_int64, vp]),
            "md_hbm_read_probe": (i32, [vp, ctypes.c_size_t, ctypes.c_uint32, vp, i32, vp]),
            "md_moe_experts_forward": (i32, [vp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "md_expert_cache_reset": (i32, [vp]),
            "md_expert_cache_plan": (i32, [vp, vp, i32, vp, vp, vp, vp]),
            "md_expert_cache_fill": (i32, [vp, vp, vp, vp, i32, vp]),
            "md_moe_cached_workspace_size": (i32, [vp, vp, i32, psz]),
            "md_moe_cached_forward": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp, vp, vp]),
            "md_moe_layer_forward_noalloc": (i32, [vp, vp, i32, vp, vp, vp, vp]),
            "md_moe_layer_stage_relaunch": (i32, [vp, vp, i32, vp, vp, vp, vp, sz, vp, i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise MDError(rc, lib().md_last_error_detail().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _workspace(nbytes, device, workspace):
    import torch
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, nbytes


def row_bytes(type_, cols):
    return lib().md_row_bytes(TYPES.get(type_, type_), cols)


class DevQMatrix:
    """A quantized matrix (or a stack of `count` experts) resident on the GPU in
    the library's device layout."""

    def __init__(self, type_, rows, cols, q, row_scale=None, count=1):
        self.type = TYPES.get(type_, type_)
        self.rows, self.cols, self.count = rows, cols, count
        self.q, self.row_scale = q, row_scale

    def desc(self, expert=0):
        rb = row_bytes(self.type, self.cols)
        off = expert * self.rows * rb
        sc = None if self.row_scale is None else self.row_scale.data_ptr() + 4 * expert * self.rows
        return QMatrixDesc(self.type, self.rows, self.cols, self.q.data_ptr() + off, sc)

    def expert(self, e):
        """The matrix of expert e of a stack, as a one-matrix view."""
        per = self.rows * row_bytes(self.type, self.cols)
        sc = None if self.row_scale is None else self.row_scale[e * self.rows:(e + 1) * self.rows]
        return DevQMatrix(self.type, self.rows, self.cols, self.q[e * per:(e + 1) * per], sc, 1)

    @property
    def nbytes(self):
        extra = 4 * self.rows * self.count if self.row_scale is not None else 0
        return self.rows * self.count * row_bytes(self.type, self.cols) + extra


def prepare_layout(type_, rows, cols, count, src, dst, stream=None):
    _check(lib().md_prepare_layout(TYPES.get(type_, type_), rows, cols, count, _ptr(src), _ptr(dst), _stream(stream)))


def qgemv_workspace_size(W, batch):
    d = W.desc()
    need = ctypes.c_size_t(0)
    _check(lib().md_qgemv_workspace_size(ctypes.byref(d), batch, ctypes.byref(need)))
    return need.value


def qgemv(W, x, y=None, workspace=None, stream=None):
    """y[b] = W x[b]; x (batch x cols) fp32 or bf16 tensor on the GPU."""
    import torch
    L = lib()
    d = W.desc()
    batch = x.shape[0] if x.dim() == 2 else 1
    xt = X_BF16 if x.dtype == torch.bfloat16 else X_F32
    if y is None:
        y = torch.empty(batch, W.rows, dtype=torch.float32, device=x.device)
    need = ctypes.c_size_t(0)
    _check(L.md_qgemv_workspace_size(ctypes.byref(d), batch, ctypes.byref(need)))
    ws, wsb = _workspace(need.value, x.device, workspace)
    _check(L.md_qgemv(ctypes.byref(d), _ptr(x), xt, batch, _ptr(y), _ptr(ws), wsb, _stream(stream)))
    return y


def route_workspace_size(T, H, E, k):
    need = ctypes.c_size_t(0)
    _check(lib().md_route_workspace_size(T, H, E, k, ctypes.byref(need)))
    return need.value


def moe_route_topk(x, Wr, bias, k, idx=None, gates=None, logits=None, workspace=None, stream=None):
    import torch
    T, H = x.shape
    E = Wr.shape[0]
    dev = x.device
    idx = torch.empty(T, k, dtype=torch.int32, device=dev) if idx is None else idx
    gates = torch.empty(T, k, dtype=torch.float32, device=dev) if gates is None else gates
    ws, wsb = _workspace(route_workspace_size(T, H, E, k), dev, workspace)
    _check(lib().md_moe_route_topk(_ptr(x), T, H, _ptr(Wr), _ptr(bias), E, k, _ptr(idx), _ptr(gates), _ptr(logits),
                                   _ptr(ws), wsb, _stream(stream)))
    return idx, gates


class FFN:
    def __init__(self, act, gate, up, down):
        self.act, self.gate, self.up, self.down = ACTS.get(act, act), gate, up, down

    def desc(self):
        return FFNDesc(self.act, self.gate.desc(), self.up.desc(), self.down.desc())


def ffn_workspace_size(ffn, T):
    d = ffn.desc()
    need = ctypes.c_size_t(0)
    _check(lib().md_ffn_workspace_size(ctypes.byref(d), T, ctypes.byref(need)))
    return need.value


def ffn_forward(ffn, x, y=None, workspace=None, stream=None):
    import torch
    T = x.shape[0]
    d = ffn.desc()
    if y is None:
        y = torch.empty(T, ffn.down.rows, dtype=torch.float32, device=x.device)
    ws, wsb = _workspace(ffn_workspace_size(ffn, T), x.device, workspace)
    _check(lib().md_ffn_forward(ctypes.byref(d), _ptr(x), T, _ptr(y), _ptr(ws), wsb, _stream(stream)))
    return y


class MoELayer:
    """Device-resident MoE layer: gate/up/down are DevQMatrix stacks of E experts."""

    def __init__(self, H, F, E, k, act, gate, up, down, Wr, bias=None, shared=None):
        self.H, self.F, self.E, self.k = H, F, E, k
        self.act = ACTS.get(act, act)
        self.gate, self.up, self.down = gate, up, down
        self.Wr, self.bias, self.shared = Wr, bias, shared
        self._desc = None

    def desc(self):
        if self._desc is None:
            d = MoELayerDesc()
            d.H, d.F, d.E, d.k, d.act, d.type = self.H, self.F, self.E, self.k, self.act, self.gate.type
            d.gate_q, d.up_q, d.down_q = _ptr(self.gate.q), _ptr(self.up.q), _ptr(self.down.q)
            d.gate_scale, d.up_scale, d.down_scale = (_ptr(self.gate.row_scale), _ptr(self.up.row_scale),
                                                      _ptr(self.down.row_scale))
            d.W_r, d.router_bias = _ptr(self.Wr), _ptr(self.bias)
            d.has_shared = 1 if self.shared is not None else 0
            if self.shared is not None:
                d.shared = self.shared.desc()
            self._desc = d
        return self._desc

    def weight_bytes(self, n_experts_read):
        """Algorithmic weight bytes of one call that reads n_experts_read experts."""
        per = (self.gate.nbytes + self.up.nbytes + self.down.nbytes) // self.E
        b = n_experts_read * per + 4 * self.E * self.H + (4 * self.E if self.bias is not None else 0)
        if self.shared is not None:
            b += self.shared.gate.nbytes + self.shared.up.nbytes + self.shared.down.nbytes
        return b


def moe_workspace_size(layer, T):
    d = layer.desc()
    need = ctypes.c_size_t(0)
    _check(lib().md_moe_workspace_size(ctypes.byref(d), T, ctypes.byref(need)))
    return need.value


def moe_layer_forward(layer, x, y=None, idx=None, gates=None, workspace=None, stream=None, residual=None):
    """y = layer(x), or residual + layer(x) when a residual ([T][H] fp32,
    possibly x or y) is given."""
    import torch
    T = x.shape[0]
    dev = x.device
    d = layer.desc()
    if y is None:
        y = torch.empty(T, layer.H, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(moe_workspace_size(layer, T), dev, workspace)
    if residual is None:
        _check(lib().md_moe_layer_forward(ctypes.byref(d), _ptr(x), T, _ptr(y), _ptr(idx), _ptr(gates), _ptr(ws), wsb,
                                          _stream(stream)))
    else:
        _check(lib().md_moe_layer_forward_residual(ctypes.byref(d), _ptr(x), T, _ptr(residual), _ptr(y), _ptr(idx),
                                                   _ptr(gates), _ptr(ws), wsb, _stream(stream)))
    return y


def moe_layer_stage_relaunch(layer, x, stage, y, workspace, idx=None, gates=None, stream=None):
    """Re-enqueue one stage ("shared", "router", "select", "gateup", "down",
    "combine") of an earlier moe_layer_forward made with the same x, y, idx,
    gates and workspace (a measurement aid)."""
    d = layer.desc()
    wsb = workspace.numel() * workspace.element_size()
    _check(lib().md_moe_layer_stage_relaunch(ctypes.byref(d), _ptr(x), x.shape[0], _ptr(y), _ptr(idx), _ptr(gates),
                                             _ptr(workspace), wsb, _stream(stream), STAGES.get(stage, stage)))


def moe_layer_forward_noalloc(layer, x, y, idx=None, gates=None, stream=None):
    """y = layer(x) with the library's built-in scratch (no workspace; the
    caller passes the output buffers).  Calls on one GPU must not overlap."""
    d = layer.desc()
    _check(lib().md_moe_layer_forward_noalloc(ctypes.byref(d), _ptr(x), x.shape[0], _ptr(y), _ptr(idx), _ptr(gates),
                                              _stream(stream)))
    return y


def moe_layer_forward_timed(layer, x, stage, start, stop, y=None, idx=None, gates=None, workspace=None,
                            stream=None):
    """moe_layer_forward that records the torch.cuda.Event pair start/stop
    around one stage ("shared", "router", "select", "gateup", "down",
    "combine") on the stream the kernels run on."""
    import torch
    T = x.shape[0]
    dev = x.device
    d = layer.desc()
    if y is None:
        y = torch.empty(T, layer.H, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(moe_workspace_size(layer, T), dev, workspace)
    _check(lib().md_moe_layer_forward_timed(ctypes.byref(d), _ptr(x), T, _ptr(y), _ptr(idx), _ptr(gates), _ptr(ws),
                                            wsb, _stream(stream), STAGES.get(stage, stage), start.cuda_event,
                                            stop.cuda_event))
    return y


def add(a, b, out=None, stream=None):
    """out = a + b (fp32 tensors of the same size on the device): the residual
    add between stacked layers."""
    import torch
    if out is None:
        out = torch.empty_like(a)
    _check(lib().md_add(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(stream)))
    return out


def hbm_read_probe(src, sink, key=0xFFFFFFFF, workgroups=0, stream=None):
    """Reads every byte of the device tensor src once (a bandwidth
    measurement).  Nothing is written unless some lane's xor of the words it
    read equals key: for zeroed src, any nonzero key leaves sink (a device
    tensor of at least 4 bytes) untouched."""
    nbytes = src.numel() * src.element_size()
    _check(lib().md_hbm_read_probe(_ptr(src), nbytes, key, _ptr(sink), workgroups, _stream(stream)))


def moe_experts_forward(layer, x, idx, gates, y=None, workspace=None, stream=None):
    """The layer's experts for a given routing (idx int32, gates fp32, [T][k]
    on the device): y[t] = sum_j gates[t][j] * expert idx[t][j] (x[t])."""
    import torch
    T = x.shape[0]
    d = layer.desc()
    if y is None:
        y = torch.empty(T, layer.H, dtype=torch.float32, device=x.device)
    ws, wsb = _workspace(moe_workspace_size(layer, T), x.device, workspace)
    _check(lib().md_moe_experts_forward(ctypes.byref(d), _ptr(x), T, _ptr(idx), _ptr(gates), _ptr(y), _ptr(ws), wsb,
                                        _stream(stream)))
    return y


class ExpertCacheState(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("S", ctypes.c_int32),
                ("slot_of_expert", ctypes.c_void_p), ("expert_in_slot", ctypes.c_void_p),
                ("uses", ctypes.c_void_p), ("last_use", ctypes.c_void_p), ("slot_idx", ctypes.c_void_p),
                ("step", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64)]


class ExpertCache:
    """The replacement state of an S-slot expert cache over E experts (host
    arrays owned here, the policy in the library)."""

    def __init__(self, E, S):
        import numpy as np
        self.slot_of_expert = np.empty(E, dtype=np.int32)
        self.expert_in_slot = np.empty(S, dtype=np.int32)
        self.uses = np.empty(S, dtype=np.int64)
        self.last_use = np.empty(S, dtype=np.int64)
        self.slot_idx = np.empty(128 * 8, dtype=np.int32)
        self.state = ExpertCacheState(E, S, self.slot_of_expert.ctypes.data, self.expert_in_slot.ctypes.data,
                                      self.uses.ctypes.data, self.last_use.ctypes.data, self.slot_idx.ctypes.data,
                                      0, 0, 0)
        self.reset()

    def reset(self):
        _check(lib().md_expert_cache_reset(ctypes.byref(self.state)))

    def plan(self, idx):
        """One policy step for the expert ids idx (host int32): returns the slot
        ids and the (expert, slot) pairs to load."""
        import numpy as np
        idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)
        n = idx.size
        slots = np.empty(n, dtype=np.int32)
        me = np.empty(n, dtype=np.int32)
        ms = np.empty(n, dtype=np.int32)
        nm = ctypes.c_int32(0)
        _check(lib().md_expert_cache_plan(ctypes.byref(self.state), idx.ctypes.data, n, slots.ctypes.data,
                                          me.ctypes.data, ms.ctypes.data, ctypes.byref(nm)))
        return slots, list(zip(me[:nm.value].tolist(), ms[:nm.value].tolist()))

    @property
    def hits(self):
        return self.state.hits

    @property
    def misses(self):
        return self.state.misses


class ExpertTier:
    """A MoE layer whose experts live in (pinned) host memory, with S slots of
    HBM caching them: `host` is a MoELayer whose expert stacks are host
    tensors (router weights on the device); the slots are allocated here."""

    def __init__(self, host, S, device="cuda", shared=None, overlap=True):
        import torch
        self.host = host
        self.S = S
        # the misses load on a stream of their own while the shared expert runs
        self.copy_stream = torch.cuda.Stream(device=device) if overlap else None
        self.copy_done = torch.cuda.Event() if overlap else None
        if self.copy_done is not None:
            self.copy_done.record(self.copy_stream)   # torch creates the HIP event at its first record

        def slots_like(m, rows):
            q = torch.empty(S * rows * row_bytes(m.type, m.cols), dtype=torch.uint8, device=device)
            sc = None if m.row_scale is None else torch.empty(S * rows, dtype=torch.float32, device=device)
            return DevQMatrix(m.type, m.rows, m.cols, q, sc, S)
        self.slots = MoELayer(host.H, host.F, S, host.k, host.act, slots_like(host.gate, host.F),
                              slots_like(host.up, host.F), slots_like(host.down, host.H), host.Wr, host.bias,
                              shared if shared is not None else host.shared)
        self.cache = ExpertCache(host.E, S)

    def workspace_size(self, T):
        need = ctypes.c_size_t(0)
        _check(lib().md_moe_cached_workspace_size(ctypes.byref(self.host.desc()), ctypes.byref(self.slots.desc()), T,
                                                  ctypes.byref(need)))
        return need.value

    def forward(self, x, y=None, idx=None, gates=None, workspace=None, stream=None):
        """y = layer(x) through the cache (one synchronisation per call)."""
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty(T, self.host.H, dtype=torch.float32, device=x.device)
        ws, wsb = _workspace(self.workspace_size(T), x.device, workspace)
        cs = self.copy_stream.cuda_stream if self.copy_stream is not None else None
        ev = self.copy_done.cuda_event if self.copy_done is not None else None
        _check(lib().md_moe_cached_forward(ctypes.byref(self.host.desc()), ctypes.byref(self.slots.desc()),
                                           ctypes.byref(self.cache.state), _ptr(x), T, _ptr(y), _ptr(idx),
                                           _ptr(gates), _ptr(ws), wsb, _stream(stream), cs, ev))
        return y
