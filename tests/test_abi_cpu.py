"""CPU checks of the C ABI: the library loads without a GPU, exports every
symbol the header declares, and rejects bad arguments with the documented
status before enqueueing anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import moe_decode_amd as md

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")

FAKE = 0x7F0000000000          # a 16-byte aligned address that is never dereferenced
FAKE_ODD = FAKE + 4


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:md_status|int32_t|int64_t|const char \*)\s*(md_\w+)\s*\(", text, re.M)))


def test_header_declares_what_the_binding_uses():
    assert declared_functions() == sorted(md.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = md.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_basic_queries():
    L = md.lib()
    assert L.md_abi_version() == 1
    assert L.md_status_string(3) == b"unsupported configuration"
    assert md.row_bytes("q8_0", 2048) == 2176
    assert md.row_bytes("q4_0", 768) == 432
    assert md.row_bytes("i4_row", 6144) == 3072
    assert md.row_bytes("i8_row", 6144) == 6144
    assert md.row_bytes("q4_1", 2560) == 1600
    assert md.row_bytes("i2_row", 6144) == 1536
    assert md.row_bytes(9, 256) == -1
    assert md.row_bytes(0, 256) == -1


def _qm(type_=md.Q8_0, rows=64, cols=256, q=FAKE, scale=None):
    return md.QMatrixDesc(type_, rows, cols, q, scale)


def _status(rc):
    return md.STATUS[rc]


def test_qgemv_errors():
    L = md.lib()
    sz = ctypes.c_size_t(0)
    assert _status(L.md_qgemv_workspace_size(None, 1, ctypes.byref(sz))) == "MD_ERR_INVALID_ARG"
    q = _qm(cols=300)
    assert _status(L.md_qgemv_workspace_size(ctypes.byref(q), 1, ctypes.byref(sz))) == "MD_ERR_UNSUPPORTED"
    q = _qm(cols=0)
    assert _status(L.md_qgemv_workspace_size(ctypes.byref(q), 1, ctypes.byref(sz))) == "MD_ERR_SHAPE"
    q = _qm()
    assert _status(L.md_qgemv_workspace_size(ctypes.byref(q), 9, ctypes.byref(sz))) == "MD_ERR_UNSUPPORTED"
    assert _status(L.md_qgemv_workspace_size(ctypes.byref(q), 0, ctypes.byref(sz))) == "MD_ERR_SHAPE"
    q = _qm(q=FAKE_ODD)
    assert _status(L.md_qgemv_workspace_size(ctypes.byref(q), 1, ctypes.byref(sz))) == "MD_ERR_ALIGNMENT"
    q = _qm(type_=md.I4_ROW)
    assert _status(L.md_qgemv_workspace_size(ctypes.byref(q), 1, ctypes.byref(sz))) == "MD_ERR_INVALID_ARG"
    assb = L.md_last_error_detail().decode()
    assert "row_scale" in assb
    q = _qm(type_=md.I2_ROW)
    assert _status(L.md_qgemv_workspace_size(ctypes.byref(q), 1, ctypes.byref(sz))) == "MD_ERR_INVALID_ARG"
    q = _qm(type_=md.I2_ROW, scale=FAKE)
    assert L.md_qgemv_workspace_size(ctypes.byref(q), 1, ctypes.byref(sz)) == 0
    q = _qm(type_=md.Q4_1, rows=4096, cols=2560)
    assert L.md_qgemv_workspace_size(ctypes.byref(q), 8, ctypes.byref(sz)) == 0
    q = _qm()
    assert _status(L.md_qgemv(ctypes.byref(q), FAKE, 7, 1, FAKE, None, 0, None)) == "MD_ERR_INVALID_ARG"
    assert _status(L.md_qgemv(ctypes.byref(q), FAKE_ODD, 0, 1, FAKE, None, 0, None)) == "MD_ERR_ALIGNMENT"
    assert _status(L.md_qgemv(ctypes.byref(q), None, 0, 1, FAKE, None, 0, None)) == "MD_ERR_INVALID_ARG"
    # a short-N shape needs a split-K workspace
    q = _qm(rows=8, cols=4096)
    assert L.md_qgemv_workspace_size(ctypes.byref(q), 1, ctypes.byref(sz)) == 0 and sz.value > 0
    assert _status(L.md_qgemv(ctypes.byref(q), FAKE, 0, 1, FAKE, None, 0, None)) == "MD_ERR_WORKSPACE"


def test_route_errors():
    L = md.lib()
    sz = ctypes.c_size_t(0)
    assert _status(L.md_route_workspace_size(1, 256, 8, 9, ctypes.byref(sz))) == "MD_ERR_SHAPE"
    assert _status(L.md_route_workspace_size(1, 256, 8, 0, ctypes.byref(sz))) == "MD_ERR_SHAPE"
    assert _status(L.md_route_workspace_size(129, 256, 8, 2, ctypes.byref(sz))) == "MD_ERR_UNSUPPORTED"
    assert _status(L.md_route_workspace_size(1, 256, 300, 2, ctypes.byref(sz))) == "MD_ERR_UNSUPPORTED"
    assert _status(L.md_route_workspace_size(1, 250, 8, 2, ctypes.byref(sz))) == "MD_ERR_UNSUPPORTED"
    assert L.md_route_workspace_size(4, 6144, 256, 8, ctypes.byref(sz)) == 0 and sz.value > 0
    assert _status(L.md_moe_route_topk(FAKE, 4, 6144, FAKE, None, 256, 8, FAKE, FAKE, None, None, 0, None)) == \
        "MD_ERR_WORKSPACE"
    assert _status(L.md_moe_route_topk(FAKE, 4, 6144, FAKE, FAKE_ODD, 256, 8, FAKE, FAKE, None, FAKE, sz.value,
                                       None)) == "MD_ERR_ALIGNMENT"


def _layer(**kw):
    d = md.MoELayerDesc()
    d.H, d.F, d.E, d.k, d.act, d.type = 256, 512, 8, 2, 0, md.Q8_0
    d.gate_q = d.up_q = d.down_q = d.W_r = FAKE
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_moe_errors():
    L = md.lib()
    sz = ctypes.c_size_t(0)
    ok = _layer()
    assert L.md_moe_workspace_size(ctypes.byref(ok), 1, ctypes.byref(sz)) == 0 and sz.value > 0
    cases = [
        (dict(k=9), 1, "MD_ERR_SHAPE"),
        (dict(k=0), 1, "MD_ERR_SHAPE"),
        (dict(E=300, k=2), 1, "MD_ERR_UNSUPPORTED"),
        (dict(H=320), 1, "MD_ERR_UNSUPPORTED"),
        (dict(act=5), 1, "MD_ERR_INVALID_ARG"),
        (dict(type=0), 1, "MD_ERR_INVALID_ARG"),
        (dict(gate_q=None), 1, "MD_ERR_INVALID_ARG"),
        (dict(down_q=FAKE_ODD), 1, "MD_ERR_ALIGNMENT"),
        (dict(type=md.I8_ROW), 1, "MD_ERR_INVALID_ARG"),
        (dict(has_shared=1), 1, "MD_ERR_INVALID_ARG"),
        (dict(type=md.I2_ROW), 1, "MD_ERR_INVALID_ARG"),          # per-row type without scales
        (dict(type=7), 1, "MD_ERR_INVALID_ARG"),
        ({}, 0, "MD_ERR_SHAPE"),
        ({}, 129, "MD_ERR_UNSUPPORTED"),
    ]
    for kw, T, want in cases:
        d = _layer(**kw)
        assert _status(L.md_moe_workspace_size(ctypes.byref(d), T, ctypes.byref(sz))) == want, (kw, T)
        assert _status(L.md_moe_layer_forward(ctypes.byref(d), FAKE, T, FAKE, None, None, FAKE, 1 << 30, None)) == \
            want, (kw, T)
    i2 = _layer(type=md.I2_ROW, gate_scale=FAKE, up_scale=FAKE, down_scale=FAKE)   # packed int2 experts
    assert L.md_moe_workspace_size(ctypes.byref(i2), 4, ctypes.byref(sz)) == 0 and sz.value > 0
    q41 = _layer(type=md.Q4_1)                                                      # Q4_1 experts
    for T in (1, 9, 128):
        assert L.md_moe_workspace_size(ctypes.byref(q41), T, ctypes.byref(sz)) == 0 and sz.value > 0
    d = _layer()
    assert _status(L.md_moe_layer_forward(ctypes.byref(d), FAKE, 1, FAKE, None, None, FAKE, 16, None)) == \
        "MD_ERR_WORKSPACE"
    assert _status(L.md_moe_layer_forward(ctypes.byref(d), FAKE, 1, FAKE_ODD, None, None, FAKE, 1 << 30, None)) == \
        "MD_ERR_ALIGNMENT"


def test_noalloc_errors_before_any_device_call():
    """The no-allocation layer call validates like md_moe_layer_forward and
    refuses a call whose scratch would exceed its 64 MiB before it looks up
    the device (so these return their codes without a GPU)."""
    L = md.lib()
    sz = ctypes.c_size_t(0)
    for kw, T, want in [(dict(k=9), 1, "MD_ERR_SHAPE"), ({}, 129, "MD_ERR_UNSUPPORTED"),
                        (dict(gate_q=None), 1, "MD_ERR_INVALID_ARG")]:
        d = _layer(**kw)
        assert _status(L.md_moe_layer_forward_noalloc(ctypes.byref(d), FAKE, T, FAKE, None, None, None)) == want
    d = _layer()
    assert _status(L.md_moe_layer_forward_noalloc(ctypes.byref(d), None, 1, FAKE, None, None, None)) == \
        "MD_ERR_INVALID_ARG"
    assert _status(L.md_moe_layer_forward_noalloc(ctypes.byref(d), FAKE, 1, FAKE_ODD, None, None, None)) == \
        "MD_ERR_ALIGNMENT"
    big = _layer(H=16384, F=16384, E=256, k=8)
    assert L.md_moe_workspace_size(ctypes.byref(big), 128, ctypes.byref(sz)) == 0 and sz.value > 64 << 20
    assert _status(L.md_moe_layer_forward_noalloc(ctypes.byref(big), FAKE, 128, FAKE, None, None, None)) == \
        "MD_ERR_UNSUPPORTED"
    assert b"64" in L.md_last_error_detail() or b"67108864" in L.md_last_error_detail()


def test_ffn_and_layout_errors():
    L = md.lib()
    sz = ctypes.c_size_t(0)
    f = md.FFNDesc(0, _qm(rows=512, cols=256), _qm(rows=512, cols=256), _qm(rows=256, cols=512))
    # fp32 h, then Q8_0 digit planes (three planes of 16 B per 16 values) and their scales,
    # of x and of h, each part rounded up to 256 bytes
    want = 3 * 512 * 4 + (3 * 16 * 48 + 256) + (3 * 32 * 48 + 512)
    assert L.md_ffn_workspace_size(ctypes.byref(f), 3, ctypes.byref(sz)) == 0 and sz.value == want
    f.down = _qm(rows=256, cols=768)
    assert _status(L.md_ffn_workspace_size(ctypes.byref(f), 3, ctypes.byref(sz))) == "MD_ERR_SHAPE"
    f.down = _qm(type_=md.Q4_0, rows=256, cols=512)
    assert _status(L.md_ffn_workspace_size(ctypes.byref(f), 3, ctypes.byref(sz))) == "MD_ERR_UNSUPPORTED"
    # Q4_1 takes the Q4_0 digit planes: the same workspace at every token count
    for T in (1, 3, 9, 128):
        ws = []
        for t in (md.Q4_0, md.Q4_1):
            f = md.FFNDesc(0, _qm(type_=t, rows=512, cols=256), _qm(type_=t, rows=512, cols=256),
                           _qm(type_=t, rows=256, cols=512))
            assert L.md_ffn_workspace_size(ctypes.byref(f), T, ctypes.byref(sz)) == 0
            ws.append(sz.value)
        assert ws[0] == ws[1] > 0, (T, ws)
    assert _status(L.md_prepare_layout(md.Q8_0, 4, 256, 1, FAKE, FAKE + 64, None)) == "MD_ERR_INVALID_ARG"
    assert _status(L.md_prepare_layout(md.Q8_0, 4, 256, 1, FAKE, FAKE_ODD, None)) == "MD_ERR_ALIGNMENT"
    assert _status(L.md_prepare_layout(md.Q8_0, 4, 100, 1, FAKE, FAKE + 4096, None)) == "MD_ERR_UNSUPPORTED"
    assert _status(L.md_prepare_layout(0, 4, 256, 1, FAKE, FAKE + 4096, None)) == "MD_ERR_INVALID_ARG"


def test_add_errors():
    L = md.lib()
    assert _status(L.md_add(FAKE, FAKE, FAKE, 0, None)) == "MD_ERR_SHAPE"
    assert _status(L.md_add(FAKE, None, FAKE, 8, None)) == "MD_ERR_INVALID_ARG"
    assert _status(L.md_add(FAKE, FAKE_ODD, FAKE, 8, None)) == "MD_ERR_ALIGNMENT"


def test_read_probe_errors():
    L = md.lib()
    f = L.md_hbm_read_probe
    assert _status(f(None, 1024, 1, FAKE, 0, None)) == "MD_ERR_INVALID_ARG"
    assert _status(f(FAKE, 1024, 1, None, 0, None)) == "MD_ERR_INVALID_ARG"
    assert _status(f(FAKE, 0, 1, FAKE, 0, None)) == "MD_ERR_SHAPE"
    assert _status(f(FAKE, 1000, 1, FAKE, 0, None)) == "MD_ERR_SHAPE"
    assert _status(f(FAKE_ODD, 1024, 1, FAKE, 0, None)) == "MD_ERR_ALIGNMENT"
    assert _status(f(FAKE, 1024, 1, FAKE, -1, None)) == "MD_ERR_INVALID_ARG"

def test_residual_forward_errors():
    L = md.lib()
    d = _layer()
    f = L.md_moe_layer_forward_residual
    assert _status(f(ctypes.byref(d), FAKE, 1, None, FAKE, None, None, FAKE, 1 << 30, None)) == "MD_ERR_INVALID_ARG"
    assert _status(f(ctypes.byref(d), FAKE, 1, FAKE_ODD, FAKE, None, None, FAKE, 1 << 30, None)) == "MD_ERR_ALIGNMENT"
    # the layer's own checks still apply
    assert _status(f(ctypes.byref(d), FAKE, 0, FAKE, FAKE, None, None, FAKE, 1 << 30, None)) == "MD_ERR_SHAPE"
    bad = _layer(k=9)
    assert _status(f(ctypes.byref(bad), FAKE, 1, FAKE, FAKE, None, None, FAKE, 1 << 30, None)) == "MD_ERR_SHAPE"
