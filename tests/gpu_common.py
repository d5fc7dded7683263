"""Shared pieces of the GPU tests: the pass criterion and cached device layers."""
import functools
import sys

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import moe_decode_amd as md
    md.lib()  # raises if the HIP library is missing: no fallback


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def within_bound(y_gpu, y_ref, S, rel=1e-4, abs_=1e-6):
    """|gpu - ref| <= rel * S + abs per element; returns (ok, max err/S)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    ok = bool(np.all(err <= rel * S + abs_))
    ratio = float(np.max(err / np.maximum(S, 1e-30))) if err.size else 0.0
    return ok, ratio


def assert_within(y_gpu, y_ref, S, what=""):
    ok, ratio = within_bound(y_gpu, y_ref, S)
    if not ok:
        bad = np.argwhere(np.abs(np.asarray(y_gpu, np.float64) - y_ref) > 1e-4 * S + 1e-6)
        raise AssertionError(f"{what}: {len(bad)} elements outside 1e-4*S+1e-6 (max err/S {ratio:.3e}); "
                             f"first {bad[:5].tolist()}")
    return ratio


@functools.lru_cache(maxsize=None)
def moe_layer(key):
    from synth import workloads as W
    from synth.device import device_moe
    say(f"[build] device layer {key}")
    return device_moe(W.spec(key))


@functools.lru_cache(maxsize=None)
def dense_matrix(key, name):
    from synth import workloads as W
    from synth.device import device_dense
    return device_dense(W.spec(key), name)


def oracle_moe(orc, sp, x):
    """Oracle forward of an MoE workload, materialising only the experts the
    tokens select (routing first, then those experts)."""
    from synth import workloads as W
    Wr, b = W.moe_router(sp)
    idx, _, _, _ = orc.route_topk(x, Wr, b, sp.k)
    experts = {int(e): W.moe_expert(sp, int(e)) for e in np.unique(idx)}
    return orc.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, experts, W.moe_shared(sp), x)
