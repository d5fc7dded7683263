"""Upload the seeded workloads to the GPU through the library's binding.

Used by the GPU tests and the benchmark only (the oracle never imports this
module).  It moves bytes; it computes nothing."""
import numpy as np
import torch

import moe_decode_amd as md
from moe_decode_amd.upload import upload_stack, upload_stack_host, upload_matrix

from . import workloads as W


def device_moe(sp, device="cuda", hashes=None):
    """The whole layer of an MoE workload resident on the GPU.  With a dict
    `hashes`, the SHA-256 of every input buffer's canonical bytes (each expert
    stack with its row scales, the router weights and bias, the shared
    expert's matrices) is stored in it, hex, under the buffer's name."""
    import hashlib
    stacks = {}
    for part in ("gate", "up", "down"):
        rows, cols = (sp.H, sp.F) if part == "down" else (sp.F, sp.H)
        h = hashlib.sha256()

        def fetch(e, part=part, h=h):
            m = W.moe_expert_part(sp, e, part)
            h.update(np.ascontiguousarray(m.data).tobytes())
            if m.scales is not None:
                h.update(np.ascontiguousarray(m.scales, dtype=np.float32).tobytes())
            return m.data, m.scales
        stacks[part] = upload_stack(sp.fmt, rows, cols, sp.E, fetch, device)
        if hashes is not None:
            hashes[f"experts.{part}"] = h.hexdigest()
    Wr, b = W.moe_router(sp)
    Wr_t = torch.from_numpy(Wr).to(device)
    b_t = None if b is None else torch.from_numpy(b).to(device)
    if hashes is not None:
        hashes["router.W_r"] = hashlib.sha256(np.ascontiguousarray(Wr).tobytes()).hexdigest()
        if b is not None:
            hashes["router.bias"] = hashlib.sha256(np.ascontiguousarray(b).tobytes()).hexdigest()
    shared = None
    sh = W.moe_shared(sp)
    if sh is not None:
        shared = md.FFN(sp.act, upload_matrix(sh["gate"], device), upload_matrix(sh["up"], device),
                        upload_matrix(sh["down"], device))
        if hashes is not None:
            for part in ("gate", "up", "down"):
                hashes[f"shared.{part}"] = hashlib.sha256(np.ascontiguousarray(sh[part].data).tobytes()).hexdigest()
    return md.MoELayer(sp.H, sp.F, sp.E, sp.k, sp.act, stacks["gate"], stacks["up"], stacks["down"], Wr_t, b_t,
                       shared)


def host_moe(sp, device="cuda"):
    """The layer with its routed experts in pinned host memory (the router
    and any shared expert on the GPU): the source of a host-memory tier."""
    stacks = {}
    for part in ("gate", "up", "down"):
        rows, cols = (sp.H, sp.F) if part == "down" else (sp.F, sp.H)

        def fetch(e, part=part):
            m = W.moe_expert_part(sp, e, part)
            return m.data, m.scales
        stacks[part] = upload_stack_host(sp.fmt, rows, cols, sp.E, fetch, device)
    Wr, b = W.moe_router(sp)
    shared = None
    sh = W.moe_shared(sp)
    if sh is not None:  # the shared expert stays resident on the GPU
        shared = md.FFN(sp.act, upload_matrix(sh["gate"], device), upload_matrix(sh["up"], device),
                        upload_matrix(sh["down"], device))
    return md.MoELayer(sp.H, sp.F, sp.E, sp.k, sp.act, stacks["gate"], stacks["up"], stacks["down"],
                       torch.from_numpy(Wr).to(device), None if b is None else torch.from_numpy(b).to(device), shared)


def device_dense(sp, name, device="cuda"):
    return upload_matrix(W.dense_matrix(sp, name), device)


def x_tensor(x, device="cuda"):
    """fp32 array -> fp32 tensor; uint16 bf16 patterns -> bf16 tensor."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x.astype(np.float32)).to(device)
