"""Weight upload: canonical-layout bytes from the host to device-layout
tensors on the GPU (the layout conversion runs in the library).

Expert stacks are streamed one expert at a time, so the host never holds a
whole multi-GB stack."""
import numpy as np
import torch

from . import DevQMatrix, prepare_layout, row_bytes, ROW_TYPES, TYPES


def upload_stack(type_, rows, cols, count, fetch, device="cuda"):
    """fetch(i) -> (canonical uint8 array rows x row_bytes, fp32 scales or None)
    for i in range(count).  Returns a DevQMatrix holding `count` matrices."""
    t = TYPES.get(type_, type_)
    rb = row_bytes(t, cols)
    per = rows * rb
    src = torch.empty(count * per, dtype=torch.uint8, device=device)
    per_row = t in ROW_TYPES
    sc = torch.empty(count * rows, dtype=torch.float32, device=device) if per_row else None
    pinned = torch.empty(per, dtype=torch.uint8, pin_memory=True)
    for i in range(count):
        data, scales = fetch(i)
        pinned.numpy()[:] = np.ascontiguousarray(data, dtype=np.uint8).reshape(-1)
        src[i * per:(i + 1) * per].copy_(pinned, non_blocking=False)
        if per_row:
            sc[i * rows:(i + 1) * rows].copy_(torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)))
    dst = torch.empty_like(src)
    prepare_layout(t, rows, cols, count, src, dst)
    torch.cuda.current_stream().synchronize()
    del src
    return DevQMatrix(t, rows, cols, dst, sc, count)


def upload_matrix(m, device="cuda"):
    """A single canonical matrix object (fmt, rows, cols, data, scales)."""
    return upload_stack(m.fmt, m.rows, m.cols, 1, lambda i: (m.data, m.scales), device)


def upload_stack_host(type_, rows, cols, count, fetch, device="cuda"):
    """As upload_stack, but the result stays in pinned host memory (in the
    device layout, which the library's layout pass produces on the GPU one
    matrix at a time): the expert set of a host-memory tier."""
    t = TYPES.get(type_, type_)
    rb = row_bytes(t, cols)
    per = rows * rb
    host = torch.empty(count * per, dtype=torch.uint8, pin_memory=True)
    per_row = t in ROW_TYPES
    sc = torch.empty(count * rows, dtype=torch.float32, pin_memory=True) if per_row else None
    src = torch.empty(per, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    for i in range(count):
        data, scales = fetch(i)
        src.copy_(torch.from_numpy(np.ascontiguousarray(data, dtype=np.uint8).reshape(-1)))
        prepare_layout(t, rows, cols, 1, src, dst)
        host[i * per:(i + 1) * per].copy_(dst)
        if per_row:
            sc[i * rows:(i + 1) * rows].copy_(torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)))
    torch.cuda.current_stream().synchronize()
    return DevQMatrix(t, rows, cols, host, sc, count)
