"""Benchmark of the MoE-layer hot path on one MI355X.

The headline step is one decode forward (router -> top-k + gates -> the 8
selected experts' gate/up + GeGLU -> down -> combine) of the 256-expert top-8
layer at hidden 6144, expert FFN 2048, packed int4 weights with per-row
scales, one token.  Every timed step takes a different token from a pool of
seeded tokens, so the selected experts change from step to step and their
bytes come from HBM (the 4.8 GB expert set is far larger than the 256 MB
Infinity Cache), as in real decode.

The same JSON line carries the metric's other half, "prefill": 128-token
chunks of that layer and of the 128-expert layer with a shared expert (four
copies of that layer in HBM, used in turn, so its 354 MB of weights are not
served from the Infinity Cache), each with tokens/s, weight GB/s, the
roofline of its dominant kernel with the matrix cores' utilisation, and the
oracle timed on a sample of the same chunk; and "decode_c3": the one-token
decode of the shared-expert layer (the same four copies), with each of its
three launches timed against the bytes it streams and the chain of plain
reads of those bytes.

Each roofline's kernel time is measured live: a number of forwards, each on
its own inputs and workspace, then that stage alone relaunched over all of
them back to back between two HIP events on the kernels' stream (the average
duration of the kernel on real inputs; HIP events around single launches,
which add the dispatch latency, are reported beside it).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--modes]
    python bench.py --copy-calibration      # plain copy kernel of known size
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (decode, 128-tok prefill) + achieved HBM GB/s on weight bytes"
HBM_PEAK_GBS = 8000.0
# dense matrix-core peaks of MI355X (no structured sparsity), in T(FL)OP/s
MFMA_PEAK_TOPS = {"bf16": 2500.0, "int8": 5000.0}
POOL = 64


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def expert_weight_bytes(sp):
    return sp.expert_bytes()


def step_weight_bytes(sp, idx):
    """Algorithmic weight bytes of one call: the distinct selected experts,
    the router, the shared expert."""
    import numpy as np
    n = len(np.unique(idx))
    return n * sp.expert_bytes() + sp.router_bytes() + sp.shared_bytes()


def gateup_bytes(sp, idx):
    import numpy as np
    from synth.formats import matrix_bytes
    return len(np.unique(idx)) * 2 * matrix_bytes(sp.fmt, sp.F, sp.H)


def token_pool(sp, T, n):
    """n seeded inputs of T tokens each (fp32, N(0, 1))."""
    import numpy as np
    rng = np.random.default_rng([sp.index, 777, T, sp.variant])
    return rng.standard_normal((n, T, sp.H)).astype(np.float32)


def run_mode(layers, sp, T, steps, warmup, stage="gateup", graph=False):
    """Time `steps` forwards of T tokens: step i takes input i of a pool of
    seeded inputs (cycled) and layer copy i of `layers` (cycled; one copy, or
    several identical copies so that consecutive steps do not find the
    weights in the Infinity Cache).  Returns a dict with per-step ms,
    tokens/s, weight bytes, the stage's time from HIP events around each of
    its launches, the per-step event-time percentiles and the host time per
    call; with graph, also the time per step of the same sequence of forwards
    captured in one HIP graph and replayed back to back."""
    import numpy as np
    import torch
    import moe_decode_amd as md

    if not isinstance(layers, (list, tuple)):
        layers = [layers]
    R = len(layers)
    pool = POOL if T == 1 else max(4, POOL // T)
    xs_np = token_pool(sp, T, pool)
    xs = torch.from_numpy(xs_np).cuda()
    y = torch.empty(T, sp.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(pool, T, sp.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, sp.k, dtype=torch.float32, device="cuda")
    ws = torch.empty(md.moe_workspace_size(layers[0], T), dtype=torch.uint8, device="cuda")

    def fwd(i):
        md.moe_layer_forward(layers[i % R], xs[i % pool], y=y, idx=idx[i % pool], gates=gates, workspace=ws)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:       # torch creates the HIP event at its first record
        a.record()
        b.record()
    for i in range(warmup):
        fwd(i)
    torch.cuda.synchronize()
    # timed region: plain forwards
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    h0 = time.perf_counter()
    for i in range(steps):
        fwd(i)
    host_s = time.perf_counter() - h0
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # the same steps again with HIP events around one stage (recorded by the
    # library on the kernels' stream)
    for i in range(steps):
        a, b = ev[i]
        md.moe_layer_forward_timed(layers[i % R], xs[i % pool], stage, a, b, y=y, idx=idx[i % pool], gates=gates,
                                   workspace=ws)
    torch.cuda.synchronize()
    stage_ms = [a.elapsed_time(b) for a, b in ev]
    # per-step percentiles from a third pass with one event between
    # consecutive steps (step i = the interval from event i to event i+1)
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    sev[0].record()
    for i in range(steps):
        fwd(i)
        sev[i + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(steps)])
    graph_ms = None
    if graph:
        g = torch.cuda.CUDAGraph()
        s_ = torch.cuda.Stream()
        s_.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_):
            with torch.cuda.graph(g, stream=s_):
                for i in range(steps):
                    fwd(i)
        torch.cuda.current_stream().wait_stream(s_)
        g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(3):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (3 * steps)
        del g
    idx_np = idx.cpu().numpy()
    wb = [step_weight_bytes(sp, idx_np[i % pool]) for i in range(steps)]
    gb = [gateup_bytes(sp, idx_np[i % pool]) for i in range(steps)]
    ms = total_ms / steps
    return {
        "T": T, "ms_per_step": ms, "tokens_per_s": T * steps / (total_ms / 1e3),
        "weight_bytes_per_step": float(np.mean(wb)),
        "weight_GBps": float(np.sum(wb)) / (total_ms / 1e3) / 1e9,
        "layer_copies": R,
        "stage": stage, "stage_ms_avg": float(np.mean(stage_ms)),
        "stage_bytes_avg": float(np.mean(gb)),
        "stage_GBps": float(np.sum(gb)) / (np.sum(stage_ms) / 1e3) / 1e9,
        "pool": pool,
        "inputs_sha256": hashlib.sha256(xs_np.tobytes()).hexdigest(),
        "step_ms_p10_p50_p90": [float(v) for v in np.percentile(step_ms, [10, 50, 90])],
        "host_us_per_call": host_s / steps * 1e6,
        "graph_ms_per_step": graph_ms,
        "idx": idx_np[:min(max(steps, warmup), pool)],   # the pool entries the calls wrote
    }


def kernel_time(layers, sp, T, stage, n_inputs, reps=3):
    """Average duration of one stage's kernels on real inputs: n_inputs
    forwards (each on its own seeded input, layer copy i mod len(layers) and
    workspace) leave their intermediate results behind; then the stage alone
    is relaunched over all of them back to back (captured in a HIP graph,
    replayed `reps` times between two HIP events on the kernels' stream).  Consecutive launches work on different
    tokens (different experts), so their weight bytes come from HBM."""
    import numpy as np
    import torch
    import moe_decode_amd as md
    if not isinstance(layers, (list, tuple)):
        layers = [layers]
    R = len(layers)
    xs = torch.from_numpy(np.random.default_rng([sp.index, 779, T, sp.variant])
                          .standard_normal((n_inputs, T, sp.H)).astype(np.float32)).cuda()
    need = md.moe_workspace_size(layers[0], T)
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(n_inputs)]
    ys = torch.empty(n_inputs, T, sp.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(n_inputs, T, sp.k, dtype=torch.int32, device="cuda")
    gts = torch.empty(n_inputs, T, sp.k, dtype=torch.float32, device="cuda")
    for p in range(n_inputs):
        md.moe_layer_forward(layers[p % R], xs[p], y=ys[p], idx=idx[p], gates=gts[p], workspace=wss[p])

    def run():
        for p in range(n_inputs):
            md.moe_layer_stage_relaunch(layers[p % R], xs[p], stage, ys[p], wss[p], idx=idx[p], gates=gts[p])

    run()
    torch.cuda.synchronize()
    # the relaunches captured in one HIP graph: a kernel shorter than the
    # host's time per call would otherwise wait for its own submission
    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            run()
    torch.cuda.current_stream().wait_stream(s_)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    del g
    ms = t0.elapsed_time(t1) / (reps * n_inputs)
    idx_np = idx.cpu().numpy()
    del wss
    return {"stage": stage, "ms_per_launch": ms, "launches": reps * n_inputs, "inputs": n_inputs, "idx": idx_np}


def mfma_stats(sp, idx, ms, dtype):
    """Matrix-core use of the grouped gate/up GEMM of a chunk: useful ops
    (2 per multiply-add of the gate and up projections of every routed
    (token, slot) pair) and issued ops (16-token tiles per active expert, times
    the passes per product: four int8 digits of the activations on the int8
    path, a bf16 high and low half on the bf16 path), per second against the
    dense peak of that dtype."""
    import numpy as np
    issue = 4 if dtype == "int8" else 2
    per_pair = 2.0 * 2 * sp.F * sp.H
    tiles = 0
    for row in idx.reshape(-1, idx.shape[-2], idx.shape[-1]):
        counts = np.bincount(row.reshape(-1), minlength=sp.E)
        tiles += int(np.sum((counts + 15) // 16))
    n_calls = idx.reshape(-1, idx.shape[-2], idx.shape[-1]).shape[0]
    useful = per_pair * idx.shape[-2] * idx.shape[-1]          # per call
    issued = per_pair * 16 * (tiles / n_calls) * issue
    peak = MFMA_PEAK_TOPS[dtype]
    u = useful / (ms / 1e3) / 1e12
    i = issued / (ms / 1e3) / 1e12
    return {"dtype": dtype, "useful_TOPS": u, "issued_TOPS": i, "peak_TOPS": peak, "useful_util": u / peak,
            "issued_util": i / peak, "passes_per_product": issue, "tiles_per_call": tiles / n_calls}


def cpu_baseline(sp, budget_s=10.0, T=1, sample_tokens=None, threads=None):
    """The oracle, as is, on a bounded sample of the same workload: forwards
    of the seeded inputs (cycled) until about budget_s seconds of oracle time
    have been spent (decode), or the first sample_tokens tokens of one
    T-token chunk (prefill: the oracle's tokens are independent, so a sample
    of a chunk's tokens times the same work per token)."""
    import numpy as np
    import oracle
    from synth import workloads as W

    threads = threads or os.cpu_count() or 1
    orc = oracle.Oracle(threads=threads)
    Wr, b = W.moe_router(sp)
    shared = W.moe_shared(sp)
    cache = {}

    def experts_for(x):
        idx, _, _, _ = orc.route_topk(x, Wr, b, sp.k)
        ex = {}
        for e in np.unique(idx):
            e = int(e)
            if e not in cache:
                if len(cache) >= 160:
                    cache.clear()
                cache[e] = W.moe_expert(sp, e)
            ex[e] = cache[e]
        return ex

    if sample_tokens is None:
        xs = token_pool(sp, 1, POOL)
        done, spent, i = 0, 0.0, 0
        while spent < budget_s:
            x = xs[i % POOL]
            i += 1
            ex = experts_for(x)
            t = time.perf_counter()
            orc.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, ex, shared, x)
            spent += time.perf_counter() - t
            done += 1
        sample = (f"{done} single-token decode forwards of this layer over a pool of {POOL} seeded tokens "
                  f"(fp64 oracle, {orc.threads} thread(s), OpenMP over output rows), {spent:.1f} s of oracle time; "
                  f"expert generation outside the timed part")
    else:
        x = token_pool(sp, T, 1)[0][:sample_tokens]
        ex = experts_for(x)
        t = time.perf_counter()
        orc.moe_forward(sp.H, sp.F, sp.E, sp.k, sp.act, Wr, b, ex, shared, x)
        spent = time.perf_counter() - t
        done = sample_tokens
        sample = (f"the first {sample_tokens} tokens of the first seeded {T}-token chunk (fp64 oracle, "
                  f"{orc.threads} thread(s); the oracle computes tokens independently), {spent:.1f} s of oracle "
                  f"time; expert generation outside the timed part")
    return {"value": done / spent, "unit": "tokens/s", "cores": orc.threads, "kind": "oracle", "sample": sample}


def traffic_record(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed PMC
    summary, if the kernel sources still hash to the ones it was taken with
    (else None)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)\s*$", text, re.M)
    h = re.search(r"^source_sha256:\s*([0-9a-f]+)\s*$", text, re.M)
    if not m or not h or h.group(1) != kernel_source_hash(kernel):
        return None
    return float(m.group(1))


KERNEL_SOURCE = {"k_gateup_t1": "decode.hip", "k_moe_mfma": "prefill.hip", "k_moe_mfma_i8": "prefill.hip"}


def kernel_source_hash(kernel=None):
    """SHA-256 of the source file that defines `kernel` and of every header
    (all HIP/C++ sources when kernel is None)."""
    import hashlib
    d = os.path.join(ROOT, "moe_decode_amd", "csrc")
    hs = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith(".hpp") or (name.endswith((".hip", ".cpp")) and kernel is None) or \
                name == KERNEL_SOURCE.get(kernel):
            hs.update(name.encode())
            hs.update(open(os.path.join(d, name), "rb").read())
    return hs.hexdigest()


def run_dense(key, name, batch, steps, warmup, rotate_bytes=1 << 30):
    """One dense quantized GEMV of a dense workload.  A call takes a few
    microseconds of GPU time, less than the Python call path, so `steps`
    calls are captured in a HIP graph and the graph's replay is timed with
    HIP events (GPU time per call, without the host).  Call i uses copy
    i mod R of the matrix, R copies filling at least rotate_bytes of HBM, so
    a call does not find its weights in the Infinity Cache (rotate_bytes 0:
    one copy, a warm-cache figure)."""
    import torch
    import moe_decode_amd as md
    from synth import workloads as W
    from synth.device import device_dense, x_tensor
    sp = W.spec(key)
    Wd = device_dense(sp, name)
    R = max(1, -(-rotate_bytes // Wd.nbytes)) if rotate_bytes else 1
    copies = [Wd]
    if R > 1:
        q = Wd.q.repeat(R)
        sc = None if Wd.row_scale is None else Wd.row_scale.repeat(R)
        n, r = Wd.q.numel(), Wd.rows
        copies = [md.DevQMatrix(Wd.type, Wd.rows, Wd.cols, q[i * n:(i + 1) * n],
                                None if sc is None else sc[i * r:(i + 1) * r]) for i in range(R)]
    x = x_tensor(W.dense_x(sp, Wd.cols, batch))
    y = torch.empty(batch, Wd.rows, dtype=torch.float32, device="cuda")
    need = md.qgemv_workspace_size(Wd, batch)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    n_calls = max(steps, R)
    for i in range(warmup):
        md.qgemv(copies[i % R], x, y=y, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            for i in range(n_calls):
                md.qgemv(copies[i % R], x, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s_)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / (reps * n_calls)
    nbytes = Wd.nbytes
    del g, copies
    torch.cuda.empty_cache()
    return {"matrix": f"{name} {Wd.rows}x{Wd.cols} {sp.fmt}", "batch": batch, "ms_per_call": ms,
            "timing": "HIP graph of the calls, replayed", "copies": R,
            "cache": "HBM: consecutive calls use different copies" if R > 1 else "warm: one copy, not HBM",
            "weight_bytes": nbytes, "weight_GBps": nbytes / (ms / 1e3) / 1e9}


def run_stack(key, n_layers, reps):
    """A stack of n_layers distinct layers of workload `key`, one token, each
    layer's output added to its input (md_moe_layer_forward_residual),
    captured in one HIP graph;
    the graph's replay is timed: per-layer time at model depth with no host
    work between layers.  The selected experts of all layers (n_layers x k
    experts) far exceed the Infinity Cache, so each replay reads HBM."""
    from dataclasses import replace
    import numpy as np
    import torch
    import moe_decode_amd as md
    from synth import workloads as W
    from synth.device import device_moe
    base = W.spec(key)
    specs = [replace(base, key=f"{key}_layer{l}", variant=base.variant + 100 + l) for l in range(n_layers)]
    t_gen = time.perf_counter()
    layers = [device_moe(sp) for sp in specs]
    torch.cuda.synchronize()
    log(f"[bench] stack of {n_layers} {key} layers resident ({time.perf_counter() - t_gen:.1f} s)")
    T = 1
    x = torch.from_numpy(np.random.default_rng([base.index, 780]).standard_normal((T, base.H)).astype(np.float32))
    x = x.cuda()
    wss = [torch.empty(md.moe_workspace_size(l, T), dtype=torch.uint8, device="cuda") for l in layers]
    curs = [x] + [torch.empty(T, base.H, device="cuda") for _ in layers]

    def run():
        for l, layer in enumerate(layers):  # the residual joins each layer's last kernel
            md.moe_layer_forward(layer, curs[l], y=curs[l + 1], workspace=wss[l], residual=curs[l])

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            run()
    torch.cuda.current_stream().wait_stream(s_)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    nbytes = n_layers * (base.k * base.expert_bytes() + base.router_bytes())
    del g, layers
    torch.cuda.empty_cache()
    return {"workload": key, "layers": n_layers, "tokens": T, "ms_per_stack": ms,
            "us_per_layer": ms * 1e3 / n_layers, "tokens_per_s": T / (ms / 1e3),
            "weight_GBps": nbytes / (ms / 1e3) / 1e9,
            "timing": "HIP graph of the stack (layer forward with the residual add per layer), replayed"}


def hbm_probe(nbytes=4 << 30, reps=5):
    """Attainable HBM read bandwidth: the library's streaming-read kernel over
    a 4 GiB buffer of random bytes (16x the Infinity Cache), a short sweep of
    grid sizes, each timed with HIP events over `reps` back-to-back reads."""
    import torch
    import moe_decode_amd as md
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sweep = []
    for wg in (2048, 8192, 32768, 65536, 131072):
        md.hbm_read_probe(src, sink, workgroups=wg)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            md.hbm_read_probe(src, sink, workgroups=wg)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        sweep.append({"workgroups": wg, "ms": ms, "GBps": nbytes / (ms / 1e3) / 1e9})
    del src
    torch.cuda.empty_cache()
    best = max(sweep, key=lambda r: r["GBps"])
    return {"bytes": nbytes, "reps": reps, "GBps": best["GBps"], "workgroups": best["workgroups"], "sweep": sweep}


def chain_floor(sizes, reps=16, pool_bytes=4 << 30):
    """Time of a chain of plain streaming reads of the given byte counts, back
    to back (the library's read probe; each read from a fresh region of a
    4 GiB buffer of random bytes, so nothing comes from the caches), captured
    in a HIP graph and replayed: what a chain of kernels that each stream
    those bytes takes at this GPU's attainable read rate, launch gaps
    included, when nothing overlaps."""
    import torch
    import moe_decode_amd as md
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    src = torch.randint(0, 256, (pool_bytes,), dtype=torch.uint8, device="cuda", generator=gen)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    per_chain = sum((n + 255) // 256 * 256 for n in sizes)
    chains = max(1, pool_bytes // per_chain)

    # each read's grid: the fastest of one, two or four 32 KB tiles per
    # workgroup, each timed alone (graph replays over fresh regions)
    def timed(nbytes, wg, n=16):
        nb = (nbytes + 15) // 16 * 16
        stride = (nb + 255) // 256 * 256
        k = max(1, min(n, pool_bytes // stride))

        def go():
            for i in range(n):
                o = (i % k) * stride
                md.hbm_read_probe(src[o:o + nb], sink, workgroups=wg)
        go()
        torch.cuda.synchronize()
        gg = torch.cuda.CUDAGraph()
        ss = torch.cuda.Stream()
        ss.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(ss):
            with torch.cuda.graph(gg, stream=ss):
                go()
        torch.cuda.current_stream().wait_stream(ss)
        gg.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        gg.replay()
        b.record()
        torch.cuda.synchronize()
        del gg
        return a.elapsed_time(b) / n

    grids = []
    for n in sizes:
        tiles = max(1, -(-n // 32768))
        cand = sorted({tiles, max(1, -(-tiles // 2)), max(1, -(-tiles // 4))})
        grids.append(min(cand, key=lambda wg: timed(n, wg)))

    def run():
        off = 0
        for c in range(reps):
            if (c % chains) == 0:
                off = 0
            for n, wg in zip(sizes, grids):
                n16 = (n + 15) // 16 * 16
                md.hbm_read_probe(src[off:off + n16], sink, workgroups=wg)
                off += (n16 + 255) // 256 * 256

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            run()
    torch.cuda.current_stream().wait_stream(s_)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del g, src
    torch.cuda.empty_cache()
    return {"bytes": list(sizes), "workgroups": grids, "us_per_chain": ms * 1e3, "GBps": sum(sizes) / (ms / 1e3) / 1e9,
            "timing": f"{reps} chains of back-to-back read-probe launches in one HIP graph"}


def environment():
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"torch": torch.__version__, "hip": torch.version.hip, "device": pr.name,
            "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "hbm_bytes": pr.total_memory, "kernel_source_sha256": kernel_source_hash(),
            "host_cpus": os.cpu_count()}


def source_hash():
    """SHA-256 over the files that make up the measured code: the library
    sources and header, its Python binding, the workload generators, the
    oracle and this script."""
    hs = hashlib.sha256()
    for sub, exts in (("include", (".h",)), ("moe_decode_amd", (".py",)), ("moe_decode_amd/csrc", (".hip", ".hpp", ".cpp")),
                      ("synth", (".py",)), ("oracle", (".c", ".h", ".py"))):
        d = os.path.join(ROOT, sub)
        for name in sorted(os.listdir(d)):
            if name.endswith(exts):
                hs.update(f"{sub}/{name}".encode())
                hs.update(open(os.path.join(d, name), "rb").read())
    hs.update(b"bench.py")
    hs.update(open(os.path.join(ROOT, "bench.py"), "rb").read())
    return hs.hexdigest()


def host_record():
    """CPU model, logical CPUs (all, and those this process may run on) and
    memory of the host, from /proc."""
    model, mem = None, None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                mem = int(line.split()[1]) * 1024
                break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": aff, "mem_bytes": mem}


def git_sha():
    """The checkout's commit, or (where the tree travelled without its
    history) the one the library was built from, as its build recorded it."""
    import subprocess
    try:
        r = subprocess.run(["git", "rev-parse", "HEAD"], cwd=ROOT, capture_output=True, text=True, timeout=10)
        if r.stdout.strip():
            return r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open(os.path.join(ROOT, "moe_decode_amd", "build_info.json")) as f:
            info = json.load(f)
        sha = info.get("git_sha")
        if sha and info.get("sources_differ_from_commit"):
            sha += " (library built from sources differing from it)"
        return sha
    except (OSError, ValueError):
        return None


def smi_snapshot():
    """GPU clocks and power from the SMI tool (a child process), or what it
    printed when it could not report them."""
    import subprocess
    for cmd in (["amd-smi", "metric", "-p", "-c", "--json"], ["rocm-smi", "--showpower", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except (OSError, subprocess.SubprocessError) as e:
            last = f"{cmd[0]}: {e}"
            continue
        if r.returncode == 0 and r.stdout.strip():
            try:
                return {"tool": " ".join(cmd), "data": json.loads(r.stdout)}
            except ValueError:
                return {"tool": " ".join(cmd), "text": r.stdout[:4000]}
        last = f"{' '.join(cmd)}: rc {r.returncode}: {(r.stderr or r.stdout)[:400]}"
    return {"error": last}


def run_tier(key, S, steps, warmup=16):
    """Decode through the host-memory expert tier: the expert set in pinned
    host memory, S slots of HBM caching it.  Tokens cycle through the seeded
    pool of 64, so a token's experts recur every 64 steps; the report gives
    the hit rate, the bytes copied for the misses and the rate of those
    copies.  Wall-clock timing: every call synchronises once (the routing is
    read back to plan the copies)."""
    import numpy as np
    import torch
    import moe_decode_amd as md
    from synth import workloads as W
    from synth.device import host_moe
    sp = W.spec(key)
    t = time.time()
    host = host_moe(sp)
    log(f"[bench] {key} expert set in pinned host memory ({time.time() - t:.1f} s)")
    tier = md.ExpertTier(host, S)
    rng = np.random.default_rng([sp.index, 777, 1, sp.variant])
    xs = torch.from_numpy(rng.standard_normal((POOL, 1, sp.H)).astype(np.float32)).cuda()
    y = torch.empty(1, sp.H, dtype=torch.float32, device="cuda")
    ws = torch.empty(tier.workspace_size(1), dtype=torch.uint8, device="cuda")
    for i in range(warmup):
        tier.forward(xs[i % POOL], y=y, workspace=ws)
    torch.cuda.synchronize()
    h0, m0 = tier.cache.hits, tier.cache.misses
    t0 = time.perf_counter()
    for i in range(steps):
        tier.forward(xs[(warmup + i) % POOL], y=y, workspace=ws)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    hits, misses = tier.cache.hits - h0, tier.cache.misses - m0
    miss_bytes = misses * sp.expert_bytes()
    del tier, host
    torch.cuda.empty_cache()
    return {"workload": key, "slots": S, "experts": sp.E, "steps": steps, "ms_per_step": dt * 1e3 / steps,
            "tokens_per_s": steps / dt, "hit_rate": hits / max(1, hits + misses),
            "miss_bytes_per_step": miss_bytes / steps, "miss_GBps": miss_bytes / dt / 1e9,
            "timing": "wall clock around the calls (each call synchronises once)"}


def copy_calibration(nbytes=1 << 30):
    """A plain 16-byte copy kernel of known size (the library's per-row-format
    layout pass, which is a copy): reads nbytes, writes nbytes."""
    import torch
    import moe_decode_amd as md
    cols = 8192
    rows = nbytes // cols
    src = torch.empty(rows * cols, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        md.prepare_layout("i8_row", rows, cols, 1, src, dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": rows * cols, "copy_bytes_written": rows * cols, "launches": 3}))


def decode_roofline(layers, sp, T, r):
    """Roofline of the dominant decode kernel (the selected experts' gate/up
    with the fused activation): its algorithmic bytes per launch over its
    average duration from back-to-back relaunches (HIP events), with the
    single-launch event time beside it."""
    import numpy as np
    kt = kernel_time(layers, sp, T, "gateup", n_inputs=32)
    kd = kernel_time(layers, sp, T, "down", n_inputs=32)
    gb = float(np.mean([gateup_bytes(sp, i) for i in kt["idx"]]))
    achieved = gb / (kt["ms_per_launch"] / 1e3) / 1e9
    kernel = "k_gateup_t1"
    return {
        "kernel": kernel + " (the selected experts' gate and up projections with the fused activation)",
        "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": traffic_record(kernel, f"{sp.key}_T{T}"),
        "bytes_per_launch": gb, "avg_launch_ms": kt["ms_per_launch"],
        "timing": f"{kt['launches']} back-to-back relaunches of the stage over {kt['inputs']} tokens' workspaces "
                  f"(HIP graph replays) between two HIP events",
        "event_launch_ms": r["stage_ms_avg"],
        "event_launch_GBps": r["stage_GBps"],
        "down_avg_launch_ms": kd["ms_per_launch"],
    }


def decode_leg(layers, sp, steps, warmup):
    """One-token decode of a layer given as identical copies used in turn:
    tokens/s, weight GB/s, each of its three launches (router; gate/up with
    the shared expert's gate/up when it rides in that launch; down with the
    combine) timed by back-to-back relaunches against the bytes it streams,
    and the chain of plain reads of those bytes as the floor of a chain of
    three launches."""
    import numpy as np
    r = run_mode(layers, sp, 1, steps, warmup, graph=True)
    n_ex = float(np.mean([len(np.unique(i)) for i in r["idx"]]))
    from synth.formats import matrix_bytes
    gu_routed = n_ex * 2 * matrix_bytes(sp.fmt, sp.F, sp.H)
    dn_routed = n_ex * matrix_bytes(sp.fmt, sp.H, sp.F)
    sh_gu = sh_dn = 0
    if sp.shared_F:
        sh_gu = 2 * matrix_bytes(sp.shared_fmt, sp.shared_F, sp.H)
        sh_dn = matrix_bytes(sp.shared_fmt, sp.H, sp.shared_F)
    stages = {"router": sp.router_bytes(), "gateup": gu_routed + sh_gu, "down": dn_routed + sh_dn}
    out = {"workload": f"{sp.key}: MoE layer decode, 1 token per step, {sp.E} experts top-{sp.k}, hidden {sp.H}, "
                       f"expert FFN {sp.F}, {sp.fmt} experts"
                       + (f", {sp.shared_fmt} shared expert (FFN {sp.shared_F})" if sp.shared_F else "")
                       + f", {len(layers)} copies of the layer in HBM used in turn",
           "steps": steps, "ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"],
           # the same steps captured in one HIP graph and replayed: the GPU's
           # time per step without the host's time per call (which is close
           # to this layer's short kernel chain)
           "graph_ms_per_step": r["graph_ms_per_step"],
           "host_us_per_call": r["host_us_per_call"],
           "weight_bytes_per_step": r["weight_bytes_per_step"], "weight_GBps": r["weight_GBps"],
           "weight_frac_of_8TBps": r["weight_GBps"] / HBM_PEAK_GBS, "launches": {}}
    for st, nbytes in stages.items():
        k = kernel_time(layers, sp, 1, st, n_inputs=32)
        out["launches"][st] = {"us": k["ms_per_launch"] * 1e3, "bytes": nbytes,
                               "GBps": nbytes / k["ms_per_launch"] / 1e6}
    floor = chain_floor([int(v) for v in stages.values()])
    out["chain_floor"] = floor
    out["step_over_chain_floor"] = r["ms_per_step"] * 1e3 / floor["us_per_chain"]
    return out


def prefill_leg(layers, sp, steps, warmup, cpu, sample_tokens, T=128):
    """A T-token chunk of a layer: tokens/s and weight GB/s over `steps`
    chunks, the roofline of the grouped gate/up GEMM with its matrix-core
    use, and the oracle on a sample of the chunk's tokens."""
    import numpy as np
    r = run_mode(layers, sp, T, steps, warmup)
    kt = kernel_time(layers, sp, T, "gateup", n_inputs=4)
    dtype = "int8" if sp.fmt.endswith("_row") else "bf16"
    kernel = "k_moe_mfma_i8" if dtype == "int8" else "k_moe_mfma"
    gb = float(np.mean([gateup_bytes(sp, i) for i in kt["idx"]]))
    achieved = gb / (kt["ms_per_launch"] / 1e3) / 1e9
    out = {
        "workload": f"{sp.key}: MoE layer, one {T}-token prefill chunk per step, {sp.E} experts top-{sp.k}, "
                    f"hidden {sp.H}, expert FFN {sp.F}, {sp.fmt} experts"
                    + (f", {sp.shared_fmt} shared expert (FFN {sp.shared_F})" if sp.shared_F else "")
                    + f", {len(layers)} cop{'y' if len(layers) == 1 else 'ies'} of the layer in HBM used in turn",
        "tokens_per_step": T, "steps": steps, "ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"],
        "weight_bytes_per_step": r["weight_bytes_per_step"], "weight_GBps": r["weight_GBps"],
        "weight_frac_of_8TBps": r["weight_GBps"] / HBM_PEAK_GBS,
        "arithmetic": ("int8 matrix cores on the weight codes against four int8 digits of 30-bit fixed-point "
                       "activation rows, exact int32 sums, fp32 combine" if dtype == "int8" else
                       "bf16 matrix cores on the exact weight codes against bf16 high and low halves of the "
                       "activations, fp32 accumulation, block scales in fp32"),
        "roofline": {
            "kernel": f"{kernel} (grouped gate/up GEMM with the fused activation)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic_record(kernel, f"{sp.key}_T{T}"),
            "bytes_per_launch": gb, "avg_launch_ms": kt["ms_per_launch"],
            "timing": f"{kt['launches']} back-to-back relaunches of the stage over {kt['inputs']} chunks' "
                      f"workspaces (HIP graph replays) between two HIP events",
            "event_launch_ms": r["stage_ms_avg"],
            "mfma": mfma_stats(sp, kt["idx"], kt["ms_per_launch"], dtype),
        },
        "step_ms_p10_p50_p90": r["step_ms_p10_p50_p90"],
        "inputs_sha256": r["inputs_sha256"],
    }
    if cpu:
        out["cpu_baseline"] = cpu_baseline(sp, T=T, sample_tokens=sample_tokens)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4_i4")
    ap.add_argument("--tokens", type=int, default=1, help="tokens per step (1 = decode; up to 128 = a prefill chunk)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="leave out the 128-token prefill legs and the c3 layer's decode leg")
    ap.add_argument("--modes", action="store_true", help="also time the other layer shapes")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--stack", type=int, default=0,
                    help="also time a stack of this many distinct layers (one token) captured in one HIP graph")
    ap.add_argument("--tier", type=int, default=0,
                    help="also time decode through a host-memory expert tier with this many HBM slots")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding of this layer is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import moe_decode_amd as md
    md.lib()
    if args.copy_calibration:
        copy_calibration()
        return

    from synth import workloads as W
    from synth.device import device_moe

    smi_before = smi_snapshot()
    sp = W.spec(args.workload)
    t = time.time()
    hashes = {}
    layer = device_moe(sp, hashes=hashes)
    torch.cuda.synchronize()
    log(f"[bench] {sp.key} resident in HBM ({time.time() - t:.1f} s to generate, hash and upload)")

    T = args.tokens
    r = run_mode(layer, sp, T, args.steps, args.warmup, graph=(T == 1))
    log(f"[bench] {sp.key} T={T}: {r['ms_per_step'] * 1e3:.1f} us/step, gate/up {r['stage_ms_avg'] * 1e3:.1f} us "
        f"(events around single launches)")
    roof = decode_roofline(layer, sp, T, r) if T <= 16 else None
    if roof:
        log(f"[bench] {sp.key} T={T}: gate/up {roof['avg_launch_ms'] * 1e3:.2f} us per launch back to back "
            f"({roof['achieved']:.0f} GB/s), down {roof['down_avg_launch_ms'] * 1e3:.2f} us")

    prefill = {}
    decode_c3 = None
    inputs = {sp.key: hashes}
    if not args.no_prefill and T == 1:
        steps_p = max(10, args.steps // 10)
        prefill[f"{sp.key}_T128"] = prefill_leg([layer], sp, steps_p, 3, not args.no_cpu_baseline, 16)
        log(f"[bench] {sp.key} T=128: {prefill[f'{sp.key}_T128']['ms_per_step'] * 1e3:.0f} us/chunk")
        del layer
        torch.cuda.empty_cache()
        s3 = W.spec("c3")
        h3 = {}
        copies = [device_moe(s3, hashes=h3)] + [device_moe(s3) for _ in range(3)]
        inputs["c3"] = h3
        prefill["c3_T128"] = prefill_leg(copies, s3, 2 * steps_p, 3, not args.no_cpu_baseline, 32)
        log(f"[bench] c3 T=128: {prefill['c3_T128']['ms_per_step'] * 1e3:.0f} us/chunk")
        decode_c3 = decode_leg(copies, s3, args.steps, args.warmup)
        log(f"[bench] c3 T=1: {decode_c3['ms_per_step'] * 1e3:.1f} us/step "
            f"({decode_c3['graph_ms_per_step'] * 1e3:.1f} as HIP-graph replays), launches "
            + ", ".join(f"{k} {v['us']:.1f} us" for k, v in decode_c3["launches"].items())
            + f"; chain of plain reads {decode_c3['chain_floor']['us_per_chain']:.1f} us")
        del copies
        torch.cuda.empty_cache()
        layer = None

    modes = {}
    if args.modes:
        if layer is None:
            layer = device_moe(sp)
        for Tm in (1, 4, 16, 128):   # 16: a speculative-decoding verify batch
            if Tm == T:
                continue
            m = run_mode(layer, sp, Tm, max(10, args.steps // (4 if Tm > 1 else 1)), 5)
            m.pop("idx")
            modes[f"{sp.key}_T{Tm}"] = m
            log(f"[bench] {sp.key} T={Tm}: {m['ms_per_step'] * 1e3:.1f} us/step")
        del layer
        layer = None
        torch.cuda.empty_cache()
        for key, name, batch in (("c1", "gate", 1), ("c1", "down", 1), ("c1", "q", 1), ("c1", "k", 1),
                                 ("c2", "w_10240x2560", 1), ("c2", "w_10240x2560", 8),
                                 ("c2", "w_2560x10240", 1), ("c2", "w_2560x10240", 8),
                                 ("q41", "w_10240x2560", 1), ("q41", "w_10240x2560", 8),
                                 ("q41", "w_2560x10240", 1), ("q41", "w_2560x10240", 8),
                                 ("i2", "gate_2048x6144", 1), ("i2", "gate_2048x6144", 4),
                                 ("i2", "down_6144x2048", 1), ("i2", "down_6144x2048", 4)):
            m = run_dense(key, name, batch, max(20, args.steps), 10)
            modes[f"{key}_{name}_b{batch}"] = m
            log(f"[bench] {key} {name} batch {batch}: {m['ms_per_call'] * 1e3:.1f} us ({m['weight_GBps']:.0f} GB/s)")
        for key, Ts in (("c4_i8", (1, 4, 128)), ("c4_i2", (1, 4, 128)), ("c4_q41", (1, 4, 128)),
                        ("c3", (1, 16, 128))):
            s2 = W.spec(key)
            # the 340 MB layer in four copies, used in turn (not served from the Infinity Cache)
            l2 = [device_moe(s2) for _ in range(4 if key == "c3" else 1)]
            for Tx in Ts:
                m = run_mode(l2, s2, Tx, max(10, args.steps // (4 if Tx > 1 else 1)), 5)
                m.pop("idx")
                modes[f"{key}_T{Tx}"] = m
                log(f"[bench] {key} T={Tx}: {m['ms_per_step'] * 1e3:.1f} us/step")
            del l2
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and T == 1:
        cpu = cpu_baseline(sp)
        one = cpu_baseline(sp, budget_s=3.0, threads=1)
        cpu["one_core"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}
        log(f"[bench] oracle: {cpu['value']:.3f} tokens/s on {cpu['cores']} threads, {one['value']:.3f} on one")

    probe = hbm_probe()
    log(f"[bench] HBM read probe: {probe['GBps']:.0f} GB/s over {probe['bytes'] >> 30} GiB")
    if roof:
        roof["hbm_read_probe_GBps"] = probe["GBps"]
        roof["frac_of_probe"] = roof["achieved"] / probe["GBps"]
        # the layer's three launches (router, gate/up, down) as plain reads of their weight bytes
        gu = roof["bytes_per_launch"]
        floor = chain_floor([sp.router_bytes(), int(gu), int(r["weight_bytes_per_step"] - gu - sp.router_bytes())])
        roof["chain_floor"] = floor
        roof["step_over_chain_floor"] = r["ms_per_step"] * 1e3 / floor["us_per_chain"]
        log(f"[bench] chain of plain reads of the same bytes: {floor['us_per_chain']:.1f} us "
            f"(step {r['ms_per_step'] * 1e3:.1f} us)")
    smi_after = smi_snapshot()

    inputs[f"{sp.key}_x_T{T}"] = r["inputs_sha256"]
    out = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32+f32",
        "data": "synthetic",
        "config": {
            "workload": f"{sp.key}: MoE layer {'decode' if T == 1 else 'forward'}, {T} token(s)/step, {sp.E} experts "
                        f"top-{sp.k}, hidden {sp.H}, expert FFN {sp.F}, {sp.fmt} weights (GeGLU), whole expert set "
                        f"resident in HBM",
            "tokens_per_step": T,
            "arithmetic": "integer dot products of weight codes with activation digit planes, exact int32 sums, "
                          "fp32 combine and accumulation" if T <= 16 else "matrix-core products, fp32 accumulation",
            "weight_bytes_per_step": r["weight_bytes_per_step"],
            "weight_GBps": r["weight_GBps"],
            "weight_frac_of_8TBps": r["weight_GBps"] / HBM_PEAK_GBS,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "prefill": prefill or None,
        "decode_c3": decode_c3,
        "timing": {
            "step_ms_p10_p50_p90": r["step_ms_p10_p50_p90"],
            "graph_ms_per_step": r["graph_ms_per_step"],
            "host_us_per_call": r["host_us_per_call"],
            "weight_frac_of_probe": r["weight_GBps"] / probe["GBps"],
            "hbm_read_probe": probe,
        },
        "records": {
            "git_sha": git_sha(),
            "source_sha256": source_hash(),
            "inputs_sha256": inputs,
            "host": host_record(),
            "smi_before": smi_before,
            "smi_after": smi_after,
        },
        "env": environment(),
    }
    if modes:
        out["modes"] = modes
    if args.stack > 0:
        out["stack"] = run_stack(args.workload, args.stack, 20)
        log(f"[bench] stack: {out['stack']['us_per_layer']:.1f} us per layer")
    if args.tier > 0:
        layer = None  # the resident copy is not needed any more
        torch.cuda.empty_cache()
        out["tier"] = run_tier(args.workload, args.tier, max(32, args.steps // 2))
        log(f"[bench] tier ({args.tier} slots): {out['tier']['tokens_per_s']:.0f} tokens/s, hit rate "
            f"{out['tier']['hit_rate']:.2f}, misses {out['tier']['miss_GBps']:.1f} GB/s")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
