/* moe_decode.h -- C ABI of libmoe_decode, the gfx950 (MI355X) library for the
 * decode / short-chunk prefill forward of a block-quantized feed-forward or
 * mixture-of-experts layer.
 *
 * The operations follow the pages' statement of the problem:
 *   - a quantized matrix-vector product over Q8_0 / Q4_0 blocks (the Camelid
 *     README, "Engine" and "Supported" sections: Q8_0 weights and Q4_0
 *     "wire GEMVs" checked against a CPU oracle) and over int8 / packed int4
 *     weights with one scale per row (the colibri summary, "model execution
 *     and memory tiers");
 *   - a router with top-k expert selection whose exact ties go to the lower
 *     expert index (the Camelid README, "Experimental lanes");
 *   - the MoE block: router -> top-k routed experts -> gated FFN (GeGLU) per
 *     selected expert -> combine, plus a dense shared-expert branch (the
 *     Camelid README, "Gemma 4": 128 experts, sparse top-8 plus a dense shared
 *     expert; the TurboFieldfare summary, "memory and expert streaming":
 *     router-chosen experts, shared branch computed alongside, prefill in
 *     chunks of at most 128 tokens reusing each expert across rows);
 *   - two more weight codecs: Q4_1 blocks (the Camelid README's bit-exact
 *     q4_1 GEMV) and packed int2 with one scale per row (the colibri summary);
 *   - a host-memory expert tier: the expert set in host RAM, a slot cache of
 *     experts in HBM (the Camelid README's experts-in-RAM lane with a VRAM
 *     expert cache; the TurboFieldfare summary's expert slots).
 *
 * Conventions (every entry point):
 *   - Pointers marked "device" are HIP device pointers, "host" are host
 *     pointers.  The caller allocates and owns every buffer and the stream; the
 *     library never allocates, frees or synchronizes (one exception, stated
 *     there: md_moe_cached_forward reads the routing back once per call).
 *     Work is enqueued on `stream` (NULL = the null stream) and completes
 *     asynchronously.
 *   - Every argument is validated on the host before anything is enqueued; a
 *     call that returns an error has enqueued nothing and written nothing
 *     (md_moe_cached_forward: nothing after the step that failed).
 *     Unsupported shapes return MD_ERR_UNSUPPORTED: there is no fallback.
 *   - Device data pointers must be 16-byte aligned (MD_ERR_ALIGNMENT).
 *   - md_last_error_detail() returns a thread-local message describing the
 *     last non-OK return on the calling thread.
 *   - Asynchronous faults surface through the HIP runtime on `stream`.
 *   - Results are deterministic: no float atomics; fixed reduction orders.
 *   - Calls that take a workspace may not overlap on the same workspace.
 *
 * Supported shapes: hidden / input widths (cols) are multiples of 256 and at
 * most 16384; rows 1..65536; E <= 256; 1 <= k <= 8; T <= 128 tokens per
 * layer call (longer prompts are split by the caller into chunks of at most
 * 128 tokens); batch <= 8 for md_qgemv.
 *
 * Accuracy contract.  Weights are decoded exactly (scale times code) and
 * every contraction y = sum_c w_c x_c is accumulated in fp32 or exactly in
 * integers; the router is accumulated in fp64 and rounded once.  The tolerance
 * the source pages' problem statement sets is
 *     |y - y_exact| <= 1e-4 * S + 1e-6,   S = sum_c |w_c x_c|,
 * and per path the library guarantees:
 *   - md_qgemv (every batch and format), and the FFN / MoE layers' chunks on
 *     block formats (Q8_0, Q4_0, Q4_1: bf16 matrix cores on the exact codes
 *     against activations split into two bf16 halves): the tolerance for
 *     every finite input.
 *   - FFN / MoE layers on the one-token kernels (up to 8 tokens, 16 on small
 *     layers; every format): the activations a 16-byte weight chunk
 *     multiplies -- a group g of 32 consecutive values for Q4_0 / Q4_1 /
 *     packed int4, 16 for Q8_0 / int8, 64 for packed int2 -- are rounded to
 *     integers of 2^-22 of the group's largest magnitude M_g before exact
 *     integer dot products.  Per contraction (gate, up, down, shared expert)
 *         |y - y_exact| <= 2^-22 * A + 2^-19 * S,
 *         A = sum_g M_g * sum_{c in g} |w_c|,
 *     which gives the tolerance whenever A <= 400 * S: a group's largest
 *     activation may exceed the typical magnitude of the activations that
 *     its weights multiply by up to about 400x.  Inputs outside that
 *     precondition (a group holding a value ~1000x the others, with the
 *     weights concentrated on the small ones) can exceed 1e-4 * S; the
 *     seeded workloads sit at A / S <= 15.
 *   - FFN / MoE layers' chunks on the per-row formats (int8, packed int4 /
 *     int2 with one scale per row: int8 matrix cores): each activation row
 *     (a token's x, a pair's h) is rounded to integers of 2^-30 of the row's
 *     largest magnitude M; per contraction
 *         |y - y_exact| <= 2^-30 * M * sum_c |w_c| + 2^-19 * S,
 *     which gives the tolerance whenever M * sum_c |w_c| <= 1e5 * S (the
 *     seeded workloads: <= 80).
 *   A layer's output additionally carries the effect of its gate/up
 *   contractions' error on h, as any fp32 evaluation does.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MD_ABI_VERSION 1

typedef enum md_status {
    MD_OK = 0,
    MD_ERR_INVALID_ARG = 1,   /* null pointer, bad enum value                 */
    MD_ERR_SHAPE = 2,         /* inconsistent dimensions                      */
    MD_ERR_UNSUPPORTED = 3,   /* valid but outside the supported set          */
    MD_ERR_ALIGNMENT = 4,     /* a device pointer is not 16-byte aligned      */
    MD_ERR_WORKSPACE = 5,     /* workspace missing or too small               */
    MD_ERR_HIP = 6            /* the HIP runtime reported a launch error      */
} md_status;

/* Weight formats.  Canonical layouts (as stored in GGUF-style files; the
 * oracle reads these):
 *   MD_Q8_0   rows of cols/32 blocks of 34 bytes: fp16 d (little-endian) then
 *             32 int8 q;  w = d * q.
 *   MD_Q4_0   rows of cols/32 blocks of 18 bytes: fp16 d then 16 bytes qs;
 *             weight j (0..15) is the low nibble n of qs[j], weight j+16 the
 *             high nibble;  w = d * (n - 8).
 *   MD_I8_ROW rows of cols int8 q; one fp32 scale s per row;  w = s * q.
 *   MD_I4_ROW rows of cols/2 bytes; weight 2j is the low nibble of byte j and
 *             2j+1 the high nibble, two's complement in [-8, 7]; one fp32
 *             scale s per row;  w = s * v.
 *   MD_Q4_1   rows of cols/32 blocks of 20 bytes: fp16 d, fp16 m, then 16
 *             bytes qs in the MD_Q4_0 nibble order, codes n in 0..15 with no
 *             offset;  w = d * n + m  (the Camelid README's bit-exact q4_1
 *             GEMV, "Experimental" rows).
 *   MD_I2_ROW rows of cols/4 bytes; weight 4j+i sits in bits 2i..2i+1 of byte
 *             j, two's complement in [-2, 1]; one fp32 scale s per row;
 *             w = s * v  (the colibri summary's packed int2 per-row format,
 *             "model execution and memory tiers").
 * Device layout (what every compute entry point reads; produced from the
 * canonical layout by md_prepare_layout, same byte count, same row stride):
 *   MD_Q8_0   per row: the cols int8 q of all blocks in order, then the
 *             cols/32 fp16 scales in order.
 *   MD_Q4_0   per row: the 16-byte qs of all blocks in order, then the
 *             cols/32 fp16 scales in order.
 *   MD_Q4_1   per row: the 16-byte qs of all blocks in order, then the
 *             cols/32 (d, m) fp16 pairs in order.
 *   MD_I8_ROW, MD_I4_ROW, MD_I2_ROW: identical to the canonical layout.
 * Every row therefore starts a run of 16-byte quant chunks that a wavefront
 * streams with coalesced 16-byte loads, scales kept out of the way.
 * Every type is taken by every entry point: md_qgemv, the FFN and MoE layers
 * (one-token kernels, grouped GEMMs) and the expert tier. */
typedef enum md_qtype {
  MD_Q8_0 = 1, MD_Q4_0 = 2, MD_I8_ROW = 3, MD_I4_ROW = 4, MD_Q4_1 = 5, MD_I2_ROW = 6
} md_qtype;

typedef enum md_xtype { MD_X_F32 = 0, MD_X_BF16 = 1 } md_xtype;

/* act(a) * u with act = tanh-form GELU (GeGLU) or SiLU (SwiGLU). */
typedef enum md_act { MD_ACT_GELU_TANH = 0, MD_ACT_SILU = 1 } md_act;

/* A quantized matrix (rows = outputs, cols = inputs), device layout. */
typedef struct md_qmatrix {
    int32_t type;              /* md_qtype                                    */
    int32_t rows, cols;
    const void *q;             /* device: rows * md_row_bytes(type, cols)     */
    const float *row_scale;    /* device: rows fp32 (the *_ROW types), else NULL */
} md_qmatrix;

/* A dense gated FFN: y = down( act(gate x) * (up x) ).
 * gate, up: F x H;  down: H x F;  all three of one type. */
typedef struct md_ffn {
    int32_t act;               /* md_act                                      */
    md_qmatrix gate, up, down;
} md_ffn;

/* One MoE layer.  The E experts of each projection are stored expert-major
 * and contiguous: expert e's gate matrix starts at gate_q + e * (F rows of
 * md_row_bytes(type, H)), its scales (the *_ROW types) at gate_scale + e*F;
 * likewise up (F x H) and down (H x F, scales at down_scale + e*H). */
typedef struct md_moe_layer {
    int32_t H, F, E, k;
    int32_t act;               /* md_act                                      */
    int32_t type;              /* md_qtype of the routed experts              */
    const void *gate_q, *up_q, *down_q;                /* device              */
    const float *gate_scale, *up_scale, *down_scale;   /* device or NULL      */
    const float *W_r;          /* device: E x H fp32 router weights           */
    const float *router_bias;  /* device: E fp32, or NULL                     */
    int32_t has_shared;        /* 1: add a dense shared expert (gate 1)       */
    md_ffn shared;             /* its gate/up F_s x H, down H x F_s           */
} md_moe_layer;

int32_t md_abi_version(void);
const char *md_status_string(md_status s);
const char *md_last_error_detail(void);

/* Bytes of one row in either layout (scales of the *_ROW types excluded);
 * -1 if cols is not valid for the type. */
int64_t md_row_bytes(int32_t type, int32_t cols);

/* Convert `count` consecutive matrices (rows x cols each) from the canonical
 * layout at `src` to the device layout at `dst` (both device, same size,
 * must not overlap).  One-time, at weight-load. */
md_status md_prepare_layout(int32_t type, int32_t rows, int32_t cols, int32_t count,
                            const void *src, void *dst, hipStream_t stream);

/* y[b][r] = sum_c w[r][c] * x[b][c] for b < batch (batch 1..8).
 * x: device, batch x cols, fp32 or bf16 (xtype); y: device, batch x rows fp32.
 * Accumulation in fp32.  Needs md_qgemv_workspace_size() bytes of workspace
 * (may be 0, then workspace may be NULL). */
md_status md_qgemv_workspace_size(const md_qmatrix *W /*host*/, int32_t batch, size_t *bytes /*host*/);
md_status md_qgemv(const md_qmatrix *W /*host*/, const void *x, int32_t xtype, int32_t batch, float *y,
                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Router for T tokens: logits l[t][e] = sum_c W_r[e][c] x[t][c] (+ bias[e]),
 * accumulated in fp64 and rounded to fp32; idx[t][0..k-1] = the k largest
 * logits in descending order, exact ties broken by the lower expert index
 * (-0 equals +0); gates[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over
 * the selected k.  idx (int32 T x k), gates (fp32 T x k) and logits (fp32
 * T x E, may be NULL) are device buffers.  Non-finite logits are outside the
 * contract (the selection is then unspecified). */
md_status md_route_workspace_size(int32_t T, int32_t H, int32_t E, int32_t k, size_t *bytes /*host*/);
md_status md_moe_route_topk(const float *x, int32_t T, int32_t H, const float *W_r, const float *bias,
                            int32_t E, int32_t k, int32_t *idx, float *gates, float *logits,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense gated FFN for T tokens (1..128): x, y device T x H fp32. */
md_status md_ffn_workspace_size(const md_ffn *f /*host*/, int32_t T, size_t *bytes /*host*/);
md_status md_ffn_forward(const md_ffn *f /*host*/, const float *x, int32_t T, float *y,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The MoE layer for T tokens (1..128):
 *   y[t] = sum_{j<k} gates[t][j] * FFN_{idx[t][j]}(x[t])  (+ shared FFN(x[t]))
 * x, y: device T x H fp32.  idx_out (int32 T x k) and gates_out (fp32 T x k)
 * receive the routing when non-NULL.  Only the selected experts' weight bytes
 * are read.  Up to 8 tokens (up to 16 on layers whose whole expert set takes
 * at most 512 MB) every (token, slot) pair runs as its own one-token problem,
 * so an expert that several tokens select is read once per such pair; the
 * layer runs as router, gate/up and down kernels (a shared expert runs inside
 * the routed launches where its shapes are covered, else as its own two
 * launches first).  Longer chunks group the pairs by expert and read each
 * selected expert once per 16-token tile of the tokens that chose it; their
 * shared expert, which needs only x, runs on a second stream of the
 * library's own (one per device, default priority, created at the device's
 * first such call) beside the routing kernels and joins `stream` before the
 * combine, so the call's work still starts after, and ends before, the
 * work around it on `stream` (a graph captured from `stream` takes the side
 * stream's launches in as a branch).  The results are those of the same
 * kernels on `stream` alone, bit for bit.  There is one code path per shape:
 * nothing in the environment selects another. */
md_status md_moe_workspace_size(const md_moe_layer *L /*host*/, int32_t T, size_t *bytes /*host*/);
md_status md_moe_layer_forward(const md_moe_layer *L /*host*/, const float *x, int32_t T, float *y,
                               int32_t *idx_out, float *gates_out,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* md_moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the scratch taken from a
 * 64 MiB array built into the library instead of a caller's workspace.
 * Every GPU the library runs on holds one such array from the library's
 * first use on it until the process ends; its address is looked up once per
 * device, on the first call with that device current.  This call allocates
 * and frees nothing and calls no allocating routine.  All calls on one GPU
 * share its array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialized by the caller; the array keeps the
 * last call's contents, and nothing in it needs to start cleared.
 * Everything runs on `stream` (no side stream).
 * Errors: as md_moe_layer_forward; a call whose scratch (the size
 * md_moe_workspace_size reports) exceeds 64 MiB -> MD_ERR_UNSUPPORTED, with
 * nothing enqueued (every layer and token count of the seeded workloads fits:
 * the largest, 128 tokens of a 256-expert layer of hidden size 6144, needs
 * about 62 MiB). */
md_status md_moe_layer_forward_noalloc(const md_moe_layer *L /*host*/, const float *x, int32_t T, float *y,
                                       int32_t *idx_out, float *gates_out, hipStream_t stream);

/* Measurement variant of md_moe_layer_forward: identical work and results,
 * every launch on `stream` (no side stream); additionally records `start` on
 * `stream` just before the launches of stage
 * `stage` and `stop` just after them (HIP events created by the caller), so
 * the elapsed time between the two events is that stage's time on the
 * stream.  A stage the call does not run (the shared expert of a layer
 * without one) records both events back to back; so do the stages that a
 * merged launch covers besides MD_STAGE_GATEUP, which then times the whole
 * merged work (few tokens, a layer with a shared expert on the shapes it
 * covers: the routed+shared gate/up and down launches). */
typedef enum md_stage {
    MD_STAGE_SHARED = 0,      /* dense shared-expert FFN                      */
    MD_STAGE_ROUTER = 1,      /* router logits                                */
    MD_STAGE_SELECT = 2,      /* top-k, gates, expert dispatch                */
    MD_STAGE_GATEUP = 3,      /* selected experts' gate/up + activation       */
    MD_STAGE_DOWN = 4,        /* selected experts' down projection            */
    MD_STAGE_COMBINE = 5      /* gate-weighted combine (+ shared)             */
} md_stage;
md_status md_moe_layer_forward_timed(const md_moe_layer *L /*host*/, const float *x, int32_t T, float *y,
                                     int32_t *idx_out, float *gates_out,
                                     void *workspace, size_t workspace_bytes, hipStream_t stream,
                                     int32_t stage, hipEvent_t start, hipEvent_t stop);

/* Measurement aid: enqueues only the launches of stage `stage` (md_stage) of
 * md_moe_layer_forward with the same arguments, which read the intermediate
 * results that an earlier such call left in `workspace` (and in idx_out /
 * gates_out); the stage's outputs are rewritten with the same values.
 * Relaunching one stage back to back over several workspaces, each left by a
 * different token's call, times that stage's kernels on their real inputs
 * with nothing else in between (HIP events around the whole run give the
 * kernels' average duration, without the dispatch latency that events around
 * one launch add).  The workspace must hold what the earlier call with the
 * same layer, x, T and outputs wrote, untouched since.  Errors: as
 * md_moe_layer_forward; a stage outside 0..5 -> MD_ERR_INVALID_ARG. */
md_status md_moe_layer_stage_relaunch(const md_moe_layer *L /*host*/, const float *x, int32_t T, float *y,
                                      int32_t *idx_out, float *gates_out, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream, int32_t stage);

/* md_moe_layer_forward with a residual: y = residual + layer(x), residual an
 * fp32 [T][H] device buffer (it may be x or y itself).  The residual is added
 * in the layer's last kernel (the down projection or the combine, after the
 * shared expert's output), so layers stack without an extra launch each (the
 * Camelid README, "Gemma 4": resident layer weights and a captured decode
 * graph).  Errors: as md_moe_layer_forward; a null residual ->
 * MD_ERR_INVALID_ARG; not 16-byte aligned -> MD_ERR_ALIGNMENT. */
md_status md_moe_layer_forward_residual(const md_moe_layer *L /*host*/, const float *x, int32_t T,
                                        const float *residual, float *y, int32_t *idx_out, float *gates_out,
                                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* y = a + b over n fp32 values (device pointers; y may alias a or b): the
 * residual add that joins stacked layers, so a stack of layers (each layer's
 * output added to its input) runs as one sequence of this library's kernels
 * that a caller can capture in a HIP graph and replay without host
 * synchronization (the Camelid README, "Gemma 4": a GPU-resident decode path
 * with resident layer weights and a captured decode graph; "Ornith 1.0 9B": a
 * device-side decode loop, the host synchronizing once per token chunk).
 * Errors: n <= 0 -> MD_ERR_SHAPE; a null pointer -> MD_ERR_INVALID_ARG;
 * pointers not 16-byte aligned -> MD_ERR_ALIGNMENT. */
md_status md_add(const float *a, const float *b, float *y, int64_t n, hipStream_t stream);

/* The experts of a layer for a given routing: y[t] = sum_j gates[t][j] *
 * FFN_{idx[t][j]}(x[t]) -- the layer forward without the router (the
 * TurboFieldfare summary, "memory and expert streaming": the runtime splits
 * the router's choices into cache hits and misses before the experts run).
 * idx, gates: device [T][k] (int32, fp32); a token's k entries must be
 * distinct; entries outside [0, E) are clamped into it.  A shared expert
 * is added as in md_moe_layer_forward.  Needs md_moe_workspace_size(L, T)
 * bytes of workspace.  Errors as md_moe_layer_forward. */
md_status md_moe_experts_forward(const md_moe_layer *L /*host*/, const float *x, int32_t T, const int32_t *idx,
                                 const float *gates, float *y, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Host-memory expert tier with an HBM slot cache (the Camelid README,
 * "Supported": experts kept in host RAM with a VRAM-resident expert cache;
 * the TurboFieldfare summary, "memory and expert streaming": a fixed number
 * of expert slots per layer, least-frequently-used replacement with a
 * recency tie-break, the router's choices split into hits and misses; the
 * colibri summary, "model execution and memory tiers": per-layer caches of
 * hot experts).  The whole expert set lives in host memory (pinned, so the
 * copies run asynchronously), S slots of the same layout in HBM.  All arrays
 * of the struct are host memory owned by the caller. */
typedef struct md_expert_cache {
  int32_t E;                 /* experts of the layer                              */
  int32_t S;                 /* HBM slots                                         */
  int32_t *slot_of_expert;   /* [E]: the slot holding expert e, or -1             */
  int32_t *expert_in_slot;   /* [S]: the expert a slot holds, or -1 (empty)       */
  int64_t *uses;             /* [S]: selections of the slot's expert since loaded */
  int64_t *last_use;         /* [S]: the plan step that last selected it          */
  int32_t *slot_idx;         /* [T*k] scratch of md_moe_cached_forward            */
  int64_t step;              /* plan steps so far                                 */
  int64_t hits, misses;      /* distinct-expert hits and misses so far            */
} md_expert_cache;

/* Empties the cache (all slots free, counters zero).  Errors: a null pointer
 * -> MD_ERR_INVALID_ARG; E or S <= 0 -> MD_ERR_SHAPE. */
md_status md_expert_cache_reset(md_expert_cache *c /*host*/);

/* One step of the replacement policy for the n = T*k expert ids in idx
 * (host): every distinct expert already in a slot is a hit (its use count
 * and last use updated); every other one, in order of first appearance,
 * takes an empty slot (lowest index first) or else evicts the slot with the
 * fewest uses, ties to the least recently used, then to the lowest index,
 * among the slots this step has not used.  Writes slot_idx[i] = the slot of
 * idx[i], and the misses as (miss_expert, miss_slot) pairs, *n_miss of them
 * (host arrays of n entries).  Errors: an id outside [0, E) or a null
 * pointer -> MD_ERR_INVALID_ARG; n outside 1..1024 -> MD_ERR_SHAPE; more
 * distinct experts than slots -> MD_ERR_UNSUPPORTED; nothing changes on
 * error. */
md_status md_expert_cache_plan(md_expert_cache *c /*host*/, const int32_t *idx, int32_t n, int32_t *slot_idx,
                               int32_t *miss_expert, int32_t *miss_slot, int32_t *n_miss);

/* Enqueues the copies of the missed experts' gate, up and down matrices (and
 * row scales) from src (E experts, usually pinned host memory) into the
 * slots of dst (a layer descriptor whose E is the slot count, in HBM) on
 * stream.  Errors: src and dst of different H, F, type, act or k ->
 * MD_ERR_SHAPE; an expert or slot out of range or a null pointer ->
 * MD_ERR_INVALID_ARG. */
md_status md_expert_cache_fill(const md_moe_layer *src /*host*/, const md_moe_layer *dst /*host*/,
                               const int32_t *miss_expert, const int32_t *miss_slot, int32_t n_miss,
                               hipStream_t stream);

/* The layer forward with the expert tier: the router and top-k on the GPU
 * (src's W_r / router_bias, device memory), one read-back of the routing
 * (this call synchronizes the stream once), the cache plan, the copies of
 * the misses, then md_moe_experts_forward on the slots with the slot ids.
 * With a copy_stream (and an event copy_done to join it), the misses load on
 * it while dst's shared expert (resident) runs on stream, and the routed
 * experts wait for the copies (the TurboFieldfare summary: misses filled
 * while the shared branch computes); a null copy_stream puts the copies on
 * stream.  idx_out / gates_out (device, nullable) receive the expert ids and
 * gates.  c->slot_idx must hold T*k entries and stay untouched until the
 * next call on the stream (an asynchronous copy reads it).  Workspace:
 * md_moe_cached_workspace_size.  A cache (and its slots) must be used from
 * one compute stream: the call's one synchronisation orders the copies into
 * the slots after the previous calls' reads of them only on that stream.
 * Errors: as md_moe_layer_forward, md_expert_cache_plan and
 * md_expert_cache_fill; a cache whose E / S differ from src->E / dst->E ->
 * MD_ERR_SHAPE; a copy_stream without an event -> MD_ERR_INVALID_ARG.  An
 * error after the plan (a copy or a launch that fails) marks the slots the
 * plan gave to missed experts empty, so their contents are never taken for
 * those experts (nor for the experts they held before). */
md_status md_moe_cached_workspace_size(const md_moe_layer *src /*host*/, const md_moe_layer *dst /*host*/, int32_t T,
                                       size_t *bytes /*host*/);
md_status md_moe_cached_forward(const md_moe_layer *src /*host*/, const md_moe_layer *dst /*host*/,
                                md_expert_cache *c /*host*/, const float *x, int32_t T, float *y, int32_t *idx_out,
                                float *gates_out, void *workspace, size_t workspace_bytes, hipStream_t stream,
                                hipStream_t copy_stream, hipEvent_t copy_done);

/* Measurement aid: reads nbytes of device memory at src once, in address
 * order, with every compute unit busy, and writes nothing unless some lane's
 * xor of the 32-bit words it read equals key (then that lane stores key at
 * sink[0]; for zeroed memory any nonzero key keeps sink untouched).  Timed over a buffer far larger than the caches it gives the HBM
 * read bandwidth this device attains, the practical ceiling of the weight
 * streams above (the Camelid README, "Gemma 4": GPU-resident decode runs at
 * the memory-bandwidth wall).  workgroups: the grid (0 picks 2048; at most
 * one workgroup per 32 KB tile is launched); each workgroup takes its tiles
 * in groups of up to four consecutive ones, every load of a group in flight
 * before any is used.
 * Errors: null pointer -> MD_ERR_INVALID_ARG; nbytes 0 or not a multiple of
 * 16 -> MD_ERR_SHAPE; src not 16-byte aligned -> MD_ERR_ALIGNMENT;
 * workgroups < 0 or > 2^20 -> MD_ERR_INVALID_ARG. */
md_status md_hbm_read_probe(const void *src, size_t nbytes, uint32_t key, uint32_t *sink, int32_t workgroups,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
