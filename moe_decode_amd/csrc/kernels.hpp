// kernels.hpp -- launch interface between the host entry points (abi.cpp)
// and the HIP kernels.  Internal to libmoe_decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace md {

// Routing hand-off in device memory.  Pair p = t*k + j is token t's slot j.
// Pairs are grouped by expert (ascending expert id, then ascending p);
// "position" q is a pair's index in that order.  h and o rows are indexed by
// position.  A dense FFN uses n_active == nullptr: one expert (0) whose
// positions are the tokens 0..T-1.
struct Disp {
  const int* n_active;     // [1]
  const int* active_e;     // [n_active]
  const int* active_off;   // [n_active + 1]  positions of each expert's pairs
  const int* pairs;        // [T*k]  pair id at each position
  int k;                   // slots per token (1 for a dense FFN)
  int T;                   // tokens (dense FFN)
  // [max_tiles(...)] work items of the grouped GEMMs, one per 16-position
  // tile of an active expert: {expert, first position, end of the expert's
  // positions, 0}, experts ascending, tiles ascending; expert -1 past the end
  const int4* items;
};

struct DispOut {
  int* n_active;
  int* active_e;
  int* active_off;
  int* pairs;
  int* pos_of_pair;
  int4* items;
  int n_items_max;
};

constexpr int kTokTile = 16;  // positions per matrix-core tile of the grouped GEMMs

// Most tokens per call on the one-token kernels ((token, slot) pairs; the
// router's partial-sum plan); more go to the grouped GEMMs.
#ifndef MD_MAX_PAIR_T
#define MD_MAX_PAIR_T 8
#endif
constexpr int kMaxPairT = MD_MAX_PAIR_T;
// The same for layers whose whole expert set is small (at most 512 MB): their
// frequently chosen experts stay in the 256 MB Infinity Cache, so re-reading
// an expert once per (token, slot) pair stays cheaper than grouping.
constexpr int kMaxPairTSmall = 16;
constexpr int64_t kSmallExpertSet = int64_t(512) << 20;

// Bound on the work items: sum over active experts of ceil(n_e / 16) is at
// most T*k / 16 + (active experts).
inline int max_tiles(int T, int k, int n_active_max) { return n_active_max + (T * k + kTokTile - 1) / kTokTile; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Digit planes (digits.hpp) of the rows of an R x K fp32 matrix, in the
// layout of weight format fmt: planes [R][K/NV][NPL] x 16 bytes, scales
// [R][K/NV].  x == nullptr: nothing to do.
struct DigJob {
  const float* x;
  int R, K, fmt;
  u32x4* planes;
  float* scales;
};
hipError_t launch_digits(const DigJob& j, hipStream_t st);

struct GemvCfg {
  int L;        // lanes per row group (8..64)
  int R;        // rows per lane group
  int B;        // tokens per pass (template width)
  int S;        // K splits (qgemv only)
  int rows_per_block;
  dim3 grid;
};

// ---- launchers (return hipGetLastError() of the launch) -------------------
int device_cus();  // compute units of the current device (cached)
hipError_t launch_prepare_layout(int fmt, int rows, int cols, int count, const void* src, void* dst,
                                 hipStream_t st);

GemvCfg qgemv_config(int fmt, int N, int K, int batch);
hipError_t launch_qgemv(int fmt, int xt, const GemvCfg& c, const uint8_t* W, const float* scales, int N, int K,
                        const void* x, int batch, float* y, float* partial, hipStream_t st);

// Router logits come as S K-slices of fp64 partials, element (s, t, e) at
// part[s*ps + t*pt + e*pe]: [t][e][s] for a few tokens (the layout the
// one-token gate/up kernel reads), [s][t][e] for a chunk (router GEMM).
struct RouterPlan {
  bool gemm;
  int S;
  int64_t ps, pt, pe;
};
// pairs: the one-token kernels consume the partials (partial-sum plan for any
// T up to kMaxPairTSmall); otherwise the plan follows T alone.
RouterPlan router_plan(int T, int H, int E, bool pairs = false);
int router_splits(int H, int E);
hipError_t launch_router_part(const float* x, int T, int H, const float* Wr, int E, int S, double* part,
                              const DigJob& j0, const DigJob& j1, hipStream_t st);
// Also runs the digit jobs j0, j1 (small-T plan only; the GEMM plan rejects
// them).  x_hi, x_lo (GEMM plan only, nullable): also write x as bf16 pairs
// (hi = bf16(x), lo = bf16(x - hi)) from the tiles the router stages.
hipError_t launch_router(const float* x, int T, int H, const float* Wr, int E, const RouterPlan& p, double* part,
                         const DigJob& j0, const DigJob& j1, hipStream_t st, unsigned short* x_hi = nullptr,
                         unsigned short* x_lo = nullptr);
hipError_t launch_select(const double* part, const RouterPlan& p, const float* bias, int T, int E, int k,
                         float* logits, int* idx, float* gates, hipStream_t st);
hipError_t launch_dispatch(const int* idx, int T, int E, int k, const DispOut& d, hipStream_t st);

// one-token decode path (decode.hip)
bool t1_supported(int fmt, int H, int F);
// x and h enter as digit planes (planes, scales) in the weights' format.
hipError_t launch_gateup_t1(int fmt, const uint8_t* gq, const uint8_t* uq, const float* gs, const float* us,
                            int64_t mat_bytes, int F, int H, int act, int E, int k, int T, const double* part, int S,
                            const float* bias, const void* xd, const float* xsc, void* hd, float* hsc, int* idx_out,
                            float* gates_out, hipStream_t st, const int* idx_in = nullptr);
hipError_t launch_down_t1(int fmt, const uint8_t* dq, const float* ds, int64_t mat_bytes, int H, int F, int k, int T,
                          const int* idx, const float* gates, const void* hd, const float* hsc, const float* y_add,
                          float* y, hipStream_t st);

// few tokens, layer with a shared expert: routed and shared gate/up in one
// launch, routed and shared down (with the combine) in another (decode.hip)
struct RsLaunch {
  int fmt;
  const uint8_t *gq, *uq, *dq;
  const float *gs, *us, *ds;                // row scales (per-row formats) or nullptr
  int64_t gu_bytes, dn_bytes;
  int F, act, H, E, k, T;
  const double* part;                       // router partials [T][E][S]
  int S;
  const float* bias;
  const void* xd;                           // x digit planes / scales (routed format)
  const float* xsc;
  void* hd;                                 // h digit planes / scales [T*k]
  float* hsc;
  int sfmt;
  const uint8_t *sgq, *suq, *sdq;
  const float *sgs, *sus, *sds;
  int Fs, sact;
  const void* sxd;
  const float* sxsc;
  void* shd;                                // [T]
  float* shsc;
  int* idx;
  float* gates;
  float* y;
  const float* residual;                    // added to y, or nullptr
  int parts = 3;                            // 1: the gate/up launch, 2: the down launch, 3: both
};
bool rs_supported(int fmt, int H, int F, int sfmt, int Fs, int k, int T);
hipError_t launch_moe_rs(const RsLaunch& L, hipStream_t st);

// prefill grouped GEMM on the matrix cores (prefill.hip)
hipError_t launch_split_bf16(const float* x, int64_t n, unsigned short* hi, unsigned short* lo, hipStream_t st);
bool mfma_supported(int K);
hipError_t launch_moe_mfma(int fmt, bool gateup, const uint8_t* wq, const uint8_t* wq2, const float* ws,
                           const float* ws2, int64_t mat_bytes, int M, int K, int act, const Disp& d, int n_items,
                           const unsigned short* a_hi, const unsigned short* a_lo, bool act_by_token, float* out,
                           unsigned short* out_hi, unsigned short* out_lo, hipStream_t st);

// dense GEMV of T <= 16 tokens on the matrix cores (block formats), K split
// in ks ranges: partials [ks][T][M] in out (reduce with launch_splitk_reduce)
int mfma_gemv_splits(int fmt, int M, int K);
hipError_t launch_mfma_gemv(int fmt, const uint8_t* wq, const float* ws, int M, int K, int T, const uint16_t* a_hi,
                            const uint16_t* a_lo, int ks, float* out, hipStream_t st);
hipError_t launch_splitk_reduce(const float* part, int S, int64_t n, float* y, hipStream_t st);

hipError_t launch_limbs(const float* a, int R, int K, int fmt, int8_t* digits, int* expo, hipStream_t st);
hipError_t launch_moe_mfma_i8(int fmt, bool gateup, const uint8_t* wq, const uint8_t* wq2, const float* ws,
                              const float* ws2, int64_t mat_bytes, int M, int K, int act, const Disp& d,
                              int n_items, const int8_t* digits, const int* expo, bool act_by_token, float* out,
                              hipStream_t st);

GemvCfg gateup_config(int fmt, int F, int H, int max_active, int T);
hipError_t launch_gateup(int fmt, const GemvCfg& c, const uint8_t* gq, const uint8_t* uq, const float* gs,
                         const float* us, int64_t mat_bytes, int F, int H, int act, const Disp& d,
                         const float* x, float* h, hipStream_t st);

GemvCfg down_config(int fmt, int H, int F, int max_active, int T);
hipError_t launch_down(int fmt, const GemvCfg& c, const uint8_t* dq, const float* ds, int64_t mat_bytes,
                       int H, int F, const Disp& d, const float* h, float* o, hipStream_t st);

hipError_t launch_add(const float* a, const float* b, float* y, int64_t n, hipStream_t st);
// Streams nbytes = 16 * n16 of src through the CUs with `grid` workgroups
// (no write unless a lane's words xor to key).
hipError_t launch_read_probe(const void* src, int64_t n16, uint32_t key, uint32_t* sink, int grid,
                             hipStream_t st);
hipError_t launch_copy_f32(const float* a, float* y, int64_t n, hipStream_t st);
// out[i] = in[i] clamped into [0, E), i < n
hipError_t launch_clamp_idx(const int* in, int n, int E, int* out, hipStream_t st);
hipError_t launch_combine(const float* o, const int* pos_of_pair, const float* gates, int T, int k, int H,
                          const float* y_shared, const float* y_residual, float* y, hipStream_t st);

}  // namespace md
