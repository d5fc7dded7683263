// abi.cpp -- the C entry points of libmoe_decode: host-side validation (every
// check runs before anything is enqueued), workspace layout, and the launch
// sequence of each operation.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "moe_decode.h"
#include "common.hpp"
#include "digits.hpp"
#include "kernels.hpp"

namespace {

thread_local char g_detail[512] = "";

md_status fail(md_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return s;
}

md_status ok() {
  g_detail[0] = 0;
  return MD_OK;
}

md_status hip_fail(hipError_t e, const char* what) {
  return fail(MD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_type(int32_t t) { return t >= MD_Q8_0 && t <= MD_I2_ROW; }
bool row_type(int32_t t) { return t == MD_I8_ROW || t == MD_I4_ROW || t == MD_I2_ROW; }

constexpr int kMaxCols = 16384;
constexpr int kMaxRows = 65536;
constexpr int kMaxT = 128;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;
constexpr int kMaxBatch = 8;
// Up to this many tokens, every (token, slot) pair runs as its own one-token
// problem in one launch; above it the pairs are grouped by expert.
using md::kMaxPairT;

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

md_status check_width(const char* what, int32_t n) {
  if (n <= 0) return fail(MD_ERR_SHAPE, "%s = %d must be positive", what, n);
  if (n % 256 || n > kMaxCols)
    return fail(MD_ERR_UNSUPPORTED, "%s = %d: supported widths are multiples of 256 up to %d", what, n, kMaxCols);
  return MD_OK;
}

md_status check_qmatrix(const char* what, const md_qmatrix* W) {
  if (!W) return fail(MD_ERR_INVALID_ARG, "%s: null matrix descriptor", what);
  if (!valid_type(W->type)) return fail(MD_ERR_INVALID_ARG, "%s: unknown type %d", what, W->type);
  if (W->rows <= 0 || W->cols <= 0) return fail(MD_ERR_SHAPE, "%s: rows %d cols %d", what, W->rows, W->cols);
  if (W->rows > kMaxRows) return fail(MD_ERR_UNSUPPORTED, "%s: rows %d > %d", what, W->rows, kMaxRows);
  md_status s = check_width(what, W->cols);
  if (s != MD_OK) return s;
  if (!W->q) return fail(MD_ERR_INVALID_ARG, "%s: null weights", what);
  if (!aligned16(W->q)) return fail(MD_ERR_ALIGNMENT, "%s: weights not 16-byte aligned", what);
  if (row_type(W->type)) {
    if (!W->row_scale) return fail(MD_ERR_INVALID_ARG, "%s: per-row type without row_scale", what);
    if (!aligned16(W->row_scale)) return fail(MD_ERR_ALIGNMENT, "%s: row_scale not 16-byte aligned", what);
  }
  return MD_OK;
}

md_status check_ffn(const md_ffn* f, int32_t H) {
  if (!f) return fail(MD_ERR_INVALID_ARG, "null FFN descriptor");
  if (f->act != MD_ACT_GELU_TANH && f->act != MD_ACT_SILU) return fail(MD_ERR_INVALID_ARG, "unknown act %d", f->act);
  md_status s;
  if ((s = check_qmatrix("ffn.gate", &f->gate)) != MD_OK) return s;
  if ((s = check_qmatrix("ffn.up", &f->up)) != MD_OK) return s;
  if ((s = check_qmatrix("ffn.down", &f->down)) != MD_OK) return s;
  if (f->gate.type != f->up.type || f->gate.type != f->down.type)
    return fail(MD_ERR_UNSUPPORTED, "ffn: gate/up/down must share one type");
  const int F = f->gate.rows;
  if (f->gate.cols != H || f->up.cols != H || f->up.rows != F || f->down.rows != H || f->down.cols != F)
    return fail(MD_ERR_SHAPE, "ffn: gate/up must be F x H and down H x F (H=%d)", H);
  return check_width("ffn F", F);
}

int max_active(int T, int E, int k) { return T * k < E ? T * k : E; }

// Digit planes of an R x K activation matrix (one-token kernels): planes,
// then scales.
struct DigBuf {
  void* planes;
  float* scales;
};
size_t dig_buf_bytes(int fmt, int R, int K) {
  return align256((size_t)R * md::dig_bytes(fmt, K)) + align256(sizeof(float) * (size_t)R * (K / md::dig_nv(fmt)));
}
DigBuf dig_buf_at(char* base, int fmt, int R, int K) {
  return DigBuf{base, reinterpret_cast<float*>(base + align256((size_t)R * md::dig_bytes(fmt, K)))};
}
md::DigJob dig_job(const float* x, int R, int K, int fmt, const DigBuf& b) {
  return md::DigJob{x, R, K, fmt, static_cast<md::u32x4*>(b.planes), b.scales};
}

// ---- MoE workspace layout ------------------------------------------------
struct MoeWs {
  size_t part, logits, idx, gates, n_active, active_e, active_off, pairs, pos, items, h, o, h_s, y_s, total;
  size_t x_hi, x_lo, h_hi, h_lo, hs_hi, hs_lo;  // bf16 pairs of the prefill path (block formats)
  size_t x_dig, x_exp, h_dig, h_exp, hs_dig, hs_exp;  // int8 digit planes (per-row formats)
  size_t xs_dig, xs_exp;  // x digits in the shared expert's order
  size_t xs_hi, xs_lo;    // x as bf16 pairs for the shared expert (its own: it may run on another stream)
  size_t xd, sxd, hd, shd;  // digit planes of x and h for the one-token kernels (routed, shared formats)
  size_t rcopy;             // the residual's copy where y, which it may be, is written before it is added
};

// Few tokens on shapes the one-token kernels cover: independent (token, slot)
// pairs; otherwise the grouped GEMM on the matrix cores.
// Measured crossover (MI355X, µs per layer call, one-token kernels vs grouped
// GEMMs): 256 experts of 19 MB (int4): 10 tokens 355 vs 354, 12: 410 vs 398;
// of 38 MB (int8): 10 tokens 554 vs 539; 128 experts of 2.65 MB with a shared
// expert: 12 tokens 122 vs 148, 16: 158 vs 163.
int pair_limit(const md_moe_layer* L) {
  const int64_t expert = 2 * (int64_t)L->F * md::row_bytes(L->type, L->H) + (int64_t)L->H * md::row_bytes(L->type, L->F);
  return (int64_t)L->E * expert <= md::kSmallExpertSet ? md::kMaxPairTSmall : kMaxPairT;
}
bool use_pairs(const md_moe_layer* L, int T) {
  return T <= pair_limit(L) && md::t1_supported(L->type, L->H, L->F) &&
         (!L->has_shared || md::t1_supported(L->shared.gate.type, L->H, L->shared.gate.rows));
}

MoeWs moe_ws(const md_moe_layer* L, int T) {
  MoeWs w{};
  const int E = L->E, k = L->k, H = L->H, F = L->F;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  w.part = take(sizeof(double) * (size_t)T * E * md::router_plan(T, H, E, use_pairs(L, T)).S);
  w.logits = take(sizeof(float) * T * E);
  w.idx = take(sizeof(int) * T * k);
  w.gates = take(sizeof(float) * T * k);
  w.n_active = take(sizeof(int));
  w.active_e = take(sizeof(int) * E);
  w.active_off = take(sizeof(int) * (E + 1));
  w.pairs = take(sizeof(int) * T * k);
  w.pos = take(sizeof(int) * T * k);
  w.h = take(sizeof(float) * (size_t)T * k * F);
  if (L->has_shared) {
    w.h_s = take(sizeof(float) * (size_t)T * L->shared.gate.rows);
    w.y_s = take(sizeof(float) * (size_t)T * H);
  }
  if (use_pairs(L, T)) {
    w.xd = take(dig_buf_bytes(L->type, T, H));
    w.hd = take(dig_buf_bytes(L->type, T * k, F));
    if (L->has_shared) {
      w.sxd = take(dig_buf_bytes(L->shared.gate.type, T, H));
      w.shd = take(dig_buf_bytes(L->shared.gate.type, T, L->shared.gate.rows));
    }
    w.rcopy = take(sizeof(float) * (size_t)T * H);
  } else {
    w.items = take(sizeof(int4) * (size_t)md::max_tiles(T, k, max_active(T, E, k)));
    w.o = take(sizeof(float) * (size_t)T * k * H);
    w.x_hi = take(2 * (size_t)T * H);
    w.x_lo = take(2 * (size_t)T * H);
    w.x_dig = take(4 * (size_t)T * H);
    w.x_exp = take(sizeof(int) * (size_t)T);
    w.h_hi = take(2 * (size_t)T * k * F);
    w.h_lo = take(2 * (size_t)T * k * F);
    w.h_dig = take(4 * (size_t)T * k * F);
    w.h_exp = take(sizeof(int) * (size_t)T * k);
    if (L->has_shared) {
      const size_t Fs = L->shared.gate.rows;
      w.hs_hi = take(2 * (size_t)T * Fs);
      w.hs_lo = take(2 * (size_t)T * Fs);
      w.hs_dig = take(4 * (size_t)T * Fs);
      w.hs_exp = take(sizeof(int) * (size_t)T);
      w.xs_dig = take(4 * (size_t)T * H);
      w.xs_exp = take(sizeof(int) * (size_t)T);
      w.xs_hi = take(2 * (size_t)T * H);
      w.xs_lo = take(2 * (size_t)T * H);
    }
  }
  w.total = off;
  return w;
}

md_status check_moe(const md_moe_layer* L, int32_t T) {
  if (!L) return fail(MD_ERR_INVALID_ARG, "null layer descriptor");
  if (T <= 0) return fail(MD_ERR_SHAPE, "T = %d must be positive", T);
  if (T > kMaxT) return fail(MD_ERR_UNSUPPORTED, "T = %d: at most %d tokens per call (split longer chunks)", T, kMaxT);
  md_status s;
  if ((s = check_width("H", L->H)) != MD_OK) return s;
  if ((s = check_width("F", L->F)) != MD_OK) return s;
  if (L->E <= 0 || L->k <= 0) return fail(MD_ERR_SHAPE, "E = %d, k = %d", L->E, L->k);
  if (L->k > L->E) return fail(MD_ERR_SHAPE, "k = %d > E = %d", L->k, L->E);
  if (L->E > kMaxE || L->k > kMaxK) return fail(MD_ERR_UNSUPPORTED, "E <= %d and k <= %d are supported", kMaxE, kMaxK);
  if (L->act != MD_ACT_GELU_TANH && L->act != MD_ACT_SILU) return fail(MD_ERR_INVALID_ARG, "unknown act %d", L->act);
  if (!valid_type(L->type)) return fail(MD_ERR_INVALID_ARG, "unknown expert type %d", L->type);
  if (!L->gate_q || !L->up_q || !L->down_q || !L->W_r) return fail(MD_ERR_INVALID_ARG, "null expert or router weights");
  if (!aligned16(L->gate_q) || !aligned16(L->up_q) || !aligned16(L->down_q) || !aligned16(L->W_r) ||
      (L->router_bias && !aligned16(L->router_bias)))
    return fail(MD_ERR_ALIGNMENT, "expert/router pointers must be 16-byte aligned");
  if (row_type(L->type)) {
    if (!L->gate_scale || !L->up_scale || !L->down_scale) return fail(MD_ERR_INVALID_ARG, "per-row type without scales");
    if (!aligned16(L->gate_scale) || !aligned16(L->up_scale) || !aligned16(L->down_scale))
      return fail(MD_ERR_ALIGNMENT, "scales must be 16-byte aligned");
  }
  if (L->has_shared) {
    if ((s = check_ffn(&L->shared, L->H)) != MD_OK) return s;
    if (L->shared.act != L->act) return fail(MD_ERR_UNSUPPORTED, "shared expert must use the layer's activation");
  }
  return MD_OK;
}

md_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MD_OK;
  if (!ws || have < need) return fail(MD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, have);
  if (!aligned16(ws)) return fail(MD_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  return MD_OK;
}

typedef unsigned short u16;

// dense FFN (or shared expert) for a chunk of tokens on the matrix cores:
// x_hi/x_lo hold x as bf16 pairs; h and its pair buffers are scratch
// Activation buffers of the chunk path: bf16 pairs feed the block formats,
// int8 digit planes the per-row formats.
struct ChunkAct {
  const u16* hi;
  const u16* lo;
  const int8_t* dig;
  const int* expo;
};

md_status run_ffn_mfma(const md_ffn* f, const ChunkAct& xa, int T, float* h, u16* h_hi, u16* h_lo, int8_t* h_dig,
                       int* h_exp, float* y, hipStream_t st) {
  const int H = f->gate.cols, F = f->gate.rows, fmt = f->gate.type;
  md::Disp d{nullptr, nullptr, nullptr, nullptr, 1, T};
  if (row_type(fmt)) {
    hipError_t e = md::launch_moe_mfma_i8(fmt, true, static_cast<const uint8_t*>(f->gate.q),
                                          static_cast<const uint8_t*>(f->up.q), f->gate.row_scale, f->up.row_scale, 0,
                                          F, H, f->act, d, 1, xa.dig, xa.expo, true, h, st);
    if (e != hipSuccess) return hip_fail(e, "ffn gate/up launch");
    e = md::launch_limbs(h, T, F, fmt, h_dig, h_exp, st);
    if (e != hipSuccess) return hip_fail(e, "digit launch");
    e = md::launch_moe_mfma_i8(fmt, false, static_cast<const uint8_t*>(f->down.q), nullptr, f->down.row_scale, nullptr,
                               0, H, F, f->act, d, 1, h_dig, h_exp, false, y, st);
    if (e != hipSuccess) return hip_fail(e, "ffn down launch");
    return MD_OK;
  }
  const u16* x_hi = xa.hi;
  const u16* x_lo = xa.lo;
  hipError_t e = md::launch_moe_mfma(fmt, true, static_cast<const uint8_t*>(f->gate.q),
                                     static_cast<const uint8_t*>(f->up.q), f->gate.row_scale, f->up.row_scale, 0, F,
                                     H, f->act, d, 1, x_hi, x_lo, true, h, h_hi, h_lo, st);
  if (e != hipSuccess) return hip_fail(e, "ffn gate/up launch");
  e = md::launch_moe_mfma(fmt, false, static_cast<const uint8_t*>(f->down.q), nullptr, f->down.row_scale, nullptr, 0,
                          H, F, f->act, d, 1, h_hi, h_lo, false, y, nullptr, nullptr, st);
  if (e != hipSuccess) return hip_fail(e, "ffn down launch");
  return MD_OK;
}

// dense FFN (or shared expert) through the MoE kernels with the identity
// dispatch.  One-token kernels: x digit planes come ready (xd_ready) or are
// made into xd; hd receives those of h.  Otherwise h (fp32) is the scratch.
md_status run_ffn(const md_ffn* f, const float* x, int T, const DigBuf* xd_ready, const DigBuf& xd, const DigBuf& hd,
                  float* h, float* y, hipStream_t st) {
  const int H = f->gate.cols, F = f->gate.rows, fmt = f->gate.type;
  if (T <= kMaxPairT && md::t1_supported(fmt, H, F)) {
    hipError_t e = hipSuccess;
    const DigBuf* xa = xd_ready;
    if (!xa) {
      e = md::launch_digits(dig_job(x, T, H, fmt, xd), st);
      if (e != hipSuccess) return hip_fail(e, "digit launch");
      xa = &xd;
    }
    e = md::launch_gateup_t1(fmt, static_cast<const uint8_t*>(f->gate.q), static_cast<const uint8_t*>(f->up.q),
                             f->gate.row_scale, f->up.row_scale, 0, F, H, f->act, 1, 1, T, nullptr, 1, nullptr,
                             xa->planes, xa->scales, hd.planes, hd.scales, nullptr, nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "ffn gate/up launch");
    e = md::launch_down_t1(fmt, static_cast<const uint8_t*>(f->down.q), f->down.row_scale, 0, H, F, 1, T, nullptr,
                           nullptr, hd.planes, hd.scales, nullptr, y, st);
    if (e != hipSuccess) return hip_fail(e, "ffn down launch");
    return MD_OK;
  }
  md::Disp d{nullptr, nullptr, nullptr, nullptr, 1, T};
  md::GemvCfg cg = md::gateup_config(fmt, F, H, 1, T);
  hipError_t e = md::launch_gateup(fmt, cg, static_cast<const uint8_t*>(f->gate.q), static_cast<const uint8_t*>(f->up.q),
                                   f->gate.row_scale, f->up.row_scale, 0, F, H, f->act, d, x, h, st);
  if (e != hipSuccess) return hip_fail(e, "ffn gate/up launch");
  md::GemvCfg cd = md::down_config(fmt, H, F, 1, T);
  e = md::launch_down(fmt, cd, static_cast<const uint8_t*>(f->down.q), f->down.row_scale, 0, H, F, d, h, y, st);
  if (e != hipSuccess) return hip_fail(e, "ffn down launch");
  return MD_OK;
}

}  // namespace

extern "C" {

int32_t md_abi_version(void) { return MD_ABI_VERSION; }

const char* md_status_string(md_status s) {
  switch (s) {
    case MD_OK: return "ok";
    case MD_ERR_INVALID_ARG: return "invalid argument";
    case MD_ERR_SHAPE: return "inconsistent shape";
    case MD_ERR_UNSUPPORTED: return "unsupported configuration";
    case MD_ERR_ALIGNMENT: return "misaligned pointer";
    case MD_ERR_WORKSPACE: return "workspace too small";
    case MD_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* md_last_error_detail(void) { return g_detail; }

int64_t md_row_bytes(int32_t type, int32_t cols) {
  if (!valid_type(type) || cols <= 0 || cols % 32) return -1;
  return md::row_bytes(type, cols);
}

md_status md_prepare_layout(int32_t type, int32_t rows, int32_t cols, int32_t count, const void* src, void* dst,
                            hipStream_t stream) {
  if (!valid_type(type)) return fail(MD_ERR_INVALID_ARG, "unknown type %d", type);
  if (rows <= 0 || count <= 0) return fail(MD_ERR_SHAPE, "rows %d count %d", rows, count);
  md_status s = check_width("cols", cols);
  if (s != MD_OK) return s;
  if (!src || !dst) return fail(MD_ERR_INVALID_ARG, "null buffer");
  if (!aligned16(src) || !aligned16(dst)) return fail(MD_ERR_ALIGNMENT, "buffers must be 16-byte aligned");
  const int64_t bytes = (int64_t)rows * count * md::row_bytes(type, cols);
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (a < b + bytes && b < a + bytes) return fail(MD_ERR_INVALID_ARG, "src and dst overlap");
  hipError_t e = md::launch_prepare_layout(type, rows, cols, count, src, dst, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "prepare_layout launch");
}

// Batches of 4 or more on block formats run on the matrix cores (the VALU
// engine re-reads every token's activations for every weight chunk).
static bool gemv_on_mfma(const md_qmatrix* W, int batch) {
  return batch >= 4 && (W->type == MD_Q8_0 || W->type == MD_Q4_0 || W->type == MD_Q4_1) &&
         md::mfma_supported(W->cols);
}

// Matrix-core GEMV workspace: [ks][batch][rows] partials (ks > 1), then the
// bf16 hi / lo halves of fp32 activations.
static size_t gemv_mfma_bytes(const md_qmatrix* W, int batch, size_t* part, size_t* pair) {
  const int ks = md::mfma_gemv_splits(W->type, W->rows, W->cols);
  *part = ks > 1 ? align256(sizeof(float) * (size_t)ks * batch * W->rows) : 0;
  *pair = align256(2 * (size_t)batch * W->cols);
  return *part + 2 * *pair;
}

md_status md_qgemv_workspace_size(const md_qmatrix* W, int32_t batch, size_t* bytes) {
  md_status s = check_qmatrix("W", W);
  if (s != MD_OK) return s;
  if (!bytes) return fail(MD_ERR_INVALID_ARG, "null bytes");
  if (batch <= 0) return fail(MD_ERR_SHAPE, "batch %d", batch);
  if (batch > kMaxBatch) return fail(MD_ERR_UNSUPPORTED, "batch %d > %d", batch, kMaxBatch);
  if (gemv_on_mfma(W, batch)) {
    size_t part, pair;
    *bytes = gemv_mfma_bytes(W, batch, &part, &pair);
    return ok();
  }
  md::GemvCfg c = md::qgemv_config(W->type, W->rows, W->cols, batch);
  *bytes = c.S > 1 ? align256(sizeof(float) * (size_t)c.S * batch * W->rows) : 0;
  return ok();
}

md_status md_qgemv(const md_qmatrix* W, const void* x, int32_t xtype, int32_t batch, float* y, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  md_status s = md_qgemv_workspace_size(W, batch, &need);
  if (s != MD_OK) return s;
  if (xtype != MD_X_F32 && xtype != MD_X_BF16) return fail(MD_ERR_INVALID_ARG, "unknown xtype %d", xtype);
  if (!x || !y) return fail(MD_ERR_INVALID_ARG, "null x or y");
  if (!aligned16(x) || !aligned16(y)) return fail(MD_ERR_ALIGNMENT, "x and y must be 16-byte aligned");
  if ((s = check_ws(workspace, workspace_bytes, need)) != MD_OK) return s;
  if (gemv_on_mfma(W, batch)) {
    size_t part, pair;
    gemv_mfma_bytes(W, batch, &part, &pair);
    char* ws = static_cast<char*>(workspace);
    const int ks = md::mfma_gemv_splits(W->type, W->rows, W->cols);
    const u16* hi = static_cast<const u16*>(x);
    const u16* lo = nullptr;  // bf16 activations have no low half
    hipError_t e = hipSuccess;
    if (xtype == MD_X_F32) {
      u16* h = reinterpret_cast<u16*>(ws + part);
      u16* l = reinterpret_cast<u16*>(ws + part + pair);
      e = md::launch_split_bf16(static_cast<const float*>(x), (int64_t)batch * W->cols, h, l, stream);
      if (e != hipSuccess) return hip_fail(e, "split launch");
      hi = h;
      lo = l;
    }
    float* out = ks > 1 ? reinterpret_cast<float*>(ws) : y;
    e = md::launch_mfma_gemv(W->type, static_cast<const uint8_t*>(W->q), W->row_scale, W->rows, W->cols, batch, hi,
                             lo, ks, out, stream);
    if (e != hipSuccess) return hip_fail(e, "matrix-core gemv launch");
    if (ks > 1) {
      e = md::launch_splitk_reduce(out, ks, (int64_t)batch * W->rows, y, stream);
      if (e != hipSuccess) return hip_fail(e, "split-K reduce launch");
    }
    return ok();
  }
  md::GemvCfg c = md::qgemv_config(W->type, W->rows, W->cols, batch);
  hipError_t e = md::launch_qgemv(W->type, xtype, c, static_cast<const uint8_t*>(W->q), W->row_scale, W->rows, W->cols,
                                  x, batch, y, static_cast<float*>(workspace), stream);
  return e == hipSuccess ? ok() : hip_fail(e, "qgemv launch");
}

md_status md_route_workspace_size(int32_t T, int32_t H, int32_t E, int32_t k, size_t* bytes) {
  if (!bytes) return fail(MD_ERR_INVALID_ARG, "null bytes");
  if (T <= 0 || E <= 0 || k <= 0) return fail(MD_ERR_SHAPE, "T %d E %d k %d", T, E, k);
  if (k > E) return fail(MD_ERR_SHAPE, "k = %d > E = %d", k, E);
  if (T > kMaxT || E > kMaxE || k > kMaxK) return fail(MD_ERR_UNSUPPORTED, "T <= %d, E <= %d, k <= %d", kMaxT, kMaxE, kMaxK);
  md_status s = check_width("H", H);
  if (s != MD_OK) return s;
  *bytes = align256(sizeof(double) * (size_t)T * E * md::router_plan(T, H, E).S) + align256(sizeof(float) * (size_t)T * E);
  return ok();
}

md_status md_moe_route_topk(const float* x, int32_t T, int32_t H, const float* W_r, const float* bias, int32_t E,
                            int32_t k, int32_t* idx, float* gates, float* logits, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  md_status s = md_route_workspace_size(T, H, E, k, &need);
  if (s != MD_OK) return s;
  if (!x || !W_r || !idx || !gates) return fail(MD_ERR_INVALID_ARG, "null x, W_r, idx or gates");
  if (!aligned16(x) || !aligned16(W_r) || !aligned16(idx) || !aligned16(gates) || (bias && !aligned16(bias)) ||
      (logits && !aligned16(logits)))
    return fail(MD_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if ((s = check_ws(workspace, workspace_bytes, need)) != MD_OK) return s;
  const md::RouterPlan rp = md::router_plan(T, H, E);
  double* part = static_cast<double*>(workspace);
  hipError_t e = md::launch_router(x, T, H, W_r, E, rp, part, md::DigJob{}, md::DigJob{}, stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  e = md::launch_select(part, rp, bias, T, E, k, logits, idx, gates, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "select launch");
}

static size_t ffn_ws_bytes(const md_ffn* f, int T) {
  const size_t H = f->gate.cols, F = f->gate.rows;
  size_t b = align256(sizeof(float) * T * F);
  if (T <= kMaxPairT) b += dig_buf_bytes(f->gate.type, T, H) + dig_buf_bytes(f->gate.type, T, F);
  if (T > kMaxPairT)
    b += 2 * align256(2 * T * H) + 2 * align256(2 * T * F) + align256(4 * T * H) + align256(4 * T * F) +
         2 * align256(sizeof(int) * T);
  return b;
}

md_status md_ffn_workspace_size(const md_ffn* f, int32_t T, size_t* bytes) {
  if (!f) return fail(MD_ERR_INVALID_ARG, "null FFN descriptor");
  md_status s = check_ffn(f, f->gate.cols);
  if (s != MD_OK) return s;
  if (!bytes) return fail(MD_ERR_INVALID_ARG, "null bytes");
  if (T <= 0) return fail(MD_ERR_SHAPE, "T %d", T);
  if (T > kMaxT) return fail(MD_ERR_UNSUPPORTED, "T %d > %d", T, kMaxT);
  *bytes = ffn_ws_bytes(f, T);
  return ok();
}

md_status md_ffn_forward(const md_ffn* f, const float* x, int32_t T, float* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  md_status s = md_ffn_workspace_size(f, T, &need);
  if (s != MD_OK) return s;
  if (!x || !y) return fail(MD_ERR_INVALID_ARG, "null x or y");
  if (!aligned16(x) || !aligned16(y)) return fail(MD_ERR_ALIGNMENT, "x and y must be 16-byte aligned");
  if ((s = check_ws(workspace, workspace_bytes, need)) != MD_OK) return s;
  char* ws = static_cast<char*>(workspace);
  float* h = reinterpret_cast<float*>(ws);
  const size_t H = f->gate.cols, F = f->gate.rows;
  if (T <= kMaxPairT) {
    char* p = ws + align256(sizeof(float) * T * F);
    const DigBuf xd = dig_buf_at(p, f->gate.type, T, (int)H);
    const DigBuf hd = dig_buf_at(p + dig_buf_bytes(f->gate.type, T, (int)H), f->gate.type, T, (int)F);
    s = run_ffn(f, x, T, nullptr, xd, hd, h, y, stream);
    return s == MD_OK ? ok() : s;
  }
  size_t off = align256(sizeof(float) * T * F);
  u16* x_hi = reinterpret_cast<u16*>(ws + off); off += align256(2 * T * H);
  u16* x_lo = reinterpret_cast<u16*>(ws + off); off += align256(2 * T * H);
  u16* h_hi = reinterpret_cast<u16*>(ws + off); off += align256(2 * T * F);
  u16* h_lo = reinterpret_cast<u16*>(ws + off); off += align256(2 * T * F);
  int8_t* x_dig = reinterpret_cast<int8_t*>(ws + off); off += align256(4 * T * H);
  int8_t* h_dig = reinterpret_cast<int8_t*>(ws + off); off += align256(4 * T * F);
  int* x_exp = reinterpret_cast<int*>(ws + off); off += align256(sizeof(int) * T);
  int* h_exp = reinterpret_cast<int*>(ws + off);
  hipError_t e = row_type(f->gate.type) ? md::launch_limbs(x, T, H, f->gate.type, x_dig, x_exp, stream)
                                        : md::launch_split_bf16(x, (int64_t)T * H, x_hi, x_lo, stream);
  if (e != hipSuccess) return hip_fail(e, "activation split launch");
  s = run_ffn_mfma(f, ChunkAct{x_hi, x_lo, x_dig, x_exp}, T, h, h_hi, h_lo, h_dig, h_exp, y, stream);
  return s == MD_OK ? ok() : s;
}

md_status md_moe_workspace_size(const md_moe_layer* L, int32_t T, size_t* bytes) {
  md_status s = check_moe(L, T);
  if (s != MD_OK) return s;
  if (!bytes) return fail(MD_ERR_INVALID_ARG, "null bytes");
  *bytes = moe_ws(L, T).total;
  return ok();
}

// residual: nullable [T][H], added to y (it may be y itself).
// A second stream per device for a chunk's shared expert: it needs only x,
// so it runs beside the routing kernels (which occupy a small part of the
// GPU) and joins the caller's stream before the combine.  Created at a
// device's first such call, default priority; each fork (event recorded on
// the caller's stream, waited on by the side stream) and each join (the
// reverse) is made under one lock, so concurrent calls cannot interleave them.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
static std::mutex g_side_mu;
static SideStream g_side[64];

static SideStream* side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    // both streams are on this device: the kernels' own end-of-kernel
    // releases make their writes visible to the other stream, so the events
    // skip the system-scope fence (a writeback and invalidation of every
    // XCD's L2 at each fork and join)
    const unsigned fl = hipEventDisableTiming | hipEventDisableSystemFence;
    if (hipEventCreateWithFlags(&a, fl) != hipSuccess || hipEventCreateWithFlags(&b, fl) != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      (void)hipStreamDestroy(st);
      return nullptr;
    }
    ss.s = st;
    ss.fork = a;
    ss.join = b;
  }
  return &ss;
}

// `from` waits for everything enqueued on `to_wait_on` so far.
static hipError_t stream_after(SideStream* ss, hipEvent_t ev, hipStream_t to_wait_on, hipStream_t from) {
  std::lock_guard<std::mutex> lk(g_side_mu);
  hipError_t e = hipEventRecord(ev, to_wait_on);
  if (e == hipSuccess) e = hipStreamWaitEvent(from, ev, 0);
  return e;
}

static md_status moe_forward(const md_moe_layer* L, const float* x, int32_t T, float* y, int32_t* idx_out,
                             float* gates_out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                             int32_t stage, hipEvent_t ev0, hipEvent_t ev1, const float* residual = nullptr,
                             int32_t only = -1, bool allow_side = false) {
  md_status s = check_moe(L, T);
  if (s != MD_OK) return s;
  if (!x || !y) return fail(MD_ERR_INVALID_ARG, "null x or y");
  if (!aligned16(x) || !aligned16(y) || (idx_out && !aligned16(idx_out)) || (gates_out && !aligned16(gates_out)))
    return fail(MD_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (stage >= 0 && (stage > MD_STAGE_COMBINE || !ev0 || !ev1))
    return fail(MD_ERR_INVALID_ARG, "timed call needs a stage in 0..5 and two events");
  const MoeWs w = moe_ws(L, T);
  if ((s = check_ws(workspace, workspace_bytes, w.total)) != MD_OK) return s;

  char* ws = static_cast<char*>(workspace);
  auto P = [&](size_t off) { return static_cast<void*>(ws + off); };
  const int H = L->H, F = L->F, E = L->E, k = L->k, fmt = L->type;
  int* idx = idx_out ? idx_out : static_cast<int*>(P(w.idx));
  float* gates = gates_out ? gates_out : static_cast<float*>(P(w.gates));
  float* y_s = L->has_shared ? static_cast<float*>(P(w.y_s)) : nullptr;
  hipError_t e = hipSuccess;
  auto mark = [&](int st, hipEvent_t ev) -> bool {
    if (st != stage) return true;
    e = hipEventRecord(ev, stream);
    return e == hipSuccess;
  };
  // only >= 0: enqueue the launches of that stage alone (they read what an
  // earlier full call left in the workspace)
  auto want = [&](int st) { return only < 0 || only == st; };

  const int64_t gu_bytes = (int64_t)F * md::row_bytes(fmt, H);
  const int64_t dn_bytes = (int64_t)H * md::row_bytes(fmt, F);
  float* logits = static_cast<float*>(P(w.logits));
  float* h = static_cast<float*>(P(w.h));
  const bool t1 = use_pairs(L, T);

  if (t1) {
    // few tokens: the router kernel also writes x's digit planes; selection
    // happens inside the gate/up kernel, the combine inside the down kernel;
    // each (token, slot) pair is an independent one-token problem
    const md::RouterPlan rp = md::router_plan(T, H, E, true);
    if (rp.gemm) return fail(MD_ERR_UNSUPPORTED, "router partial layout does not match the one-token kernels");
    double* part = static_cast<double*>(P(w.part));
    const DigBuf xd = dig_buf_at(ws + w.xd, fmt, T, H);
    const DigBuf hd = dig_buf_at(ws + w.hd, fmt, T * k, F);
    DigBuf sxd{}, shd{};
    md::DigJob js{};
    if (L->has_shared) {
      const int sfmt = L->shared.gate.type;
      sxd = dig_buf_at(ws + w.sxd, sfmt, T, H);
      shd = dig_buf_at(ws + w.shd, sfmt, T, L->shared.gate.rows);
      js = dig_job(x, T, H, sfmt, sxd);
    }
    // the paths that add the residual in a launch of its own after y is
    // written keep a copy of it when it is y itself
    const float* res_late = residual;
    auto keep_residual = [&]() -> bool {
      if (residual != y) return true;
      float* c = static_cast<float*>(P(w.rcopy));
      if (md::launch_copy_f32(residual, c, (int64_t)T * H, stream) != hipSuccess) return false;
      res_late = c;
      return true;
    };
    if (!mark(MD_STAGE_ROUTER, ev0)) return hip_fail(e, "event record");
    if (want(MD_STAGE_ROUTER)) {
      e = md::launch_router(x, T, H, L->W_r, E, rp, part, dig_job(x, T, H, fmt, xd), js, stream);
      if (e != hipSuccess) return hip_fail(e, "router launch");
    }
    if (L->has_shared && md::rs_supported(fmt, H, F, L->shared.gate.type, L->shared.gate.rows, k, T)) {
      // the shared expert inside the routed launches
      if (!mark(MD_STAGE_ROUTER, ev1) || !mark(MD_STAGE_SHARED, ev0) || !mark(MD_STAGE_SHARED, ev1) ||
          !mark(MD_STAGE_SELECT, ev0) || !mark(MD_STAGE_SELECT, ev1) || !mark(MD_STAGE_GATEUP, ev0))
        return hip_fail(e, "event record");
      const md_ffn& sf = L->shared;
      md::RsLaunch rl{};
      rl.fmt = fmt;
      rl.gq = static_cast<const uint8_t*>(L->gate_q);
      rl.uq = static_cast<const uint8_t*>(L->up_q);
      rl.dq = static_cast<const uint8_t*>(L->down_q);
      rl.gs = L->gate_scale;
      rl.us = L->up_scale;
      rl.ds = L->down_scale;
      rl.gu_bytes = gu_bytes;
      rl.dn_bytes = dn_bytes;
      rl.F = F; rl.act = L->act; rl.H = H; rl.E = E; rl.k = k; rl.T = T;
      rl.part = part; rl.S = rp.S; rl.bias = L->router_bias;
      rl.xd = xd.planes; rl.xsc = xd.scales; rl.hd = hd.planes; rl.hsc = hd.scales;
      rl.sfmt = sf.gate.type;
      rl.sgq = static_cast<const uint8_t*>(sf.gate.q);
      rl.suq = static_cast<const uint8_t*>(sf.up.q);
      rl.sdq = static_cast<const uint8_t*>(sf.down.q);
      rl.sgs = row_type(sf.gate.type) ? sf.gate.row_scale : nullptr;
      rl.sus = row_type(sf.gate.type) ? sf.up.row_scale : nullptr;
      rl.sds = row_type(sf.gate.type) ? sf.down.row_scale : nullptr;
      rl.Fs = sf.gate.rows; rl.sact = sf.act;
      rl.sxd = sxd.planes; rl.sxsc = sxd.scales; rl.shd = shd.planes; rl.shsc = shd.scales;
      rl.idx = idx; rl.gates = gates; rl.y = y; rl.residual = residual;
      rl.parts = (want(MD_STAGE_GATEUP) ? 1 : 0) | (want(MD_STAGE_DOWN) ? 2 : 0);
      if (rl.parts) {
        e = md::launch_moe_rs(rl, stream);
        if (e != hipSuccess) return hip_fail(e, "routed+shared launch");
      }
      if (!mark(MD_STAGE_GATEUP, ev1) || !mark(MD_STAGE_DOWN, ev0) || !mark(MD_STAGE_DOWN, ev1) ||
          !mark(MD_STAGE_COMBINE, ev0) || !mark(MD_STAGE_COMBINE, ev1))
        return hip_fail(e, "event record");
      return ok();
    }
    if (!mark(MD_STAGE_ROUTER, ev1) || !mark(MD_STAGE_SHARED, ev0)) return hip_fail(e, "event record");
    if (L->has_shared && want(MD_STAGE_SHARED)) {
      s = run_ffn(&L->shared, x, T, &sxd, sxd, shd, static_cast<float*>(P(w.h_s)), y_s, stream);
      if (s != MD_OK) return s;
    }
    if (!mark(MD_STAGE_SHARED, ev1) || !mark(MD_STAGE_SELECT, ev0) || !mark(MD_STAGE_SELECT, ev1) ||
        !mark(MD_STAGE_GATEUP, ev0))
      return hip_fail(e, "event record");
    if (want(MD_STAGE_GATEUP)) {
      e = md::launch_gateup_t1(fmt, static_cast<const uint8_t*>(L->gate_q), static_cast<const uint8_t*>(L->up_q),
                               L->gate_scale, L->up_scale, gu_bytes, F, H, L->act, E, k, T, part, rp.S,
                               L->router_bias, xd.planes, xd.scales, hd.planes, hd.scales, idx, gates, stream);
      if (e != hipSuccess) return hip_fail(e, "gate/up launch");
    }
    if (!mark(MD_STAGE_GATEUP, ev1) || !mark(MD_STAGE_DOWN, ev0)) return hip_fail(e, "event record");
    if (want(MD_STAGE_DOWN)) {
      if (y_s && residual && !keep_residual()) return hip_fail(hipGetLastError(), "residual copy");
      e = md::launch_down_t1(fmt, static_cast<const uint8_t*>(L->down_q), L->down_scale, dn_bytes, H, F, k, T, idx,
                             gates, hd.planes, hd.scales, y_s ? y_s : residual, y, stream);
      if (e != hipSuccess) return hip_fail(e, "down launch");
      if (y_s && residual) {  // the addend slot held the shared output
        e = md::launch_add(y, res_late, y, (int64_t)T * H, stream);
        if (e != hipSuccess) return hip_fail(e, "residual launch");
      }
    }
    if (!mark(MD_STAGE_DOWN, ev1) || !mark(MD_STAGE_COMBINE, ev0) || !mark(MD_STAGE_COMBINE, ev1))
      return hip_fail(e, "event record");
    return ok();
  }

  // shared expert: independent of the routing, enqueued first
  ChunkAct xa{nullptr, nullptr, nullptr, nullptr};
  if (!mark(MD_STAGE_SHARED, ev0)) return hip_fail(e, "event record");
  const md::RouterPlan rp = md::router_plan(T, H, E);
  // the router GEMM writes the routed experts' bf16 pair of x from the tiles
  // it stages (one launch less before the grouped GEMMs)
  const bool pair_by_router = rp.gemm && !row_type(fmt);
  {
    // the activation forms the chunk path's kernels need (enqueued with the
    // shared expert's stage; pointers set up for every stage)
    const bool need_pair = !row_type(fmt);
    const bool need_dig = row_type(fmt);
    if (need_pair) {
      xa.hi = static_cast<u16*>(P(w.x_hi));
      xa.lo = static_cast<u16*>(P(w.x_lo));
      if (want(MD_STAGE_SHARED) && !pair_by_router) {
        e = md::launch_split_bf16(x, (int64_t)T * H, static_cast<u16*>(P(w.x_hi)), static_cast<u16*>(P(w.x_lo)),
                                  stream);
        if (e != hipSuccess) return hip_fail(e, "split launch");
      }
    }
    if (need_dig) {
      xa.dig = static_cast<int8_t*>(P(w.x_dig));
      xa.expo = static_cast<int*>(P(w.x_exp));
      if (want(MD_STAGE_SHARED)) {
        e = md::launch_limbs(x, T, H, fmt, static_cast<int8_t*>(P(w.x_dig)), static_cast<int*>(P(w.x_exp)),
                             stream);
        if (e != hipSuccess) return hip_fail(e, "digit launch");
      }
    }
  }
  // a plain call runs the shared expert on the side stream; every exit after
  // the fork joins it back into the caller's stream
  SideStream* side = nullptr;
  struct Join {
    SideStream* ss = nullptr;
    hipStream_t caller = nullptr;
    hipError_t now() {
      if (!ss) return hipSuccess;
      SideStream* t = ss;
      ss = nullptr;
      return stream_after(t, t->join, t->s, caller);
    }
    ~Join() { (void)now(); }
  } join;
  if (L->has_shared && want(MD_STAGE_SHARED)) {
    hipStream_t sst = stream;
    if (allow_side && stage < 0 && only < 0 && (side = side_stream()) != nullptr) {
      e = stream_after(side, side->fork, stream, side->s);
      if (e != hipSuccess) return hip_fail(e, "side stream fork");
      join.ss = side;
      join.caller = stream;
      sst = side->s;
    }
    ChunkAct xs = xa;
    const int sfmt = L->shared.gate.type;
    if (row_type(sfmt)) {  // x digits in the shared expert's own column order
      e = md::launch_limbs(x, T, H, sfmt, static_cast<int8_t*>(P(w.xs_dig)),
                           static_cast<int*>(P(w.xs_exp)), sst);
      if (e != hipSuccess) return hip_fail(e, "digit launch");
      xs.dig = static_cast<int8_t*>(P(w.xs_dig));
      xs.expo = static_cast<int*>(P(w.xs_exp));
    } else {  // its own bf16 pair of x, made on its stream
      xs.hi = static_cast<u16*>(P(w.xs_hi));
      xs.lo = static_cast<u16*>(P(w.xs_lo));
      e = md::launch_split_bf16(x, (int64_t)T * H, static_cast<u16*>(P(w.xs_hi)), static_cast<u16*>(P(w.xs_lo)), sst);
      if (e != hipSuccess) return hip_fail(e, "split launch");
    }
    s = run_ffn_mfma(&L->shared, xs, T, static_cast<float*>(P(w.h_s)), static_cast<u16*>(P(w.hs_hi)),
                     static_cast<u16*>(P(w.hs_lo)), static_cast<int8_t*>(P(w.hs_dig)), static_cast<int*>(P(w.hs_exp)),
                     y_s, sst);
    if (s != MD_OK) return s;
  }
  if (!mark(MD_STAGE_SHARED, ev1) || !mark(MD_STAGE_ROUTER, ev0)) return hip_fail(e, "event record");
  double* part = static_cast<double*>(P(w.part));
  if (want(MD_STAGE_ROUTER)) {
    e = md::launch_router(x, T, H, L->W_r, E, rp, part, md::DigJob{}, md::DigJob{}, stream,
                          pair_by_router ? static_cast<u16*>(P(w.x_hi)) : nullptr,
                          pair_by_router ? static_cast<u16*>(P(w.x_lo)) : nullptr);
    if (e != hipSuccess) return hip_fail(e, "router launch");
  }
  if (!mark(MD_STAGE_ROUTER, ev1) || !mark(MD_STAGE_SELECT, ev0)) return hip_fail(e, "event record");

  // a chunk of tokens: group the (token, slot) pairs by expert, then one
  // grouped GEMM per stage on the matrix cores, each expert read once
  const int n_items = md::max_tiles(T, k, max_active(T, E, k));
  md::DispOut dout{static_cast<int*>(P(w.n_active)), static_cast<int*>(P(w.active_e)),
                   static_cast<int*>(P(w.active_off)), static_cast<int*>(P(w.pairs)), static_cast<int*>(P(w.pos)),
                   static_cast<int4*>(P(w.items)), n_items};
  if (want(MD_STAGE_SELECT)) {
    e = md::launch_select(part, rp, L->router_bias, T, E, k, logits, idx, gates, stream);
    if (e != hipSuccess) return hip_fail(e, "select launch");
    e = md::launch_dispatch(idx, T, E, k, dout, stream);
    if (e != hipSuccess) return hip_fail(e, "dispatch launch");
  }
  if (!mark(MD_STAGE_SELECT, ev1) || !mark(MD_STAGE_GATEUP, ev0)) return hip_fail(e, "event record");

  md::Disp d{dout.n_active, dout.active_e, dout.active_off, dout.pairs, k, T, dout.items};
  const int A = n_items;
  float* o = static_cast<float*>(P(w.o));
  if (row_type(fmt)) {
    int8_t* h_dig = static_cast<int8_t*>(P(w.h_dig));
    int* h_exp = static_cast<int*>(P(w.h_exp));
    if (want(MD_STAGE_GATEUP)) {
      e = md::launch_moe_mfma_i8(fmt, true, static_cast<const uint8_t*>(L->gate_q),
                                 static_cast<const uint8_t*>(L->up_q), L->gate_scale, L->up_scale, gu_bytes, F, H,
                                 L->act, d, A, xa.dig, xa.expo, true, h, stream);
      if (e != hipSuccess) return hip_fail(e, "gate/up launch");
    }
    if (!mark(MD_STAGE_GATEUP, ev1) || !mark(MD_STAGE_DOWN, ev0)) return hip_fail(e, "event record");
    if (want(MD_STAGE_DOWN)) {
      e = md::launch_limbs(h, T * k, F, fmt, h_dig, h_exp, stream);
      if (e != hipSuccess) return hip_fail(e, "digit launch");
      e = md::launch_moe_mfma_i8(fmt, false, static_cast<const uint8_t*>(L->down_q), nullptr, L->down_scale, nullptr,
                                 dn_bytes, H, F, L->act, d, A, h_dig, h_exp, false, o, stream);
      if (e != hipSuccess) return hip_fail(e, "down launch");
    }
  } else {
    u16* h_hi = static_cast<u16*>(P(w.h_hi));
    u16* h_lo = static_cast<u16*>(P(w.h_lo));
    if (want(MD_STAGE_GATEUP)) {
      e = md::launch_moe_mfma(fmt, true, static_cast<const uint8_t*>(L->gate_q), static_cast<const uint8_t*>(L->up_q),
                              L->gate_scale, L->up_scale, gu_bytes, F, H, L->act, d, A, xa.hi, xa.lo, true, h, h_hi,
                              h_lo, stream);
      if (e != hipSuccess) return hip_fail(e, "gate/up launch");
    }
    if (!mark(MD_STAGE_GATEUP, ev1) || !mark(MD_STAGE_DOWN, ev0)) return hip_fail(e, "event record");
    if (want(MD_STAGE_DOWN)) {
      e = md::launch_moe_mfma(fmt, false, static_cast<const uint8_t*>(L->down_q), nullptr, L->down_scale, nullptr,
                              dn_bytes, H, F, L->act, d, A, h_hi, h_lo, false, o, nullptr, nullptr, stream);
      if (e != hipSuccess) return hip_fail(e, "down launch");
    }
  }
  if (!mark(MD_STAGE_DOWN, ev1) || !mark(MD_STAGE_COMBINE, ev0)) return hip_fail(e, "event record");
  if ((e = join.now()) != hipSuccess) return hip_fail(e, "side stream join");
  if (want(MD_STAGE_COMBINE)) {
    e = md::launch_combine(o, dout.pos_of_pair, gates, T, k, H, y_s, residual, y, stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  if (!mark(MD_STAGE_COMBINE, ev1)) return hip_fail(e, "event record");
  return ok();
}

// The experts of a layer for a given routing (idx, gates: device [T][k]):
// the stages of moe_forward after the router, in two phases so that a caller
// can put other work between them: the shared expert (into the workspace),
// then the routed experts with the combine, which adds the shared output.
// The routing is first copied into the workspace with every entry clamped
// into [0, E), so no entry can address outside the expert stacks.
static md_status experts_check(const md_moe_layer* L, const float* x, int32_t T, const int32_t* idx_in,
                               const float* gates_in, const float* y, size_t workspace_bytes, const void* workspace) {
  md_status s = check_moe(L, T);
  if (s != MD_OK) return s;
  if (!x || !y || !idx_in || !gates_in) return fail(MD_ERR_INVALID_ARG, "null x, y, idx or gates");
  if (!aligned16(x) || !aligned16(y) || !aligned16(idx_in) || !aligned16(gates_in))
    return fail(MD_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  return check_ws(const_cast<void*>(workspace), workspace_bytes, moe_ws(L, T).total);
}

// Phase 1: the shared expert's output for the T tokens (nullptr without one).
static md_status shared_phase(const md_moe_layer* L, const float* x, int32_t T, char* ws, hipStream_t stream,
                              float** y_s_out) {
  *y_s_out = nullptr;
  if (!L->has_shared) return MD_OK;
  const MoeWs w = moe_ws(L, T);
  auto P = [&](size_t off) { return static_cast<void*>(ws + off); };
  const int H = L->H, sfmt = L->shared.gate.type;
  float* y_s = static_cast<float*>(P(w.y_s));
  md_status s;
  if (use_pairs(L, T)) {
    const DigBuf sxd = dig_buf_at(ws + w.sxd, sfmt, T, H);
    const DigBuf shd = dig_buf_at(ws + w.shd, sfmt, T, L->shared.gate.rows);
    s = run_ffn(&L->shared, x, T, nullptr, sxd, shd, static_cast<float*>(P(w.h_s)), y_s, stream);
  } else {
    ChunkAct xs{nullptr, nullptr, nullptr, nullptr};
    hipError_t e;
    if (row_type(sfmt)) {
      e = md::launch_limbs(x, T, H, sfmt, static_cast<int8_t*>(P(w.xs_dig)), static_cast<int*>(P(w.xs_exp)), stream);
      xs.dig = static_cast<int8_t*>(P(w.xs_dig));
      xs.expo = static_cast<int*>(P(w.xs_exp));
    } else {
      e = md::launch_split_bf16(x, (int64_t)T * H, static_cast<u16*>(P(w.x_hi)), static_cast<u16*>(P(w.x_lo)), stream);
      xs.hi = static_cast<u16*>(P(w.x_hi));
      xs.lo = static_cast<u16*>(P(w.x_lo));
    }
    if (e != hipSuccess) return hip_fail(e, "shared activation launch");
    s = run_ffn_mfma(&L->shared, xs, T, static_cast<float*>(P(w.h_s)), static_cast<u16*>(P(w.hs_hi)),
                     static_cast<u16*>(P(w.hs_lo)), static_cast<int8_t*>(P(w.hs_dig)), static_cast<int*>(P(w.hs_exp)),
                     y_s, stream);
  }
  if (s != MD_OK) return s;
  *y_s_out = y_s;
  return MD_OK;
}

// Phase 2: the routed experts; y = their gated sum + y_add (nullable).
static md_status routed_phase(const md_moe_layer* L, const float* x, int32_t T, const int32_t* idx_in,
                              const float* gates_in, const float* y_add, float* y, char* ws, hipStream_t stream) {
  const MoeWs w = moe_ws(L, T);
  auto P = [&](size_t off) { return static_cast<void*>(ws + off); };
  const int H = L->H, F = L->F, E = L->E, k = L->k, fmt = L->type;
  const int64_t gu_bytes = (int64_t)F * md::row_bytes(fmt, H);
  const int64_t dn_bytes = (int64_t)H * md::row_bytes(fmt, F);
  int* idx = static_cast<int*>(P(w.idx));
  hipError_t e = md::launch_clamp_idx(idx_in, T * k, E, idx, stream);
  if (e != hipSuccess) return hip_fail(e, "routing copy launch");
  float* h = static_cast<float*>(P(w.h));
  if (use_pairs(L, T)) {
    const DigBuf xd = dig_buf_at(ws + w.xd, fmt, T, H);
    const DigBuf hd = dig_buf_at(ws + w.hd, fmt, T * k, F);
    e = md::launch_digits(dig_job(x, T, H, fmt, xd), stream);
    if (e != hipSuccess) return hip_fail(e, "digit launch");
    e = md::launch_gateup_t1(fmt, static_cast<const uint8_t*>(L->gate_q), static_cast<const uint8_t*>(L->up_q),
                             L->gate_scale, L->up_scale, gu_bytes, F, H, L->act, E, k, T, nullptr, 1, nullptr,
                             xd.planes, xd.scales, hd.planes, hd.scales, nullptr, nullptr, stream, idx);
    if (e != hipSuccess) return hip_fail(e, "gate/up launch");
    e = md::launch_down_t1(fmt, static_cast<const uint8_t*>(L->down_q), L->down_scale, dn_bytes, H, F, k, T, idx,
                           gates_in, hd.planes, hd.scales, y_add, y, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "down launch");
  }
  ChunkAct xa{nullptr, nullptr, nullptr, nullptr};
  if (row_type(fmt)) {
    e = md::launch_limbs(x, T, H, fmt, static_cast<int8_t*>(P(w.x_dig)), static_cast<int*>(P(w.x_exp)), stream);
    xa.dig = static_cast<int8_t*>(P(w.x_dig));
    xa.expo = static_cast<int*>(P(w.x_exp));
  } else {
    e = md::launch_split_bf16(x, (int64_t)T * H, static_cast<u16*>(P(w.x_hi)), static_cast<u16*>(P(w.x_lo)), stream);
    xa.hi = static_cast<u16*>(P(w.x_hi));
    xa.lo = static_cast<u16*>(P(w.x_lo));
  }
  if (e != hipSuccess) return hip_fail(e, "activation launch");
  const int n_items = md::max_tiles(T, k, max_active(T, E, k));
  md::DispOut dout{static_cast<int*>(P(w.n_active)), static_cast<int*>(P(w.active_e)),
                   static_cast<int*>(P(w.active_off)), static_cast<int*>(P(w.pairs)), static_cast<int*>(P(w.pos)),
                   static_cast<int4*>(P(w.items)), n_items};
  e = md::launch_dispatch(idx, T, E, k, dout, stream);
  if (e != hipSuccess) return hip_fail(e, "dispatch launch");
  md::Disp d{dout.n_active, dout.active_e, dout.active_off, dout.pairs, k, T, dout.items};
  float* o = static_cast<float*>(P(w.o));
  if (row_type(fmt)) {
    int8_t* h_dig = static_cast<int8_t*>(P(w.h_dig));
    int* h_exp = static_cast<int*>(P(w.h_exp));
    e = md::launch_moe_mfma_i8(fmt, true, static_cast<const uint8_t*>(L->gate_q), static_cast<const uint8_t*>(L->up_q),
                               L->gate_scale, L->up_scale, gu_bytes, F, H, L->act, d, n_items, xa.dig, xa.expo, true,
                               h, stream);
    if (e == hipSuccess) e = md::launch_limbs(h, T * k, F, fmt, h_dig, h_exp, stream);
    if (e == hipSuccess)
      e = md::launch_moe_mfma_i8(fmt, false, static_cast<const uint8_t*>(L->down_q), nullptr, L->down_scale, nullptr,
                                 dn_bytes, H, F, L->act, d, n_items, h_dig, h_exp, false, o, stream);
  } else {
    u16* h_hi = static_cast<u16*>(P(w.h_hi));
    u16* h_lo = static_cast<u16*>(P(w.h_lo));
    e = md::launch_moe_mfma(fmt, true, static_cast<const uint8_t*>(L->gate_q), static_cast<const uint8_t*>(L->up_q),
                            L->gate_scale, L->up_scale, gu_bytes, F, H, L->act, d, n_items, xa.hi, xa.lo, true, h,
                            h_hi, h_lo, stream);
    if (e == hipSuccess)
      e = md::launch_moe_mfma(fmt, false, static_cast<const uint8_t*>(L->down_q), nullptr, L->down_scale, nullptr,
                              dn_bytes, H, F, L->act, d, n_items, h_hi, h_lo, false, o, nullptr, nullptr, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "expert launch");
  e = md::launch_combine(o, dout.pos_of_pair, gates_in, T, k, H, y_add, nullptr, y, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "combine launch");
}

static md_status experts_forward(const md_moe_layer* L, const float* x, int32_t T, const int32_t* idx_in,
                                 const float* gates_in, float* y, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  md_status s = experts_check(L, x, T, idx_in, gates_in, y, workspace_bytes, workspace);
  if (s != MD_OK) return s;
  char* ws = static_cast<char*>(workspace);
  float* y_s = nullptr;
  if ((s = shared_phase(L, x, T, ws, stream, &y_s)) != MD_OK) return s;
  return routed_phase(L, x, T, idx_in, gates_in, y_s, y, ws, stream);
}

md_status md_moe_layer_forward(const md_moe_layer* L, const float* x, int32_t T, float* y, int32_t* idx_out,
                               float* gates_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return moe_forward(L, x, T, y, idx_out, gates_out, workspace, workspace_bytes, stream, -1, nullptr, nullptr,
                     nullptr, -1, true);
}

}  // extern "C"

// ---- the layer forward that allocates nothing -------------------------------
//
// Scratch of md_moe_layer_forward_noalloc: an array in the library's code
// object, so every GPU the library runs on holds one copy of it (at its own
// address) until the process ends.  Host code reaches a device's copy only
// through the address hipGetSymbolAddress returns on that device (the array's
// name on the host is a stand-in, not a device address).  Nothing in it needs
// to start at zero: every kernel of the layer writes what a later one reads.

constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up once per device,
// with that device current).
md_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MD_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MD_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MD_OK;
}
}  // namespace

extern "C" {

md_status md_moe_layer_forward_noalloc(const md_moe_layer* L, const float* x, int32_t T, float* y, int32_t* idx_out,
                                       float* gates_out, hipStream_t stream) {
  md_status s = check_moe(L, T);
  if (s != MD_OK) return s;
  if (!x || !y) return fail(MD_ERR_INVALID_ARG, "null x or y");
  if (!aligned16(x) || !aligned16(y) || (idx_out && !aligned16(idx_out)) || (gates_out && !aligned16(gates_out)))
    return fail(MD_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  const size_t need = moe_ws(L, T).total;
  if (need > kScratchBytes)
    return fail(MD_ERR_UNSUPPORTED,
                "this layer call needs %zu bytes of scratch, more than the %zu bytes built in "
                "(md_moe_layer_forward takes a workspace of any size)", need, kScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != MD_OK) return s;
  return moe_forward(L, x, T, y, idx_out, gates_out, ws, kScratchBytes, stream, -1, nullptr, nullptr);
}

md_status md_moe_layer_forward_timed(const md_moe_layer* L, const float* x, int32_t T, float* y, int32_t* idx_out,
                                     float* gates_out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                     int32_t stage, hipEvent_t start, hipEvent_t stop) {
  if (stage < 0) return fail(MD_ERR_INVALID_ARG, "stage %d", stage);
  return moe_forward(L, x, T, y, idx_out, gates_out, workspace, workspace_bytes, stream, stage, start, stop);
}

md_status md_moe_layer_stage_relaunch(const md_moe_layer* L, const float* x, int32_t T, float* y, int32_t* idx_out,
                                      float* gates_out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                      int32_t stage) {
  if (stage < MD_STAGE_SHARED || stage > MD_STAGE_COMBINE) return fail(MD_ERR_INVALID_ARG, "stage %d", stage);
  return moe_forward(L, x, T, y, idx_out, gates_out, workspace, workspace_bytes, stream, -1, nullptr, nullptr,
                     nullptr, stage);
}

md_status md_moe_layer_forward_residual(const md_moe_layer* L, const float* x, int32_t T, const float* residual,
                                        float* y, int32_t* idx_out, float* gates_out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (!residual) return fail(MD_ERR_INVALID_ARG, "residual is null");
  if (!aligned16(residual)) return fail(MD_ERR_ALIGNMENT, "residual not 16-byte aligned");
  return moe_forward(L, x, T, y, idx_out, gates_out, workspace, workspace_bytes, stream, -1, nullptr, nullptr,
                     residual, -1, true);
}

md_status md_add(const float* a, const float* b, float* y, int64_t n, hipStream_t stream) {
  if (n <= 0) return fail(MD_ERR_SHAPE, "n = %lld must be positive", (long long)n);
  if (!a || !b || !y) return fail(MD_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(a) || !aligned16(b) || !aligned16(y)) return fail(MD_ERR_ALIGNMENT, "pointers not 16-byte aligned");
  const hipError_t e = md::launch_add(a, b, y, n, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "add launch");
}

md_status md_moe_experts_forward(const md_moe_layer* L, const float* x, int32_t T, const int32_t* idx,
                                 const float* gates, float* y, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return experts_forward(L, x, T, idx, gates, y, workspace, workspace_bytes, stream);
}

// ---- host-memory expert tier ------------------------------------------------

md_status md_expert_cache_reset(md_expert_cache* c) {
  if (!c || !c->slot_of_expert || !c->expert_in_slot || !c->uses || !c->last_use)
    return fail(MD_ERR_INVALID_ARG, "null cache or cache array");
  if (c->E <= 0 || c->S <= 0) return fail(MD_ERR_SHAPE, "E = %d, S = %d", c->E, c->S);
  for (int e = 0; e < c->E; ++e) c->slot_of_expert[e] = -1;
  for (int j = 0; j < c->S; ++j) {
    c->expert_in_slot[j] = -1;
    c->uses[j] = 0;
    c->last_use[j] = 0;
  }
  c->step = 0;
  c->hits = 0;
  c->misses = 0;
  return ok();
}

md_status md_expert_cache_plan(md_expert_cache* c, const int32_t* idx, int32_t n, int32_t* slot_idx,
                               int32_t* miss_expert, int32_t* miss_slot, int32_t* n_miss) {
  if (!c || !c->slot_of_expert || !c->expert_in_slot || !c->uses || !c->last_use)
    return fail(MD_ERR_INVALID_ARG, "null cache or cache array");
  if (!idx || !slot_idx || !miss_expert || !miss_slot || !n_miss) return fail(MD_ERR_INVALID_ARG, "null argument");
  if (n <= 0 || n > kMaxT * kMaxK) return fail(MD_ERR_SHAPE, "n = %d outside 1..%d", n, kMaxT * kMaxK);
  // validate everything before any state changes
  int distinct[kMaxT * kMaxK];
  int nd = 0;
  for (int i = 0; i < n; ++i) {
    const int e = idx[i];
    if (e < 0 || e >= c->E) return fail(MD_ERR_INVALID_ARG, "idx[%d] = %d outside [0, %d)", i, e, c->E);
    bool seen = false;
    for (int j = 0; j < nd && !seen; ++j) seen = distinct[j] == e;
    if (!seen) distinct[nd++] = e;
  }
  if (nd > c->S) return fail(MD_ERR_UNSUPPORTED, "%d distinct experts in one call, %d slots", nd, c->S);
  const int64_t step = ++c->step;
  // hits first: they keep their slots for this call
  for (int j = 0; j < nd; ++j) {
    const int sl = c->slot_of_expert[distinct[j]];
    if (sl >= 0) {
      c->uses[sl] += 1;
      c->last_use[sl] = step;
      c->hits += 1;
    }
  }
  // misses in order of first appearance: an empty slot (lowest index), else
  // the least frequently used slot not used in this call, ties to the least
  // recently used, then to the lowest index
  int nm = 0;
  for (int j = 0; j < nd; ++j) {
    const int e = distinct[j];
    if (c->slot_of_expert[e] >= 0) continue;
    int v = -1;
    for (int sl = 0; sl < c->S && v < 0; ++sl)
      if (c->expert_in_slot[sl] < 0) v = sl;
    if (v < 0) {
      for (int sl = 0; sl < c->S; ++sl) {
        if (c->last_use[sl] == step) continue;
        if (v < 0 || c->uses[sl] < c->uses[v] || (c->uses[sl] == c->uses[v] && c->last_use[sl] < c->last_use[v]))
          v = sl;
      }
    }
    // (nd <= S guarantees a victim: at most nd - 1 other slots are in use by this call)
    if (c->expert_in_slot[v] >= 0) c->slot_of_expert[c->expert_in_slot[v]] = -1;
    c->expert_in_slot[v] = e;
    c->slot_of_expert[e] = v;
    c->uses[v] = 1;
    c->last_use[v] = step;
    c->misses += 1;
    miss_expert[nm] = e;
    miss_slot[nm] = v;
    ++nm;
  }
  for (int i = 0; i < n; ++i) slot_idx[i] = c->slot_of_expert[idx[i]];
  *n_miss = nm;
  return ok();
}

static md_status check_tier_pair(const md_moe_layer* src, const md_moe_layer* dst) {
  if (!src || !dst) return fail(MD_ERR_INVALID_ARG, "null layer descriptor");
  if (src->H != dst->H || src->F != dst->F || src->type != dst->type || src->act != dst->act || src->k != dst->k)
    return fail(MD_ERR_SHAPE, "host experts and slots differ in shape, type, act or k");
  if (!src->gate_q || !src->up_q || !src->down_q || !dst->gate_q || !dst->up_q || !dst->down_q)
    return fail(MD_ERR_INVALID_ARG, "null expert weights");
  if (row_type(src->type) && (!src->gate_scale || !src->up_scale || !src->down_scale || !dst->gate_scale ||
                              !dst->up_scale || !dst->down_scale))
    return fail(MD_ERR_INVALID_ARG, "per-row type without scales");
  return MD_OK;
}

md_status md_expert_cache_fill(const md_moe_layer* src, const md_moe_layer* dst, const int32_t* miss_expert,
                               const int32_t* miss_slot, int32_t n_miss, hipStream_t stream) {
  md_status s = check_tier_pair(src, dst);
  if (s != MD_OK) return s;
  if (n_miss < 0) return fail(MD_ERR_SHAPE, "n_miss = %d", n_miss);
  if (n_miss > 0 && (!miss_expert || !miss_slot)) return fail(MD_ERR_INVALID_ARG, "null miss list");
  for (int i = 0; i < n_miss; ++i) {
    if (miss_expert[i] < 0 || miss_expert[i] >= src->E || miss_slot[i] < 0 || miss_slot[i] >= dst->E)
      return fail(MD_ERR_INVALID_ARG, "miss %d: expert %d / slot %d out of range", i, miss_expert[i], miss_slot[i]);
  }
  const int64_t gb = (int64_t)src->F * md::row_bytes(src->type, src->H);
  const int64_t db = (int64_t)src->H * md::row_bytes(src->type, src->F);
  auto cp = [&](const void* from, int64_t fi, void* to, int64_t ti, int64_t bytes) {
    return hipMemcpyAsync(static_cast<char*>(to) + ti * bytes, static_cast<const char*>(from) + fi * bytes,
                          (size_t)bytes, hipMemcpyDefault, stream);
  };
  for (int i = 0; i < n_miss; ++i) {
    const int e = miss_expert[i], sl = miss_slot[i];
    hipError_t r = cp(src->gate_q, e, const_cast<void*>(dst->gate_q), sl, gb);
    if (r == hipSuccess) r = cp(src->up_q, e, const_cast<void*>(dst->up_q), sl, gb);
    if (r == hipSuccess) r = cp(src->down_q, e, const_cast<void*>(dst->down_q), sl, db);
    if (r == hipSuccess && row_type(src->type)) {
      r = cp(src->gate_scale, e, const_cast<float*>(dst->gate_scale), sl, 4 * (int64_t)src->F);
      if (r == hipSuccess) r = cp(src->up_scale, e, const_cast<float*>(dst->up_scale), sl, 4 * (int64_t)src->F);
      if (r == hipSuccess) r = cp(src->down_scale, e, const_cast<float*>(dst->down_scale), sl, 4 * (int64_t)src->H);
    }
    if (r != hipSuccess) return hip_fail(r, "expert copy");
  }
  return ok();
}

// Workspace of md_moe_cached_forward: the router's, the routing (expert ids,
// gates, slot ids), then the slot layer's experts forward.
struct CachedWs {
  size_t route, idx, gates, slots, experts, total;
};
static md_status cached_ws(const md_moe_layer* src, const md_moe_layer* dst, int T, CachedWs& w) {
  size_t route = 0;
  md_status s = md_route_workspace_size(T, src->H, src->E, src->k, &route);
  if (s != MD_OK) return s;
  if ((s = check_moe(dst, T)) != MD_OK) return s;
  w.route = 0;
  w.idx = align256(route);
  w.gates = w.idx + align256(sizeof(int) * T * src->k);
  w.slots = w.gates + align256(sizeof(float) * T * src->k);
  w.experts = w.slots + align256(sizeof(int) * T * src->k);
  w.total = w.experts + moe_ws(dst, T).total;
  return MD_OK;
}

md_status md_moe_cached_workspace_size(const md_moe_layer* src, const md_moe_layer* dst, int32_t T, size_t* bytes) {
  md_status s = check_tier_pair(src, dst);
  if (s != MD_OK) return s;
  if (!bytes) return fail(MD_ERR_INVALID_ARG, "null bytes");
  CachedWs w{};
  if ((s = cached_ws(src, dst, T, w)) != MD_OK) return s;
  *bytes = w.total;
  return ok();
}

md_status md_moe_cached_forward(const md_moe_layer* src, const md_moe_layer* dst, md_expert_cache* c, const float* x,
                                int32_t T, float* y, int32_t* idx_out, float* gates_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, hipStream_t copy_stream,
                                hipEvent_t copy_done) {
  md_status s = check_tier_pair(src, dst);
  if (s != MD_OK) return s;
  if (!c || !c->slot_idx) return fail(MD_ERR_INVALID_ARG, "null cache or cache scratch");
  if (c->E != src->E || c->S != dst->E) return fail(MD_ERR_SHAPE, "cache of %d experts / %d slots for a %d-expert "
                                                    "layer with %d slots", c->E, c->S, src->E, dst->E);
  if (!src->W_r) return fail(MD_ERR_INVALID_ARG, "null router weights");
  if (copy_stream && !copy_done) return fail(MD_ERR_INVALID_ARG, "a copy stream needs an event");
  if (!x || !y) return fail(MD_ERR_INVALID_ARG, "null x or y");
  if (!aligned16(x) || !aligned16(y) || (idx_out && !aligned16(idx_out)) || (gates_out && !aligned16(gates_out)))
    return fail(MD_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  CachedWs w{};
  if ((s = cached_ws(src, dst, T, w)) != MD_OK) return s;
  if ((s = check_ws(workspace, workspace_bytes, w.total)) != MD_OK) return s;
  char* ws = static_cast<char*>(workspace);
  const int n = T * src->k;
  int* idx = idx_out ? idx_out : reinterpret_cast<int*>(ws + w.idx);
  float* gates = gates_out ? gates_out : reinterpret_cast<float*>(ws + w.gates);
  int* slots = reinterpret_cast<int*>(ws + w.slots);
  // 1. routing on the GPU, 2. read back (the one synchronisation), 3. the
  // cache decides hits and misses, 4. misses copied from host memory,
  // 5. the slot ids, 6. the experts on the slots
  s = md_moe_route_topk(x, T, src->H, src->W_r, src->router_bias, src->E, src->k, idx, gates, nullptr, ws + w.route,
                        w.idx - w.route, stream);
  if (s != MD_OK) return s;
  int host_idx[kMaxT * kMaxK];
  hipError_t e = hipMemcpyAsync(host_idx, idx, sizeof(int) * n, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "routing read-back");
  int miss_e[kMaxT * kMaxK], miss_s[kMaxT * kMaxK], nm = 0;
  if ((s = md_expert_cache_plan(c, host_idx, n, c->slot_idx, miss_e, miss_s, &nm)) != MD_OK) return s;
  // the misses load on the copy stream while the shared expert (resident)
  // runs on the compute stream; the routed experts wait for both
  auto rest = [&]() -> md_status {
    md_status r = md_expert_cache_fill(src, dst, miss_e, miss_s, nm, copy_stream ? copy_stream : stream);
    if (r != MD_OK) return r;
    if (copy_stream && (e = hipEventRecord(copy_done, copy_stream)) != hipSuccess) return hip_fail(e, "event record");
    e = hipMemcpyAsync(slots, c->slot_idx, sizeof(int) * n, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "slot ids copy");
    char* xws = ws + w.experts;
    float* y_s = nullptr;
    if ((r = shared_phase(dst, x, T, xws, stream, &y_s)) != MD_OK) return r;
    if (copy_stream && (e = hipStreamWaitEvent(stream, copy_done, 0)) != hipSuccess) return hip_fail(e, "event wait");
    return routed_phase(dst, x, T, slots, gates, y_s, y, xws, stream);
  };
  s = rest();
  if (s != MD_OK) {
    // the plan already gave the missed experts their slots, whose copies may
    // not have run or may have run in part: the slots are marked empty, so
    // no later call takes what they hold for a resident expert
    for (int i = 0; i < nm; ++i) {
      c->slot_of_expert[miss_e[i]] = -1;
      c->expert_in_slot[miss_s[i]] = -1;
      c->uses[miss_s[i]] = 0;
      c->last_use[miss_s[i]] = 0;
    }
  }
  return s;
}

md_status md_hbm_read_probe(const void* src, size_t nbytes, uint32_t key, uint32_t* sink, int32_t workgroups,
                             hipStream_t stream) {
  if (!src || !sink) return fail(MD_ERR_INVALID_ARG, "null pointer");
  if (nbytes == 0 || nbytes % 16) return fail(MD_ERR_SHAPE, "nbytes = %zu must be a positive multiple of 16", nbytes);
  if (!aligned16(src)) return fail(MD_ERR_ALIGNMENT, "src not 16-byte aligned");
  if (workgroups < 0 || workgroups > (1 << 20))
    return fail(MD_ERR_INVALID_ARG, "workgroups = %d outside 0..1048576", workgroups);
  const hipError_t e = md::launch_read_probe(src, (int64_t)(nbytes / 16), key, sink,
                                             workgroups ? workgroups : 2048, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "read probe launch");
}

}  // extern "C"
