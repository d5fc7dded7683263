// gemv.hip -- decode-path contractions over quantized rows (gfx950, wave64).
//
// One engine serves every decode-shaped contraction: a wave is split into
// G = 64/L groups of L lanes; a group owns R rows; lane t of a group walks the
// 16-byte chunks t, t+L, t+2L, ... of those R rows (R independent 16-byte
// loads in flight per step), decodes them in registers and accumulates in
// fp32 against the activations of up to B tokens.  The L partial sums of a
// row are then combined with cross-lane shuffles.  Rows are read once per
// pass; when an expert serves more than B tokens the pass repeats.
//
//   k_qgemv    dense y = W x (batch <= 8), split-K across blocks for short-N
//              shapes with a fixed-order second pass (no atomics)
//   k_gateup   per active expert: a = W_g x, u = W_u x, h = act(a) * u
//   k_down     per active expert: o = W_d h
//   k_combine  y[t] = sum_j g[t][j] * o[pos(t, j)] (+ shared), slot order
#include "common.hpp"
#include "kernels.hpp"

namespace md {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

// chunks cs[0..N) of the R rows (all in range) against the activations,
// their weight loads issued together; sums in chunk order
template <int FMT, int XT, int R, int B, int N>
MD_DEV void chunks_dot(const uint8_t* const (&rowp)[R], int K, const int (&cs)[N], const void* const (&xp)[B],
                       float (&acc)[R][B]) {
  constexpr int W = Fmt<FMT>::WPC;
  u32x4 w[N][R];
  float sc[N][R], mn[N][R];
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r) w[u][r] = ld_stream(rowp[r] + 16 * (int64_t)cs[u]);
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sc[u][r] = chunk_scale<FMT>(rowp[r], K, cs[u]);
      if constexpr (FMT == Q4_1) mn[u][r] = chunk_min_q4_1(rowp[r], K, cs[u]);
    }
  // one token, at most 64 activations in all: those of every chunk loaded here too
  constexpr bool XPRE = B == 1 && N > 1 && N * W <= 64;
  float xpre[XPRE ? N : 1][W];
  if constexpr (XPRE) {
#pragma unroll
    for (int u = 0; u < N; ++u) load_x<FMT, XT>(xp[0], cs[u], xpre[u]);
  }
  // keep every load above issued before the first product (the scheduler
  // would otherwise interleave them with the products and wait on each)
  if constexpr (N > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < N; ++u) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float xv[W];
      if constexpr (XPRE) {
#pragma unroll
        for (int i = 0; i < W; ++i) xv[i] = xpre[u][i];
      } else {
        load_x<FMT, XT>(xp[b], cs[u], xv);
      }
      float sx = 0.f;  // Q4_1: the block's sum of activations, for its minimum
      if constexpr (FMT == Q4_1) {
#pragma unroll
        for (int i = 0; i < W; ++i) sx += xv[i];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float d = dot_chunk<FMT>(w[u][r], xv);
        if constexpr (Fmt<FMT>::ROW) acc[r][b] += d;
        else if constexpr (FMT == Q4_1) acc[r][b] = fmaf(sc[u][r], d, fmaf(mn[u][r], sx, acc[r][b]));
        else acc[r][b] = fmaf(sc[u][r], d, acc[r][b]);
      }
    }
  }
}

// Lane t of a group of L sums chunks c0 + t, c0 + t + L, ... below c1, in
// order.  One row of one or two tokens (long rows: one row per lane group):
// passes of 64 weights' chunks (four Q8_0/int8 chunks, two 4-bit ones) with
// all their loads in flight; two rows of 16-weight chunks for one token: two
// chunks of each; then the last few chunks one at a time, as for the other
// shapes, whose loads the loop's unrolling overlaps.
template <int FMT, int XT, int L, int R, int B>
MD_DEV void rows_dot(const uint8_t* const (&rowp)[R], int K, int c0, int c1, int t,
                     const void* const (&xp)[B], float (&acc)[R][B]) {
  constexpr int W = Fmt<FMT>::WPC;
  constexpr int U = (R == 1 && B <= 2) ? 64 / W : (R == 2 && B == 1 && W <= 16) ? 2 : 1;
  int c = c0 + t;
  if constexpr (U > 1) {
    for (; c + (U - 1) * L < c1; c += U * L) {
      int cs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) cs[u] = c + u * L;
      chunks_dot<FMT, XT, R, B, U>(rowp, K, cs, xp, acc);
    }
  }
#pragma unroll 2
  for (; c < c1; c += L) {
    const int cs[1] = {c};
    chunks_dot<FMT, XT, R, B, 1>(rowp, K, cs, xp, acc);
  }
}

template <int XT>
MD_DEV const void* xrow(const void* x, int64_t elem) {
  if constexpr (XT == XF32) return static_cast<const float*>(x) + elem;
  else return static_cast<const uint16_t*>(x) + elem;
}

// ------------------------------------------------------------------ qgemv

template <int FMT, int XT, int L, int R, int B>
__global__ __launch_bounds__(kBlock) void k_qgemv(const uint8_t* __restrict__ W, const float* __restrict__ scales,
                                                  int N, int K, const void* __restrict__ x, int nb,
                                                  float* __restrict__ out, int S) {
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / L, t = lane % L;
  const int row0 = ((blockIdx.x * kWaves + wave) * G + g) * R;
  if (row0 >= N) return;
  const int nc = nchunks(FMT, K);
  const int c0 = (int)((int64_t)blockIdx.y * nc / S), c1 = (int)((int64_t)(blockIdx.y + 1) * nc / S);
  const int64_t rb = row_bytes(FMT, K);
  const uint8_t* rowp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rowp[r] = W + (int64_t)min(row0 + r, N - 1) * rb;
  const void* xp[B];
#pragma unroll
  for (int b = 0; b < B; ++b) xp[b] = xrow<XT>(x, (int64_t)min(b, nb - 1) * K);
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.f;
  rows_dot<FMT, XT, L, R, B>(rowp, K, c0, c1, t, xp, acc);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = group_sum<L>(acc[r][b]);
  if (t == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r;
      if (row >= N) break;
      const float s = Fmt<FMT>::ROW ? scales[row] * row_post<FMT>() : 1.0f;
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (b < nb) out[((int64_t)blockIdx.y * nb + b) * N + row] = acc[r][b] * s;
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_splitk_reduce(const float* __restrict__ part, int S, int64_t n,
                                                          float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  float a = 0.f;
  for (int s = 0; s < S; ++s) a += part[(int64_t)s * n + i];
  y[i] = a;
}

hipError_t launch_splitk_reduce(const float* part, int S, int64_t n, float* y, hipStream_t st) {
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, part, S, n, y);
  return hipGetLastError();
}

static int pow2_divisor_le64(int n) {
  int L = 64;
  while (L > 1 && n % L) L >>= 1;
  return L;
}

GemvCfg qgemv_config(int fmt, int N, int K, int batch) {
  GemvCfg c{};
  const int nc = nchunks(fmt, K);
  // lanes per row group: the largest power of two (8..64) dividing the chunk
  // count, so lanes share the chunks evenly; at least 8 (rows of fewer chunks,
  // packed int2 at 256 columns, leave lanes idle)
  c.L = std::max(8, pow2_divisor_le64(nc));
  c.B = batch <= 1 ? 1 : batch <= 2 ? 2 : batch <= 4 ? 4 : 8;
  const int G = 64 / c.L;
  // rows per lane group: about four 16-byte row chunks in flight per lane
  // (measured: more makes each wave's chain longer than the extra overlap
  // gains), fewer if the grid would then hold less than 1024 waves; K is
  // split (uneven ranges allowed, a second pass adds the slices) only for
  // grids still below that, every K-slice keeping >= 2 chunks per lane
  // (packed int2 at batch 2: four rows would spill, 64 activations a chunk)
  const int rmax = c.B <= 2 && !(fmt == I2_ROW && c.B == 2) ? 4 : 2;
  const int cpl = nc / c.L;
  c.R = 1;
  while (c.R < rmax && 2 * c.R * cpl <= 4) c.R *= 2;
  auto blocks = [&](int R) { return (N + kWaves * G * R - 1) / (kWaves * G * R); };
  while (c.R > 1 && (int64_t)blocks(c.R) * kWaves < 1024) c.R /= 2;
  c.rows_per_block = kWaves * G * c.R;
  const int bx = blocks(c.R);
  c.S = 1;
  while ((int64_t)bx * kWaves * c.S < 1024 && nc / (2 * c.S) >= 2 * c.L && c.S < 16) c.S *= 2;
  c.grid = dim3(bx, c.S);
  return c;
}

template <int FMT, int XT>
static hipError_t qgemv_fx(const GemvCfg& c, const uint8_t* W, const float* s, int N, int K, const void* x,
                           int nb, float* out, hipStream_t st) {
#define MD_Q(L_, R_, B_) \
  if (c.L == L_ && c.R == R_ && c.B == B_) { \
    hipLaunchKernelGGL((k_qgemv<FMT, XT, L_, R_, B_>), c.grid, dim3(kBlock), 0, st, W, s, N, K, x, nb, out, c.S); \
    return hipGetLastError(); }
#define MD_QL(L_) MD_Q(L_, 4, 1) MD_Q(L_, 2, 1) MD_Q(L_, 1, 1) MD_Q(L_, 4, 2) MD_Q(L_, 2, 2) MD_Q(L_, 1, 2) \
                  MD_Q(L_, 2, 4) MD_Q(L_, 1, 4) MD_Q(L_, 2, 8) MD_Q(L_, 1, 8)
  MD_QL(64) MD_QL(32) MD_QL(16) MD_QL(8)
#undef MD_QL
#undef MD_Q
  return hipErrorInvalidConfiguration;
}

hipError_t launch_qgemv(int fmt, int xt, const GemvCfg& c, const uint8_t* W, const float* scales, int N, int K,
                        const void* x, int batch, float* y, float* partial, hipStream_t st) {
  float* out = c.S > 1 ? partial : y;
  hipError_t e = hipErrorInvalidValue;
#define MD_F(F_) \
  if (fmt == F_) e = xt == XF32 ? qgemv_fx<F_, XF32>(c, W, scales, N, K, x, batch, out, st) \
                                : qgemv_fx<F_, XBF16>(c, W, scales, N, K, x, batch, out, st);
  MD_F(Q8_0) MD_F(Q4_0) MD_F(I8_ROW) MD_F(I4_ROW) MD_F(Q4_1) MD_F(I2_ROW)
#undef MD_F
  if (e != hipSuccess || c.S == 1) return e;
  const int64_t n = (int64_t)batch * N;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, partial, c.S,
                     n, y);
  return hipGetLastError();
}

// ------------------------------------------------------------------ MoE

struct ExpertRange {
  int e, p0, p1;
};

MD_DEV bool expert_range(const Disp& d, int slot, ExpertRange& r) {
  if (d.n_active == nullptr) {  // dense FFN: one expert, positions = tokens
    if (slot != 0) return false;
    r.e = 0; r.p0 = 0; r.p1 = d.T;
    return true;
  }
  if (slot >= *d.n_active) return false;
  r.e = d.active_e[slot];
  r.p0 = d.active_off[slot];
  r.p1 = d.active_off[slot + 1];
  return true;
}

MD_DEV int pos_token(const Disp& d, int q) { return d.n_active == nullptr ? q : d.pairs[q] / d.k; }

// Gate/up with the fused activation.  A group owns P row pairs (gate row f and
// up row f), i.e. R = 2P streamed rows.
template <int FMT, int L, int P, int B>
__global__ __launch_bounds__(kBlock) void k_gateup(const uint8_t* __restrict__ gq, const uint8_t* __restrict__ uq,
                                                   const float* __restrict__ gs, const float* __restrict__ us,
                                                   int64_t mat_bytes, int F, int H, int act, Disp d,
                                                   const float* __restrict__ x, float* __restrict__ h) {
  constexpr int G = 64 / L, R = 2 * P;
  ExpertRange er;
  if (!expert_range(d, blockIdx.y, er)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / L, t = lane % L;
  const int f0 = ((blockIdx.x * kWaves + wave) * G + g) * P;
  if (f0 >= F) return;
  const int64_t rb = row_bytes(FMT, H);
  const uint8_t* Gm = gq + (int64_t)er.e * mat_bytes;
  const uint8_t* Um = uq + (int64_t)er.e * mat_bytes;
  const uint8_t* rowp[R];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int f = min(f0 + p, F - 1);
    rowp[p] = Gm + (int64_t)f * rb;
    rowp[P + p] = Um + (int64_t)f * rb;
  }
  const int nc = nchunks(FMT, H);
  for (int q0 = er.p0; q0 < er.p1; q0 += B) {
    const void* xp[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xp[b] = x + (int64_t)pos_token(d, min(q0 + b, er.p1 - 1)) * H;
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = 0.f;
    rows_dot<FMT, XF32, L, R, B>(rowp, H, 0, nc, t, xp, acc);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = group_sum<L>(acc[r][b]);
    if (t == 0) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int f = f0 + p;
        if (f >= F) break;
        float sg = 1.f, su = 1.f;
        if constexpr (Fmt<FMT>::ROW) {
          sg = gs[(int64_t)er.e * F + f] * row_post<FMT>();
          su = us[(int64_t)er.e * F + f] * row_post<FMT>();
        }
#pragma unroll
        for (int b = 0; b < B; ++b)
          if (q0 + b < er.p1) h[(int64_t)(q0 + b) * F + f] = act_f(act, acc[p][b] * sg) * (acc[P + p][b] * su);
      }
    }
  }
}

template <int FMT, int L, int R, int B>
__global__ __launch_bounds__(kBlock) void k_down(const uint8_t* __restrict__ dq, const float* __restrict__ ds,
                                                 int64_t mat_bytes, int H, int F, Disp d,
                                                 const float* __restrict__ h, float* __restrict__ o) {
  constexpr int G = 64 / L;
  ExpertRange er;
  if (!expert_range(d, blockIdx.y, er)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / L, t = lane % L;
  const int i0 = ((blockIdx.x * kWaves + wave) * G + g) * R;
  if (i0 >= H) return;
  const int64_t rb = row_bytes(FMT, F);
  const uint8_t* Dm = dq + (int64_t)er.e * mat_bytes;
  const uint8_t* rowp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rowp[r] = Dm + (int64_t)min(i0 + r, H - 1) * rb;
  const int nc = nchunks(FMT, F);
  for (int q0 = er.p0; q0 < er.p1; q0 += B) {
    const void* xp[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xp[b] = h + (int64_t)min(q0 + b, er.p1 - 1) * F;
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = 0.f;
    rows_dot<FMT, XF32, L, R, B>(rowp, F, 0, nc, t, xp, acc);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = group_sum<L>(acc[r][b]);
    if (t == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = i0 + r;
        if (i >= H) break;
        const float s = Fmt<FMT>::ROW ? ds[(int64_t)er.e * H + i] * row_post<FMT>() : 1.0f;
#pragma unroll
        for (int b = 0; b < B; ++b)
          if (q0 + b < er.p1) o[(int64_t)(q0 + b) * H + i] = acc[r][b] * s;
      }
    }
  }
}

// y[t][i] = sum_j g[t][j] * o[pos(t,j)][i]  (+ y_shared[t][i]) (+ y_residual[t][i]),
// slot order, then the shared output, then the residual.
__global__ __launch_bounds__(kBlock) void k_combine(const float* __restrict__ o, const int* __restrict__ pos_of_pair,
                                                    const float* __restrict__ gates, int T, int k, int H,
                                                    const float* __restrict__ ys, const float* yr, float* y) {
  const int H4 = H / 4;
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= (int64_t)T * H4) return;
  const int t = (int)(i / H4), c = (int)(i % H4);
  // the positions and gates of the token's k <= 8 slots first, then all their
  // rows' loads in flight together, summed in slot order
  int pj[8];
  float gj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pj[j] = j < k ? pos_of_pair[t * k + j] : 0;
    gj[j] = j < k ? gates[t * k + j] : 0.f;
  }
  float4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = j < k ? reinterpret_cast<const float4*>(o + (int64_t)pj[j] * H)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      a.x = fmaf(gj[j], v[j].x, a.x); a.y = fmaf(gj[j], v[j].y, a.y);
      a.z = fmaf(gj[j], v[j].z, a.z); a.w = fmaf(gj[j], v[j].w, a.w);
    }
  }
  if (ys) {
    const float4 v = reinterpret_cast<const float4*>(ys + (int64_t)t * H)[c];
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  if (yr) {  // may be y itself: read before the write by the same thread
    const float4 v = reinterpret_cast<const float4*>(yr + (int64_t)t * H)[c];
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  reinterpret_cast<float4*>(y + (int64_t)t * H)[c] = a;
}

static int choose_R(int rows, int G, int experts, const int* opts, int nopt) {
  for (int i = 0; i < nopt; ++i) {
    const int per_wave = G * opts[i];
    const int64_t waves = (int64_t)((rows + per_wave - 1) / per_wave) * experts;
    if (waves >= 2048) return opts[i];
  }
  return opts[nopt - 1];
}

GemvCfg gateup_config(int fmt, int F, int H, int max_active, int T) {
  GemvCfg c{};
  c.L = std::max(8, pow2_divisor_le64(nchunks(fmt, H)));
  const int G = 64 / c.L;
  c.B = T == 1 ? 1 : 4;
  const int opts1[] = {2, 1};
  const int P = c.B == 1 ? choose_R(F, G, max_active, opts1, 2) : 1;
  c.R = 2 * P;
  c.rows_per_block = kWaves * G * P;  // row pairs per block
  c.grid = dim3((F + c.rows_per_block - 1) / c.rows_per_block, max_active);
  c.S = 1;
  return c;
}

GemvCfg down_config(int fmt, int H, int F, int max_active, int T) {
  GemvCfg c{};
  c.L = std::max(8, pow2_divisor_le64(nchunks(fmt, F)));
  const int G = 64 / c.L;
  c.B = T == 1 ? 1 : 4;
  const int opts[] = {4, 2, 1};
  c.R = c.B == 1 ? choose_R(H, G, max_active, opts, 3) : 1;
  c.rows_per_block = kWaves * G * c.R;
  c.grid = dim3((H + c.rows_per_block - 1) / c.rows_per_block, max_active);
  c.S = 1;
  return c;
}

template <int FMT>
static hipError_t gateup_f(const GemvCfg& c, const uint8_t* gq, const uint8_t* uq, const float* gs, const float* us,
                           int64_t mb, int F, int H, int act, const Disp& d, const float* x, float* h,
                           hipStream_t st) {
  const int P = c.R / 2;
#define MD_G(L_, P_, B_) \
  if (c.L == L_ && P == P_ && c.B == B_) { \
    hipLaunchKernelGGL((k_gateup<FMT, L_, P_, B_>), c.grid, dim3(kBlock), 0, st, gq, uq, gs, us, mb, F, H, act, d, \
                       x, h); \
    return hipGetLastError(); }
#define MD_GL(L_) MD_G(L_, 2, 1) MD_G(L_, 1, 1) MD_G(L_, 1, 4)
  MD_GL(64) MD_GL(32) MD_GL(16) MD_GL(8)
#undef MD_GL
#undef MD_G
  return hipErrorInvalidConfiguration;
}

hipError_t launch_gateup(int fmt, const GemvCfg& c, const uint8_t* gq, const uint8_t* uq, const float* gs,
                         const float* us, int64_t mat_bytes, int F, int H, int act, const Disp& d,
                         const float* x, float* h, hipStream_t st) {
  switch (fmt) {
    case Q8_0: return gateup_f<Q8_0>(c, gq, uq, gs, us, mat_bytes, F, H, act, d, x, h, st);
    case Q4_0: return gateup_f<Q4_0>(c, gq, uq, gs, us, mat_bytes, F, H, act, d, x, h, st);
    case I8_ROW: return gateup_f<I8_ROW>(c, gq, uq, gs, us, mat_bytes, F, H, act, d, x, h, st);
    case I4_ROW: return gateup_f<I4_ROW>(c, gq, uq, gs, us, mat_bytes, F, H, act, d, x, h, st);
    case I2_ROW: return gateup_f<I2_ROW>(c, gq, uq, gs, us, mat_bytes, F, H, act, d, x, h, st);
    case Q4_1: return gateup_f<Q4_1>(c, gq, uq, gs, us, mat_bytes, F, H, act, d, x, h, st);
  }
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t down_f(const GemvCfg& c, const uint8_t* dq, const float* ds, int64_t mb, int H, int F,
                         const Disp& d, const float* h, float* o, hipStream_t st) {
#define MD_D(L_, R_, B_) \
  if (c.L == L_ && c.R == R_ && c.B == B_) { \
    hipLaunchKernelGGL((k_down<FMT, L_, R_, B_>), c.grid, dim3(kBlock), 0, st, dq, ds, mb, H, F, d, h, o); \
    return hipGetLastError(); }
#define MD_DL(L_) MD_D(L_, 4, 1) MD_D(L_, 2, 1) MD_D(L_, 1, 1) MD_D(L_, 1, 4)
  MD_DL(64) MD_DL(32) MD_DL(16) MD_DL(8)
#undef MD_DL
#undef MD_D
  return hipErrorInvalidConfiguration;
}

hipError_t launch_down(int fmt, const GemvCfg& c, const uint8_t* dq, const float* ds, int64_t mat_bytes, int H,
                       int F, const Disp& d, const float* h, float* o, hipStream_t st) {
  switch (fmt) {
    case Q8_0: return down_f<Q8_0>(c, dq, ds, mat_bytes, H, F, d, h, o, st);
    case Q4_0: return down_f<Q4_0>(c, dq, ds, mat_bytes, H, F, d, h, o, st);
    case I8_ROW: return down_f<I8_ROW>(c, dq, ds, mat_bytes, H, F, d, h, o, st);
    case I4_ROW: return down_f<I4_ROW>(c, dq, ds, mat_bytes, H, F, d, h, o, st);
    case I2_ROW: return down_f<I2_ROW>(c, dq, ds, mat_bytes, H, F, d, h, o, st);
    case Q4_1: return down_f<Q4_1>(c, dq, ds, mat_bytes, H, F, d, h, o, st);
  }
  return hipErrorInvalidValue;
}

// y = a + b, fp32, n values (16-byte chunks, then the tail).
__global__ __launch_bounds__(kBlock) void k_add(const float* __restrict__ a, const float* __restrict__ b,
                                                float* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t n4 = n / 4;
  if (i < n4) {
    const float4 u = reinterpret_cast<const float4*>(a)[i], v = reinterpret_cast<const float4*>(b)[i];
    reinterpret_cast<float4*>(y)[i] = make_float4(u.x + v.x, u.y + v.y, u.z + v.z, u.w + v.w);
  } else if (i < n4 + (n & 3)) {
    const int64_t j = 4 * n4 + (i - n4);
    y[j] = a[j] + b[j];
  }
}

__global__ __launch_bounds__(kBlock) void k_copy_f32(const float* __restrict__ a, float* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) y[i] = a[i];
}

hipError_t launch_copy_f32(const float* a, float* y, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, a, y, n);
  return hipGetLastError();
}

hipError_t launch_add(const float* a, const float* b, float* y, int64_t n, hipStream_t st) {
  const int64_t threads = n / 4 + (n & 3);
  hipLaunchKernelGGL(k_add, dim3((unsigned)((threads + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, a, b, y, n);
  return hipGetLastError();
}

// The attainable HBM read bandwidth, the practical ceiling of every weight
// stream here: each workgroup reads groups of U tiles of kBlock x kProbeU
// 16-byte chunks (the kernels' streaming loads), groups taken in address order
// across the grid, all U x kProbeU loads of a lane in flight before any is
// used (U = the tiles per workgroup the grid implies, 1 to 4).  Indexes past
// the end are clamped (the last chunk is read again) so no load sits under a
// branch.  A lane stores the xor of the words it read only when that equals
// `key`, which the caller picks so that it does not happen for the data; the
// loads cannot be dropped.
constexpr int kProbeU = 8;

template <int U>
__global__ __launch_bounds__(kBlock) void k_read_probe(const uint4* __restrict__ src, int64_t n16, uint32_t key,
                                                       uint32_t* sink) {
  constexpr int64_t group = (int64_t)U * kBlock * kProbeU;
  const uint8_t* base8 = reinterpret_cast<const uint8_t*>(src);
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * group; base < n16; base += (int64_t)gridDim.x * group) {
    u32x4 v[U * kProbeU];
#pragma unroll
    for (int j = 0; j < U * kProbeU; ++j) {
      const int64_t i = base + j * kBlock + threadIdx.x;
      v[j] = ld_stream(base8 + 16 * (i < n16 ? i : n16 - 1));
    }
#pragma unroll
    for (int j = 0; j < U * kProbeU; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  if (acc == key) sink[0] = acc;
}

hipError_t launch_read_probe(const void* src, int64_t n16, uint32_t key, uint32_t* sink, int grid,
                             hipStream_t st) {
  const int64_t tiles = (n16 + (int64_t)kBlock * kProbeU - 1) / ((int64_t)kBlock * kProbeU);
  const int g = (int)std::min<int64_t>(grid, tiles);
  const int64_t per = (tiles + g - 1) / g;  // tiles per workgroup
  const uint4* s4 = static_cast<const uint4*>(src);
  if (per >= 4) {
    hipLaunchKernelGGL(k_read_probe<4>, dim3((unsigned)std::min<int64_t>(g, (tiles + 3) / 4)), dim3(kBlock), 0, st,
                       s4, n16, key, sink);
  } else if (per >= 2) {
    hipLaunchKernelGGL(k_read_probe<2>, dim3((unsigned)((tiles + 1) / 2)), dim3(kBlock), 0, st, s4, n16, key, sink);
  } else {
    hipLaunchKernelGGL(k_read_probe<1>, dim3((unsigned)tiles), dim3(kBlock), 0, st, s4, n16, key, sink);
  }
  return hipGetLastError();
}

// A given routing made safe to index with: entries clamped into [0, E).
__global__ __launch_bounds__(kBlock) void k_clamp_idx(const int* __restrict__ in, int n, int E, int* __restrict__ out) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < n) out[i] = min(max(in[i], 0), E - 1);
}

hipError_t launch_clamp_idx(const int* in, int n, int E, int* out, hipStream_t st) {
  hipLaunchKernelGGL(k_clamp_idx, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, in, n, E, out);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o, const int* pos_of_pair, const float* gates, int T, int k, int H,
                          const float* y_shared, const float* y_residual, float* y, hipStream_t st) {
  const int64_t n = (int64_t)T * (H / 4);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, o, pos_of_pair,
                     gates, T, k, H, y_shared, y_residual, y);
  return hipGetLastError();
}

}  // namespace md
