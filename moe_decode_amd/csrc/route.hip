// route.hip -- the chunk router GEMM, top-k selection with softmax gates for
// many tokens, the expert dispatch, and the weight layout pass (gfx950, wave64).
//
// The logits are formed from fp64 partials over K-slices (added in slice
// order, plus the bias, rounded once to fp32).  Selection uses 64-bit keys: the order-preserving image of the fp32 logit in
// the high word (with -0 folded onto +0) and the complemented expert index in
// the low word, so one integer maximum picks the largest logit and, among
// exact ties, the lower expert index -- the tie rule of the Camelid README,
// "Experimental lanes".
#include "common.hpp"
#include "kernels.hpp"
#include "rows.hpp"

namespace md {

typedef unsigned short u16;

// -------------------------------------------------------------- router

// Chunk router: logits partials of many tokens as a GEMM on the fp64 matrix
// cores (v_mfma_f64_16x16x4_f64).  Block (ex, ty, s) covers experts 64*ex..,
// tokens 64*ty.. and K-slice s; each wave owns 2 x 2 tiles of 16 experts x 16
// tokens.  W_r and x tiles are staged as fp32 in LDS (transposed, padded),
// each operand widened to fp64 as it is read (exact), and each product of two
// fp32 values is exact in fp64; the K-slice's terms accumulate in fp64.
constexpr int kRG = 64;   // experts / tokens per block tile
constexpr int kRKC = 32;  // K per LDS stage

// Per 4-wide K step a lane widens one W_r and one x element per tile row /
// column from the LDS stage.  Operand layout of the 16x16x4 fp64 MFMA
// (checked on the device): A[i][k] and B[k][j] at lane 16 k + i (j), result
// D[4 v + lane / 16][lane % 16] in element v.  The next stage's tiles are
// fetched into registers while a stage is used.
typedef double f64x4 __attribute__((ext_vector_type(4)));
//
// x_hi, x_lo (nullable): the blocks of the first expert tile also write the
// bf16 pair of every x value they stage (together they stage each value
// once), so the grouped GEMMs' activation forms need no launch of their own.
__global__ __launch_bounds__(256) void k_router_mfma(const float* __restrict__ x, int T, int H,
                                                     const float* __restrict__ Wr, int E, int Ks,
                                                     double* __restrict__ part, u16* __restrict__ x_hi,
                                                     u16* __restrict__ x_lo) {
  __shared__ float sw[kRKC][kRG + 1];
  __shared__ float sx[kRKC][kRG + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.x * kRG, t0 = blockIdx.y * kRG, sl = blockIdx.z;
  const int kbeg = sl * Ks;
  const int li = lane & 15, kq = lane >> 4;
  const int er0 = 2 * (wave & 1), tc0 = 2 * (wave >> 1);  // this wave's first tile row / column
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  float4 pw[2], px[2];
  auto fetch = [&](int kc) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + 256 * r, row = idx >> 3, c4 = idx & 7;
      pw[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      px[r] = pw[r];
      if (e0 + row < E) pw[r] = *reinterpret_cast<const float4*>(Wr + (int64_t)(e0 + row) * H + kc + 4 * c4);
      if (t0 + row < T) px[r] = *reinterpret_cast<const float4*>(x + (int64_t)(t0 + row) * H + kc + 4 * c4);
    }
  };
  fetch(kbeg);
  for (int kc = kbeg; kc < kbeg + Ks; kc += kRKC) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + 256 * r, row = idx >> 3, c4 = idx & 7;
      sw[4 * c4 + 0][row] = pw[r].x; sw[4 * c4 + 1][row] = pw[r].y;
      sw[4 * c4 + 2][row] = pw[r].z; sw[4 * c4 + 3][row] = pw[r].w;
      sx[4 * c4 + 0][row] = px[r].x; sx[4 * c4 + 1][row] = px[r].y;
      sx[4 * c4 + 2][row] = px[r].z; sx[4 * c4 + 3][row] = px[r].w;
      if (x_hi && blockIdx.x == 0 && t0 + row < T) {
        const float v[4] = {px[r].x, px[r].y, px[r].z, px[r].w};
        u16 h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 b = (__bf16)v[i];
          h[i] = __builtin_bit_cast(u16, b);
          l[i] = __builtin_bit_cast(u16, (__bf16)(v[i] - (float)b));
        }
        const int64_t o = (int64_t)(t0 + row) * H + kc + 4 * c4;
        *reinterpret_cast<ushort4*>(x_hi + o) = make_ushort4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<ushort4*>(x_lo + o) = make_ushort4(l[0], l[1], l[2], l[3]);
      }
    }
    __syncthreads();
    if (kc + kRKC < kbeg + Ks) fetch(kc + kRKC);
#pragma unroll
    for (int k4 = 0; k4 < kRKC; k4 += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = (double)sw[k4 + kq][16 * (er0 + a) + li];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = (double)sx[k4 + kq][16 * (tc0 + b) + li];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int t = t0 + 16 * (tc0 + b) + li;
      if (t >= T) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e = e0 + 16 * (er0 + a) + 4 * v + kq;
        if (e < E) part[((int64_t)sl * T + t) * E + e] = acc[a][b][v];
      }
    }
}

#ifndef MD_ROUTER_GEMM_BLOCKS
#define MD_ROUTER_GEMM_BLOCKS 256
#endif

RouterPlan router_plan(int T, int H, int E, bool pairs) {
  RouterPlan p{};
  if (T <= kMaxPairT || (pairs && T <= kMaxPairTSmall)) {  // one block per (expert, K-slice); partials [t][e][s]
    p.gemm = false;
    p.S = router_splits(H, E);
    p.ps = 1;
    p.pt = (int64_t)E * p.S;
    p.pe = p.S;
    return p;
  }
  // tiles x K-slices: the fewest slices giving MD_ROUTER_GEMM_BLOCKS blocks,
  // with at least two LDS stages per slice; partials [s][t][e]
  const int tiles = ((E + kRG - 1) / kRG) * ((T + kRG - 1) / kRG);
  const int units = H / kRKC;
  int S = 1;
  for (int d = 1; d <= units; ++d) {
    if (units % d || H / d < 2 * kRKC) continue;
    S = d;
    if (tiles * d >= MD_ROUTER_GEMM_BLOCKS) break;
  }
  p.gemm = true;
  p.S = S;
  p.ps = (int64_t)T * E;
  p.pt = E;
  p.pe = 1;
  return p;
}

hipError_t launch_router(const float* x, int T, int H, const float* Wr, int E, const RouterPlan& p, double* part,
                         const DigJob& j0, const DigJob& j1, hipStream_t st, u16* x_hi, u16* x_lo) {
  if (!p.gemm) {
    if (x_hi || x_lo) return hipErrorInvalidValue;
    return launch_router_part(x, T, H, Wr, E, p.S, part, j0, j1, st);
  }
  if (j0.x || j1.x || (x_hi == nullptr) != (x_lo == nullptr)) return hipErrorInvalidValue;
  const dim3 grid((E + kRG - 1) / kRG, (T + kRG - 1) / kRG, p.S);
  hipLaunchKernelGGL(k_router_mfma, grid, dim3(256), 0, st, x, T, H, Wr, E, H / p.S, part, x_hi, x_lo);
  return hipGetLastError();
}

// -------------------------------------------------------------- select

// One workgroup per token.  Thread e forms expert e's logit: the S partials
// added in slice order, then the bias, rounded once to fp32.  Wave 0 then
// takes the k winners one at a time (topk_rounds); lane j
// computes exp(l_j - l_0) in fp64, the sum runs over j in order, and lane j
// writes gate j.
__global__ __launch_bounds__(256) void k_select(const double* __restrict__ part, int S, int64_t ps, int64_t pt,
                                                int64_t pe, const float* __restrict__ bias, int T, int E, int k,
                                                float* __restrict__ logits, int* __restrict__ idx,
                                                float* __restrict__ gates) {
  __shared__ float s_l[256];
  const int t = blockIdx.x, e = threadIdx.x, lane = threadIdx.x & 63;
  if (e < E) {
    const double* p = part + t * pt + e * pe;
    // up to 32 slices' partials loaded before the first add (one memory
    // round trip instead of one per eight), then added in slice order
    double a = 0.0;
    for (int s = 0; s < S; s += 32) {
      const int n = S - s < 32 ? S - s : 32;
      double v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = i < n ? p[(int64_t)(s + i) * ps] : 0.0;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (i < n) a += v[i];
    }
    if (bias) a += (double)bias[e];
    const float l = (float)a;
    if (logits) logits[(int64_t)t * E + e] = l;
    s_l[e] = l;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = lane + 64 * i < E ? order_key32(s_l[lane + 64 * i]) : 0u;
  float my_l = 0.f;
  int sel[8];
  topk_rounds(key, k, lane, sel, my_l);
  int my_e = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (lane == j) my_e = sel[j];
  const double m = (double)__shfl(my_l, 0, 64);
  const double ex = lane < k ? exp((double)my_l - m) : 0.0;
  double z = 0.0;
  for (int j = 0; j < k; ++j) z += __shfl(ex, j, 64);
  if (lane < k) {
    idx[t * k + lane] = my_e;
    gates[t * k + lane] = (float)(ex / z);
  }
}

hipError_t launch_select(const double* part, const RouterPlan& p, const float* bias, int T, int E, int k,
                         float* logits, int* idx, float* gates, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(T), dim3(256), 0, st, part, p.S, p.ps, p.pt, p.pe, bias, T, E, k,
                     logits, idx, gates);
  return hipGetLastError();
}

// -------------------------------------------------------------- dispatch

// One workgroup (1024 threads): a stable counting sort of the T*k pairs by
// expert.  Per-expert token bitmasks give each pair its rank among the pairs
// of its expert (pairs of one expert are ordered by token, and a token
// selects an expert at most once); exclusive scans give the offsets and the
// list of active experts in ascending order, and the work items of the
// grouped GEMMs (16-position tiles of each active expert).
__global__ __launch_bounds__(1024) void k_dispatch(const int* __restrict__ idx, int T, int E, int k, DispOut d) {
  __shared__ uint32_t mask[256][4];
  __shared__ int cnt[256], poff[256], apos[256], ioff[256];
  __shared__ int s_items;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // one pair per thread (T * k <= 1024, checked at launch); its expert is
  // read once and kept for the rank pass at the end
  const int p = threadIdx.x;
  const bool has_pair = p < T * k;
  const int my_e = has_pair ? idx[p] : 0;
  for (int i = threadIdx.x; i < 256 * 4; i += 1024) (&mask[0][0])[i] = 0u;
  __syncthreads();
  if (has_pair) {
    const int t = p / k;
    atomicOr(&mask[my_e][t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    const int e = threadIdx.x;
    cnt[e] = e < E ? __popc(mask[e][0]) + __popc(mask[e][1]) + __popc(mask[e][2]) + __popc(mask[e][3]) : 0;
  }
  __syncthreads();
  if (wave == 0) {
    int run_p = 0, run_a = 0, run_i = 0;
    for (int base = 0; base < 256; base += 64) {
      const int e = base + lane;
      const int c = cnt[e];
      const int a = c > 0 ? 1 : 0;
      const int n = (c + kTokTile - 1) / kTokTile;
      int ic = c, ia = a, in = n;  // inclusive scans across the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int pc = __shfl_up(ic, off, 64), pa = __shfl_up(ia, off, 64), pn = __shfl_up(in, off, 64);
        if (lane >= off) { ic += pc; ia += pa; in += pn; }
      }
      poff[e] = run_p + ic - c;
      apos[e] = run_a + ia - a;
      ioff[e] = run_i + in - n;
      run_p += __shfl(ic, 63, 64);
      run_a += __shfl(ia, 63, 64);
      run_i += __shfl(in, 63, 64);
    }
    if (lane == 0) {
      *d.n_active = run_a;
      d.active_off[run_a] = T * k;
      s_items = run_i;
    }
  }
  __syncthreads();
  if (threadIdx.x < E && cnt[threadIdx.x] > 0) {
    const int e = threadIdx.x;
    d.active_e[apos[e]] = e;
    d.active_off[apos[e]] = poff[e];
    for (int i = 0; i * kTokTile < cnt[e]; ++i)
      d.items[ioff[e] + i] = make_int4(e, poff[e] + i * kTokTile, poff[e] + cnt[e], 0);
  }
  for (int i = s_items + (int)threadIdx.x; i < d.n_items_max; i += 1024) d.items[i] = make_int4(-1, 0, 0, 0);
  if (has_pair) {
    const int t = p / k, e = my_e;
    int rank = 0;
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(mask[e][w]);
    rank += __popc(mask[e][t >> 5] & ((1u << (t & 31)) - 1u));
    const int q = poff[e] + rank;
    d.pairs[q] = p;
    d.pos_of_pair[p] = q;
  }
}

hipError_t launch_dispatch(const int* idx, int T, int E, int k, const DispOut& d, hipStream_t st) {
  if (T < 1 || k < 1 || T * k > 1024 || T > 128 || E > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(1024), 0, st, idx, T, E, k, d);
  return hipGetLastError();
}

// -------------------------------------------------------------- layout

// Canonical -> device layout, one thread per 32-weight block (Q8_0, Q4_0,
// Q4_1) or per 16 bytes (per-row formats, a plain copy).
__global__ __launch_bounds__(256) void k_prepare_q(int fmt, int64_t nblocks, int nb, const uint8_t* __restrict__ src,
                                                   uint8_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const int64_t row = i / nb;
  const int j = (int)(i % nb);
  if (fmt == Q8_0) {
    const uint8_t* s = src + row * (int64_t)nb * 34 + (int64_t)j * 34;
    uint8_t* r = dst + row * (int64_t)nb * 34;
    for (int b = 0; b < 32; ++b) r[32 * j + b] = s[2 + b];
    r[32 * nb + 2 * j] = s[0];
    r[32 * nb + 2 * j + 1] = s[1];
  } else if (fmt == Q4_0) {
    const uint8_t* s = src + row * (int64_t)nb * 18 + (int64_t)j * 18;
    uint8_t* r = dst + row * (int64_t)nb * 18;
    for (int b = 0; b < 16; ++b) r[16 * j + b] = s[2 + b];
    r[16 * nb + 2 * j] = s[0];
    r[16 * nb + 2 * j + 1] = s[1];
  } else {  // Q4_1: qs, then the (d, m) pair
    const uint8_t* s = src + row * (int64_t)nb * 20 + (int64_t)j * 20;
    uint8_t* r = dst + row * (int64_t)nb * 20;
    for (int b = 0; b < 16; ++b) r[16 * j + b] = s[4 + b];
    for (int b = 0; b < 4; ++b) r[16 * nb + 4 * j + b] = s[b];
  }
}

__global__ __launch_bounds__(256) void k_copy16(int64_t n16, const uint4* __restrict__ src, uint4* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

hipError_t launch_prepare_layout(int fmt, int rows, int cols, int count, const void* src, void* dst,
                                 hipStream_t st) {
  const int64_t nrows = (int64_t)rows * count;
  if (fmt == Q8_0 || fmt == Q4_0 || fmt == Q4_1) {
    const int nb = cols / 32;
    const int64_t n = nrows * nb;
    hipLaunchKernelGGL(k_prepare_q, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, fmt, n, nb,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst));
  } else {
    const int64_t n16 = nrows * row_bytes(fmt, cols) / 16;
    hipLaunchKernelGGL(k_copy16, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, n16,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst));
  }
  return hipGetLastError();
}

}  // namespace md
