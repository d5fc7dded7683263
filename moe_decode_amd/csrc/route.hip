// route.hip -- top-k selection with softmax gates for many tokens, the expert
// dispatch, and the weight layout pass (gfx950, wave64).
//
// The logits are formed from k_router_part's fp64 partials (added in a fixed
// order, plus the bias, rounded once to fp32).  Selection uses 64-bit keys: the order-preserving image of the fp32 logit in
// the high word (with -0 folded onto +0) and the complemented expert index in
// the low word, so one integer maximum picks the largest logit and, among
// exact ties, the lower expert index -- the tie rule of the Camelid README,
// "Experimental lanes".
#include "common.hpp"
#include "kernels.hpp"

namespace md {

// -------------------------------------------------------------- select

MD_DEV uint32_t order_key(float l) {
  uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

MD_DEV uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// One workgroup (1024 threads).  Wave w handles tokens w, w+16, ...
// Then (when d != nullptr) a stable counting sort of the T*k pairs by expert:
// per-expert token bitmasks give each pair its rank among the pairs of its
// expert (pairs of one expert are ordered by token, and a token selects an
// expert at most once), exclusive scans give the offsets and the list of
// active experts in ascending order.
__global__ __launch_bounds__(1024) void k_route_finalize(const double* __restrict__ part, int S,
                                                         const float* __restrict__ bias, int T, int E, int k,
                                                         float* __restrict__ logits, int* __restrict__ idx,
                                                         float* __restrict__ gates, DispOut d, int do_disp) {
  __shared__ uint32_t mask[256][4];
  __shared__ int sel[128 * 8];
  __shared__ int cnt[256], poff[256], apos[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 256 * 4; i += 1024) (&mask[0][0])[i] = 0u;
  __syncthreads();

  for (int t = wave; t < T; t += 16) {
    uint64_t key[4];
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      key[i] = 0;
      lv[i] = 0.f;
      if (e < E) {
        double a = 0.0;
        for (int s = 0; s < S; ++s) a += part[((int64_t)t * E + e) * S + s];
        if (bias) a += (double)bias[e];
        const float l = (float)a;
        if (logits) logits[(int64_t)t * E + e] = l;
        lv[i] = l;
        key[i] = ((uint64_t)order_key(l) << 32) | (uint32_t)(~(uint32_t)e);
      }
    }
    float sl[8];
    int se[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = (int)(~(uint32_t)best);
      se[j] = e;
      // the owner lane retires the winner and publishes its logit
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == e) { key[i] = 0; l = lv[i]; }
      sl[j] = __shfl(l, e & 63, 64);
    }
    if (lane == 0) {
      const double m = (double)sl[0];
      double z = 0.0, ex[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k) { ex[j] = exp((double)sl[j] - m); z += ex[j]; }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < k) {
          idx[t * k + j] = se[j];
          gates[t * k + j] = (float)(ex[j] / z);
          sel[t * k + j] = se[j];
        }
      }
    }
    if (do_disp && lane < k) {
      int e = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j == lane) e = se[j];
      atomicOr(&mask[e][t >> 5], 1u << (t & 31));
    }
  }
  if (!do_disp) return;
  __syncthreads();
  // per-expert pair counts, active flags; exclusive scans by wave 0
  if (threadIdx.x < 256) {
    const int e = threadIdx.x;
    cnt[e] = e < E ? __popc(mask[e][0]) + __popc(mask[e][1]) + __popc(mask[e][2]) + __popc(mask[e][3]) : 0;
  }
  __syncthreads();
  if (wave == 0) {
    int run_p = 0, run_a = 0;
    for (int base = 0; base < 256; base += 64) {
      const int e = base + lane;
      const int c = cnt[e];
      const int a = c > 0 ? 1 : 0;
      int ic = c, ia = a;  // inclusive scans across the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int pc = __shfl_up(ic, off, 64), pa = __shfl_up(ia, off, 64);
        if (lane >= off) { ic += pc; ia += pa; }
      }
      poff[e] = run_p + ic - c;
      apos[e] = run_a + ia - a;
      run_p += __shfl(ic, 63, 64);
      run_a += __shfl(ia, 63, 64);
    }
    if (lane == 0) {
      *d.n_active = run_a;
      d.active_off[run_a] = T * k;
    }
  }
  __syncthreads();
  if (threadIdx.x < E && cnt[threadIdx.x] > 0) {
    const int e = threadIdx.x;
    d.active_e[apos[e]] = e;
    d.active_off[apos[e]] = poff[e];
  }
  for (int p = threadIdx.x; p < T * k; p += 1024) {
    const int t = p / k, e = sel[p];
    int rank = 0;
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(mask[e][w]);
    rank += __popc(mask[e][t >> 5] & ((1u << (t & 31)) - 1u));
    const int q = poff[e] + rank;
    d.pairs[q] = p;
    d.pos_of_pair[p] = q;
  }
}

hipError_t launch_route_finalize(const double* part, int S, const float* bias, int T, int E, int k, float* logits,
                                 int* idx, float* gates, const DispOut* d, hipStream_t st) {
  DispOut dd = d ? *d : DispOut{nullptr, nullptr, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL(k_route_finalize, dim3(1), dim3(1024), 0, st, part, S, bias, T, E, k, logits, idx, gates, dd,
                     d ? 1 : 0);
  return hipGetLastError();
}

// -------------------------------------------------------------- layout

// Canonical -> device layout, one thread per 32-weight block (Q8_0, Q4_0) or
// per 16 bytes (per-row formats, a plain copy).
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
  } else {
    const uint8_t* s = src + row * (int64_t)nb * 18 + (int64_t)j * 18;
    uint8_t* r = dst + row * (int64_t)nb * 18;
    for (int b = 0; b < 16; ++b) r[16 * j + b] = s[2 + b];
    r[16 * nb + 2 * j] = s[0];
    r[16 * nb + 2 * j + 1] = s[1];
  }
}

__global__ __launch_bounds__(256) void k_copy16(int64_t n16, const uint4* __restrict__ src, uint4* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

hipError_t launch_prepare_layout(int fmt, int rows, int cols, int count, const void* src, void* dst,
                                 hipStream_t st) {
  const int64_t nrows = (int64_t)rows * count;
  if (fmt == Q8_0 || fmt == Q4_0) {
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
