// decode.hip -- the one-token decode path of the MoE layer (gfx950, wave64).
//
// Three launches per layer call (five with a shared expert):
//   k_router_part  logits = W_r x (+ b) with fp64 accumulation, K split in S
//                  slices across workgroups (fp64 partials).
//   k_gateup_t1    each workgroup first forms the logits (partials added in a
//                  fixed order, plus the bias, rounded once to fp32) and
//                  selects the top-k experts (64-bit order keys: larger
//                  logit, then lower index),
//                  then streams gate and up rows of its slot's expert against
//                  the activations held in VGPRs, and writes h = act(a) * u.
//   k_down_t1      each workgroup owns a tile of output rows; wave j streams
//                  the down rows of slot j's expert against h_j held in VGPRs;
//                  the per-slot partials meet in LDS and are combined in slot
//                  order with the gates (+ the shared expert's output).
// The shared expert (a dense gated FFN) runs through the same two kernels in
// dense mode before the routed ones.
//
// Streaming: a lane group of L lanes owns a row; each lane owns one 16-byte
// chunk position per K-slice, so the activations it multiplies never change
// and stay in registers for every row the wave visits.  Activations enter as
// integer digit planes (digits.hpp): one v_dot8 (4-bit weights) or v_dot4
// (8-bit) per weight word and digit plane, exact int32 sums, one fp32 combine
// per chunk.  The router kernel writes the digit planes of x; the gate/up
// kernel writes those of h (each workgroup covers whole digit groups).  Row loads run in a
// rolling window (several rows in flight while one is decoded).  Partial sums of the rows a lane group visited are reduced with
// one transposed butterfly (N-1 exchanges for N rows instead of N log L).
#include <type_traits>

#include "common.hpp"
#include "digits.hpp"
#include "kernels.hpp"
#include "rows.hpp"

namespace md {

#ifndef MD_GU_MAXNP
#define MD_GU_MAXNP 8
#endif
#ifndef MD_DN_ROWS
#define MD_DN_ROWS 8
#endif
constexpr int kNRW = MD_DN_ROWS;   // output rows per workgroup in k_down_t1
#ifndef MD_DN_ROWS_PACKED
#define MD_DN_ROWS_PACKED 32
#endif
// Packed int4/int2 per-row weights: the h planes a lane loads are large next
// to the weight bytes of a row, so each wave streams 32 rows against them
// (measured: int2 layer 35.3 -> 32.0 us, int4 39.0 -> 38.3 us per token; the
// block formats and int8 stay at 8)
constexpr int dn_nrw(int fmt) { return (fmt == I2_ROW || fmt == I4_ROW) ? MD_DN_ROWS_PACKED : kNRW; }

// The digit planes of rows [0, R) of a row-major R x K fp32 matrix (K a
// multiple of 256), spread over nb workgroups (this one is b): each takes as
// few whole groups as cover them all (at most 256 values per pass).
MD_DEV void dig_rows(const DigJob& j, uint32_t* ys, int b, int nb) {
  if (!j.x) return;
  const int nv = dig_nv(j.fmt);
  const int64_t G = (int64_t)j.R * j.K / nv;
  int64_t per = (G + nb - 1) / nb;
  if (per > 256 / nv) per = 256 / nv;
  if (per < 1) per = 1;
  for (int64_t g0 = (int64_t)b * per; g0 < G; g0 += (int64_t)nb * per) {
    const int cnt = (int)(G - g0 < per ? G - g0 : per);
    const int n = cnt * nv;
    const float v = (int)threadIdx.x < n ? j.x[g0 * nv + threadIdx.x] : 0.f;
    switch (j.fmt) {
      case Q8_0: dig_block<Q8_0>(v, n, ys, j.planes + g0 * Dig<Q8_0>::NPL, j.scales + g0); break;
      case Q4_0: dig_block<Q4_0>(v, n, ys, j.planes + g0 * Dig<Q4_0>::NPL, j.scales + g0); break;
      case Q4_1: dig_block<Q4_1>(v, n, ys, j.planes + g0 * Dig<Q4_1>::NPL, j.scales + g0); break;
      case I8_ROW: dig_block<I8_ROW>(v, n, ys, j.planes + g0 * Dig<I8_ROW>::NPL, j.scales + g0); break;
      case I2_ROW: dig_block<I2_ROW>(v, n, ys, j.planes + g0 * Dig<I2_ROW>::NPL, j.scales + g0); break;
      default: dig_block<I4_ROW>(v, n, ys, j.planes + g0 * Dig<I4_ROW>::NPL, j.scales + g0); break;
    }
  }
}

// Workgroups that one pass of dig_rows needs for a job (0 without a job).
__host__ __device__ static int dig_blocks(const DigJob& j) {
  if (!j.x) return 0;
  const int nv = dig_nv(j.fmt);
  const int64_t G = (int64_t)j.R * j.K / nv;
  return (int)((G + 256 / nv - 1) / (256 / nv));
}

__global__ __launch_bounds__(256) void k_digits(DigJob j) {
  __shared__ uint32_t ys[256];
  dig_rows(j, ys, blockIdx.x, gridDim.x);
}

hipError_t launch_digits(const DigJob& j, hipStream_t st) {
  const int64_t n = (int64_t)j.R * j.K;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_digits, dim3(blocks), dim3(256), 0, st, j);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router

// Block (e, s): expert e, K-slice s of S; the four waves split the slice,
// each lane accumulates in fp64 for up to 4 tokens at a time, and the wave
// sums are added in a fixed order into part[t][e][s].  The consumer adds the
// S partials in order, then the bias, and rounds once to fp32.
// fp64 sum over the wave by DPP lane moves (quads, mirrored half-rows and
// rows, then the row broadcasts carry the total to lane 63); fixed order.
MD_DEV double wave_sum_f64_dpp(double v) {
  auto step = [&](auto ctrl, auto row_mask) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
    const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp(0, lo, decltype(ctrl)::value, decltype(row_mask)::value,
                                                                0xF, false);
    const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp(0, hi, decltype(ctrl)::value, decltype(row_mask)::value,
                                                                0xF, false);
    v += __longlong_as_double((long long)(((uint64_t)phi << 32) | plo));
  };
  step(std::integral_constant<int, 0xB1>{}, std::integral_constant<int, 0xF>{});   // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{}, std::integral_constant<int, 0xF>{});   // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{}, std::integral_constant<int, 0xF>{});  // row_half_mirror
  step(std::integral_constant<int, 0x140>{}, std::integral_constant<int, 0xF>{});  // row_mirror
  step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});  // row_bcast:15 into rows 1, 3
  step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});  // row_bcast:31 into rows 2, 3
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Block (e, s): expert e, K-slice s of S; the four waves split the slice,
// each lane accumulates in fp64 for up to 4 tokens at a time, and the wave
// sums are added in a fixed order into part[t][e][s].  The consumer adds the
// S partials in order, then the bias, and rounds once to fp32.  A lane's
// W_r values (at most kRV float4) are loaded once, before any product, and
// each token's activations likewise.  Workgroups past E*S run the digit jobs
// beside the router work.
constexpr int kRV = 8;
__global__ __launch_bounds__(256) void k_router_part(const float* __restrict__ x, int T, int H,
                                                     const float* __restrict__ Wr, int E, int S,
                                                     double* __restrict__ part, DigJob j0, DigJob j1) {
  __shared__ double red[4][4];
  __shared__ uint32_t ys[256];
  const int nr = E * S;
  if ((int)blockIdx.x >= nr) {
    // the activations' digit planes for the expert kernels (independent of
    // the routing): the first dig_blocks(j0) workgroups take the first job,
    // the rest the second, so each makes one pass (two passes in one
    // workgroup were the launch's longest path on the shared-expert layer)
    const int b = blockIdx.x - nr, n0 = dig_blocks(j0), n1 = gridDim.x - nr - n0;
    if (b < n0) dig_rows(j0, ys, b, n0);
    else dig_rows(j1, ys, b - n0, n1);
    return;
  }
  const int e = blockIdx.x / S, sl = blockIdx.x % S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = H / S / 4;             // elements per wave, a multiple of 64
  const int k0 = sl * (H / S) + wave * ks;
  const float* w = Wr + (int64_t)e * H + k0;
  const int nv = ks / 256;              // float4 per lane when ks is a multiple of 256
  const bool vec = (ks % 256) == 0 && nv <= kRV;
  float4 wv[kRV];
  if (vec) {
#pragma unroll
    for (int u = 0; u < kRV; ++u)
      if (u < nv) wv[u] = reinterpret_cast<const float4*>(w)[lane + 64 * u];
  }
  for (int t0 = 0; t0 < T; t0 += 4) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (vec) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (t0 + b < T) {
          const float4* xp = reinterpret_cast<const float4*>(x + (int64_t)(t0 + b) * H + k0);
          float4 xv[kRV];
#pragma unroll
          for (int u = 0; u < kRV; ++u)
            if (u < nv) xv[u] = xp[lane + 64 * u];
#pragma unroll
          for (int u = 0; u < kRV; ++u) {
            if (u < nv) {
              acc[b] = fma((double)wv[u].x, (double)xv[u].x, acc[b]);
              acc[b] = fma((double)wv[u].y, (double)xv[u].y, acc[b]);
              acc[b] = fma((double)wv[u].z, (double)xv[u].z, acc[b]);
              acc[b] = fma((double)wv[u].w, (double)xv[u].w, acc[b]);
            }
          }
        }
      }
    } else {
      for (int j = lane; j < ks; j += 64) {
        const double wd = (double)w[j];
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (t0 + b < T) acc[b] = fma(wd, (double)x[(int64_t)(t0 + b) * H + k0 + j], acc[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (t0 + b < T) {
        const double v = wave_sum_f64_dpp(acc[b]);
        if (lane == 0) red[wave][b] = v;
      }
    }
    __syncthreads();
    if (threadIdx.x < 4 && t0 + (int)threadIdx.x < T) {
      const int b = threadIdx.x;
      part[((int64_t)(t0 + b) * E + e) * S + sl] = ((red[0][b] + red[1][b]) + red[2][b]) + red[3][b];
    }
    __syncthreads();
  }
}

#ifndef MD_ROUTER_BLOCKS
#define MD_ROUTER_BLOCKS 128
#endif
// K-slices per expert: the fewest that give at least MD_ROUTER_BLOCKS blocks
// (128-expert layer: one slice instead of two, so each gate/up workgroup's
// top-k reads half the partials: router 3.58 -> 3.44 us, gate/up 8.75 -> 8.62)
int router_splits(int H, int E) {
  const int units = H / 256;  // K-slices stay multiples of 256
  int S = 1;
  for (int c = 1; c <= 8; ++c)
    if (units % c == 0) { S = c; if (E * c >= MD_ROUTER_BLOCKS) break; }
  return S;
}

hipError_t launch_router_part(const float* x, int T, int H, const float* Wr, int E, int S, double* part,
                              const DigJob& j0, const DigJob& j1, hipStream_t st) {
  const int nd = dig_blocks(j0) + dig_blocks(j1);
  hipLaunchKernelGGL(k_router_part, dim3(E * S + nd), dim3(256), 0, st, x, T, H, Wr, E, S, part, j0, j1);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gate/up

struct GateUpT1 {
  const uint8_t* gq;
  const uint8_t* uq;
  const float* gs;
  const float* us;
  int64_t mat_bytes;
  int F, H, act, E, k;
  const double* part;    // router partials [T][E][S]; nullptr: dense mode (expert 0, one slot per token)
  const float* bias;     // router bias [E] or nullptr
  int S;
  const u32x4* xd;       // x digit planes [T][H/NV][NPL]
  const float* xsc;      // x digit scales [T][H/NV]
  u32x4* hd;             // h digit planes [T*slots][F/NV][NPL]
  float* hsc;            // h digit scales [T*slots][F/NV]
  int* idx_out;          // [T][k], written by the blocks with blockIdx.x == 0 and slot 0
  float* gates_out;
  int KS, RGW;           // K-slices per row, row-group waves per block
  const int* idx_in;     // [T][k] a given routing (part == nullptr): slot j of token t is expert idx_in[t][j]
};

// Block = KS * RGW waves.  Wave (rg, ks) streams kNP row pairs (gate row f
// and up row f) per lane group over K-slice ks.  With KS > 1 the slices meet
// in LDS.  blockIdx.y = t * slots + j: token t's slot j (each pair of a
// several-token call is an independent one-token problem).  The block's rows
// are whole digit groups of h, whose planes it writes for the down kernel.
// At least 6 waves per SIMD (<= 80 VGPRs): two 12-wave workgroups per CU
// (packed int2: 4 waves, <= 128 VGPRs, for its twelve activation planes).
template <int FMT, int L, int kNP, bool kLoop>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(FMT == I2_ROW ? 4 : 6))) void k_gateup_t1(
    GateUpT1 a) {
  using D = Dig<FMT>;
  constexpr int G = 64 / L;
  extern __shared__ float lds[];  // [npairs] h values, then [RGW][G][kNP][KS][2] slice sums
  __shared__ int s_sel[8];
  __shared__ uint32_t ys[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slots = (a.part || a.idx_in) ? a.k : 1;
  const int tok = blockIdx.y / slots, slot = blockIdx.y % slots;
  const int npairs = a.RGW * G * kNP;
  const int ngx = a.H / D::NV;

  // The token's activation planes do not depend on the expert: their loads
  // are in flight while wave 0 selects it (int4 layer 38.0 -> 36.2 us per
  // token).  Not for packed int2, whose twelve planes held across the top-k
  // made its step 1.5 us slower.
  constexpr bool kPre = FMT != I2_ROW;
  const int ngh = a.F / D::NV;
  GuTile u{nullptr, nullptr, nullptr, nullptr, a.F, a.H, a.act, a.KS, a.RGW, a.xd + (int64_t)tok * ngx * D::NPL,
           a.xsc + (int64_t)tok * ngx, a.hd + (int64_t)blockIdx.y * ngh * D::NPL, a.hsc + (int64_t)blockIdx.y * ngh};
  ActDig<FMT, 1> xa;
  if constexpr (kPre) gu_act<FMT, L>(u, xa);

  int e = a.idx_in ? a.idx_in[tok * a.k + slot] : 0;
  if (a.part) {
    if (wave == 0) {
      int sel[8];
      float gts[8];
      const bool first = blockIdx.x == 0 && slot == 0;
      wave_topk(a.part + (int64_t)tok * a.E * a.S, a.S, a.bias, a.E, a.k, lane, sel, gts, first, slot + 1);
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < a.k) {
            s_sel[j] = sel[j];
            if (first) { a.idx_out[tok * a.k + j] = sel[j]; a.gates_out[tok * a.k + j] = gts[j]; }
          }
        }
      }
    }
    __syncthreads();
    e = s_sel[slot];
  }

  u.Gm = a.gq + (int64_t)e * a.mat_bytes;
  u.Um = a.uq + (int64_t)e * a.mat_bytes;
  u.gs = Fmt<FMT>::ROW ? a.gs + (int64_t)e * a.F : nullptr;
  u.us = Fmt<FMT>::ROW ? a.us + (int64_t)e * a.F : nullptr;
  if constexpr (kLoop) {
    // more row tiles than resident workgroups: each loops over its tiles of
    // this slot, so the top-k runs once per workgroup
    const int ntiles = (a.F + npairs - 1) / npairs;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x)
      gu_tile<FMT, L, kNP>(u, tile * npairs, lds, ys, kPre ? &xa : nullptr);
  } else {
    gu_tile<FMT, L, kNP>(u, blockIdx.x * npairs, lds, ys, kPre ? &xa : nullptr);
  }
}

// ------------------------------------------------------------------ down

struct DownT1 {
  const uint8_t* dq;
  const float* ds;
  int64_t mat_bytes;
  int H, F, k;
  const int* idx;        // [T][k]; nullptr: dense mode (expert 0, gate 1, one slot)
  const float* gates;    // [T][k]
  const u32x4* hd;       // h digit planes [T*k][F/NV][NPL]
  const float* hsc;      // h digit scales [T*k][F/NV]
  const float* y_add;    // [T][H], nullable: added to the combined result
  float* y;              // [T][H]
};

// Block = k waves; wave j streams kNRW output rows of token t's slot j
// expert (t = blockIdx.y).
template <int FMT, int L, int CPL>
__global__ __launch_bounds__(512) void k_down_t1(DownT1 a) {
  using D = Dig<FMT>;
  constexpr int NRW = dn_nrw(FMT);
  __shared__ float red[8][NRW];
  // Packed int4: j is the wave's slot, taken as wave-uniform so the expert
  // index is one scalar load, and the pair's h planes (which do not depend on
  // the expert) are in flight while it returns (down 14.06 -> 13.60 us on the
  // int4 layer; the same for int8 and int2 was 0.4 and 0.1 us slower).
  constexpr bool kPre = FMT == I4_ROW;
  const int j = kPre ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int tok = blockIdx.y, p = tok * a.k + j;
  const int ngh = a.F / D::NV;
  const u32x4* hd = a.hd + (int64_t)p * ngh * D::NPL;
  const float* hsc = a.hsc + (int64_t)p * ngh;
  ActDig<FMT, CPL> ha;
  if constexpr (kPre) load_act<FMT, L, CPL>(ha, hd, hsc, (threadIdx.x & 63) % L);
  const int e = a.idx ? a.idx[p] : 0;
  dn_rows<FMT, L, CPL, NRW>(a.dq + (int64_t)e * a.mat_bytes, Fmt<FMT>::ROW ? a.ds + (int64_t)e * a.H : nullptr, a.H, a.F,
                            hd, hsc, blockIdx.x * NRW, red[j], kPre ? &ha : nullptr);
  __syncthreads();
  if (threadIdx.x < NRW) {
    const int i = blockIdx.x * NRW + threadIdx.x;
    if (i < a.H) {
      float v = 0.f;
      if (a.idx) {
        for (int q = 0; q < a.k; ++q) v = fmaf(a.gates[tok * a.k + q], red[q][threadIdx.x], v);
      } else {
        v = red[0][threadIdx.x];
      }
      if (a.y_add) v += a.y_add[(int64_t)tok * a.H + i];
      a.y[(int64_t)tok * a.H + i] = v;
    }
  }
}

// ------------------------------------------------------------------ routed + shared

// A layer with a shared expert: the shared expert's gate/up tiles run in the
// routed gate/up launch (its own format and geometry, same workgroup size),
// and its down rows in the routed down launch as one more wave per workgroup,
// added after the gated routed rows -- the same order and arithmetic as the
// separate launches, in two launches fewer.  These layers are small (a few
// waves per SIMD), so every wave issues all its row loads up front: one
// memory round trip instead of a chain of them.
struct SharedGU {
  const uint8_t* gq;
  const uint8_t* uq;
  const float* gs;       // row scales (per-row formats) or nullptr
  const float* us;
  int F, act, KS, RGW, ntiles;
  const u32x4* xd;       // x digit planes in the shared expert's format [T][H/NV][NPL]
  const float* xsc;
  u32x4* hd;             // its h digit planes [T][F/NV][NPL]
  float* hsc;
};

// Blocks [0, T*k*rtiles): routed pair bid / rtiles, row tile bid % rtiles;
// then T*ntiles shared blocks (token, row tile).
#ifndef MD_RS_NP
#define MD_RS_NP 4
#endif
constexpr int kRsNP = MD_RS_NP;                 // row pairs per lane group
constexpr int kRsThreads = 256 * (8 / kRsNP);   // the same rows per workgroup

template <int FMT, int L, int kNP, int SFMT, int SL, int SNP>
__global__ __launch_bounds__(kRsThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_gateup_rs(GateUpT1 a,
                                                                                             SharedGU sh,
                                                                                             int rtiles, int T) {
  extern __shared__ float lds[];
  __shared__ int s_sel[8];
  __shared__ uint32_t ys[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrb = T * a.k * rtiles;
  const int bid = blockIdx.x;
  if (bid < nrb) {
    using D = Dig<FMT>;
    constexpr int G = 64 / L;
    const int pair = bid / rtiles, tile = bid % rtiles, tok = pair / a.k, slot = pair % a.k;
    if (wave == 0) {
      int sel[8];
      float gts[8];
      const bool first = tile == 0 && slot == 0;
      wave_topk(a.part + (int64_t)tok * a.E * a.S, a.S, a.bias, a.E, a.k, lane, sel, gts, first, slot + 1);
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < a.k) {
            s_sel[j] = sel[j];
            if (first) { a.idx_out[tok * a.k + j] = sel[j]; a.gates_out[tok * a.k + j] = gts[j]; }
          }
        }
      }
    }
    __syncthreads();
    const int e = s_sel[slot];
    const int ngx = a.H / D::NV, ngh = a.F / D::NV;
    const GuTile u{a.gq + (int64_t)e * a.mat_bytes, a.uq + (int64_t)e * a.mat_bytes,
                   Fmt<FMT>::ROW ? a.gs + (int64_t)e * a.F : nullptr, Fmt<FMT>::ROW ? a.us + (int64_t)e * a.F : nullptr,
                   a.F, a.H, a.act, a.KS, a.RGW, a.xd + (int64_t)tok * ngx * D::NPL, a.xsc + (int64_t)tok * ngx,
                   a.hd + (int64_t)pair * ngh * D::NPL, a.hsc + (int64_t)pair * ngh};
    gu_tile<FMT, L, kNP, false, kNP>(u, tile * (a.RGW * G * kNP), lds, ys);
  } else {
    using D = Dig<SFMT>;
    constexpr int G = 64 / SL;
    const int r = bid - nrb, tok = r / sh.ntiles, tile = r % sh.ntiles;
    const int ngx = a.H / D::NV, ngh = sh.F / D::NV;
    const GuTile u{sh.gq, sh.uq, sh.gs, sh.us, sh.F, a.H, sh.act, sh.KS, sh.RGW,
                   sh.xd + (int64_t)tok * ngx * D::NPL, sh.xsc + (int64_t)tok * ngx,
                   sh.hd + (int64_t)tok * ngh * D::NPL, sh.hsc + (int64_t)tok * ngh};
    gu_tile<SFMT, SL, SNP, false, SNP>(u, tile * (sh.RGW * G * SNP), lds, ys);
  }
}

struct SharedDN {
  const uint8_t* dq;
  const float* ds;       // row scales (per-row formats) or nullptr
  int F;
  const u32x4* hd;       // h digit planes [T][F/NV][NPL]
  const float* hsc;
};

#ifndef MD_RS_SDW
#define MD_RS_SDW 4
#endif
constexpr int kSDW = MD_RS_SDW;   // waves that share the shared expert's down rows

// Block = k + kSDW waves: wave j < k streams kNRW rows of token t's slot j
// expert, waves k.. the same rows of the shared expert, kNRW / kSDW rows each
// (t = blockIdx.y).
template <int FMT, int L, int CPL, int SFMT, int SL, int SCPL>
__global__ __launch_bounds__(64 * (8 + kSDW)) void k_down_rs(DownT1 a, SharedDN sh) {
  static_assert(kNRW % kSDW == 0, "shared down rows per wave");
  __shared__ float red[9][kNRW];
  const int j = threadIdx.x >> 6;
  const int tok = blockIdx.y;
  if (j < a.k) {
    using D = Dig<FMT>;
    const int p = tok * a.k + j, e = a.idx[p];
    const int ngh = a.F / D::NV;
    dn_rows<FMT, L, CPL, kNRW>(a.dq + (int64_t)e * a.mat_bytes, Fmt<FMT>::ROW ? a.ds + (int64_t)e * a.H : nullptr,
                               a.H, a.F, a.hd + (int64_t)p * ngh * D::NPL, a.hsc + (int64_t)p * ngh,
                               blockIdx.x * kNRW, red[j]);
  } else {
    using D = Dig<SFMT>;
    const int ngh = sh.F / D::NV;
    constexpr int NR = kNRW / kSDW;
    const int q = j - a.k;
    dn_rows<SFMT, SL, SCPL, NR>(sh.dq, sh.ds, a.H, sh.F, sh.hd + (int64_t)tok * ngh * D::NPL,
                                sh.hsc + (int64_t)tok * ngh, blockIdx.x * kNRW + q * NR, red[a.k] + q * NR);
  }
  __syncthreads();
  if (threadIdx.x < kNRW) {
    const int i = blockIdx.x * kNRW + threadIdx.x;
    if (i < a.H) {
      float v = 0.f;
      for (int q = 0; q < a.k; ++q) v = fmaf(a.gates[tok * a.k + q], red[q][threadIdx.x], v);
      v += red[a.k][threadIdx.x];
      if (a.y_add) v += a.y_add[(int64_t)tok * a.H + i];  // the residual (may be y itself)
      a.y[(int64_t)tok * a.H + i] = v;
    }
  }
}

// ------------------------------------------------------------------ launch

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

static int pow2_div(int n) {
  int L = 64;
  while (L > 1 && n % L) L >>= 1;
  return L;
}

// Gate/up geometry: lane groups of L lanes over KS K-slices, RGW row-group
// waves per slice, NP row pairs per lane group; the block's G*RGW*NP rows
// form whole digit groups of h (a multiple of NV, at most 256).
struct GuGeom {
  int L, G, KS, RGW, NP;
};

static bool gu_geom(int fmt, int F, int H, int slots, GuGeom& q) {
  const int nc = nchunks(fmt, H);
  q.L = pow2_div(nc);
  if (q.L < 8) return false;
  q.G = 64 / q.L;
  q.KS = nc / q.L;
  q.RGW = q.KS >= 4 ? 1 : 4 / q.KS;
  // row pairs per lane group: as many as keep >= 2048 waves in flight
  q.NP = MD_GU_MAXNP;
  while (q.NP > 2 && (int64_t)((F + q.RGW * q.G * q.NP - 1) / (q.RGW * q.G * q.NP)) * slots * q.KS * q.RGW < 2048)
    q.NP /= 2;
  const int NV = dig_nv(fmt);
  while ((q.RGW * q.G * q.NP) % NV) {
    if (q.NP < MD_GU_MAXNP) q.NP *= 2;
    else q.RGW *= 2;
  }
  return q.KS * q.RGW <= 16 && q.RGW * q.G * q.NP <= 256;
}

bool t1_supported(int fmt, int H, int F) {
  GuGeom q;
  if (!gu_geom(fmt, F, H, 1, q) || !gu_geom(fmt, F, H, 64, q)) return false;
  const int ncd = nchunks(fmt, F);
  const int Ld = pow2_div(ncd);
  if (Ld < 8) return false;
  const int cpl = ncd / Ld;
  return cpl == 1 || cpl == 2 || cpl == 3;
}

hipError_t launch_gateup_t1(int fmt, const uint8_t* gq, const uint8_t* uq, const float* gs, const float* us,
                            int64_t mat_bytes, int F, int H, int act, int E, int k, int T, const double* part, int S,
                            const float* bias, const void* xd, const float* xsc, void* hd, float* hsc, int* idx_out,
                            float* gates_out, hipStream_t st, const int* idx_in) {
  if (part && idx_in) return hipErrorInvalidValue;
  const int slots = ((part || idx_in) ? k : 1) * T;
  GuGeom q;
  if (!gu_geom(fmt, F, H, slots, q)) return hipErrorInvalidConfiguration;
  GateUpT1 a{gq, uq, gs, us, mat_bytes, F, H, act, E, k, part, bias, S, static_cast<const u32x4*>(xd), xsc,
             static_cast<u32x4*>(hd), hsc, idx_out, gates_out, q.KS, q.RGW, idx_in};
  const int L = q.L, NP = q.NP;
  const int pairs_per_block = q.RGW * q.G * NP;
  // row tiles per slot; the grid holds at most what is resident at once, and
  // each workgroup loops over its tiles (the top-k runs once per workgroup)
  const int ntiles = (F + pairs_per_block - 1) / pairs_per_block;
  const dim3 block(64 * q.KS * q.RGW);
  const size_t lds = sizeof(float) * (pairs_per_block + (q.KS > 1 ? 2 * q.KS * pairs_per_block : 0));
#define MD_GU(F_, L_, N_) \
  if (fmt == F_ && L == L_ && NP == N_) { \
    static int occ = 0; \
    if (!occ && (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gateup_t1<F_, L_, N_, true>, block.x, lds) != \
                 hipSuccess || occ < 1)) occ = 1; \
    const int per_slot = (int)(((int64_t)device_cus() * occ + slots - 1) / slots); \
    if (ntiles <= per_slot) { \
      hipLaunchKernelGGL((k_gateup_t1<F_, L_, N_, false>), dim3(ntiles, slots), block, lds, st, a); \
    } else { \
      hipLaunchKernelGGL((k_gateup_t1<F_, L_, N_, true>), dim3(per_slot < 1 ? 1 : per_slot, slots), block, lds, st, a); \
    } \
    return hipGetLastError(); }
#define MD_GUL(F_) MD_GU(F_, 64, 8) MD_GU(F_, 32, 8) MD_GU(F_, 16, 8) MD_GU(F_, 8, 8) \
                   MD_GU(F_, 64, 4) MD_GU(F_, 32, 4) MD_GU(F_, 16, 4) MD_GU(F_, 8, 4) \
                   MD_GU(F_, 64, 2) MD_GU(F_, 32, 2) MD_GU(F_, 16, 2) MD_GU(F_, 8, 2)
  MD_GUL(Q8_0) MD_GUL(Q4_0) MD_GUL(I8_ROW) MD_GUL(I4_ROW) MD_GUL(I2_ROW) MD_GUL(Q4_1)
#undef MD_GUL
#undef MD_GU
  return hipErrorInvalidConfiguration;
}

hipError_t launch_down_t1(int fmt, const uint8_t* dq, const float* ds, int64_t mat_bytes, int H, int F, int k, int T,
                          const int* idx, const float* gates, const void* hd, const float* hsc, const float* y_add,
                          float* y, hipStream_t st) {
  const int nc = nchunks(fmt, F);
  const int L = pow2_div(nc), CPL = nc / L;
  DownT1 a{dq, ds, mat_bytes, H, F, idx ? k : 1, idx, gates, static_cast<const u32x4*>(hd), hsc, y_add, y};
  const int nrw = dn_nrw(fmt);
  const dim3 grid((H + nrw - 1) / nrw, T), block(64 * a.k);
#define MD_DN(F_, L_, C_) \
  if (fmt == F_ && L == L_ && CPL == C_) { \
    hipLaunchKernelGGL((k_down_t1<F_, L_, C_>), grid, block, 0, st, a); return hipGetLastError(); }
#define MD_DNL(F_, L_) MD_DN(F_, L_, 1) MD_DN(F_, L_, 2) MD_DN(F_, L_, 3)
#define MD_DNF(F_) MD_DNL(F_, 64) MD_DNL(F_, 32) MD_DNL(F_, 16) MD_DNL(F_, 8)
  MD_DNF(Q8_0) MD_DNF(Q4_0) MD_DNF(I8_ROW) MD_DNF(I4_ROW) MD_DNF(I2_ROW) MD_DNF(Q4_1)
#undef MD_DNF
#undef MD_DNL
#undef MD_DN
  return hipErrorInvalidConfiguration;
}

// ---- routed + shared

// The instantiated shape family: Q4_0 experts (hidden 2048: 64-lane row
// groups, 8 row pairs; FFN 768: 8-lane groups, 3 chunks per lane) with a Q8_0
// shared expert (64-lane groups, 8 row pairs; FFN 2048: 64 lanes, 2 chunks).
struct RsGeom {
  GuGeom r, s;
  int Ld, CPLd, Lsd, CPLsd;
};
static bool rs_geom(int fmt, int H, int F, int sfmt, int Fs, int k, int T, RsGeom& g) {
  if (k > 8) return false;
  if (!gu_geom(fmt, F, H, T * k, g.r) || !gu_geom(sfmt, Fs, H, T, g.s)) return false;
  // the same rows per workgroup on more waves, fewer row pairs each
  for (GuGeom* q : {&g.r, &g.s})
    if (q->NP == 8 && kRsNP < 8) { q->RGW *= 8 / kRsNP; q->NP = kRsNP; }
  if (g.r.KS * g.r.RGW != g.s.KS * g.s.RGW) return false;   // one workgroup size
  if (64 * g.r.KS * g.r.RGW > kRsThreads) return false;     // the kernel's bound
  const int ncd = nchunks(fmt, F), ncs = nchunks(sfmt, Fs);
  g.Ld = pow2_div(ncd);
  g.Lsd = pow2_div(ncs);
  g.CPLd = ncd / g.Ld;
  g.CPLsd = ncs / g.Lsd;
  return fmt == Q4_0 && sfmt == Q8_0 && g.r.L == 64 && g.r.NP == kRsNP && g.s.L == 64 && g.s.NP == kRsNP && g.Ld == 8 &&
         g.CPLd == 3 && g.Lsd == 64 && g.CPLsd == 2;
}

bool rs_supported(int fmt, int H, int F, int sfmt, int Fs, int k, int T) {
  RsGeom g;
  return rs_geom(fmt, H, F, sfmt, Fs, k, T, g);
}

hipError_t launch_moe_rs(const RsLaunch& L, hipStream_t st) {
  RsGeom g;
  if (!rs_geom(L.fmt, L.H, L.F, L.sfmt, L.Fs, L.k, L.T, g)) return hipErrorInvalidConfiguration;
  const int rpb = g.r.RGW * g.r.G * g.r.NP, spb = g.s.RGW * g.s.G * g.s.NP;
  const int rtiles = (L.F + rpb - 1) / rpb, stiles = (L.Fs + spb - 1) / spb;
  GateUpT1 a{L.gq, L.uq, L.gs, L.us, L.gu_bytes, L.F, L.H, L.act, L.E, L.k, L.part, L.bias, L.S,
             static_cast<const u32x4*>(L.xd), L.xsc, static_cast<u32x4*>(L.hd), L.hsc, L.idx, L.gates, g.r.KS, g.r.RGW};
  SharedGU sh{L.sgq, L.suq, L.sgs, L.sus, L.Fs, L.sact, g.s.KS, g.s.RGW, stiles,
              static_cast<const u32x4*>(L.sxd), L.sxsc, static_cast<u32x4*>(L.shd), L.shsc};
  const int mx = rpb > spb ? rpb : spb;
  const int ks = g.r.KS > g.s.KS ? g.r.KS : g.s.KS;
  const size_t lds = sizeof(float) * (mx + (ks > 1 ? 2 * ks * mx : 0));
  const int nblk = L.T * L.k * rtiles + L.T * stiles;
  if (L.parts & 1) {
    hipLaunchKernelGGL((k_gateup_rs<Q4_0, 64, kRsNP, Q8_0, 64, kRsNP>), dim3(nblk), dim3(64 * g.r.KS * g.r.RGW), lds, st, a,
                       sh, rtiles, L.T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (L.parts & 2) {
    DownT1 d{L.dq, L.ds, L.dn_bytes, L.H, L.F, L.k, L.idx, L.gates, static_cast<const u32x4*>(L.hd), L.hsc,
             L.residual, L.y};
    SharedDN sd{L.sdq, L.sds, L.Fs, static_cast<const u32x4*>(L.shd), L.shsc};
    hipLaunchKernelGGL((k_down_rs<Q4_0, 8, 3, Q8_0, 64, 2>), dim3((L.H + kNRW - 1) / kNRW, L.T), dim3(64 * (L.k + kSDW)),
                       0, st, d, sd);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace md
