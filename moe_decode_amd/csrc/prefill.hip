// prefill.hip -- grouped GEMM of a token chunk through its experts on the
// bf16 matrix cores (gfx950 v_mfma_f32_16x16x32_bf16).
//
// Every expert's weight rows are read from HBM once per call and reused for
// all the tokens routed to it (the TurboFieldfare summary, "memory and expert
// streaming": prefill in chunks of at most 128 tokens reusing each loaded
// expert across the prompt rows).
//
// A block owns 64 weight rows of one active expert (gate/up stage: gate rows
// f0..f0+31 and up rows f0..f0+31, so the activation fuses in the epilogue;
// down stage: 64 output rows) and one tile of 16 of the expert's tokens (the
// work item blockIdx.y of the routing hand-off); an expert with more tokens
// has its rows streamed once per tile, the repeats (adjacent work items)
// served mostly from the on-chip caches.  K runs in tiles of
// 256 weights: the next two tiles' weights, scales and activations are loaded
// with coalesced 16-byte loads into registers while the current tile,
// double-buffered in LDS, feeds the matrix cores.
//
// Exactness: every weight code is an integer of at most 8 significant bits
// (4-bit codes are taken as 16 * value, see common.hpp), so its bf16 image is
// exact; activations enter as a bf16 pair hi + lo with hi = bf16(x) and
// lo = bf16(x - hi) (16 significant bits); the MFMA accumulates in fp32.
// A 32-wide MFMA step covers exactly one Q8_0/Q4_0/Q4_1 block, so the block
// scale is applied to the step's partial sums before they join the
// accumulator (Q4_1 adds its minimum times the block's activation sum, which
// one more MFMA per step forms for all rows at once); per-row scales are
// applied once at the end.
#include "common.hpp"
#include "kernels.hpp"

namespace md {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int kRows = 64;         // weight rows per block
constexpr int kKT = 256;          // K tile (8 MFMA steps of 32)
constexpr int kTok = kTokTile;    // tokens per MFMA tile
constexpr int kAST = kKT + 8;     // LDS row stride of an activation tile (16-byte pad: the 16
                                  // token rows of one operand read land in distinct banks)

// -------------------------------------------------------- activations -> bf16 pair

__global__ __launch_bounds__(256) void k_split_bf16(const float* __restrict__ x, int64_t n, u16* __restrict__ hi,
                                                    u16* __restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  const __bf16 h = (__bf16)v;
  const __bf16 l = (__bf16)(v - (float)h);
  hi[i] = __builtin_bit_cast(u16, h);
  lo[i] = __builtin_bit_cast(u16, l);
}

hipError_t launch_split_bf16(const float* x, int64_t n, u16* hi, u16* lo, hipStream_t st) {
  hipLaunchKernelGGL(k_split_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n, hi, lo);
  return hipGetLastError();
}

// -------------------------------------------------------- grouped GEMM

template <int FMT>
struct Tile {
  static constexpr bool B8 = (FMT == Q8_0 || FMT == I8_ROW);
  static constexpr int WB = B8 ? kKT : FMT == I2_ROW ? kKT / 4 : kKT / 2;  // weight bytes per row per K tile
  static constexpr int WSTR = WB + 16;                 // LDS row stride (bank spread)
  static constexpr int WCH = kRows * WB / 16;          // 16-byte weight chunks per tile
  static constexpr int WPT = WCH / 256;                // chunks per thread (2 or 4)
  static constexpr bool BLK = (FMT == Q8_0 || FMT == Q4_0 || FMT == Q4_1);
  static constexpr int SCW = FMT == Q4_1 ? 16 : 8;    // fp16 words of block constants per row per K tile
};

struct MfmaArgs {
  const uint8_t* wq;     // gate (gate/up stage) or down weights, expert-major
  const uint8_t* wq2;    // up weights (gate/up stage)
  const float* ws;       // per-row scales of wq (per-row formats)
  const float* ws2;
  int64_t mat_bytes;     // bytes per expert matrix
  int M, K;              // rows per matrix (F or H), columns
  int act;
  Disp d;
  const u16* a_hi;       // activation pairs, rows of K
  const u16* a_lo;       // nullptr: activations exactly bf16 (no low half)
  int act_by_token;      // activation row = token of the position (x) or the position (h)
  float* out;            // h [pos][F] or o [pos][H]
  u16* out_hi;           // h as a bf16 pair for the next stage (gate/up stage)
  u16* out_lo;
  int ks;                // dense mode: K splits (blockIdx.z); partial sums go to out + z*T*M
};

template <int FMT>
MD_DEV bf16x8 decode_a(const uint8_t* p) {
  bf16x8 a;
  if constexpr (Tile<FMT>::B8) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const unsigned w[2] = {u.x, u.y};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < 4; ++b) a[4 * h + b] = (__bf16)(float)(signed char)(w[h] >> (8 * b));
  } else if constexpr (FMT == Q4_1) {
    // the Q4_0 order, unsigned codes: each masked byte is 16 * n
    const unsigned v = *reinterpret_cast<const unsigned*>(p);
    const unsigned lo = opaque((v << 4) & 0xF0F0F0F0u), hi = opaque(v & 0xF0F0F0F0u);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      a[b] = (__bf16)(float)(unsigned char)(lo >> (8 * b));
      a[4 + b] = (__bf16)(float)(unsigned char)(hi >> (8 * b));
    }
  } else if constexpr (FMT == Q4_0) {
    // bytes b: low nibble = step weight 4q+b, high = 16+4q+b; elements [lo0..3, hi0..3]
    const unsigned v = *reinterpret_cast<const unsigned*>(p) ^ 0x88888888u;
    const unsigned lo = opaque((v << 4) & 0xF0F0F0F0u), hi = opaque(v & 0xF0F0F0F0u);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      a[b] = (__bf16)(float)(signed char)(lo >> (8 * b));
      a[4 + b] = (__bf16)(float)(signed char)(hi >> (8 * b));
    }
  } else {  // I4_ROW: byte b holds step weights 8q+2b (low) and 8q+2b+1 (high)
    const unsigned u = *reinterpret_cast<const unsigned*>(p);
    const unsigned lo = opaque((u << 4) & 0xF0F0F0F0u), hi = opaque(u & 0xF0F0F0F0u);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      a[2 * b] = (__bf16)(float)(signed char)(lo >> (8 * b));
      a[2 * b + 1] = (__bf16)(float)(signed char)(hi >> (8 * b));
    }
  }
  return a;
}

// Activation operand: the 8 values of token j that pair with decode_a's
// elements for lane group q in step s.
template <int FMT>
MD_DEV bf16x8 load_b(const u16* tile, int j, int s, int q) {
  // (4-bit blocks: the tile was staged with x[4q..4q+3] and x[16+4q..16+4q+3]
  // of every block side by side, so one 16-byte read serves all formats)
  const uint4 v = *reinterpret_cast<const uint4*>(tile + j * kAST + 32 * s + 8 * q);
  return __builtin_bit_cast(bf16x8, v);
}

#ifndef MD_BF_WAVES
#define MD_BF_WAVES 2
#endif
// RT: 16-row MFMA tiles per wave; each activation fragment read from LDS
// feeds RT products (64*RT rows per block; gate/up: 32*RT gate + 32*RT up).
// LO: the activations carry a low bf16 half (a_lo != nullptr).
template <int FMT, int GU, int RT, bool LO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MD_BF_WAVES))) void k_moe_mfma(MfmaArgs a) {
  using TL = Tile<FMT>;
  constexpr int BR = 64 * RT;
  constexpr int WCH = BR * TL::WB / 16, WPT = WCH / 256;
  // gate/up: a thread's pieces i < WPT/2 lie in the gate rows, the rest in the up rows
  static_assert(!GU || WPT % 2 == 0, "gate and up rows split the pieces evenly");
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][BR * TL::WSTR];
  __shared__ __attribute__((aligned(16))) uint16_t s_sc[2][BR * TL::SCW];
  __shared__ __attribute__((aligned(16))) u16 s_hi[2][kTok * kAST];
  __shared__ __attribute__((aligned(16))) u16 s_lo[2][kTok * kAST];
  __shared__ float s_up[BR / 2][kTok];

  struct { int e, p0, p1; } er;
  if (a.d.n_active == nullptr) {  // dense FFN: one expert, positions = tokens
    if (blockIdx.y != 0) return;
    er.e = 0; er.p0 = 0; er.p1 = a.d.T;
  } else {  // work item blockIdx.y: one 16-position tile of an active expert
    const int4 it = a.d.items[blockIdx.y];
    if (it.x < 0) return;
    er.e = it.x; er.p0 = it.y; er.p1 = it.z;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, li = lane & 15;
  const int64_t rb = row_bytes(FMT, a.K);
  int kt_begin = 0, kt_end = a.K / kKT;
  int ksplit = 0;
  if (a.d.n_active == nullptr && a.ks > 1) {  // dense mode, K split over blockIdx.z
    ksplit = (int)blockIdx.z;
    const int n = kt_end;
    kt_begin = (int)((int64_t)ksplit * n / a.ks);
    kt_end = (int)((int64_t)(ksplit + 1) * n / a.ks);
  }
  const int nkt = kt_end - kt_begin;
  // block rows: gate/up stage -> BR/2 gate + BR/2 up rows of f0..
  const int r0 = GU ? blockIdx.x * (BR / 2) : blockIdx.x * BR;

  auto pos_token = [&](int pos) { return a.d.n_active == nullptr ? pos : a.d.pairs[pos] / a.d.k; };

  {
    const int t0 = er.p0 + (ksplit ? 0 : (int)blockIdx.z) * kTok;  // this block's 16-token tile
    if (t0 >= er.p1) return;
    const int nt = min(kTok, er.p1 - t0);
    // this thread's activation rows for staging: token slot jj = tid / 16, piece pp = tid % 16
    const int jj = tid >> 4, pp = tid & 15;
    constexpr bool has_lo = LO;
    // Tiles are read through buffer resources: an offset past a resource's
    // end reads zeros without a memory access, so the lanes with nothing to
    // load (empty token slots, lanes past the scale rows) and the tiles past
    // the last one issue the same loads as the others.  With no branch around
    // a load, the compiled loop waits only for the older of the two tiles in
    // flight (where the paths of a conditional load meet it waits for all).
    const uint8_t* wg = a.wq + (int64_t)er.e * a.mat_bytes;
    const uint8_t* wu = GU ? a.wq2 + (int64_t)er.e * a.mat_bytes : wg;
    const int mat_len = (int)((int64_t)a.M * rb);
    const rsrc_t res_g = make_res(wg, mat_len), res_u = make_res(wu, mat_len);
    const int a_rows = a.act_by_token ? a.d.T : a.d.T * a.d.k;
    const int a_len = (int)((int64_t)a_rows * a.K * 2);
    const rsrc_t res_ah = make_res(a.a_hi, a_len), res_al = make_res(has_lo ? a.a_lo : a.a_hi, a_len);
    uint32_t woff[WPT];  // this thread's weight pieces, tile 0 of the matrix
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + 256 * i, r = c / (TL::WB / 16), piece = c % (TL::WB / 16);
      const int f = min(r0 + (GU ? r % (BR / 2) : r), a.M - 1);
      woff[i] = (uint32_t)((int64_t)f * rb) + 16u * piece;
    }
    // block scales, BR rows x SCW fp16 words per tile, spread over all 256
    // threads: SPT bytes each, TPR threads per row (gate/up: the gate rows'
    // scales fall to threads 0..127, waves 0 and 1)
    constexpr int SPT = BR * TL::SCW * 2 / 256, TPR = TL::SCW * 2 / SPT;
    static_assert(!TL::BLK || ((SPT == 4 || SPT == 8) && TPR * BR == 256), "scale pieces");
    const int sc_row = tid / TPR, sc_part = tid % TPR;
    const bool up_wave = GU && __builtin_amdgcn_readfirstlane(tid) >= 128;
    const rsrc_t res_s = up_wave ? res_u : res_g;
    const uint32_t soff = (uint32_t)((int64_t)min(r0 + (GU ? sc_row % (BR / 2) : sc_row), a.M - 1) * rb) +
                          (uint32_t)(FMT == Q8_0 ? a.K : (a.K / 32) * 16) + (uint32_t)(SPT * sc_part);
    uint32_t aoff = 0;  // this thread's activation piece (token slot jj)
    if (jj < nt) {
      const int row = a.act_by_token ? pos_token(t0 + jj) : t0 + jj;
      aoff = (uint32_t)((int64_t)row * a.K * 2) + 32u * pp;
    }
    const bool a_lane = jj < nt;
    // two register sets: tile kt+1 waits in one while tile kt+2 is in flight
    u32x4 rw[2][WPT];
    uint32_t rs[2][2] = {};
    uint4 rh[2][2], rl[2][2];
    auto gload = [&](int ktl, int set) {
      const int kt = kt_begin + ktl;
      const bool tile = ktl < nkt;
#pragma unroll
      for (int i = 0; i < WPT; ++i)
        rw[set][i] = buf_load<kAuxStream>(GU && i >= WPT / 2 ? res_u : res_g,
                                          past(tile, woff[i] + (uint32_t)kt * TL::WB));
      if constexpr (TL::BLK) {
        const uint32_t o = past(tile, soff + (uint32_t)(2 * TL::SCW * kt));
        if constexpr (SPT == 8) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(res_s, o, 0, 0);
          rs[set][0] = v[0];
          rs[set][1] = v[1];
        } else {
          rs[set][0] = __builtin_amdgcn_raw_buffer_load_b32(res_s, o, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t o = past(tile && a_lane, aoff + (uint32_t)kt * (2 * kKT) + 16u * i);
        rh[set][i] = __builtin_bit_cast(uint4, buf_load(res_ah, o));
        rl[set][i] = has_lo ? __builtin_bit_cast(uint4, buf_load(res_al, o)) : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto lstore = [&](int buf, int set) {
#pragma unroll
      for (int i = 0; i < WPT; ++i) {
        const int c = tid + 256 * i, r = c / (TL::WB / 16), piece = c % (TL::WB / 16);
        *reinterpret_cast<u32x4*>(&s_w[buf][r * TL::WSTR + 16 * piece]) = rw[set][i];
      }
      if constexpr (TL::BLK) {
        if constexpr (FMT == Q4_1) {
          // (d, m) pairs step-major, [step][row][2]: a lane's four rows of a
          // step are one 16-byte read; this thread holds steps 2 sc_part, +1
#pragma unroll
          for (int j = 0; j < 2; ++j)
            *reinterpret_cast<uint32_t*>(&s_sc[buf][2 * ((2 * sc_part + j) * BR + sc_row)]) = rs[set][j];
        } else {
          // block scales step-major, [step][row]: the four consecutive rows
          // of a lane's MFMA outputs read their step's scales as one 8-byte
          // load; this thread holds SPT / 2 consecutive steps
#pragma unroll
          for (int j = 0; j < SPT / 2; ++j)
            s_sc[buf][((SPT / 2) * sc_part + j) * BR + sc_row] = (uint16_t)(rs[set][j >> 1] >> (16 * (j & 1)));
        }
      }
      if constexpr (FMT == Q4_0 || FMT == Q4_1) {
        // nibble order: x[4q..4q+3] and x[16+4q..16+4q+3] of a block side by side
        const int base = jj * kAST + 32 * (pp >> 1) + 4 * (pp & 1);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          *reinterpret_cast<uint2*>(&s_hi[buf][base + 16 * i]) = make_uint2(rh[set][i].x, rh[set][i].y);
          *reinterpret_cast<uint2*>(&s_hi[buf][base + 16 * i + 8]) = make_uint2(rh[set][i].z, rh[set][i].w);
          *reinterpret_cast<uint2*>(&s_lo[buf][base + 16 * i]) = make_uint2(rl[set][i].x, rl[set][i].y);
          *reinterpret_cast<uint2*>(&s_lo[buf][base + 16 * i + 8]) = make_uint2(rl[set][i].z, rl[set][i].w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          *reinterpret_cast<uint4*>(&s_hi[buf][jj * kAST + 16 * pp + 8 * i]) = rh[set][i];
          *reinterpret_cast<uint4*>(&s_lo[buf][jj * kAST + 16 * pp + 8 * i]) = rl[set][i];
        }
      }
    };

    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wr = wave * 16 * RT;  // this wave's first block row
    auto compute = [&](int buf) {
#pragma unroll
      for (int s = 0; s < kKT / 32; ++s) {
        const bf16x8 bh = load_b<FMT>(s_hi[buf], li, s, q);
        const bf16x8 bl = has_lo ? load_b<FMT>(s_lo[buf], li, s, q) : bf16x8{};
        // Q4_1: 16 times the block's sum of each token's activations (an
        // operand of 16.0 in every row), for the block minimum
        f32x4 zs = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FMT == Q4_1) {
          const bf16x8 sixteen = __builtin_bit_cast(bf16x8, u32x4{0x41804180u, 0x41804180u, 0x41804180u, 0x41804180u});
          zs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sixteen, bh, zs, 0, 0, 0);
          if (has_lo) zs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sixteen, bl, zs, 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const uint8_t* wp =
              &s_w[buf][(wr + 16 * rt + li) * TL::WSTR + (TL::B8 ? 32 * s + 8 * q : 16 * s + 4 * q)];
          const bf16x8 av = decode_a<FMT>(wp);
          if constexpr (TL::BLK) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, z, 0, 0, 0);
            if (has_lo) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, z, 0, 0, 0);
            if constexpr (FMT == Q4_1) {
              const u32x4 dm = *reinterpret_cast<const u32x4*>(&s_sc[buf][2 * (s * BR + wr + 16 * rt + 4 * q)]);
#pragma unroll
              for (int v = 0; v < 4; ++v)
                acc[rt][v] = fmaf(h2f((uint16_t)(dm[v] & 0xFFFFu)), z[v],
                                  fmaf(h2f((uint16_t)(dm[v] >> 16)), zs[v], acc[rt][v]));
            } else {
              const uint2 sc4 = *reinterpret_cast<const uint2*>(&s_sc[buf][s * BR + wr + 16 * rt + 4 * q]);
              const unsigned sw[2] = {sc4.x, sc4.y};
#pragma unroll
              for (int v = 0; v < 4; ++v)
                acc[rt][v] = fmaf(h2f((uint16_t)(sw[v >> 1] >> (16 * (v & 1)))), z[v], acc[rt][v]);
            }
          } else {
            acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, acc[rt], 0, 0, 0);
            if (has_lo) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, acc[rt], 0, 0, 0);
          }
        }
      }
    };
    // Loop top: LDS buffer 0 holds tile kt, register set 1 tile kt+1.  The
    // loop runs while tile kt+2 exists, so its LDS stores are unconditional
    // (a store skipped on some path would leave that path's loads pending
    // at the loop top, and the compiled loop would wait for them there); the
    // last one or two tiles are computed after it.
    gload(0, 0);
    gload(1, 1);
    lstore(0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 < nkt; kt += 2) {
      gload(kt + 2, 0);
      compute(0);
      lstore(1, 1);
      __syncthreads();
      gload(kt + 3, 1);
      compute(1);
      lstore(0, 0);
      __syncthreads();
    }
    compute(0);
    if (kt + 1 < nkt) {
      lstore(1, 1);
      __syncthreads();
      compute(1);
    }

    // 4-bit codes entered as 16 * value (Q4_1: its block sums as 16 * sum):
    // one exact power-of-two scaling of the sums instead of one per step
    if constexpr (FMT == Q4_0 || FMT == Q4_1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[rt][v] *= 0.0625f;
    }
    // epilogue: lane holds rows wr + 16 rt + 4q + v (v < 4) of token column li
    const int j = li;
    if constexpr (GU) {
      if (wave >= 2) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int v = 0; v < 4; ++v) s_up[wr - BR / 2 + 16 * rt + 4 * q + v][j] = acc[rt][v];
      }
      __syncthreads();
      if (wave < 2 && j < nt) {
        const int pos = t0 + j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rr = wr + 16 * rt + 4 * q + v, f = r0 + rr;
            if (f < a.M) {
              float av = acc[rt][v], uv = s_up[rr][j];
              if constexpr (Fmt<FMT>::ROW) {
                av *= a.ws[(int64_t)er.e * a.M + f] * row_post<FMT>();
                uv *= a.ws2[(int64_t)er.e * a.M + f] * row_post<FMT>();
              }
              const float hv = act_f(a.act, av) * uv;
              const int64_t o = (int64_t)pos * a.M + f;
              a.out[o] = hv;
              const __bf16 hh = (__bf16)hv;
              a.out_hi[o] = __builtin_bit_cast(u16, hh);
              a.out_lo[o] = __builtin_bit_cast(u16, (__bf16)(hv - (float)hh));
            }
          }
        }
      }
    } else {
      if (j < nt) {
        const int pos = t0 + j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int i = r0 + wr + 16 * rt + 4 * q + v;
            if (i < a.M) {
              float ov = acc[rt][v];
              if constexpr (Fmt<FMT>::ROW) ov *= a.ws[(int64_t)er.e * a.M + i] * row_post<FMT>();
              a.out[((int64_t)ksplit * a.d.T + pos) * a.M + i] = ov;
            }
          }
        }
      }
    }
  }
}

bool mfma_supported(int K) { return K % kKT == 0; }

// Dense GEMV of a small batch (T <= 16 tokens) on the matrix cores: rows in
// blocks of 64*RT, K split in ks ranges of whole tiles (partials [ks][T][M]).
int mfma_gemv_splits(int fmt, int M, int K) {
  const int RT = (fmt == Q4_0 || fmt == I4_ROW) ? 2 : 1;
  const int rb = (M + 64 * RT - 1) / (64 * RT), nkt = K / kKT;
  int ks = 1;
  while (rb * ks < 512 && nkt / (2 * ks) >= 2) ks *= 2;
  return ks;
}

hipError_t launch_mfma_gemv(int fmt, const uint8_t* wq, const float* ws, int M, int K, int T, const u16* a_hi,
                            const u16* a_lo, int ks, float* out, hipStream_t st) {
  if (T < 1 || T > kTok || ks < 1) return hipErrorInvalidValue;
  const Disp d{nullptr, nullptr, nullptr, nullptr, 1, T};
  MfmaArgs a{wq, nullptr, ws, nullptr, 0, M, K, 0, d, a_hi, a_lo, 0, out, nullptr, nullptr, ks};
  // (Q4_1: one row tile per wave; two would spill with its minimum terms)
  const int RT = (fmt == Q4_0 || fmt == I4_ROW) ? 2 : 1;
  const dim3 grid((M + 64 * RT - 1) / (64 * RT), 1, ks);
  if (fmt == Q8_0 && a_lo) hipLaunchKernelGGL((k_moe_mfma<Q8_0, 0, 1, true>), grid, dim3(256), 0, st, a);
  else if (fmt == Q8_0) hipLaunchKernelGGL((k_moe_mfma<Q8_0, 0, 1, false>), grid, dim3(256), 0, st, a);
  else if (fmt == Q4_0 && a_lo) hipLaunchKernelGGL((k_moe_mfma<Q4_0, 0, 2, true>), grid, dim3(256), 0, st, a);
  else if (fmt == Q4_0) hipLaunchKernelGGL((k_moe_mfma<Q4_0, 0, 2, false>), grid, dim3(256), 0, st, a);
  else if (fmt == Q4_1 && a_lo) hipLaunchKernelGGL((k_moe_mfma<Q4_1, 0, 1, true>), grid, dim3(256), 0, st, a);
  else if (fmt == Q4_1) hipLaunchKernelGGL((k_moe_mfma<Q4_1, 0, 1, false>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_moe_mfma(int fmt, bool gateup, const uint8_t* wq, const uint8_t* wq2, const float* ws,
                           const float* ws2, int64_t mat_bytes, int M, int K, int act, const Disp& d, int n_items,
                           const u16* a_hi, const u16* a_lo, bool act_by_token, float* out, u16* out_hi,
                           u16* out_lo, hipStream_t st) {
  MfmaArgs a{wq, wq2, ws, ws2, mat_bytes, M, K, act, d, a_hi, a_lo, act_by_token ? 1 : 0, out, out_hi, out_lo, 1};
  // 4-bit codes: two row tiles per wave (activation fragment reads per weight
  // byte halve); 8-bit codes: one (twice the weight bytes per tile)
  const int RT = (fmt == Q4_0 || fmt == I4_ROW) ? 2 : 1;
  const int rows_per_block = (gateup ? 32 : 64) * RT;
  // token tiles: an expert holds at most T tokens (one per token)
  const int tiles = d.items ? 1 : (d.T + kTok - 1) / kTok;
  const dim3 grid((M + rows_per_block - 1) / rows_per_block, d.items ? n_items : 1, tiles);
  // (the per-row formats take the int8 path below)
  if (!a_lo) return hipErrorInvalidValue;
#define MD_MF(F_, RT_) \
  if (fmt == F_ && RT == RT_) { \
    if (gateup) hipLaunchKernelGGL((k_moe_mfma<F_, 1, RT_, true>), grid, dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((k_moe_mfma<F_, 0, RT_, true>), grid, dim3(256), 0, st, a); \
    return hipGetLastError(); }
  MD_MF(Q8_0, 1) MD_MF(Q4_0, 2) MD_MF(Q4_1, 1)
#undef MD_MF
  return hipErrorInvalidValue;
}

// ================================================================ int8 path
//
// For the per-row-scale formats the codes feed v_mfma_i32_16x16x64_i8 as they
// are (int8 codes directly; 4-bit codes as the exact bytes 16 * value).  Each
// activation row a (a token's x or a position's h) is written as a 30-bit
// fixed-point integer X = rint(a * 2^(30 - E)), E the binary exponent that
// bounds max|a| (|X| < 2^30), split into four balanced int8 digits,
// X = d0 + 256 d1 + 65536 d2 + 2^24 d3 (d_i in [-128, 127]).  One MFMA per
// digit accumulates exact int32 sums; the epilogue forms
// (2^24 acc3 + 2^16 acc2 + 2^8 acc1 + acc0) * 2^(E - 30) in fp32.  The digits
// resolve |a| to 2^-31 of the row maximum, so the only rounding left is the
// fp32 combine.

constexpr int kLST = kKT + 16;    // LDS stride of a digit plane row (bank spread)

// Digit planes [R][4][K] (int8) and exponents [R].  perm 1 (packed int4):
// within every 8 columns the even columns come first (the order in which a
// packed-int4 word's low and high nibbles are laid out as bytes); perm 2
// (packed int2): within every 16 columns, column 4b + i goes to 4i + b (bit
// pair i of the 4 bytes of a weight word forms one byte lane each).
// One workgroup per row, one thread per 16 columns (K / 16 of them, the
// workgroup rounded up to whole waves, at most 16): 16-byte loads of the
// values, the row maximum by lane exchanges and LDS, and each digit plane's
// 16 bytes stored at once.
__global__ __launch_bounds__(1024) void k_limbs(const float* __restrict__ a, int K, int perm,
                                                int8_t* __restrict__ digits, int* __restrict__ expo) {
  __shared__ float red[16];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (int)(blockDim.x >> 6);
  const bool mine = 16 * tid < K;  // threads past the row's groups hold zeros and store nothing
  const float* row = a + (int64_t)r * K + 16 * tid;
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = mine ? reinterpret_cast<const float4*>(row)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = 0.f;
  for (int w = 0; w < nw; ++w) m = fmaxf(m, red[w]);
  int E = 0;
  if (m > 0.f) frexpf(m, &E);  // m = f * 2^E, f in [0.5, 1): |a| < 2^E
  if (tid == 0) expo[r] = E;
  if (!mine) return;
  // Y = X + bias: bytes 0-2 are digits 0-2 plus 128, byte 3 the top digit
  uint32_t y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = (uint32_t)(int)rintf(ldexpf(v[i], 30 - E)) + 0x00808080u;
  // position p of the group holds column src(p)
  auto src = [&](int p) {
    if (perm == 1) { const int h = p & 7, b = p & 8; return b + (h < 4 ? 2 * h : 2 * (h - 4) + 1); }
    if (perm == 2) return 4 * (p & 3) + (p >> 2);
    return p;
  };
  int8_t* out = digits + (int64_t)r * 4 * K + 16 * tid;
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const uint32_t byte = l < 3 ? (((y[src(p)] >> (8 * l)) & 0xFFu) ^ 0x80u) : ((y[src(p)] >> 24) & 0xFFu);
      w[p >> 2] |= byte << (8 * (p & 3));
    }
    *reinterpret_cast<uint4*>(out + (int64_t)l * K) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_limbs(const float* a, int R, int K, int fmt, int8_t* digits, int* expo, hipStream_t st) {
  const int perm = fmt == I4_ROW ? 1 : fmt == I2_ROW ? 2 : 0;
  // K is a multiple of 256 and at most 16384: K / 16 threads in whole waves
  if (K % 256 || K > 16384 || R < 1) return hipErrorInvalidValue;
  const int threads = (K / 16 + 63) / 64 * 64;
  hipLaunchKernelGGL(k_limbs, dim3(R), dim3(threads), 0, st, a, K, perm, digits, expo);
  return hipGetLastError();
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct MfmaI8Args {
  const uint8_t* wq;
  const uint8_t* wq2;
  const float* ws;
  const float* ws2;
  int64_t mat_bytes;
  int M, K, act;
  Disp d;
  const int8_t* digits;  // activation digit planes [rows][4][K]
  const int* expo;       // [rows]
  int act_by_token;
  float* out;            // h [pos][F] or o [pos][H]
  int R;                 // row blocks per workgroup
};

template <int FMT>
MD_DEV i32x4 decode_a8(const uint8_t* p) {
  if constexpr (FMT == I8_ROW) {
    return *reinterpret_cast<const i32x4*>(p);
  } else if constexpr (FMT == I2_ROW) {  // 4 bytes = 16 weights; bytes 64*v, bit pair i of every byte first
    const unsigned u = *reinterpret_cast<const unsigned*>(p);
    i32x4 r;
    r[0] = (int)opaque((u << 6) & 0xC0C0C0C0u);
    r[1] = (int)opaque((u << 4) & 0xC0C0C0C0u);
    r[2] = (int)opaque((u << 2) & 0xC0C0C0C0u);
    r[3] = (int)opaque(u & 0xC0C0C0C0u);
    return r;
  } else {  // I4_ROW: 8 bytes = 16 weights; bytes 16*v, even weights first in every 8
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    i32x4 r;
    r[0] = (int)opaque((u.x << 4) & 0xF0F0F0F0u);
    r[1] = (int)opaque(u.x & 0xF0F0F0F0u);
    r[2] = (int)opaque((u.y << 4) & 0xF0F0F0F0u);
    r[3] = (int)opaque(u.y & 0xF0F0F0F0u);
    return r;
  }
}

// RT: 16-row MFMA tiles per wave; each digit-plane fragment read from LDS
// feeds RT products (the block covers 64*RT rows: for gate/up 32*RT gate rows
// and the same up rows).
#ifndef MD_I8_WAVES
#define MD_I8_WAVES 2
#endif
#ifndef MD_I8_R_LONG
#define MD_I8_R_LONG 1
#endif
#ifndef MD_I8_R_SHORT
#define MD_I8_R_SHORT 4
#endif
template <int FMT, int GU, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MD_I8_WAVES))) void k_moe_mfma_i8(MfmaI8Args a) {
  using TL = Tile<FMT>;
  constexpr int KB = TL::B8 ? 16 : FMT == I2_ROW ? 4 : 8;  // weight bytes per lane per 64-wide step
  constexpr int BR = 64 * RT;          // weight rows per block
  constexpr int WCH = BR * TL::WB / 16, WPT = WCH / 256;
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][BR * TL::WSTR];
  __shared__ __attribute__((aligned(16))) int8_t s_d[2][4 * kTok * kLST];
  __shared__ float s_up[BR / 2][kTok];
  __shared__ int s_e[kTok];

  struct { int e, p0, p1; } er;
  if (a.d.n_active == nullptr) {
    if (blockIdx.y != 0) return;
    er.e = 0; er.p0 = 0; er.p1 = a.d.T;
  } else {  // work item blockIdx.y: one 16-position tile of an active expert
    const int4 it = a.d.items[blockIdx.y];
    if (it.x < 0) return;
    er.e = it.x; er.p0 = it.y; er.p1 = it.z;
  }
  const int t0 = er.p0 + (int)blockIdx.z * kTok;
  if (t0 >= er.p1) return;
  const int nt = min(kTok, er.p1 - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, li = lane & 15;
  const int64_t rb = row_bytes(FMT, a.K);
  const int nkt = a.K / kKT;
  // this block's row blocks: rb_first .. rb_first + nrb - 1, streamed as one
  // sequence of nrb * nkt weight tiles (the loads run on across row blocks)
  constexpr int RPB = GU ? BR / 2 : BR;  // matrix rows per row block
  const int nrb_all = (a.M + RPB - 1) / RPB;
  const int rb_first = blockIdx.x * a.R;
  const int nrb = min(a.R, nrb_all - rb_first);
  const int NT = nrb * nkt;
  auto act_row = [&](int jj) {
    const int pos = t0 + jj;
    return a.act_by_token ? (a.d.n_active == nullptr ? pos : a.d.pairs[pos] / a.d.k) : pos;
  };
  // staging: thread (jj, pp) moves bytes [16 pp, 16 pp + 16) of each digit plane of token slot jj
  const int jj = tid >> 4, pp = tid & 15;
  if (tid < kTok) s_e[tid] = tid < nt ? a.expo[act_row(tid)] : 0;
  // Tiles are read through buffer resources (offsets past a resource's end
  // read zeros without a memory access), so empty token slots and the tiles
  // past the last issue the same loads as the rest: no branch around a load,
  // and the compiled loop waits only for the older of the two tiles in flight.
  const int mat_len = (int)((int64_t)a.M * rb);
  const rsrc_t res_g = make_res(a.wq + (int64_t)er.e * a.mat_bytes, mat_len);
  const rsrc_t res_u = make_res((GU ? a.wq2 : a.wq) + (int64_t)er.e * a.mat_bytes, mat_len);
  const int a_rows = a.act_by_token ? a.d.T : a.d.T * a.d.k;
  const rsrc_t res_d = make_res(a.digits, (int)((int64_t)a_rows * 4 * a.K));
  const bool d_lane = jj < nt;
  const uint32_t doff = d_lane ? (uint32_t)((int64_t)act_row(jj) * 4 * a.K) + 16u * pp : 0u;

  u32x4 rw[2][WPT];
  uint4 rd[2][4];
  auto gload = [&](int ti, int set) {
    const int rbi = ti / nkt, kt = ti - rbi * nkt;
    const bool tile = ti < NT;
    const int r0 = (rb_first + rbi) * RPB;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + 256 * i, r = c / (TL::WB / 16), piece = c % (TL::WB / 16);
      const int f = min(r0 + (GU ? r % (BR / 2) : r), a.M - 1);
      const uint32_t o = (uint32_t)((int64_t)f * rb) + (uint32_t)(kt * TL::WB + 16 * piece);
      rw[set][i] = buf_load<kAuxStream>(GU && i >= WPT / 2 ? res_u : res_g, past(tile, o));
    }
#pragma unroll
    for (int l = 0; l < 4; ++l)
      rd[set][l] = __builtin_bit_cast(uint4, buf_load(res_d, past(tile && d_lane, doff + (uint32_t)(l * a.K + kt * kKT))));
  };
  auto lstore = [&](int buf, int set) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + 256 * i, r = c / (TL::WB / 16), piece = c % (TL::WB / 16);
      *reinterpret_cast<u32x4*>(&s_w[buf][r * TL::WSTR + 16 * piece]) = rw[set][i];
    }
#pragma unroll
    for (int l = 0; l < 4; ++l)
      *reinterpret_cast<uint4*>(&s_d[buf][(l * kTok + jj) * kLST + 16 * pp]) = rd[set][l];
  };
  i32x4 acc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int l = 0; l < 4; ++l) acc[rt][l] = i32x4{0, 0, 0, 0};
  const int wr = wave * 16 * RT;
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kKT / 64; ++s) {
      i32x4 av[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        av[rt] = decode_a8<FMT>(&s_w[buf][(wr + 16 * rt + li) * TL::WSTR + KB * (4 * s + q)]);
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const i32x4 bv = *reinterpret_cast<const i32x4*>(&s_d[buf][(l * kTok + li) * kLST + 64 * s + 16 * q]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][l] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[rt], bv, acc[rt][l], 0, 0, 0);
      }
    }
  };
  // epilogue of row block rbi: lane holds rows wr + 16 rt + 4q + v of token column li
  auto finish = [&](int rbi) {
    const int r0 = (rb_first + rbi) * RPB;
    const int j = li;
    const float ex = ldexpf(1.0f, s_e[j] - 30);
    float val[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        val[rt][v] = (fmaf((float)acc[rt][3][v], 16777216.0f, (float)acc[rt][2][v] * 65536.0f) +
                      fmaf((float)acc[rt][1][v], 256.0f, (float)acc[rt][0][v])) * ex;
    if constexpr (GU) {
      // waves 0, 1: gate rows; waves 2, 3: the same rows of up
      if (wave >= 2) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int v = 0; v < 4; ++v) s_up[wr - BR / 2 + 16 * rt + 4 * q + v][j] = val[rt][v];
      }
      __syncthreads();
      if (wave < 2 && j < nt) {
        const int pos = t0 + j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rr = wr + 16 * rt + 4 * q + v, f = r0 + rr;
            if (f < a.M) {
              const float av = val[rt][v] * a.ws[(int64_t)er.e * a.M + f] * row_post<FMT>();
              const float uv = s_up[rr][j] * a.ws2[(int64_t)er.e * a.M + f] * row_post<FMT>();
              a.out[(int64_t)pos * a.M + f] = act_f(a.act, av) * uv;
            }
          }
        }
      }
    } else {
      if (j < nt) {
        const int pos = t0 + j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int i = r0 + wr + 16 * rt + 4 * q + v;
            if (i < a.M)
              a.out[(int64_t)pos * a.M + i] = val[rt][v] * a.ws[(int64_t)er.e * a.M + i] * row_post<FMT>();
          }
        }
      }
    }
  };
  auto end_of_row_block = [&](int ti) {
    if ((ti + 1) % nkt == 0) {
      finish(ti / nkt);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int l = 0; l < 4; ++l) acc[rt][l] = i32x4{0, 0, 0, 0};
    }
  };
  // Loop top: LDS buffer 0 holds tile ti, register set 1 tile ti+1; the loop
  // runs while tile ti+2 exists, so its LDS stores are unconditional, and the
  // last one or two tiles are computed after it.
  gload(0, 0);
  gload(1, 1);
  lstore(0, 0);
  __syncthreads();
  int ti = 0;
  for (; ti + 2 < NT; ti += 2) {
    gload(ti + 2, 0);
    compute(0);
    end_of_row_block(ti);
    lstore(1, 1);
    __syncthreads();
    gload(ti + 3, 1);
    compute(1);
    end_of_row_block(ti + 1);
    lstore(0, 0);
    __syncthreads();
  }
  compute(0);
  end_of_row_block(ti);
  if (ti + 1 < NT) {
    lstore(1, 1);
    __syncthreads();
    compute(1);
    end_of_row_block(ti + 1);
  }
}

hipError_t launch_moe_mfma_i8(int fmt, bool gateup, const uint8_t* wq, const uint8_t* wq2, const float* ws,
                              const float* ws2, int64_t mat_bytes, int M, int K, int act, const Disp& d,
                              int n_items, const int8_t* digits, const int* expo, bool act_by_token, float* out,
                              hipStream_t st) {
  MfmaI8Args a{wq, wq2, ws, ws2, mat_bytes, M, K, act, d, digits, expo, act_by_token ? 1 : 0, out, 1};
  // int4 weights: two row tiles per wave (LDS reads of the activation digits
  // per weight byte halve); int8: one (its weight tiles are twice as large)
  const int RT = fmt == I4_ROW || fmt == I2_ROW ? 2 : 1;
  const int rows_per_block = (gateup ? 32 : 64) * RT;
  const int tiles = d.items ? 1 : (d.T + kTok - 1) / kTok;
  // row blocks per workgroup: short rows (few K tiles) stream several row
  // blocks back to back so the load pipeline's fill is paid once
  const int nkt = K / kKT;
  a.R = nkt >= 16 ? MD_I8_R_LONG : MD_I8_R_SHORT;
  const int nrb = (M + rows_per_block - 1) / rows_per_block;
  const dim3 grid((nrb + a.R - 1) / a.R, d.items ? n_items : 1, tiles);
#define MD_MF8(F_, RT_) \
  if (fmt == F_ && RT == RT_) { \
    if (gateup) hipLaunchKernelGGL((k_moe_mfma_i8<F_, 1, RT_>), grid, dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((k_moe_mfma_i8<F_, 0, RT_>), grid, dim3(256), 0, st, a); \
    return hipGetLastError(); }
  MD_MF8(I8_ROW, 1) MD_MF8(I4_ROW, 2) MD_MF8(I2_ROW, 2)
#undef MD_MF8
  return hipErrorInvalidValue;
}

}  // namespace md
