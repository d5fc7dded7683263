// common.hpp -- device helpers of libmoe_decode (gfx950, wave64).
//
// Weight rows are streamed in 16-byte chunks (one global_load_dwordx4 per
// lane, consecutive lanes on consecutive chunks, so a wavefront reads 1 KiB of
// one row per instruction).  A chunk holds:
//   Q8_0   16 int8 weights, scale = the fp16 d of block c/2
//   Q4_0   one block: 32 nibbles (low nibbles = weights 0..15, high = 16..31)
//   I8_ROW 16 int8 weights (scale per row)
//   I4_ROW 32 two's-complement nibbles, low nibble of byte b = weight 2b
//   Q4_1   one block: 32 unsigned nibbles in the Q4_0 order; scale d and
//          minimum m of the block (w = d n + m)
//   I2_ROW 64 two's-complement bit pairs, bits 2i..2i+1 of byte b = weight
//          4b+i (scale per row)
// Decoding happens in VGPRs.  int8 goes through the sign-extending byte
// convert.  A 4-bit code is made a two's-complement nibble (Q4_0: n XOR 8 is
// n - 8) and moved into the high half of a byte with a 0xF0F0F0F0 mask, so each
// byte holds exactly 16 * value as an int8 and converts with the same
// sign-extending byte convert; the factor 1/16 is folded into the scale.  No
// offset correction is needed, so an all-zero row gives exactly zero.  Q4_1
// codes carry no offset: masked the same way they convert with the unsigned
// byte convert, and the block's m times the block's sum of activations is
// added.  A 2-bit code moved into the top two bits of a byte is 64 * value.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#define MD_DEV __device__ __forceinline__

namespace md {

enum : int { Q8_0 = 1, Q4_0 = 2, I8_ROW = 3, I4_ROW = 4, Q4_1 = 5, I2_ROW = 6 };
enum : int { ACT_GELU_TANH = 0, ACT_SILU = 1 };
enum : int { XF32 = 0, XBF16 = 1 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int FMT> struct Fmt;
template <> struct Fmt<Q8_0>   { static constexpr int WPC = 16; static constexpr bool ROW = false; };
template <> struct Fmt<Q4_0>   { static constexpr int WPC = 32; static constexpr bool ROW = false; };
template <> struct Fmt<I8_ROW> { static constexpr int WPC = 16; static constexpr bool ROW = true; };
template <> struct Fmt<I4_ROW> { static constexpr int WPC = 32; static constexpr bool ROW = true; };
template <> struct Fmt<Q4_1>   { static constexpr int WPC = 32; static constexpr bool ROW = false; };
template <> struct Fmt<I2_ROW> { static constexpr int WPC = 64; static constexpr bool ROW = true; };

__host__ __device__ constexpr int64_t row_bytes(int fmt, int K) {
  return fmt == Q8_0 ? (int64_t)K / 32 * 34
       : fmt == Q4_0 ? (int64_t)K / 32 * 18
       : fmt == I8_ROW ? (int64_t)K
       : fmt == Q4_1 ? (int64_t)K / 32 * 20
       : fmt == I2_ROW ? (int64_t)K / 4
       : (int64_t)K / 2;
}
__host__ __device__ constexpr int wpc(int fmt) {
  return (fmt == Q8_0 || fmt == I8_ROW) ? 16 : fmt == I2_ROW ? 64 : 32;
}
__host__ __device__ constexpr int nchunks(int fmt, int K) { return K / wpc(fmt); }

// Hide known bits from the optimizer so each masked byte converts with one
// sign-extending byte convert (SDWA) instead of a bit-field extract plus a
// convert per nibble.
MD_DEV unsigned opaque(unsigned v) { asm volatile("" : "+v"(v)); return v; }

#ifndef MD_NT_LOADS
#define MD_NT_LOADS 1
#endif
MD_DEV u32x4 ld_stream(const uint8_t* p) {
#if MD_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

// Raw buffer resource over the n bytes at p (descriptor word 3 of the gfx9
// family: dword data, range-checked).  A read at an offset past n returns
// zeros and touches no memory; kPast is past the end of every resource here
// (all are under 2 GiB, so offset + kPast never wraps).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
MD_DEV rsrc_t make_res(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
constexpr uint32_t kPast = 0x80000000u;
MD_DEV uint32_t past(bool ok, uint32_t off) { return ok ? off : kPast; }
constexpr int kAuxStream = MD_NT_LOADS ? 2 : 0;  // nontemporal hint for streamed weights
template <int AUX = 0>
MD_DEV u32x4 buf_load(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
}

MD_DEV float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Scale that multiplies chunk c of a row (block formats, including the 1/16
// of the 4-bit decode); 1 for per-row formats (their scale is applied once per
// row, times row_post<FMT>()).
template <int FMT>
MD_DEV float chunk_scale(const uint8_t* row, int K, int c) {
  if constexpr (FMT == Q8_0) {
    return h2f(*reinterpret_cast<const uint16_t*>(row + K + 2 * (c >> 1)));
  } else if constexpr (FMT == Q4_0) {
    return h2f(*reinterpret_cast<const uint16_t*>(row + (K / 32) * 16 + 2 * c)) * 0.0625f;
  } else if constexpr (FMT == Q4_1) {
    return h2f(*reinterpret_cast<const uint16_t*>(row + (K / 32) * 16 + 4 * c)) * 0.0625f;
  } else {
    return 1.0f;
  }
}

// Q4_1: the minimum m of block c.
MD_DEV float chunk_min_q4_1(const uint8_t* row, int K, int c) {
  return h2f(*reinterpret_cast<const uint16_t*>(row + (K / 32) * 16 + 4 * c + 2));
}

template <int FMT>
constexpr float row_post() { return FMT == I4_ROW ? 0.0625f : FMT == I2_ROW ? 0.015625f : 1.0f; }

// Load the WPC activations of chunk c (fp32 or bf16 source).
template <int FMT, int XT>
MD_DEV void load_x(const void* xp, int c, float* xv) {
  constexpr int W = Fmt<FMT>::WPC;
  if constexpr (XT == XF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(xp) + c * W);
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      float4 v = p[i];
      xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xp) + c * W);
#pragma unroll
    for (int i = 0; i < W / 8; ++i) {
      uint4 v = p[i];
      unsigned u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
        xv[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
      }
    }
  }
}

// Dot product of one chunk's integer codes with its activations (the block or
// row scale is applied by the caller).  4-bit formats return 16x the value.
template <int FMT>
MD_DEV float dot_chunk(u32x4 w, const float* xv) {
  float a0 = 0.f, a1 = 0.f;
  if constexpr (FMT == Q8_0 || FMT == I8_ROW) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      unsigned u = w[m];
      a0 = fmaf((float)(signed char)(u), xv[4 * m], a0);
      a1 = fmaf((float)(signed char)(u >> 8), xv[4 * m + 1], a1);
      a0 = fmaf((float)(signed char)(u >> 16), xv[4 * m + 2], a0);
      a1 = fmaf((float)(signed char)(u >> 24), xv[4 * m + 3], a1);
    }
  } else if constexpr (FMT == Q4_0) {
    // byte b of word m: low nibble = weight 4m+b, high nibble = weight 16+4m+b
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const unsigned v = w[m] ^ 0x88888888u;                 // n - 8 as two's complement
      const unsigned lo = opaque((v << 4) & 0xF0F0F0F0u), hi = opaque(v & 0xF0F0F0F0u);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        a0 = fmaf((float)(signed char)(lo >> (8 * b)), xv[4 * m + b], a0);
        a1 = fmaf((float)(signed char)(hi >> (8 * b)), xv[16 + 4 * m + b], a1);
      }
    }
  } else if constexpr (FMT == Q4_1) {
    // the Q4_0 order, unsigned codes: each masked byte is 16 * n
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const unsigned lo = opaque((w[m] << 4) & 0xF0F0F0F0u), hi = opaque(w[m] & 0xF0F0F0F0u);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        a0 = fmaf((float)(unsigned char)(lo >> (8 * b)), xv[4 * m + b], a0);
        a1 = fmaf((float)(unsigned char)(hi >> (8 * b)), xv[16 + 4 * m + b], a1);
      }
    }
  } else if constexpr (FMT == I2_ROW) {
    // byte b of word m holds weights 16m+4b+i in bits 2i..2i+1; plane i moves
    // them to the top of each byte: 64 * value as an int8
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const unsigned p[4] = {opaque((w[m] << 6) & 0xC0C0C0C0u), opaque((w[m] << 4) & 0xC0C0C0C0u),
                             opaque((w[m] << 2) & 0xC0C0C0C0u), opaque(w[m] & 0xC0C0C0C0u)};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (float)(signed char)(p[i] >> (8 * b));
          if (i & 1) a1 = fmaf(v, xv[16 * m + 4 * b + i], a1);
          else a0 = fmaf(v, xv[16 * m + 4 * b + i], a0);
        }
      }
    }
  } else {  // I4_ROW: byte b of word m: low nibble = weight 8m+2b, high = 8m+2b+1
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const unsigned lo = opaque((w[m] << 4) & 0xF0F0F0F0u), hi = opaque(w[m] & 0xF0F0F0F0u);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        a0 = fmaf((float)(signed char)(lo >> (8 * b)), xv[8 * m + 2 * b], a0);
        a1 = fmaf((float)(signed char)(hi >> (8 * b)), xv[8 * m + 2 * b + 1], a1);
      }
    }
  }
  return a0 + a1;
}

// ---- lane exchanges without LDS traffic (gfx950)
//
// xor_lanes<OFF>(x): the value of lane (lane ^ OFF).  Quads and the 8-lane
// halves of a row by DPP, across rows by the permlane swaps.
template <int CTRL>
MD_DEV float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int OFF>
MD_DEV float xor_lanes(float x) {
  if constexpr (OFF == 1) return dpp_f<0xB1>(x);        // quad_perm [1,0,3,2]
  else if constexpr (OFF == 2) return dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  else if constexpr (OFF == 4)                          // swizzle, bit mode: and 0x1F, xor 4
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
  else if constexpr (OFF == 8) return dpp_f<0x128>(x);  // row_ror:8 (xor 8 within a row of 16)
  else if constexpr (OFF == 16) {                       // rows 0<->1, 2<->3
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(((threadIdx.x & 16) ? r[0] : r[1]));
  } else {                                              // halves of the wave
    static_assert(OFF == 32, "lane offset");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(((threadIdx.x & 32) ? r[0] : r[1]));
  }
}

// Reduction over groups of 2*OFF lanes, one step: every lane combines its
// value with one other lane's so that, after the steps OFF, OFF/2, ..., 1,
// each lane holds the group's total.  Step 4 pairs lane i with i ^ 7 within
// 8 lanes (the row half-mirror), which covers the same lanes together with
// the steps 2 and 1 that follow it.
template <int OFF, typename Op>
MD_DEV float allreduce_step(float x, Op op) {
  if constexpr (OFF == 4) return op(x, dpp_f<0x141>(x));  // row_half_mirror
  else return op(x, xor_lanes<OFF>(x));
}

template <int OFF, typename Op>
MD_DEV float allreduce_from(float x, Op op) {
  if constexpr (OFF >= 1) return allreduce_from<OFF / 2>(allreduce_step<OFF>(x, op), op);
  else return x;
}

// Sum / maximum over the L consecutive lanes of a lane group (L a power of
// two <= 64), returned to every lane of the group.
template <int L>
MD_DEV float group_sum(float v) {
  return allreduce_from<L / 2>(v, [](float x, float y) { return x + y; });
}
template <int L>
MD_DEV float group_max(float v) {
  return allreduce_from<L / 2>(v, [](float x, float y) { return fmaxf(x, y); });
}

MD_DEV double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// tanh-form GELU and SiLU in fp32.
MD_DEV float act_f(int act, float z) {
  if (act == ACT_SILU) return z / (1.0f + expf(-z));
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}

}  // namespace md
