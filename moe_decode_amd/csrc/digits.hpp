// digits.hpp -- activations as integer digit planes for the integer dot
// instructions of gfx950 (v_dot8_i32_i4, v_dot4_i32_i8).
//
// A group is the NV activations that one 16-byte weight chunk multiplies.
// The group is scaled by a power of two 2^s, chosen from its largest
// magnitude, and rounded to integers X with |X| <= 2^22.  X is written in
// balanced base 16 (six digits in [-8, 7], 4-bit weights) or balanced base 256
// (three digits in [-128, 127], 8-bit weights): adding the bias
// B = sum_j 8*16^j (or 128*256^j) makes every nibble (byte) of Y = X + B the
// digit plus 8 (128), so flipping its top bit gives the digit as a two's-
// complement nibble (byte).  (Packed int2 weights use base 16 with two planes
// per digit, one for the even and one for the odd weights of each nibble.)  Plane j packs digit j of every value of the group
// into the nibble or byte position of the weight it multiplies, so one dot
// instruction per weight word forms  sum_i w_i * d_j(X_i)  exactly in int32,
// and  sum_j base^j * P_j = sum_i w_i X_i.  The chunk's value is that integer
// times 2^-s; the only rounding is that of x to X (at most 2^-22 of the
// group's largest magnitude per value) and of the final fp32 combine.  (Seven
// or four planes, 2^-26, measured 4-6% slower on the large one-token layers;
// the tolerance 1e-4 * sum|w x| is met with a wide margin at 2^-22.)
#pragma once

#include "common.hpp"

namespace md {

// Plane p holds digit digit(p) of the group's values; nibble (byte) i of its
// word m belongs to value pos(p, m, i).
template <int FMT> struct Dig;
template <> struct Dig<Q4_0> {
  static constexpr int NV = 32, NPL = 6, SB = 22, SH = 4, PER = 8;
  static constexpr uint32_t BIAS = 0x00888888u, FLIP = 0x88888888u;
  static constexpr int digit(int p) { return p; }
  // word m, nibble i <- value: low nibble of byte b is weight 4m+b, high is 16+4m+b
  static constexpr int pos(int, int m, int i) { return (i & 1) ? 16 + 4 * m + (i >> 1) : 4 * m + (i >> 1); }
};
// Q4_1: the Q4_0 nibble order; its codes are unsigned, entered as n - 8 like
// Q4_0's, with (8d + m) times the group's activation sum added per block.
template <> struct Dig<Q4_1> : Dig<Q4_0> {};
template <> struct Dig<I4_ROW> {
  static constexpr int NV = 32, NPL = 6, SB = 22, SH = 4, PER = 8;
  static constexpr uint32_t BIAS = 0x00888888u, FLIP = 0x88888888u;
  static constexpr int digit(int p) { return p; }
  static constexpr int pos(int, int m, int i) { return 8 * m + i; }
};
// Packed int2: a 16-byte chunk holds 64 weights; nibble i of weight word m
// holds weights 16m+2i (bits 0-1) and 16m+2i+1 (bits 2-3).  Each digit has
// two planes: plane 2j pairs digit j of the even weights' activations with
// those nibbles, plane 2j+1 digit j of the odd ones'.
template <> struct Dig<I2_ROW> {
  static constexpr int NV = 64, NPL = 12, SB = 22, SH = 4, PER = 8;
  static constexpr uint32_t BIAS = 0x00888888u, FLIP = 0x88888888u;
  static constexpr int digit(int p) { return p >> 1; }
  static constexpr int pos(int p, int m, int i) { return 16 * m + 2 * i + (p & 1); }
};
template <> struct Dig<Q8_0> {
  static constexpr int NV = 16, NPL = 3, SB = 22, SH = 8, PER = 4;
  static constexpr uint32_t BIAS = 0x00808080u, FLIP = 0x80808080u;
  static constexpr int digit(int p) { return p; }
  static constexpr int pos(int, int m, int i) { return 4 * m + i; }
};
template <> struct Dig<I8_ROW> : Dig<Q8_0> {};

__host__ __device__ constexpr int dig_nv(int fmt) {
  return (fmt == Q8_0 || fmt == I8_ROW) ? 16 : fmt == I2_ROW ? 64 : 32;
}
__host__ __device__ constexpr int dig_npl(int fmt) {
  return (fmt == Q8_0 || fmt == I8_ROW) ? 3 : fmt == I2_ROW ? 12 : 6;
}
// bytes of digit planes per group, and per K activations
__host__ __device__ constexpr int64_t dig_group_bytes(int fmt) { return 16 * dig_npl(fmt); }
__host__ __device__ constexpr int64_t dig_bytes(int fmt, int K) { return (int64_t)(K / dig_nv(fmt)) * dig_group_bytes(fmt); }

// Shift s of a group whose largest magnitude is m: m < 2^e, s = SB - e,
// limited so that 2^-s stays a normal number for tiny groups.
template <int FMT>
MD_DEV int dig_shift(float m) {
  int e = 0;
  (void)frexpf(m, &e);
  const int s = Dig<FMT>::SB - e;
  return s > 120 ? 120 : s;
}

// Biased integer image of one value (its nibbles / bytes are digit + 8 / 128).
template <int FMT>
MD_DEV uint32_t dig_biased(float v, int s) {
  return (uint32_t)(int)rintf(ldexpf(v, s)) + Dig<FMT>::BIAS;
}

// Word (plane p, weight word m) of a group from the biased images Y[0..NV).
template <int FMT, typename GetY>
MD_DEV uint32_t dig_word(int p, int m, GetY Y) {
  using D = Dig<FMT>;
  constexpr uint32_t mask = (1u << D::SH) - 1u;
  const int j = D::digit(p);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < D::PER; ++i) w |= ((Y(D::pos(p, m, i)) >> (D::SH * j)) & mask) << (D::SH * i);
  return w ^ D::FLIP;
}

// One thread writes a whole group: planes (NPL x 4 words) and the scale 2^-s.
template <int FMT>
MD_DEV void dig_group(const float* v, uint32_t* planes, float* scale) {
  using D = Dig<FMT>;
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < D::NV; ++i) m = fmaxf(m, fabsf(v[i]));
  const int s = dig_shift<FMT>(m);
  uint32_t Y[D::NV];
#pragma unroll
  for (int i = 0; i < D::NV; ++i) Y[i] = dig_biased<FMT>(v[i], s);
#pragma unroll
  for (int j = 0; j < D::NPL; ++j)
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) planes[4 * j + mm] = dig_word<FMT>(j, mm, [&](int p) { return Y[p]; });
  *scale = ldexpf(1.0f, -s);
}

// Running plane sums of one lane: the integer dot instructions accumulate
// into a[] without being cleared between chunks, and a chunk's value is the
// difference of the combined sums before and after it (lo, hi hold the last
// combination).  All of it is exact two's-complement arithmetic: a sum that
// wraps still gives the right difference, since each chunk's own combination
// fits easily in 32 bits.
template <int FMT>
struct DigAcc {
  int a[Dig<FMT>::NPL];
  int lo, hi;
  MD_DEV DigAcc() : lo(0), hi(0) {
#pragma unroll
    for (int j = 0; j < Dig<FMT>::NPL; ++j) a[j] = 0;
  }
};

// Value of one chunk: w = the chunk's 4 weight words, d = its group's planes,
// sc = 2^-s.  Returns sum_i w_i x_i (before the weights' block or row scale).
template <int FMT>
MD_DEV float dig_chunk(u32x4 w, const u32x4* d, float sc, DigAcc<FMT>& r) {
  using D = Dig<FMT>;
  if constexpr (FMT == I2_ROW) {
    // even weights sign-extended from bits 0-1 to whole nibbles; odd weights
    // stay in bits 2-3, i.e. nibbles of 4 * value: 4 * sum = sum_j 16^j (4 E_j + O_j)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t e = w[m] & 0x33333333u, sg = e & 0x22222222u;
      const uint32_t we = e | (sg << 1) | (sg << 2), wo = w[m] & 0xCCCCCCCCu;
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        r.a[2 * j] = __builtin_amdgcn_sdot8((int)we, (int)d[2 * j][m], r.a[2 * j], false);
        r.a[2 * j + 1] = __builtin_amdgcn_sdot8((int)wo, (int)d[2 * j + 1][m], r.a[2 * j + 1], false);
      }
    }
    uint32_t p[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) p[j] = 4u * (uint32_t)r.a[2 * j] + (uint32_t)r.a[2 * j + 1];
    const uint32_t lo = p[0] + 16u * (p[1] + 16u * (p[2] + 16u * p[3])), hi = p[4] + 16u * p[5];
    const int dlo = (int)(lo - (uint32_t)r.lo), dhi = (int)(hi - (uint32_t)r.hi);
    r.lo = (int)lo;
    r.hi = (int)hi;
    return fmaf((float)dhi, sc * 16384.0f, (float)dlo * (sc * 0.25f));
  }
  if constexpr (FMT == Q4_0 || FMT == Q4_1) w ^= u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};  // n - 8
#pragma unroll
  for (int j = 0; j < D::NPL; ++j) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if constexpr (D::SH == 4)
        r.a[j] = __builtin_amdgcn_sdot8((int)w[m], (int)d[j][m], r.a[j], false);
      else
        r.a[j] = __builtin_amdgcn_sdot4((int)w[m], (int)d[j][m], r.a[j], false);
    }
  }
  uint32_t lo, hi;  // unsigned: wrap-around is defined
  if constexpr (D::SH == 4) {
    lo = (uint32_t)r.a[0] + 16u * ((uint32_t)r.a[1] + 16u * ((uint32_t)r.a[2] + 16u * (uint32_t)r.a[3]));
    hi = (uint32_t)r.a[4] + 16u * (uint32_t)r.a[5];
  } else {
    lo = (uint32_t)r.a[0] + 256u * (uint32_t)r.a[1];
    hi = (uint32_t)r.a[2];
  }
  const int dlo = (int)(lo - (uint32_t)r.lo), dhi = (int)(hi - (uint32_t)r.hi);
  r.lo = (int)lo;
  r.hi = (int)hi;
  return fmaf((float)dhi, sc * 65536.0f, (float)dlo * sc);
}

// The same with the plane sums cleared for the chunk (no state carried).
template <int FMT>
MD_DEV float dig_chunk(u32x4 w, const u32x4* d, float sc) {
  DigAcc<FMT> r;
  return dig_chunk<FMT>(w, d, sc, r);
}

// Block scale of chunk c for the digit path (no 1/16: nibbles enter as values).
template <int FMT>
MD_DEV float dig_block_scale(const uint8_t* row, int K, int c) {
  if constexpr (FMT == Q8_0) {
    return h2f(*reinterpret_cast<const uint16_t*>(row + K + 2 * (c >> 1)));
  } else if constexpr (FMT == Q4_0) {
    return h2f(*reinterpret_cast<const uint16_t*>(row + (K / 32) * 16 + 2 * c));
  } else {
    return 1.0f;
  }
}

// Q4_1: block c's scale d and minimum m, one 4-byte read.
MD_DEV void dig_block_dm_q4_1(const uint8_t* row, int K, int c, float& d, float& m) {
  const uint32_t dm = *reinterpret_cast<const uint32_t*>(row + (K / 32) * 16 + 4 * c);
  d = h2f((uint16_t)(dm & 0xFFFFu));
  m = h2f((uint16_t)(dm >> 16));
}

// Sum of a 4-bit group's values as the planes hold them, times sc: each
// plane's digits summed by one dot against all-ones nibbles, then combined
// in base 16 (|sum X| <= 32 * 2^22, exact in int32).
template <int FMT>
MD_DEV float dig_group_sum(const u32x4* d, float sc) {
  static_assert(Dig<FMT>::SH == 4 && Dig<FMT>::NV == 32, "4-bit groups of 32");
  int s[Dig<FMT>::NPL];
#pragma unroll
  for (int j = 0; j < Dig<FMT>::NPL; ++j) {
    int a = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) a = __builtin_amdgcn_sdot8((int)d[j][m], 0x11111111, a, false);
    s[j] = a;
  }
  int X = s[Dig<FMT>::NPL - 1];
#pragma unroll
  for (int j = Dig<FMT>::NPL - 2; j >= 0; --j) X = 16 * X + s[j];
  return (float)X * sc;
}

}  // namespace md
