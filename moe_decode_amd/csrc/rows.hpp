// rows.hpp -- wave-level building blocks of the one-token kernels (gfx950,
// wave64): lane-group reductions, 16-byte row streaming against activation
// digit planes held in registers, digit planes of a workgroup's values, and
// the single-wave router top-k.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "digits.hpp"

namespace md {

#ifndef MD_GU_WINDOW
#define MD_GU_WINDOW 2
#endif
#ifndef MD_DN_WINDOW
#define MD_DN_WINDOW 8
#endif
#ifndef MD_GU_RUN
#define MD_GU_RUN 0
#endif

// One level of the transposed butterfly: lanes with (t & OFF) == 0 return
// a + a(partner), the others b + b(partner), partner = lane ^ OFF (the same
// sums, bit for bit, in either formulation).
template <int OFF>
MD_DEV float butterfly_level(float a, float b, int t) {
  if constexpr (OFF == 32) {
    // r[0] = [a of lanes 0-31, b of lanes 0-31], r[1] = [a of 32-63, b of 32-63]
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (OFF == 16) {
    // r[0] = [a row 0, b row 0, a row 2, b row 2], r[1] = [a row 1, b row 1, a row 3, b row 3]
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    // m = all ones on the upper lane of each pair: it sends a and keeps b;
    // the lower lane the other way round.  Bit-field selects keep both
    // candidates in registers (a select between array elements would be
    // turned into a computed index and a chain of compares).
    const uint32_t m = (t & OFF) ? 0xFFFFFFFFu : 0u;
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    const float send = __uint_as_float((ua & m) | (ub & ~m));
    const float keep = __uint_as_float((ub & m) | (ua & ~m));
    return keep + xor_lanes<OFF>(send);
  }
}

template <int N, int L, int S>
MD_DEV void butterfly_levels(float (&v)[N], int t) {
  if constexpr ((N >> S) > 1) {
    constexpr int half = (N >> S) / 2, off = L >> (S + 1);
#pragma unroll
    for (int i = 0; i < half; ++i) v[i] = butterfly_level<off>(v[i], v[i + half], t);
    butterfly_levels<N, L, S + 1>(v, t);
  }
}

// Sum over the L lanes of a group for N rows at once.  On return lane t holds
// the full sum of row (t / (L/N)) % N.
template <int N, int L>
MD_DEV float butterfly(float (&v)[N], int t) {
  static_assert(N <= L, "more rows than lanes");
  butterfly_levels<N, L, 0>(v, t);
  return group_sum<L / N>(v[0]);
}

template <int FMT, int CPL>
struct RowBuf {
  u32x4 w[CPL];
  float s[CPL];
  float m[FMT == Q4_1 ? CPL : 1];  // Q4_1: 8d + m of each block
};

template <int FMT, int L, int CPL>
MD_DEV void load_row(RowBuf<FMT, CPL>& b, const uint8_t* row, int K, int c0) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) b.w[i] = ld_stream(row + 16 * (int64_t)(c0 + L * i));
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if constexpr (FMT == Q4_1) {
      float d, m;
      dig_block_dm_q4_1(row, K, c0 + L * i, d, m);
      b.s[i] = d;
      b.m[i] = fmaf(8.0f, d, m);
    } else {
      b.s[i] = dig_block_scale<FMT>(row, K, c0 + L * i);
    }
  }
}

// Activation digit planes of the CPL chunks a lane owns (Q4_1: with each
// group's activation sum).
template <int FMT, int CPL>
struct ActDig {
  u32x4 d[CPL][Dig<FMT>::NPL];
  float sc[CPL];
  float xs[FMT == Q4_1 ? CPL : 1];
};

// kCoh: the planes were written by another workgroup of the same launch
// (agent-scope atomic loads, which see the writer's agent-scope stores).
template <int FMT, int L, int CPL, bool kCoh = false>
MD_DEV void load_act(ActDig<FMT, CPL>& x, const u32x4* planes, const float* scales, int c0) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
#pragma unroll
    for (int j = 0; j < Dig<FMT>::NPL; ++j) {
      const u32x4* p = planes + (int64_t)(c0 + L * i) * Dig<FMT>::NPL + j;
      if constexpr (kCoh) {
        const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
        const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        x.d[i][j] = u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
      } else {
        x.d[i][j] = *p;
      }
    }
    if constexpr (kCoh)
      x.sc[i] = __hip_atomic_load(scales + c0 + L * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      x.sc[i] = scales[c0 + L * i];
    if constexpr (FMT == Q4_1) x.xs[i] = dig_group_sum<FMT>(x.d[i], x.sc[i]);
  }
}

// kRun: carry the plane sums in r across calls (fewer instructions, more
// live registers); otherwise each chunk starts from zero.
template <int FMT, int CPL, bool kRun = true>
MD_DEV float row_dot(const RowBuf<FMT, CPL>& b, const ActDig<FMT, CPL>& x, DigAcc<FMT>& r) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const float v = kRun ? dig_chunk<FMT>(b.w[i], x.d[i], x.sc[i], r) : dig_chunk<FMT>(b.w[i], x.d[i], x.sc[i]);
    if constexpr (FMT == Q4_1)  // d * sum (n - 8) X + (8d + m) * sum X
      acc = fmaf(b.s[i], v, fmaf(b.m[i], x.xs[i], acc));
    else
      acc = Fmt<FMT>::ROW ? acc + v : fmaf(b.s[i], v, acc);
  }
  return acc;
}

// Store that another workgroup of the same launch reads (agent scope).
template <bool kCoh, typename V>
MD_DEV void put(V* p, V v) {
  if constexpr (kCoh)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Digit planes of n values held one per thread (thread q: value q; n a
// multiple of NV and at most blockDim.x): group g's planes go to
// planes[g * NPL .. ] and its scale to scales[g].  ys: LDS scratch of n words.
// Every thread of the block must call it (it synchronises).
template <int FMT, bool kCoh = false>
MD_DEV void dig_block(float v, int n, uint32_t* ys, u32x4* planes, float* scales) {
  using D = Dig<FMT>;
  const int q = threadIdx.x;
  const float m = group_max<D::NV>(q < n ? fabsf(v) : 0.f);
  const int s = dig_shift<FMT>(m);
  if (q < n) {
    ys[q] = dig_biased<FMT>(v, s);
    if (q % D::NV == 0) put<kCoh>(scales + q / D::NV, ldexpf(1.0f, -s));
  }
  __syncthreads();
  uint32_t* out = reinterpret_cast<uint32_t*>(planes);
  const int nw = n / D::NV * D::NPL * 4;
  for (int i = q; i < nw; i += blockDim.x) {
    const int g = i / (D::NPL * 4), w = i % (D::NPL * 4);
    put<kCoh>(out + i, dig_word<FMT>(w / 4, w % 4, [&](int p) { return ys[g * D::NV + p]; }));
  }
  __syncthreads();
}

// ------------------------------------------------------------------ top-k


// Maximum of a 32-bit unsigned value over the wave, returned to every lane
// (uniform).  Lane moves by DPP only: within quads, then mirrored half-rows and
// rows (each row of 16 lanes then holds its maximum), then the row broadcasts
// carry it to lane 63, which is read back.
MD_DEV uint32_t wave_max_u32(uint32_t v) {
  // lanes a row broadcast does not write read 0, the identity of the maximum
  // (so each lane move can fold into the max instruction as a DPP operand)
  auto step = [&](auto ctrl, auto row_mask) {
    const uint32_t p = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, decltype(ctrl)::value,
                                                              decltype(row_mask)::value, 0xF, false);
    v = p > v ? p : v;
  };
  step(std::integral_constant<int, 0xB1>{}, std::integral_constant<int, 0xF>{});   // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{}, std::integral_constant<int, 0xF>{});   // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{}, std::integral_constant<int, 0xF>{});  // row_half_mirror
  step(std::integral_constant<int, 0x140>{}, std::integral_constant<int, 0xF>{});  // row_mirror
  step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});  // row_bcast:15 into rows 1, 3
  step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

MD_DEV uint32_t order_key32(float l) {
  uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit of an order key (-0 comes back as +0).
MD_DEV float key_logit(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// Selection rounds over 32-bit order keys held as lane l: experts l, l + 64,
// l + 128, l + 192 (0 marks a taken or absent expert: every finite logit maps
// above it).  Each round takes the wave maximum of the keys; among the experts
// that hold it (an exact tie) the lowest index wins: the first of the four
// slots with a match, and within it the lowest lane.  sel[j] (every lane) is
// the j-th winner; lane j's my_l is its logit.  Only the first nr <= k
// winners are formed (sel[j] = 0 for j >= nr).
MD_DEV void topk_rounds(uint32_t (&key)[4], int nr, int lane, int (&sel)[8], float& my_l) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel[j] = 0;
    if (j >= nr) continue;
    const uint32_t best = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
    int e = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t hit = __ballot(key[i] == best);
      if (!found && hit != 0) {
        e = 64 * i + (int)__builtin_ctzll(hit);
        found = true;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == e) key[i] = 0u;
    if (lane == j) my_l = key_logit(best);
    sel[j] = e;
  }
}

// Wave-level top-k of one token's E logits (E <= 256), formed from the S
// router partials of each expert (added in slice order, plus the bias,
// rounded once to fp32), by topk_rounds over order-preserving 32-bit images
// of the logits.  All lanes return the same experts in selection order (the
// first min(k, need) of them; all k when the gates are asked for) and, when
// asked, the gates: lane j forms exp(l_j - l_0) in fp64, the sum
// runs over j in order, gate j = its term / sum, rounded to fp32.
MD_DEV void wave_topk(const double* __restrict__ part, int S, const float* __restrict__ bias, int E, int k, int lane,
                      int (&sel)[8], float (&gts)[8], bool want_gates, int need = 8) {
  // every load is issued before the first use (indices clamped, results of
  // lanes past E dropped), so the logits cost one memory round trip per slice
  double a[4];
  float b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = part[(int64_t)min(lane + 64 * i, E - 1) * S];
  if (bias) {
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = bias[min(lane + 64 * i, E - 1)];
  }
  for (int s = 1; s < S; ++s) {
    double p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = part[(int64_t)min(lane + 64 * i, E - 1) * S + s];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] += p[i];
  }
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (bias) a[i] += (double)b[i];
    key[i] = lane + 64 * i < E ? order_key32((float)a[i]) : 0u;
  }
  float my_l = 0.f;
  topk_rounds(key, want_gates ? k : min(k, need), lane, sel, my_l);
  if (want_gates) {
    const double m = (double)__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(my_l)));
    const double ex = lane < k ? exp((double)my_l - m) : 0.0;
    double z = 0.0;
    for (int j = 0; j < k; ++j) {
      const uint64_t u = (uint64_t)__double_as_longlong(ex);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, j);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), j);
      z += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
    const float g = (float)(ex / z);
#pragma unroll
    for (int j = 0; j < 8; ++j) gts[j] = j < k ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), j)) : 0.f;
  }
}

// ------------------------------------------------------------------ tiles

// Gate/up rows of one (token, slot) pair for one workgroup: KS*RGW waves;
// wave (rg, ks) streams kNP row pairs per lane group over K-slice ks, rows
// [f0, f0 + RGW*G*kNP).  h = act(gate) * up goes through LDS (lds: the h
// values, then 2*KS per row of slice sums) and leaves as digit planes of the
// down matrix's format (the same format).  Waves past KS*RGW only take part
// in the barriers; every thread of the workgroup must call it.  kCoh: the h
// planes are read by other workgroups of the same launch.  kWin: row pairs in
// flight per lane group (kNP: every row load issued up front).
struct GuTile {
  const uint8_t* Gm;      // the expert's gate matrix (device layout)
  const uint8_t* Um;      // its up matrix
  const float* gs;        // row scales of gate / up (per-row formats) or nullptr
  const float* us;
  int F, H, act, KS, RGW;
  const u32x4* xd;        // x digit planes of the token (group 0)
  const float* xsc;
  u32x4* hd;              // h digit planes of the pair (group 0)
  float* hsc;
};

// The activation planes a lane of gu_tile multiplies: chunk ks * L + t of the
// token (expert-independent, so a caller may load them before it knows the
// expert and pass them in as pre).
template <int FMT, int L>
MD_DEV void gu_act(const GuTile& a, ActDig<FMT, 1>& xa) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = wave % a.KS, t = lane % L;
  if (wave / a.KS < a.RGW) load_act<FMT, L, 1>(xa, a.xd, a.xsc, ks * L + t);
}

template <int FMT, int L, int kNP, bool kCoh = false, int kWin = MD_GU_WINDOW>
MD_DEV void gu_tile(const GuTile& a, int f0, float* lds, uint32_t* ys, const ActDig<FMT, 1>* pre = nullptr) {
  using D = Dig<FMT>;
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / L, t = lane % L;
  const int ks = wave % a.KS, rg = wave / a.KS;
  const int npairs = a.RGW * G * kNP;
  float* hv = lds;
  float* red = lds + npairs;
  auto finish = [&](int q, float av, float uv) {
    const int f = f0 + q;
    float sg = 1.f, sv = 1.f;
    if (f < a.F && a.gs) {
      sg = a.gs[f];
      sv = a.us[f];
    }
    hv[q] = f < a.F ? act_f(a.act, av * sg) * (uv * sv) : 0.f;
  };
  if (rg < a.RGW) {
    const int c0 = ks * L + t;  // this lane's chunk (one chunk per lane per slice)
    ActDig<FMT, 1> xa;
    if (pre) xa = *pre;
    else load_act<FMT, L, 1>(xa, a.xd, a.xsc, c0);
    const int fb = f0 + (rg * G + g) * kNP;
    const int64_t rb = row_bytes(FMT, a.H);
    float pg[kNP], pu[kNP];
    {
      // rolling window: kD row pairs in flight while one pair is decoded
      constexpr int kD = kNP < kWin ? kNP : kWin;
      RowBuf<FMT, 1> bg[kD], bu[kD];
      DigAcc<FMT> ra;  // one running state serves the gate and up rows alike
      auto rowp = [&](const uint8_t* M, int p) { return M + (int64_t)min(fb + p, a.F - 1) * rb; };
#pragma unroll
      for (int p = 0; p < kD; ++p) {
        load_row<FMT, L, 1>(bg[p], rowp(a.Gm, p), a.H, c0);
        load_row<FMT, L, 1>(bu[p], rowp(a.Um, p), a.H, c0);
      }
#pragma unroll
      for (int p = 0; p < kNP; ++p) {
        pg[p] = row_dot<FMT, 1, MD_GU_RUN>(bg[p % kD], xa, ra);
        pu[p] = row_dot<FMT, 1, MD_GU_RUN>(bu[p % kD], xa, ra);
        if (p + kD < kNP) {
          load_row<FMT, L, 1>(bg[p % kD], rowp(a.Gm, p + kD), a.H, c0);
          load_row<FMT, L, 1>(bu[p % kD], rowp(a.Um, p + kD), a.H, c0);
        }
      }
    }
    const float sa = butterfly<kNP, L>(pg, t);
    const float su = butterfly<kNP, L>(pu, t);
    const int r = (t / (L / kNP)) % kNP;
    if ((t % (L / kNP)) == 0) {
      const int q = (rg * G + g) * kNP + r;
      if (a.KS == 1) {
        finish(q, sa, su);
      } else {
        red[(q * a.KS + ks) * 2] = sa;
        red[(q * a.KS + ks) * 2 + 1] = su;
      }
    }
  }
  if (a.KS > 1) {
    __syncthreads();
    for (int q = threadIdx.x; q < npairs; q += blockDim.x) {
      const float* rq = red + q * a.KS * 2;
      float av = 0.f, uv = 0.f;
      for (int s = 0; s < a.KS; ++s) { av += rq[2 * s]; uv += rq[2 * s + 1]; }
      finish(q, av, uv);
    }
  }
  __syncthreads();
  // digit planes of the tile's h values (rows past F form whole groups and are skipped)
  const int n = min(npairs, a.F - f0);
  dig_block<FMT, kCoh>(threadIdx.x < npairs ? hv[threadIdx.x] : 0.f, n, ys, a.hd + (int64_t)(f0 / D::NV) * D::NPL,
                       a.hsc + f0 / D::NV);
}

// One wave, NRW output rows [i0, i0 + NRW) of a row-major H x F down matrix
// Dm (lane groups of L lanes, NR = NRW / (64 / L) rows each), against h digit
// planes (hd, hsc: the pair's group 0).  Writer lanes store row i0 + j's value
// (times its row scale when ds != nullptr) to out[j]; rows past H are not
// written.  kCoh: h was written, and out is read, by other workgroups of the
// same launch.
template <int FMT, int L, int CPL, int NRW, bool kCoh = false>
MD_DEV void dn_rows(const uint8_t* Dm, const float* ds, int H, int F, const u32x4* hd, const float* hsc, int i0,
                    float* out, const ActDig<FMT, CPL>* pre = nullptr) {
  constexpr int G = 64 / L, NR = NRW / G;
  static_assert(NRW % G == 0 && NR <= L, "rows per wave");
  const int lane = threadIdx.x & 63;
  const int g = lane / L, t = lane % L;
  ActDig<FMT, CPL> ha;
  if (pre) ha = *pre;
  else load_act<FMT, L, CPL, kCoh>(ha, hd, hsc, t);
  const int ib = i0 + g * NR;
  const int64_t rb = row_bytes(FMT, F);
  float part[NR];
  {
    // rolling window: kD rows in flight while one row is decoded
    constexpr int kD = NR < MD_DN_WINDOW ? NR : MD_DN_WINDOW;
    RowBuf<FMT, CPL> b[kD];
    DigAcc<FMT> ra;
    auto rowp = [&](int r) { return Dm + (int64_t)min(ib + r, H - 1) * rb; };
#pragma unroll
    for (int r = 0; r < kD; ++r) load_row<FMT, L, CPL>(b[r], rowp(r), F, t);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      part[r] = row_dot<FMT, CPL>(b[r % kD], ha, ra);
      if (r + kD < NR) load_row<FMT, L, CPL>(b[r % kD], rowp(r + kD), F, t);
    }
  }
  const float s = butterfly<NR, L>(part, t);
  const int r = (t / (L / NR)) % NR;
  const int i = ib + r;
  if ((t % (L / NR)) == 0 && i < H) put<kCoh>(out + g * NR + r, ds ? s * ds[i] : s);
}

}  // namespace md
