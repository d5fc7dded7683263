// fused.hip -- the MoE layer for a few tokens after the router, as one
// persistent kernel (gfx950, wave64).
//
// The work is cut into tiles that workgroups take in ticket order from one
// atomic counter:
//   gate/up tiles  (pair, rows of F): the gate/up tile body of the one-token
//                  kernels (x digit planes in registers, 16-byte row streaming,
//                  h written as digit planes); then the pair's counter rises.
//   down tiles     (pair, 96 output rows): each wave streams 8 rows of the
//                  pair's expert against h's digit planes into o[pair][row].
//                  The tile that completes a (token, row block) over all of
//                  the token's pairs adds them in slot order with the gates
//                  (then the shared expert's rows) into y.
// A pair is a token's routed slot j (pairs t*k + j) or its shared expert
// (pairs T*k + t).  All gate/up tickets come before any down ticket, so a
// down tile only waits (bounded spin) for gate/up tiles that running
// workgroups already hold and that wait on nothing: progress never depends on
// how many workgroups are resident.  Each workgroup forms the top-k of the
// call's tokens once from the router's partials while its first ticket is in
// flight.  Data handed between workgroups (h planes, o) is written with
// agent-scope atomic stores; each wave waits for its stores to complete
// before the barrier that precedes the counter update, and readers load it
// with agent-scope atomic loads after the barrier that follows the wait.
// (Full agent-scope fences would write back and invalidate the L2 each time,
// which costs far more than the tiles themselves.)
#include "common.hpp"
#include "digits.hpp"
#include "kernels.hpp"
#include "rows.hpp"

namespace md {

constexpr int kFW = 12;            // waves per workgroup
constexpr int kFRW = 8;            // down rows per wave in a down tile
constexpr int kFDR = kFW * kFRW;   // down rows per tile
constexpr int kFLds = 1024;        // LDS floats for a gate/up tile (h values + slice sums)

// Lane geometry of one expert format: gate/up lane groups of LG lanes, NPG
// row pairs per lane group and tile; down lane groups of LD lanes with CPLD
// chunks per lane.
template <int FMT_, int LG_, int NPG_, int LD_, int CPLD_>
struct XCfg {
  static constexpr int FMT = FMT_, LG = LG_, NPG = NPG_, LD = LD_, CPLD = CPLD_;
};
struct NoShared {
  static constexpr int FMT = 0;
};

struct FusedExp {
  const uint8_t* gq;      // gate matrices (one per expert, gu_bytes apart)
  const uint8_t* uq;
  const uint8_t* dq;      // down matrices (dn_bytes apart)
  const float* gs;        // row scales (per-row formats) or nullptr
  const float* us;
  const float* ds;
  int64_t gu_bytes, dn_bytes;
  int F, act, KS, RGW, rows;   // gate/up geometry; rows per gate/up tile
  int nG;                      // gate/up tiles per pair
  const u32x4* xd;             // x digit planes [T][H/NV][NPL], scales [T][H/NV]
  const float* xsc;
  u32x4* hd;                   // h digit planes [pairs][F/NV][NPL], scales
  float* hsc;
};

struct FusedArgs {
  FusedExp r, s;               // routed experts, shared expert (s.gq == nullptr: none)
  int H, E, k, T;
  const double* part;          // router partials [T][E][S]
  int S;
  const float* bias;
  float* o;                    // [T*k + T][H] per-pair down outputs
  float* y;                    // [T][H]
  int* idx_out;                // [T][k]
  float* gates_out;
  int* ctr;                    // [0] tickets, [1] unused, [2 ..) gate/up done per pair, then [T][nD] row blocks done
  int nD;                      // down tiles per pair
  int nG, nTot;                // gate/up tiles in all, tiles in all
};

MD_DEV float ld_coh(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Every memory operation of this wave issued so far has completed.
MD_DEV void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until *p >= target; false after about a second (2^20 polls).
MD_DEV bool spin_until(const int* p, int target) {
  for (int it = 0; it < (1 << 20); ++it) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// e: expert; t: token (x planes); hq: the pair's index in x.hd (routed: t*k + j,
// shared: t)
template <class X>
MD_DEV GuTile gu_args(const FusedExp& x, int e, int t, int hq, int H) {
  using D = Dig<X::FMT>;
  const int ngx = H / D::NV, ngh = x.F / D::NV;
  return GuTile{x.gq + (int64_t)e * x.gu_bytes, x.uq + (int64_t)e * x.gu_bytes,
                x.gs ? x.gs + (int64_t)e * x.F : nullptr, x.us ? x.us + (int64_t)e * x.F : nullptr,
                x.F, H, x.act, x.KS, x.RGW,
                x.xd + (int64_t)t * ngx * D::NPL, x.xsc + (int64_t)t * ngx,
                x.hd + (int64_t)hq * ngh * D::NPL, x.hsc + (int64_t)hq * ngh};
}

template <class X>
MD_DEV void dn_wave(const FusedExp& x, int e, int hq, int H, int i0, float* out) {
  using D = Dig<X::FMT>;
  const int ngh = x.F / D::NV;
  dn_rows<X::FMT, X::LD, X::CPLD, kFRW, true>(x.dq + (int64_t)e * x.dn_bytes, x.ds ? x.ds + (int64_t)e * H : nullptr, H, x.F,
                                       x.hd + (int64_t)hq * ngh * D::NPL, x.hsc + (int64_t)hq * ngh, i0, out);
}

template <class R, class SH>
__global__ __launch_bounds__(kFW * 64) void k_moe_fused(FusedArgs a) {
  __shared__ float lds[kFLds];
  __shared__ uint32_t ys[256];
  __shared__ int s_sel[8][8];
  __shared__ float s_gate[8][8];
  __shared__ int s_tk, s_last, s_fail;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nr = a.T * a.k;
  if (threadIdx.x == 0) {
    s_tk = atomicAdd(a.ctr, 1);
    s_fail = 0;
  }
  // the top-k of every token (wave t: token t)
  if (wave < a.T) {
    int sel[8];
    float gts[8];
    wave_topk(a.part + (int64_t)wave * a.E * a.S, a.S, a.bias, a.E, a.k, lane, sel, gts, true);
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < a.k) {
          s_sel[wave][j] = sel[j];
          s_gate[wave][j] = gts[j];
          if (blockIdx.x == 0) {
            a.idx_out[wave * a.k + j] = sel[j];
            a.gates_out[wave * a.k + j] = gts[j];
          }
        }
      }
    }
  }
  __syncthreads();
  int tk = s_tk;
  __syncthreads();
  while (tk < a.nTot) {
    int nxt = 0;
    if (threadIdx.x == 0) nxt = atomicAdd(a.ctr, 1);  // the next ticket, in flight during this tile
    if (tk < a.nG) {
      // ---- gate/up tile
      int q;
      if (tk < nr * a.r.nG) {
        q = tk / a.r.nG;
        const int ti = tk % a.r.nG, t = q / a.k;
        const GuTile u = gu_args<R>(a.r, s_sel[t][q % a.k], t, q, a.H);
        gu_tile<R::FMT, R::LG, R::NPG, true>(u, ti * a.r.rows, lds, ys);
      } else {
        if constexpr (SH::FMT != 0) {
          const int rr = tk - nr * a.r.nG, t = rr / a.s.nG, ti = rr % a.s.nG;
          q = nr + t;
          const GuTile u = gu_args<SH>(a.s, 0, t, t, a.H);
          gu_tile<SH::FMT, SH::LG, SH::NPG, true>(u, ti * a.s.rows, lds, ys);
        } else {
          q = 0;  // unreachable: no shared tiles are counted
        }
      }
      drain();
      __syncthreads();
      if (threadIdx.x == 0) atomicAdd(a.ctr + 2 + q, 1);
    } else {
      // ---- down tile
      const int d = tk - a.nG, q = d / a.nD, ti = d % a.nD;
      const bool sh = q >= nr;
      const int t = sh ? q - nr : q / a.k;
      if (threadIdx.x == 0 && !spin_until(a.ctr + 2 + q, sh ? a.s.nG : a.r.nG)) s_fail = 1;
      __syncthreads();
      const int i0 = ti * kFDR + wave * kFRW;
      if (i0 < a.H) {
        float* out = a.o + (int64_t)q * a.H + i0;
        if (!sh) {
          dn_wave<R>(a.r, s_sel[t][q % a.k], q, a.H, i0, out);
        } else {
          if constexpr (SH::FMT != 0) dn_wave<SH>(a.s, 0, t, a.H, i0, out);
        }
      }
      drain();
      __syncthreads();
      if (threadIdx.x == 0) {
        const int nslots = a.k + (a.s.gq ? 1 : 0);
        const int old = atomicAdd(a.ctr + 2 + nr + a.T + t * a.nD + ti, 1);
        s_last = old == nslots - 1;
      }
      __syncthreads();
      if (s_last) {
        for (int rr = threadIdx.x; rr < kFDR; rr += blockDim.x) {
          const int i = ti * kFDR + rr;
          if (i < a.H) {
            float v = 0.f;
            for (int j = 0; j < a.k; ++j) v = fmaf(s_gate[t][j], ld_coh(a.o + (int64_t)(t * a.k + j) * a.H + i), v);
            if (a.s.gq) v += ld_coh(a.o + (int64_t)(nr + t) * a.H + i);
            a.y[(int64_t)t * a.H + i] = s_fail ? __builtin_nanf("") : v;
          }
        }
      }
    }
    if (threadIdx.x == 0) s_tk = nxt;
    __syncthreads();
    tk = s_tk;
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launch

static int pow2_lanes(int n) {
  int L = 64;
  while (L > 1 && n % L) L >>= 1;
  return L;
}

// Geometry of one expert format in the fused kernel; false if the shapes do
// not fit (then the caller uses the separate one-token kernels).
struct FGeom {
  int LG, G, KS, RGW, NPG, rows, LD, CPLD;
};
static bool fused_geom(int fmt, int H, int F, FGeom& g) {
  const int ncg = nchunks(fmt, H), ncd = nchunks(fmt, F);
  g.LG = pow2_lanes(ncg);
  g.LD = pow2_lanes(ncd);
  if (g.LG < 8 || g.LD < 8) return false;
  g.G = 64 / g.LG;
  g.KS = ncg / g.LG;
  if (kFW % g.KS) return false;
  g.RGW = kFW / g.KS;
  const int NV = dig_nv(fmt);
  g.NPG = 0;
  for (int np = 1; np <= 8; np *= 2)
    if ((g.RGW * g.G * np) % NV == 0) { g.NPG = np; break; }
  if (!g.NPG) return false;
  g.rows = g.RGW * g.G * g.NPG;
  if (g.rows > 256 || g.rows * (1 + (g.KS > 1 ? 2 * g.KS : 0)) > kFLds) return false;
  g.CPLD = ncd / g.LD;
  return g.CPLD >= 1 && g.CPLD <= 3;
}

template <class R, class SH>
static hipError_t launch_cfg(const FusedArgs& a, hipStream_t st) {
  static int per_cu = 0;
  if (!per_cu) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_moe_fused<R, SH>, kFW * 64, 0) != hipSuccess || n < 1) n = 1;
    per_cu = n;
  }
  int grid = device_cus() * per_cu;
  if (grid > a.nTot) grid = a.nTot;
  hipLaunchKernelGGL((k_moe_fused<R, SH>), dim3(grid), dim3(kFW * 64), 0, st, a);
  return hipGetLastError();
}

// The instantiated shapes: 4-bit or 8-bit per-row experts with hidden width
// a multiple of 64 chunks and FFN width 2048; Q4_0 experts of width 768 with
// a Q8_0 shared expert of width 2048 (hidden 2048); small Q8_0 layers.
using CfgI4 = XCfg<I4_ROW, 64, 8, 64, 1>;
using CfgI8 = XCfg<I8_ROW, 64, 8, 64, 2>;
using CfgQ4n = XCfg<Q4_0, 64, 8, 8, 3>;
using CfgQ8s = XCfg<Q8_0, 64, 8, 64, 2>;
using CfgQ8t = XCfg<Q8_0, 16, 1, 32, 1>;

template <class X>
static bool matches(int fmt, const FGeom& g) {
  return fmt == X::FMT && g.LG == X::LG && g.NPG == X::NPG && g.LD == X::LD && g.CPLD == X::CPLD;
}

// Fills the geometry fields of a.r / a.s and the tile counts; false if no
// instantiation covers the shapes.
static int pick(FusedArgs& a, int fmt, int sfmt, bool has_shared) {
  FGeom gr{}, gs{};
  if (!fused_geom(fmt, a.H, a.r.F, gr)) return -1;
  if (has_shared && !fused_geom(sfmt, a.H, a.s.F, gs)) return -1;
  int id = -1;
  if (!has_shared) {
    if (matches<CfgI4>(fmt, gr)) id = 0;
    else if (matches<CfgI8>(fmt, gr)) id = 1;
    else if (matches<CfgQ8t>(fmt, gr)) id = 2;
  } else if (matches<CfgQ4n>(fmt, gr) && matches<CfgQ8s>(sfmt, gs)) {
    id = 3;
  }
  if (id < 0) return -1;
  a.r.KS = gr.KS; a.r.RGW = gr.RGW; a.r.rows = gr.rows; a.r.nG = (a.r.F + gr.rows - 1) / gr.rows;
  if (has_shared) {
    a.s.KS = gs.KS; a.s.RGW = gs.RGW; a.s.rows = gs.rows; a.s.nG = (a.s.F + gs.rows - 1) / gs.rows;
  } else {
    a.s.nG = 0;
  }
  a.nD = (a.H + kFDR - 1) / kFDR;
  const int pairs = a.T * a.k + (has_shared ? a.T : 0);
  a.nG = a.T * a.k * a.r.nG + (has_shared ? a.T * a.s.nG : 0);
  a.nTot = a.nG + pairs * a.nD;
  return id;
}

bool fused_supported(int fmt, int H, int F, int sfmt, int Fs, bool has_shared) {
  FusedArgs a{};
  a.H = H; a.r.F = F; a.s.F = Fs; a.T = 1; a.k = 1;
  return pick(a, fmt, sfmt, has_shared) >= 0;
}

int fused_counter_words(int T, int k, int H) {
  return 2 + T * (k + 1) + T * ((H + kFDR - 1) / kFDR);
}

hipError_t launch_moe_fused(const FusedLaunch& L, hipStream_t st) {
  FusedArgs a{};
  a.r = FusedExp{L.gq, L.uq, L.dq, L.gs, L.us, L.ds, L.gu_bytes, L.dn_bytes, L.F, L.act, 0, 0, 0, 0,
                 static_cast<const u32x4*>(L.xd), L.xsc, static_cast<u32x4*>(L.hd), L.hsc};
  a.s = FusedExp{L.sgq, L.suq, L.sdq, L.sgs, L.sus, L.sds, 0, 0, L.Fs, L.sact, 0, 0, 0, 0,
                 static_cast<const u32x4*>(L.sxd), L.sxsc, static_cast<u32x4*>(L.shd), L.shsc};
  a.H = L.H; a.E = L.E; a.k = L.k; a.T = L.T;
  a.part = L.part; a.S = L.S; a.bias = L.bias;
  a.o = L.o; a.y = L.y; a.idx_out = L.idx_out; a.gates_out = L.gates_out; a.ctr = L.ctr;
  const bool has_shared = L.sgq != nullptr;
  if (L.T < 1 || L.T > 8 || L.k < 1 || L.k > 8) return hipErrorInvalidValue;
  switch (pick(a, L.fmt, L.sfmt, has_shared)) {
    case 0: return launch_cfg<CfgI4, NoShared>(a, st);
    case 1: return launch_cfg<CfgI8, NoShared>(a, st);
    case 2: return launch_cfg<CfgQ8t, NoShared>(a, st);
    case 3: return launch_cfg<CfgQ4n, CfgQ8s>(a, st);
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace md
