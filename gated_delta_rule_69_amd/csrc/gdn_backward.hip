// Backward pass of the token recurrence (reverse mode), every variant: FG2, FG2+, KDA,
// GDN, ASYM, and DeltaProduct as its sequence of Householder sub-steps.
//
// Per step, with X = Diag(alpha) S_{t-1}, u = w - X^T b, S_t = X + a u^T,
// o_t = S_t^T q_t and G = dL/dS_t (the later steps' gradient plus q_t do_t^T):
//   dq = S_t do,  dw = G^T a,  da = G u,  db = -X dw,  dX = G - b dw^T,
//   dalpha = rowsum(dX . S_{t-1}),  dL/dS_{t-1} = Diag(alpha) dX,
// then the chain rule through the variant's (a, b, w, alpha) map (FG2-GDN reading
// notes, section 2.2 eq. (11) and section 2.3 eq. (13); GDN2-stability page, eq. (1)).
//
// Only two things are sequential: the state S runs forward, and the state gradient
// runs backward as G <- Diag(alpha) (I - b a^T) G + q do^T, which does not involve S.
// So the pass is split into:
//  1. the operand kernel: every step's a, b, alpha, q rows and w, do columns, once,
//     in float32 (the later kernels do not branch on the variant);
//  2. the chain kernel: the S and G recursions side by side, in separate waves, each
//     over narrow column slices; S is stored at the start and G at the end of every
//     64-step interval;
//  3. the interval kernel: every (batch*head, 16-column slice, interval) on its own.
//     It recomputes the interval's states from the stored S (keeping one state in
//     four in a per-workgroup scratch slot, and four states at a time in registers)
//     and walks the interval backwards from the stored G, writing the slice's row
//     partials and the column-complete dw;
//  4. the reduce kernel: slices summed in a fixed order, then the variant's chain rule.
// Every sum runs in a fixed order: the results are deterministic.
//
// Lane layout of the chain and interval kernels (rows on lanes): lane l owns state
// rows l*NR .. l*NR+NR-1 (NR = max(dk / 64, 1); lanes past dk hold zeros) and all CW
// columns of its slice in registers. Sums over a slice's columns stay inside a lane;
// sums over rows are wave reductions: a transposing butterfly over the lane bits
// below CW (each exchange halves the values a lane carries, DPP within 16-lane rows)
// and then plain pair sums over the remaining lane bits, which leaves the total of
// column bitrev(l mod CW) in lane l; a DPP move (quad_perm or row_newbcast) then gives
// every lane any column's total.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCB = 64;        // steps per checkpoint interval
constexpr int kSub = 4;        // steps whose states the interval kernel holds in registers
constexpr int kCW = 16;        // columns of an interval-kernel wave (a row-partial slice)
constexpr int kChainCW = 4;    // columns of a chain-kernel wave
constexpr int kChainRing = 16; // steps of operands a chain wave keeps in flight
constexpr int kSlots = 1024;   // interval-kernel waves, each with a scratch slot
constexpr int kPad = kChainRing;  // operand padding (steps) before and after a sequence
static_assert(kSub <= kPad, "an interval block reads at most kSub - 1 steps past the end");

__host__ __device__ constexpr int rows_per_lane(int64_t dk) { return dk >= 64 ? int(dk / 64) : 1; }
// Column slices an interval-kernel workgroup takes (one wave each): their row partials
// are summed in LDS, so the workspace holds one partial set per group of slices.
__host__ __device__ constexpr int slices_per_group(int64_t dv) { return dv >= 64 ? 4 : int(dv / kCW); }

// Workspace (float offsets). T counts steps here (tokens x n_h for DeltaProduct).
//   rows [B*H][kPad + steps + kPad][4][dk]   a, b, alpha, q      (kPad steps of padding on
//   cols [B*H][kPad + steps + kPad][2][dv]   w, do                both sides, never used)
//   ck   [B*H][intervals][dk][dv]   S before the interval's first step
//   gk   [B*H][intervals][dk][dv]   dL/dS after the interval's last step
//   sub  [waves][kCB / kSub][NR * kCW / 4][64 lanes] float4   interval-kernel states
//   part [slice groups][B*H][steps][4][dk]   dq, da, db, dalpha partials per group
//   dw   [B*H][steps][dv]
struct BwdLayout {
  int64_t rows, cols, ck, gk, sub, part, dw, total;
  int64_t nck, items, slots;
};

__host__ __device__ inline BwdLayout bwd_layout(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  BwdLayout L;
  const int64_t bh = B * H;
  const int64_t bth = B * T * H;
  L.nck = (T + kCB - 1) / kCB;
  const int64_t wpg = slices_per_group(dv), groups = dv / kCW / wpg;
  L.items = bh * groups * L.nck;  // interval-kernel workgroup items
  L.slots = L.items < kSlots / wpg ? L.items : kSlots / wpg;  // its workgroups
  const int64_t bsp = bh * (T + 2 * kPad);  // padded steps
  L.rows = 0;
  L.cols = L.rows + bsp * 4 * dk;
  L.ck = L.cols + bsp * 2 * dv;
  L.gk = L.ck + bh * L.nck * dk * dv;
  L.sub = L.gk + bh * L.nck * dk * dv;
  L.part = L.sub + L.slots * wpg * (kCB / kSub) * 64 * rows_per_lane(dk) * kCW;
  L.dw = L.part + groups * bth * 4 * dk;
  L.total = L.dw + bth * dv;
  if (L.total < 64) L.total = 64;  // a valid empty problem still reports a nonzero size
  return L;
}

// ---- wave reductions in the rows-on-lanes layout ------------------------------------

// The value lane l ^ M holds (M < 16: DPP inside 16-lane rows).
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  const int v = __float_as_int(x);
  // (bound_ctrl set where every lane has a source: lets the move fuse into its add)
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, true));  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, true));  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    // lanes 0-3 and 8-11 of a row (banks 0, 2) read lane + 4 (row_shl:4), lanes
    // 4-7 and 12-15 (banks 1, 3) read lane - 4 (row_shr:4)
    int r = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xf, 0x5, false);
    r = __builtin_amdgcn_update_dpp(r, v, 0x114, 0xf, 0xa, false);
    return __int_as_float(r);
  } else {
    static_assert(M == 8, "lane_xor: M is 1, 2, 4 or 8");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, true));  // row_ror:8
  }
}

// x + (x of lane l ^ M), the same bits in both lanes of the pair.
template <int M>
__device__ __forceinline__ float pair_sum(float x) {
  if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  } else if constexpr (M == 32) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  } else {
    return x + lane_xor<M>(x);
  }
}

// One transposing level: a lane with bit M clear keeps the lower half of its n = CW / M
// values and adds the partner's lower half; a lane with bit M set keeps the upper half.
template <int M, int CW>
__device__ __forceinline__ void transpose_level(float (&v)[CW], int lane) {
  constexpr int n = CW / M;
  const bool hi = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < n / 2; ++i) {
    const float lo = v[i], up = v[i + n / 2];
    const float keep = hi ? up : lo;
    const float send = hi ? lo : up;
    v[i] = keep + lane_xor<M>(send);
  }
}

// Column sums over the 64 lanes of v[CW] (each lane's partials of CW columns).
// Returns in lane l the total of column col_lane<CW>(l mod CW); v is consumed.
template <int CW>
__device__ __forceinline__ float col_sum(float (&v)[CW], int lane) {
  static_assert(CW == 2 || CW == 4 || CW == 8 || CW == 16, "col_sum: CW is 2, 4, 8 or 16");
  transpose_level<1, CW>(v, lane);
  if constexpr (CW > 2) transpose_level<2, CW>(v, lane);
  if constexpr (CW > 4) transpose_level<4, CW>(v, lane);
  if constexpr (CW > 8) transpose_level<8, CW>(v, lane);
  float x = v[0];
  if constexpr (CW <= 2) x = pair_sum<2>(x);
  if constexpr (CW <= 4) x = pair_sum<4>(x);
  if constexpr (CW <= 8) x = pair_sum<8>(x);
  x = pair_sum<16>(x);
  return pair_sum<32>(x);
}

// Bit reversal over log2(CW) bits: the column whose total col_sum leaves in lane
// l (l < CW), and, being an involution, the lane that holds column c.
template <int CW>
__host__ __device__ constexpr int col_lane(int c) {
  int r = 0;
  for (int b = 1, rb = CW / 2; b < CW; b <<= 1, rb >>= 1)
    if (c & b) r |= rb;
  return r;
}

// The total of column c in every lane, after col_sum: DPP from the lane holding it in
// the lane's own quad (CW <= 4, quad_perm) or 16-lane row (row_newbcast). c must fold
// to a constant (unrolled loops), so that the switch leaves one DPP move.
#define GDN_BCAST_CASE(n, ctrl) \
  case n:                      \
    return __int_as_float(__builtin_amdgcn_update_dpp(0, v, ctrl, 0xf, 0xf, true));
template <int CW>
__device__ __forceinline__ float col_bcast(float x, int c) {
  const int v = __float_as_int(x);
  if constexpr (CW <= 4) {
    switch (col_lane<CW>(c)) {
      GDN_BCAST_CASE(0, 0x00) GDN_BCAST_CASE(1, 0x55) GDN_BCAST_CASE(2, 0xaa) GDN_BCAST_CASE(3, 0xff)
    }
  } else {
    switch (col_lane<CW>(c)) {
      GDN_BCAST_CASE(0, 0x150) GDN_BCAST_CASE(1, 0x151) GDN_BCAST_CASE(2, 0x152) GDN_BCAST_CASE(3, 0x153)
      GDN_BCAST_CASE(4, 0x154) GDN_BCAST_CASE(5, 0x155) GDN_BCAST_CASE(6, 0x156) GDN_BCAST_CASE(7, 0x157)
      GDN_BCAST_CASE(8, 0x158) GDN_BCAST_CASE(9, 0x159) GDN_BCAST_CASE(10, 0x15a) GDN_BCAST_CASE(11, 0x15b)
      GDN_BCAST_CASE(12, 0x15c) GDN_BCAST_CASE(13, 0x15d) GDN_BCAST_CASE(14, 0x15e) GDN_BCAST_CASE(15, 0x15f)
    }
  }
  return 0.0f;
}
#undef GDN_BCAST_CASE

// ---- 1. operand kernel -------------------------------------------------------------
// One wave per (batch*head, step): rows a, b, alpha, q and columns w, do in float32.
// q and do act after a token's last step (DeltaProduct: zero for the earlier steps),
// the gate at its first.
template <typename In>
__global__ __launch_bounds__(256) void bwd_ops_kernel(Problem p, const In* __restrict__ d_o,
                                                      float* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const int64_t NS = p.steps, T = p.T, H = p.H, DK = p.dk, dv = p.dv;
  const int nh = p.n_h;
  const BwdLayout L = bwd_layout(p.B, NS, H, DK, dv);
  const int64_t x = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // bh * NS + s
  if (x >= p.B * H * NS) return;
  const int64_t bh = x / NS, s = x % NS;
  const int64_t b = bh / H, h = bh % H;
  const int64_t t = s / nh;
  const int sub = int(s - t * nh);
  const int64_t th = (b * T + t) * H + h;  // token-head
  const int64_t sr = th * nh + sub;        // step row ([B, T, H, n_h] for DeltaProduct)
  const bool last = sub == nh - 1;
  const In* q = static_cast<const In*>(p.q);
  const In* k = static_cast<const In*>(p.k);
  const In* v = static_cast<const In*>(p.v);
  const In* al = static_cast<const In*>(p.alpha);
  const In* be = static_cast<const In*>(p.beta);
  const In* bev = static_cast<const In*>(p.beta_v);
  const In* jv = static_cast<const In*>(p.j);
  const In* et = static_cast<const In*>(p.eta);
  auto ld = [](const In* y) { return IO<In>::ld(y); };
  const int64_t xp = bh * (NS + 2 * kPad) + kPad + s;
  float* rw = ws + L.rows + xp * 4 * DK;
  float* cl = ws + L.cols + xp * 2 * dv;
  const int var = p.variant;
  // per-step scalars
  float sc = 0.0f, gate = 1.0f;
  if (var == GDN_VARIANT_DELTAPRODUCT) {
    sc = ld(be + sr);
    gate = sub == 0 ? ld(al + th) : 1.0f;
  } else if (var == GDN_VARIANT_ASYM) {
    sc = ld(et + th);
  } else if (var == GDN_VARIANT_KDA || var == GDN_VARIANT_GDN) {
    sc = sqrtf(ld(be + th));
    if (var == GDN_VARIANT_GDN) gate = ld(al + th);
  }
  for (int64_t e = lane; e < DK; e += 64) {
    const float kr = ld(k + sr * DK + e);
    float a, bb, alpha;
    if (var == GDN_VARIANT_DELTAPRODUCT) {
      a = kr, bb = sc * kr, alpha = gate;
    } else if (var == GDN_VARIANT_ASYM) {
      a = kr, bb = ld(jv + th * DK + e) * sc, alpha = ld(al + th * DK + e);
    } else if (var == GDN_VARIANT_FG2) {
      a = kr * sqrtf(ld(be + th * DK + e)), bb = a, alpha = ld(al + th * DK + e);
    } else {
      a = kr * sc, bb = a, alpha = var == GDN_VARIANT_KDA ? ld(al + th * DK + e) : gate;
    }
    rw[e] = a;
    rw[DK + e] = bb;
    rw[2 * DK + e] = alpha;
    rw[3 * DK + e] = last ? ld(q + th * DK + e) : 0.0f;
  }
  for (int64_t c = lane; c < dv; c += 64) {
    const float vc = ld(v + sr * dv + c);
    float w;
    if (var == GDN_VARIANT_FG2) w = vc * sqrtf(ld(bev ? bev + th * dv + c : be + th * DK + c));
    else w = sc * vc;
    cl[c] = w;
    cl[dv + c] = last ? ld(d_o + th * dv + c) : 0.0f;
  }
}

// One step's operands in the rows-on-lanes layout: this lane's rows of a, b, alpha
// (and q), and one column value (w or do of column col_lane(l mod CW)).
template <int NR>
struct Op {
  float a[NR], b[NR], al[NR], q[NR];
  float w, d;
};

// Inactive lanes (rows past dk) read row 0 and keep zeros.
template <int NR, bool WQ, bool WW, bool WD>
__device__ __forceinline__ void load_op(const float* rows, const float* cols, int64_t s, int64_t DK,
                                        int64_t dv, int r0, bool act, int col, Op<NR>& o) {
  const float* rw = rows + s * 4 * DK + (act ? r0 : 0);
  float a[NR], b[NR], al[NR], q[NR];
  if constexpr (NR == 2) {
    const float2 x = *reinterpret_cast<const float2*>(rw);
    const float2 y = *reinterpret_cast<const float2*>(rw + DK);
    const float2 z = *reinterpret_cast<const float2*>(rw + 2 * DK);
    a[0] = x.x, a[1] = x.y, b[0] = y.x, b[1] = y.y, al[0] = z.x, al[1] = z.y;
    if constexpr (WQ) {
      const float2 w = *reinterpret_cast<const float2*>(rw + 3 * DK);
      q[0] = w.x, q[1] = w.y;
    }
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      a[r] = rw[r], b[r] = rw[DK + r], al[r] = rw[2 * DK + r];
      if constexpr (WQ) q[r] = rw[3 * DK + r];
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    o.a[r] = act ? a[r] : 0.0f;
    o.b[r] = act ? b[r] : 0.0f;
    o.al[r] = act ? al[r] : 0.0f;
    o.q[r] = WQ && act ? q[r] : 0.0f;
  }
  const float* cl = cols + s * 2 * dv + col;
  o.w = WW ? cl[0] : 0.0f;
  o.d = WD ? cl[dv] : 0.0f;
}

// S <- X + a u^T with X = Diag(alpha) S, u = w - X^T b (a forward step). Returns u of
// column col_lane(l mod CW).
template <int NR, int CW>
__device__ __forceinline__ float fwd_step(float (&S)[NR][CW], const Op<NR>& o, int lane) {
  float part[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) part[c] = 0.0f;
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      S[r][c] *= o.al[r];
      part[c] += o.b[r] * S[r][c];
    }
  const float u = o.w - col_sum<CW>(part, lane);
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const float uc = col_bcast<CW>(u, c);
#pragma unroll
    for (int r = 0; r < NR; ++r) S[r][c] += o.a[r] * uc;
  }
  return u;
}

// G <- Diag(alpha) (G' - b dw^T), G' = G + q do^T, dw = G'^T a (a backward step of the
// state gradient alone).
template <int NR, int CW>
__device__ __forceinline__ void grad_step(float (&G)[NR][CW], const Op<NR>& o, int lane) {
  float part[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const float dc = col_bcast<CW>(o.d, c);
    part[c] = 0.0f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      G[r][c] += o.q[r] * dc;
      part[c] += G[r][c] * o.a[r];
    }
  }
  const float dw = col_sum<CW>(part, lane);
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const float dwc = col_bcast<CW>(dw, c);
#pragma unroll
    for (int r = 0; r < NR; ++r) G[r][c] = o.al[r] * (G[r][c] - o.b[r] * dwc);
  }
}

// ---- 2. chain kernel ----------------------------------------------------------------
// Four waves per workgroup, one per CW-column slice; the first B*H*dv/CW waves run S
// forward from s0, the rest run the state gradient backward from dL/dS_T.
template <int DK, int CW>
__global__ __launch_bounds__(256) void bwd_chain_kernel(Problem p, const float* __restrict__ dsf,
                                                        float* __restrict__ ds0, float* __restrict__ ws) {
  constexpr int NR = rows_per_lane(DK);
  constexpr int D = kChainRing;
  const int lane = threadIdx.x & 63;
  const int64_t NS = p.steps, H = p.H, dv = p.dv;
  const BwdLayout L = bwd_layout(p.B, NS, H, DK, dv);
  const int ncs = int(dv / CW);
  const int64_t nw = p.B * H * ncs;  // waves per chain
  const int64_t wid = int64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool grad = wid >= nw;
  const int64_t w2 = grad ? wid - nw : wid;
  const int64_t bh = w2 / ncs;
  const int cbase = int(w2 % ncs) * CW;
  const int r0 = lane * NR;
  const bool act = DK >= 64 || r0 < DK;
  const int col = cbase + col_lane<CW>(lane & (CW - 1));
  // step s of this head at rows + s * 4 dk (s in [-kPad, NS + kPad))
  const float* rows = ws + L.rows + (bh * (NS + 2 * kPad) + kPad) * 4 * DK;
  const float* cols = ws + L.cols + (bh * (NS + 2 * kPad) + kPad) * 2 * dv;
  const size_t sbase = size_t(bh) * DK * size_t(dv);
  float* ckp = ws + (grad ? L.gk : L.ck) + bh * L.nck * DK * dv;
  const float* init = grad ? dsf : p.s0;

  float X[NR][CW];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int c = 0; c < CW; ++c)
      X[r][c] = (act && init) ? init[sbase + size_t(r0 + r) * dv + cbase + c] : 0.0f;
  auto store = [&](float* dst) __attribute__((always_inline)) {
    if (!act) return;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float* d = dst + size_t(r0 + r) * dv + cbase;
      if constexpr (CW % 4 == 0) {
#pragma unroll
        for (int c = 0; c < CW; c += 4)
          *reinterpret_cast<float4*>(d + c) = make_float4(X[r][c], X[r][c + 1], X[r][c + 2], X[r][c + 3]);
      } else {
#pragma unroll
        for (int c = 0; c < CW; ++c) d[c] = X[r][c];
      }
    }
  };

  // Operands of the next D steps stay in flight in a register ring. The steady state
  // runs whole groups of D steps aligned to multiples of D (kCB is one), so its loads
  // are unconditional and each step waits only for its own slot; the ragged end
  // (fewer than D steps) runs separately.
  static_assert(kCB % D == 0, "checkpoint interval is a multiple of the ring depth");
  if (NS == 0) {  // nothing to run: dL/dS_0 is dL/dS_T
    if (grad && ds0) store(ds0 + sbase);
    return;
  }
  Op<NR> ring[D];
  const int64_t nfull = NS / D;  // whole groups [D g, D g + D)
  const int64_t tail0 = nfull * D;
  if (!grad) {
#pragma unroll
    for (int i = 0; i < D; ++i) {  // in slot order, as the loop refills them
      load_op<NR, false, true, false>(rows, cols, i, DK, dv, r0, act, col, ring[i]);
      asm volatile("" ::: "memory");
    }
    for (int64_t g = 0; g < nfull; ++g) {
      const int64_t s0 = g * D;
      if (s0 % kCB == 0) store(ckp + (s0 / kCB) * DK * dv);
      // opaque to the optimizer, which would otherwise turn the refills back into
      // loads at the point of use (the next group's addresses are the same)
      int64_t nb = s0 + D;
      asm volatile("" : "+s"(nb));
#pragma unroll
      for (int i = 0; i < D; ++i) {
        fwd_step<NR, CW>(X, ring[i], lane);
        load_op<NR, false, true, false>(rows, cols, nb + i, DK, dv, r0, act, col, ring[i]);
        __builtin_amdgcn_sched_barrier(0);  // keep the refill here, D steps ahead of its use
      }
    }
#pragma unroll
    for (int i = 0; i < D; ++i) {  // the ring holds steps tail0 .. tail0 + D - 1
      const int64_t s = tail0 + i;
      if (s < NS) {
        if (s % kCB == 0) store(ckp + (s / kCB) * DK * dv);
        fwd_step<NR, CW>(X, ring[i], lane);
      }
    }
    return;
  }
  // the ragged end first (steps NS - 1 down to tail0), loading as it goes
  for (int64_t s = NS - 1; s >= tail0; --s) {
    Op<NR> o;
    load_op<NR, true, false, true>(rows, cols, s, DK, dv, r0, act, col, o);
    if (s == NS - 1 || (s + 1) % kCB == 0) store(ckp + (s / kCB) * DK * dv);
    grad_step<NR, CW>(X, o, lane);
  }
#pragma unroll
  for (int i = 0; i < D; ++i) {
    load_op<NR, true, false, true>(rows, cols, tail0 - 1 - i, DK, dv, r0, act, col, ring[i]);
    asm volatile("" ::: "memory");
  }
  for (int64_t g = nfull - 1; g >= 0; --g) {
    const int64_t s0 = g * D + D - 1;  // an interval's last step can only be a group's first
    if (s0 == NS - 1 || (s0 + 1) % kCB == 0) store(ckp + (s0 / kCB) * DK * dv);
    int64_t nb = s0 - D;
    asm volatile("" : "+s"(nb));
#pragma unroll
    for (int i = 0; i < D; ++i) {
      grad_step<NR, CW>(X, ring[i], lane);
      load_op<NR, true, false, true>(rows, cols, nb - i, DK, dv, r0, act, col, ring[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (ds0) store(ds0 + sbase);
}

// ---- 3. interval kernel -------------------------------------------------------------
// WPG waves per workgroup, one per 16-column slice of a group of slices, persistent
// over the items (batch*head, interval, slice group). Pass A runs the interval forward
// from its stored S and keeps the state before every kSub-step block in the wave's
// slot; pass B takes the blocks in reverse: it recomputes the block's kSub states into
// the wave's LDS and walks them back. The waves' row partials of a step are summed in
// LDS in wave order (one barrier a step) and written once per group.
template <int DK, int WPG>
__global__ __launch_bounds__(64 * WPG) void bwd_interval_kernel(Problem p, float* __restrict__ ws) {
  constexpr int NR = rows_per_lane(DK);
  constexpr int CW = kCW;
  constexpr int NV = NR * CW / 4;  // float4 per lane of a state
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t NS = p.steps, H = p.H, dv = p.dv;
  const int ngroups = int(dv / CW) / WPG;
  const BwdLayout L = bwd_layout(p.B, NS, H, DK, dv);
  const int64_t bth = p.B * NS * H;  // step rows
  const int r0 = lane * NR;
  const bool act = DK >= 64 || r0 < DK;
  const int lc = col_lane<CW>(lane & (CW - 1));
  float4* slot = reinterpret_cast<float4*>(ws + L.sub) + (int64_t(blockIdx.x) * WPG + wave) * (kCB / kSub) * NV * 64;
  __shared__ float4 sts_all[WPG][kSub * NV * 64];  // each wave's block states, lane order
  __shared__ float xch[WPG > 1 ? 2 : 1][WPG][4][DK];  // row partials of a step, by parity
  float4* sts = sts_all[wave];
  int par = 0;  // exchange buffer of the next step (the same sequence in every wave)
  float* part = ws + L.part;
  float* dwg = ws + L.dw;

  using St = float[NR][CW];
  auto save = [&](float4* dst, const St& S) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int r = (4 * i) / CW, c = (4 * i) % CW;
      dst[i * 64 + lane] = make_float4(S[r][c], S[r][c + 1], S[r][c + 2], S[r][c + 3]);
    }
  };
  auto restore = [&](const float4* src, St& S) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int r = (4 * i) / CW, c = (4 * i) % CW;
      const float4 x = src[i * 64 + lane];
      S[r][c] = x.x, S[r][c + 1] = x.y, S[r][c + 2] = x.z, S[r][c + 3] = x.w;
    }
  };

  for (int64_t item = blockIdx.x; item < L.items; item += gridDim.x) {
    const int grp = int(item % ngroups);
    const int slice = grp * WPG + wave;
    const int64_t rest = item / ngroups;
    const int64_t ci = rest % L.nck, bh = rest / L.nck;
    const int cbase = slice * CW;
    const int64_t t0 = ci * kCB, t1 = min(NS, t0 + kCB);
    const int nb = int((t1 - t0 + kSub - 1) / kSub);
    const float* rows = ws + L.rows + (bh * (NS + 2 * kPad) + kPad) * 4 * DK;
    const float* cols = ws + L.cols + (bh * (NS + 2 * kPad) + kPad) * 2 * dv;
    auto load_blk = [&](int m, Op<NR> (&o)[kSub]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        // past the interval's end: the next steps or padding, never used
        const int64_t s = t0 + int64_t(m) * kSub + i;
        load_op<NR, true, true, true>(rows, cols, s, DK, dv, r0, act, cbase + lc, o[i]);
      }
    };

    float S[NR][CW], G[NR][CW];
    {
      const float* sck = ws + L.ck + (bh * L.nck + ci) * DK * dv + cbase;
      const float* gck = ws + L.gk + (bh * L.nck + ci) * DK * dv + cbase;
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < CW; c += 4) {
          const float4 x = act ? *reinterpret_cast<const float4*>(sck + size_t(r0 + r) * dv + c) : float4{};
          const float4 y = act ? *reinterpret_cast<const float4*>(gck + size_t(r0 + r) * dv + c) : float4{};
          S[r][c] = x.x, S[r][c + 1] = x.y, S[r][c + 2] = x.z, S[r][c + 3] = x.w;
          G[r][c] = y.x, G[r][c + 1] = y.y, G[r][c + 2] = y.z, G[r][c + 3] = y.w;
        }
    }

    // pass A: blocks 0 .. nb-2 forward, the state before each kept in the slot; S
    // ends as the state before block nb-1, and cur holds that block's operands
    Op<NR> cur[kSub], nxt[kSub];
    load_blk(0, cur);
    for (int m = 0; m + 1 < nb; ++m) {
      load_blk(m + 1, nxt);
      save(slot + int64_t(m) * NV * 64, S);
#pragma unroll
      for (int i = 0; i < kSub; ++i) fwd_step<NR, CW>(S, cur[i], lane);  // full block (m < nb - 1)
#pragma unroll
      for (int i = 0; i < kSub; ++i) cur[i] = nxt[i];
    }

    // pass B: blocks in reverse; the last one (possibly short) first, so that the
    // loop over whole blocks has no conditional memory operation (each block waits
    // only for its own prefetched operands)
    auto run_block = [&](const int m, auto whole) __attribute__((always_inline)) {
      constexpr bool W = decltype(whole)::value;
      const int mp = m > 0 ? m - 1 : 0;  // prefetch (block 0 again at the end: unused)
      load_blk(mp, nxt);
      float Sn[NR][CW];
      restore(slot + int64_t(mp) * NV * 64, Sn);
      const int64_t sb = t0 + int64_t(m) * kSub;
      const int n = W ? kSub : int(min<int64_t>(kSub, t1 - sb));
      // the state before each step of the block, in this wave's LDS, and each step's u
      // (this lane's column); the block's last step runs too, for its u
      float ul[kSub];
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        save(sts + i * NV * 64, S);
        ul[i] = (W || i < n) ? fwd_step<NR, CW>(S, cur[i], lane) : 0.0f;
      }
      auto back = [&](const int i) __attribute__((always_inline)) {
        const Op<NR>& o = cur[i];
        float Sp[NR][CW];
        restore(sts + i * NV * 64, Sp);
        const int64_t s = sb + i;
        float X[NR][CW];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int c = 0; c < CW; ++c) X[r][c] = o.al[r] * Sp[r][c];
        float u = ul[i];
        // u^T do over the slice's columns (lanes 0..15 of every row hold distinct ones)
        float udo = u * o.d;
        udo = pair_sum<1>(udo);
        udo = pair_sum<2>(udo);
        udo = pair_sum<4>(udo);
        udo = pair_sum<8>(udo);
        // dq = S_t do = X do + a (u^T do); G += q do^T; dw = G^T a
        float dq[NR], gw[CW];
#pragma unroll
        for (int r = 0; r < NR; ++r) dq[r] = o.a[r] * udo;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
          const float dc = col_bcast<CW>(o.d, c);
          gw[c] = 0.0f;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            dq[r] += X[r][c] * dc;
            G[r][c] += o.q[r] * dc;
            gw[c] += G[r][c] * o.a[r];
          }
        }
        const float dw = col_sum<CW>(gw, lane);
        asm volatile("" : "+v"(u));  // broadcast u here, after the reduction
        // da = G u; db = -X dw; dX = G - b dw^T; dalpha = rowsum(dX . S_{t-1}); G = Diag(alpha) dX
        float da[NR], db[NR], dal[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) da[r] = db[r] = dal[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
          const float uc = col_bcast<CW>(u, c);
          const float dwc = col_bcast<CW>(dw, c);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            da[r] += G[r][c] * uc;
            db[r] -= X[r][c] * dwc;
            const float dX = G[r][c] - o.b[r] * dwc;
            dal[r] += dX * Sp[r][c];
            G[r][c] = o.al[r] * dX;
          }
        }
        const int64_t pr = bh * NS + s;  // this head's step s
        if (lane < CW) dwg[pr * dv + cbase + lc] = dw;
        float* pw = part + (int64_t(grp) * bth + pr) * 4 * DK;
        if constexpr (WPG == 1) {
          if (act) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
              pw[r0 + r] = dq[r];
              pw[DK + r0 + r] = da[r];
              pw[2 * DK + r0 + r] = db[r];
              pw[3 * DK + r0 + r] = dal[r];
            }
          }
        } else {
          float(*xb)[4][DK] = xch[par];
          if (act) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
              xb[wave][0][r0 + r] = dq[r];
              xb[wave][1][r0 + r] = da[r];
              xb[wave][2][r0 + r] = db[r];
              xb[wave][3][r0 + r] = dal[r];
            }
          }
          __syncthreads();
          // the sum over the group's slices, one quantity per wave (two for WPG = 2)
#pragma unroll
          for (int q = wave; q < 4; q += WPG) {
#pragma unroll
            for (int row = lane; row < DK; row += 64) {
              float sum = xb[0][q][row];
#pragma unroll
              for (int w = 1; w < WPG; ++w) sum += xb[w][q][row];
              pw[q * DK + row] = sum;
            }
          }
          par ^= 1;
        }
      };
      static_assert(kSub == 4, "the reverse walk below is written out for four steps");
      if (W || n > 3) back(3);
      if (W || n > 2) back(2);
      if (W || n > 1) back(1);
      back(0);
#pragma unroll
      for (int i = 0; i < kSub; ++i) cur[i] = nxt[i];
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < CW; ++c) S[r][c] = Sn[r][c];
    };
    run_block(nb - 1, std::false_type{});
    for (int m = nb - 2; m >= 0; --m) run_block(m, std::true_type{});
  }
}

// ---- 4. reduce kernel -------------------------------------------------------------
// One wave per step row: the partials summed over the slices in order, then the
// variant's chain rule.
template <typename In, int DK>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(Problem p, GradPtrs g, const float* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const int64_t T = p.T, H = p.H, dv = p.dv;
  const int ns = int(dv / kCW) / slices_per_group(dv);  // partial sets (slice groups)
  const int nh = p.n_h;
  const int64_t bth = p.B * T * H * nh;  // step rows
  const BwdLayout L = bwd_layout(p.B, p.steps, H, DK, dv);
  const float* part = ws + L.part;
  const float* dwg = ws + L.dw;
  const In* k = static_cast<const In*>(p.k);
  const In* v = static_cast<const In*>(p.v);
  const In* be = static_cast<const In*>(p.beta);
  const In* bev = static_cast<const In*>(p.beta_v);
  const In* jv = static_cast<const In*>(p.j);
  const In* et = static_cast<const In*>(p.eta);
  auto ld = [](const In* x) { return IO<In>::ld(x); };
  const int64_t stride = int64_t(gridDim.x) * (blockDim.x / 64);
  for (int64_t th = int64_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6); th < bth; th += stride) {
    // the partials of step row th = ((b T + t) H + h) n_h + sub sit at head b H + h, step t n_h + sub
    const int64_t tok = th / nh;
    const int64_t bt = tok / H;
    const int64_t prow = ((bt / T) * H + tok % H) * p.steps + (bt % T) * nh + (th - tok * nh);
    if (p.variant == GDN_VARIANT_DELTAPRODUCT) {  // th is a step row (token x n_h + step)
      const int sub = int(th - tok * nh);
      const float bt = ld(be + th);
      float sb = 0.0f, sal = 0.0f;
      for (int r = lane; r < DK; r += 64) {
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int w2 = 0; w2 < ns; ++w2) {
          const float* pr = part + (int64_t(w2) * bth + prow) * 4 * DK;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) s4[qd] += pr[qd * DK + r];
        }
        g.dk[th * DK + r] = s4[1] + bt * s4[2];
        sb += ld(k + th * DK + r) * s4[2];
        sal += s4[3];
        if (sub == nh - 1) g.dq[tok * DK + r] = s4[0];
      }
      for (int cc = lane; cc < dv; cc += 64) {
        const float dw = dwg[prow * dv + cc];
        g.dv[th * dv + cc] = bt * dw;
        sb += ld(v + th * dv + cc) * dw;
      }
      const float tb = wave_sum(sb);
      if (lane == 0) g.dbeta[th] = tb;
      if (sub == 0) {
        const float ta = wave_sum(sal);
        if (lane == 0) g.dalpha[tok] = ta;  // the gate acts at the first step
      }
      continue;
    }
    float sk = 0.0f, sv = 0.0f, sj = 0.0f, sal = 0.0f;  // per-token sums
    const float sbeta = (p.variant == GDN_VARIANT_KDA || p.variant == GDN_VARIANT_GDN) ? sqrtf(ld(be + th)) : 1.0f;
    const float e = p.variant == GDN_VARIANT_ASYM ? ld(et + th) : 0.0f;
    for (int r = lane; r < DK; r += 64) {
      float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int w2 = 0; w2 < ns; ++w2) {
        const float* pr = part + (int64_t(w2) * bth + prow) * 4 * DK;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) s4[qd] += pr[qd * DK + r];
      }
      const float dab = s4[1] + s4[2], dal = s4[3];
      const int64_t ir = th * DK + r;
      g.dq[ir] = s4[0];
      const float kr = ld(k + ir);
      if (p.variant == GDN_VARIANT_FG2) {
        const float s = sqrtf(ld(be + ir));
        g.dk[ir] = s * dab;
        g.dalpha[ir] = dal;
        float db = kr * dab;
        if (!bev) db += ld(v + th * dv + r) * dwg[prow * dv + r];  // shared beta (dk == dv)
        g.dbeta[ir] = db / (2.0f * s);
      } else if (p.variant == GDN_VARIANT_ASYM) {
        g.dk[ir] = s4[1];
        g.dj[ir] = e * s4[2];
        g.dalpha[ir] = dal;
        sj += ld(jv + ir) * s4[2];
      } else {
        g.dk[ir] = sbeta * dab;
        sk += kr * dab;
        if (p.variant == GDN_VARIANT_KDA) g.dalpha[ir] = dal;
        else sal += dal;
      }
    }
    for (int cc = lane; cc < dv; cc += 64) {
      const float dw = dwg[prow * dv + cc];
      const int64_t ic = th * dv + cc;
      const float vc = ld(v + ic);
      if (p.variant == GDN_VARIANT_FG2) {
        if (bev) {
          const float s = sqrtf(ld(bev + ic));
          g.dv[ic] = s * dw;
          g.dbeta_v[ic] = vc * dw / (2.0f * s);
        } else {
          g.dv[ic] = sqrtf(ld(be + th * DK + cc)) * dw;
        }
      } else if (p.variant == GDN_VARIANT_ASYM) {
        g.dv[ic] = e * dw;
        sv += vc * dw;
      } else {
        g.dv[ic] = sbeta * dw;
        sv += vc * dw;
      }
    }
    if (p.variant == GDN_VARIANT_KDA || p.variant == GDN_VARIANT_GDN) {
      const float tot = wave_sum(sk + sv);
      if (lane == 0) g.dbeta[th] = tot / (2.0f * sbeta);
      if (p.variant == GDN_VARIANT_GDN) {
        const float ta = wave_sum(sal);
        if (lane == 0) g.dalpha[th] = ta;
      }
    } else if (p.variant == GDN_VARIANT_ASYM) {
      const float tot = wave_sum(sj + sv);
      if (lane == 0) g.deta[th] = tot;
    }
  }
}

template <typename In, int DK>
int launch_dk(const Problem& p, const In* dO, const float* dsf, const GradPtrs& g, float* ws, hipStream_t s) {
  const BwdLayout L = bwd_layout(p.B, p.steps, p.H, DK, p.dv);
  const int64_t nsteps = p.B * p.H * p.steps;
  if (nsteps > 0) {
    // one wave a step: the grid fits 32 bits for any workspace that can exist (at least
    // 16 dk + 8 dv bytes a step, so 2^34 steps would need hundreds of terabytes)
    bwd_ops_kernel<In><<<dim3(unsigned((nsteps + 3) / 4)), dim3(256), 0, s>>>(p, dO, ws);
    int e = int(hipGetLastError());
    if (e != 0) return e;
  }
  // dv / kChainCW is a multiple of 4: whole workgroups, and the S and G halves split
  // between workgroups
  const int64_t chain_waves = 2 * p.B * p.H * (p.dv / kChainCW);
  bwd_chain_kernel<DK, kChainCW><<<dim3(unsigned(chain_waves / 4)), dim3(256), 0, s>>>(p, dsf, g.ds0, ws);
  int e = int(hipGetLastError());
  if (e != 0 || nsteps == 0) return e;
  switch (slices_per_group(p.dv)) {
    case 1: bwd_interval_kernel<DK, 1><<<dim3(unsigned(L.slots)), dim3(64), 0, s>>>(p, ws); break;
    case 2: bwd_interval_kernel<DK, 2><<<dim3(unsigned(L.slots)), dim3(128), 0, s>>>(p, ws); break;
    default: bwd_interval_kernel<DK, 4><<<dim3(unsigned(L.slots)), dim3(256), 0, s>>>(p, ws); break;
  }
  e = int(hipGetLastError());
  if (e != 0) return e;
  const int64_t waves = p.B * p.T * p.H * p.n_h;
  const int64_t blocks = (waves + 3) / 4;
  bwd_reduce_kernel<In, DK><<<dim3(unsigned(blocks < (int64_t(1) << 20) ? blocks : (int64_t(1) << 20))), dim3(256), 0, s>>>(p, g, ws);
  return int(hipGetLastError());
}

template <typename In>
int launch_in(const Problem& p, const void* d_o, const float* dsf, const GradPtrs& g, float* ws,
              hipStream_t s) {
  const In* dO = static_cast<const In*>(d_o);
  switch (p.dk) {
    case 16: return launch_dk<In, 16>(p, dO, dsf, g, ws, s);
    case 32: return launch_dk<In, 32>(p, dO, dsf, g, ws, s);
    case 64: return launch_dk<In, 64>(p, dO, dsf, g, ws, s);
    case 128: return launch_dk<In, 128>(p, dO, dsf, g, ws, s);
    default: return int(hipErrorInvalidValue);
  }
}

}  // namespace

size_t bwd_workspace_bytes(const Problem& p) {
  return size_t(bwd_layout(p.B, p.steps, p.H, p.dk, p.dv).total) * sizeof(float);
}

int launch_recurrent_bwd(const Problem& p, const void* d_o, const float* dsf, const GradPtrs& g,
                         void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* w = static_cast<float*>(ws);
  return p.dtype == GDN_DTYPE_BF16 ? launch_in<uint16_t>(p, d_o, dsf, g, w, s)
                                   : launch_in<float>(p, d_o, dsf, g, w, s);
}

}  // namespace gdn
