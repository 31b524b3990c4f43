// Backward pass of the token recurrence (reverse mode), every variant: FG2, FG2+, KDA,
// GDN, ASYM, and DeltaProduct as its sequence of Householder sub-steps.
//
// Per step S_t = (I - a b^T) Diag(alpha) S_{t-1} + a w^T and o_t = S_t^T q_t (FG2-GDN
// reading notes, section 2.2 eq. (11) and section 2.3 eq. (13); GDN2-stability page,
// eq. (1)); each variant is a map onto the per-step rows a, b, alpha, q and columns w.
// The pass runs on chunks of 16 steps in the WY / UT form the forward pass uses
// (reading notes, section 2.4). For a chunk with start state S and in-chunk inclusive
// cumulative log decay G (per key channel, G_C at its last step):
//   B+ = b e^G,  A- = a e^-G,  Q+ = q e^G,  A^ = a e^(G_C - G),  Gamma = e^(G_C)
//   M = strict_tril(B+ A-^T),  P = tril(Q+ A-^T),  T = (I + M)^-1
//   W = T B+,  U~ = T W_v,  U = U~ - W S,  O = Q+ S + P U,  S' = Gamma S + A^^T U.
// With D = dL/dS' and dO, reverse mode through these products gives
//   dU = P^T dO + A^ D,  dR = T^T dU (the gradient of W_v, i.e. of w),
//   dP = tril(dO U^T),   dM = -strict_tril(dR U^T),
//   dS = Gamma D + Q+^T dO - W^T dU = Gamma D - W^T (A^ D) + (Q+ - P W)^T dO,
//   dQ+ = dO S^T + dP A-,  dB+ = -dR S^T + dM A-,  dA- = dP^T Q+ + dM^T B+,  dA^ = U D^T,
// and the decay through dG = q.dq + b.db - a.da: d log alpha_l is the sum of dG over the
// steps from l on, plus the Gamma term, plus the A^ terms of the steps before l.
//
// e^-G is never formed: the Grams and the products with A- take factors split at the
// chunk's step 8, e^(G - G_8) on the B+ / Q+ side and e^(G_8 - G) on the A- side, so no
// factor spans more than 8 steps of decay; e^G, e^(G_C - G) and Gamma are at most 1.
// Every factor is a product of the alphas it spans.
//
// Kernels (all arithmetic in float32, products on fp32 MFMA):
//  1. operands: every step's a, b, alpha, q rows and w, do columns (the variant's map),
//     then identity steps up to a whole chunk;
//  2. records: per chunk, the Grams, T by forward substitution, W, U~, A^, Q+ - P W and
//     Gamma, each stored in the lane order of the products that read it;
//  3. recursions: the state forward and its gradient backward over the chunks, one
//     four-wave workgroup per (batch*head, 16 value columns) and direction; the state
//     before every even chunk and the gradient after every odd one are stored;
//  4. intra-chunk gradients: the chunks in pairs, one wave each; each wave rebuilds
//     the matrix its partner lacks from its own chunk's record;
//  5. reduce: the variant's chain rule.
// Every sum runs in a fixed order: the results are deterministic.
//
// MFMA layout (16x16x4 fp32, one wave): in a 16 x 16 tile, lane l = i + 16 g supplies
// A[i][4g + e] and B[4g + e][i] for e = 0..3, and receives D[4g + e][i]. So an output
// tile can be fed back as a B operand, or as the A operand of the transposed matrix,
// and swapping the operands of a product yields its transpose. Two storage orders of
// a 16-row matrix X follow: the fragment order (lane i + 16g holds X[4g + e][16t + i])
// and the row order (lane i + 16g holds X[i][16t + 4g + e]), both one float4 per lane
// and tile.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kC = 16;        // steps a chunk
constexpr int kPad = 2 * kC;  // operand rows after a sequence (identity steps fill its last chunk pair)

// Record of one chunk (float offsets): W (fragment, row order), A^ (fragment, row
// order), Q+ - P W (fragment), U~ (fragment, row order), Gamma, T and P (row-major 16 x 16).
__host__ __device__ constexpr int64_t rec_floats(int64_t dk, int64_t dv) { return 80 * dk + 32 * dv + dk + 512; }
template <int DK, int DV>
struct Rec {
  static constexpr int Wf = 0, Wr = 16 * DK, Af = 32 * DK, Ar = 48 * DK, Cf = 64 * DK;
  static constexpr int Uf = 80 * DK, Ur = 80 * DK + 16 * DV, Gm = 80 * DK + 32 * DV;
  static constexpr int Tm = Gm + DK, Pm = Tm + 256, size = Pm + 256;
  static_assert(size == rec_floats(DK, DV), "record size");
};

// Workspace (float offsets); NS steps a head (tokens x n_h for DeltaProduct):
//   rows [B*H][NS + kPad][4][dk]   a, b, alpha, q
//   cols [B*H][NS + kPad][2][dv]   w, do
//   rec  [B*H][chunks][rec_floats]
//   sst  [B*H][chunks/2][dk/16][dv/16][64 lanes][4]   state before chunk 2m (fragment order)
//   dst  [B*H][chunks/2][dk/16][dv/16][64 lanes][4]   dL/dS after chunk 2m + 1
//   part [B*H][NS][4][dk]   dq, da, db, dalpha of each step
//   dw   [B*H][NS][dv]
struct BwdLayout {
  int64_t rows, cols, rec, sst, dst, part, dw, total;
  int64_t nc, rs;  // chunks and operand rows a head
};

__host__ __device__ inline BwdLayout bwd_layout(int64_t B, int64_t NS, int64_t H, int64_t dk, int64_t dv) {
  BwdLayout L;
  const int64_t bh = B * H;
  L.nc = ((NS + kC - 1) / kC + 1) & ~int64_t(1);  // an even number: chunks go in pairs
  L.rs = NS + kPad;
  L.rows = 0;
  L.cols = L.rows + bh * L.rs * 4 * dk;
  L.rec = L.cols + bh * L.rs * 2 * dv;
  L.sst = L.rec + bh * L.nc * rec_floats(dk, dv);
  L.dst = L.sst + bh * (L.nc / 2) * dk * dv;
  L.part = L.dst + bh * (L.nc / 2) * dk * dv;
  L.dw = L.part + bh * NS * 4 * dk;
  L.total = L.dw + bh * NS * dv;
  if (L.total < 64) L.total = 64;  // a valid empty problem still reports a nonzero size
  return L;
}

__device__ __forceinline__ float4v ld4(const float* p) { return *reinterpret_cast<const float4v*>(p); }
__device__ __forceinline__ void st4(float* p, float4v v) { *reinterpret_cast<float4v*>(p) = v; }
__device__ __forceinline__ float4v zero4() { return float4v{0.0f, 0.0f, 0.0f, 0.0f}; }

// D += A B over one 16-wide slice of the summed index (four MFMA 16x16x4).
__device__ __forceinline__ float4v mma4(float4v a, float4v b, float4v acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}

// A 16 x 16 tile in the fragment order (lane i + 16g holds X[4g+e][i]) returned in the
// row order (X[i][4g+e]) through a 16 x 20 float LDS tile of the calling wave: one
// 16-byte write of the lane's column, four reads of its row (rows 20 floats apart put
// the four lane groups on different banks). A wave's LDS accesses complete in order;
// the empty asm statements keep the compiler from reordering them.
__device__ __forceinline__ float4v lds_transpose(float* tr, float4v x, int l) {
  const int i = l & 15, g = l >> 4;
  *reinterpret_cast<float4v*>(tr + i * 20 + 4 * g) = x;
  asm volatile("" ::: "memory");
  float4v y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = tr[(4 * g + e) * 20 + i];
  asm volatile("" ::: "memory");
  return y;
}

// Sum of x over the lane groups below this lane's (lanes l - 16, l - 32, l - 48).
__device__ __forceinline__ float group_prefix(float x, int l) {
  const int g = l >> 4;
  const float x1 = __shfl(x, (l + 48) & 63, 64);
  const float x2 = __shfl(x, (l + 32) & 63, 64);
  const float x3 = __shfl(x, (l + 16) & 63, 64);
  return (g >= 1 ? x1 : 0.0f) + (g >= 2 ? x2 : 0.0f) + (g >= 3 ? x3 : 0.0f);
}
// Sum of x over the lane groups above this lane's.
__device__ __forceinline__ float group_suffix(float x, int l) {
  const int g = l >> 4;
  const float x1 = __shfl(x, (l + 16) & 63, 64);
  const float x2 = __shfl(x, (l + 32) & 63, 64);
  const float x3 = __shfl(x, (l + 48) & 63, 64);
  return (g <= 2 ? x1 : 0.0f) + (g <= 1 ? x2 : 0.0f) + (g == 0 ? x3 : 0.0f);
}

// Decay factors of one channel at steps s = 4g .. 4g+3 of a chunk (fragment order),
// from its decays alpha at those steps: eg = e^(G_s), eh = e^(G_C - G_s), up =
// e^(G_s - G_8), dn = e^(G_8 - G_s) and gam = e^(G_C). Each is a product of the
// alphas over just the steps it spans (up and dn at most 8 of them), never an
// exponential of a difference of cumulative log decays, which would carry the
// rounding of sums as large as 16 |log alpha| into every factor. Every kernel forms
// the factors here, in the same order, so all of them see the same values.
struct Decay {
  float eg[4], eh[4], up[4], dn[4], gam;
};
__device__ __forceinline__ Decay chunk_decay(const float (&al)[4], int l) {
  const int g = l >> 4, i = l & 15;
  float ip[4], es[4], ipx[4];  // in-group inclusive prefix, exclusive suffix, prefix after the first
  ip[0] = al[0];
  ipx[0] = 1.0f;
  ipx[1] = al[1];
#pragma unroll
  for (int e = 1; e < 4; ++e) ip[e] = ip[e - 1] * al[e];
  ipx[2] = ipx[1] * al[2];
  ipx[3] = ipx[2] * al[3];
  es[3] = 1.0f;
#pragma unroll
  for (int e = 2; e >= 0; --e) es[e] = al[e + 1] * es[e + 1];
  const float t0 = __shfl(ip[3], i, 64), t1 = __shfl(ip[3], 16 + i, 64);  // group products
  const float t2 = __shfl(ip[3], 32 + i, 64), t3 = __shfl(ip[3], 48 + i, 64);
  const float a8 = __shfl(al[0], 32 + i, 64);     // alpha at step 8
  const float p911 = __shfl(ipx[3], 32 + i, 64);  // alphas of steps 9 .. 11
  const float before = g == 0 ? 1.0f : g == 1 ? t0 : g == 2 ? t0 * t1 : (t0 * t1) * t2;
  const float after = g == 3 ? 1.0f : g == 2 ? t3 : g == 1 ? t2 * t3 : t1 * (t2 * t3);
  Decay d;
  d.gam = ((t0 * t1) * t2) * t3;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    d.eg[e] = before * ip[e];
    d.eh[e] = es[e] * after;
    const float u = g == 2 ? ipx[e] : p911 * ip[e];        // steps 8 .. 15: alphas of steps 9 .. s
    const float w = g == 1 ? es[e] * a8 : (es[e] * t1) * a8;  // steps 0 .. 7: alphas of steps s+1 .. 8
    d.up[e] = g >= 2 ? u : 1.0f / w;
    d.dn[e] = g >= 2 ? 1.0f / u : w;
  }
  return d;
}

// ---- 1. operand kernel ------------------------------------------------------------
// One wave per step: a, b, alpha, q rows and w, do columns in float32:
//   FG2:   a = b = sqrt(beta) k, w = sqrt(beta) v (sqrt(beta_v) v for FG2+), alpha per channel
//   KDA:   a = b = sqrt(beta) k, w = sqrt(beta) v, alpha per channel
//   GDN:   the same with a scalar alpha
//   DeltaProduct sub-step i: a = k_i, b = beta_i k_i, w = beta_i v_i
//   ASYM:  a = k, b = eta j, w = eta v, alpha = D
// q and do act after a token's last step (DeltaProduct: zero for the earlier steps),
// the gate at its first. Steps from the end of the sequence to the end of its last
// chunk are identity steps (nothing erased, written or read; no decay).
// R consecutive elements (R = 1 or 2; the address aligned to R elements) as floats.
template <int R>
__device__ __forceinline__ void ldr(const float* p, float (&o)[R]) {
  if constexpr (R == 2) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    o[0] = x.x, o[1] = x.y;
  } else {
    o[0] = *p;
  }
}
template <int R>
__device__ __forceinline__ void ldr(const uint16_t* p, float (&o)[R]) {
  if constexpr (R == 2) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(p);
    o[0] = __uint_as_float(x << 16), o[1] = __uint_as_float(x & 0xffff0000u);
  } else {
    o[0] = bf16_to_f32(*p);
  }
}
template <int R>
__device__ __forceinline__ void str(float* p, const float (&x)[R]) {
  if constexpr (R == 2) *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  else *p = x[0];
}
// channels a lane takes in a row of d: d / 64 consecutive ones (lanes past d idle below 64)
__host__ __device__ constexpr int lane_run(int d) { return d >= 64 ? d / 64 : 1; }

template <typename In, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_ops_kernel(Problem p, const In* __restrict__ d_o,
                                                      float* __restrict__ ws) {
  constexpr int RK = lane_run(DK), RV = lane_run(DV);
  const int lane = threadIdx.x & 63;
  const int64_t NS = p.steps, T = p.T, H = p.H;
  const int nh = p.n_h;
  const BwdLayout L = bwd_layout(p.B, NS, H, DK, DV);
  const int64_t NP = L.nc * kC;
  const int64_t x = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // bh * NP + s
  if (x >= p.B * H * NP) return;
  const int64_t bh = x / NP, s = x % NP;
  float* rw = ws + L.rows + (bh * L.rs + s) * 4 * DK;
  float* cl = ws + L.cols + (bh * L.rs + s) * 2 * DV;
  const int ek = lane * RK, ev = lane * RV;  // this lane's first channel and column
  const bool kl = ek < DK, vl = ev < DV;
  if (s >= NS) {
    float z[RK], one[RK];
#pragma unroll
    for (int r = 0; r < RK; ++r) z[r] = 0.0f, one[r] = 1.0f;
    if (kl) {
      str<RK>(rw + ek, z);
      str<RK>(rw + DK + ek, z);
      str<RK>(rw + 2 * DK + ek, one);
      str<RK>(rw + 3 * DK + ek, z);
    }
    float zv[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) zv[r] = 0.0f;
    if (vl) {
      str<RV>(cl + ev, zv);
      str<RV>(cl + DV + ev, zv);
    }
    return;
  }
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
  if (kl) {
    float kr[RK], a[RK], bb[RK], alpha[RK], qq[RK], x1[RK], x2[RK];
    ldr<RK>(k + sr * DK + ek, kr);
    if (var == GDN_VARIANT_ASYM || var == GDN_VARIANT_FG2 || var == GDN_VARIANT_KDA) ldr<RK>(al + th * DK + ek, x1);
    if (var == GDN_VARIANT_ASYM) ldr<RK>(jv + th * DK + ek, x2);
    if (var == GDN_VARIANT_FG2) ldr<RK>(be + th * DK + ek, x2);
    if (last) ldr<RK>(q + th * DK + ek, qq);
#pragma unroll
    for (int r = 0; r < RK; ++r) {
      if (var == GDN_VARIANT_DELTAPRODUCT) {
        a[r] = kr[r], bb[r] = sc * kr[r], alpha[r] = gate;
      } else if (var == GDN_VARIANT_ASYM) {
        a[r] = kr[r], bb[r] = x2[r] * sc, alpha[r] = x1[r];
      } else if (var == GDN_VARIANT_FG2) {
        a[r] = kr[r] * sqrtf(x2[r]), bb[r] = a[r], alpha[r] = x1[r];
      } else {
        a[r] = kr[r] * sc, bb[r] = a[r], alpha[r] = var == GDN_VARIANT_KDA ? x1[r] : gate;
      }
      if (!last) qq[r] = 0.0f;
    }
    str<RK>(rw + ek, a);
    str<RK>(rw + DK + ek, bb);
    str<RK>(rw + 2 * DK + ek, alpha);
    str<RK>(rw + 3 * DK + ek, qq);
  }
  if (vl) {
    float vc[RV], w[RV], dd[RV], bs[RV];
    ldr<RV>(v + sr * DV + ev, vc);
    if (var == GDN_VARIANT_FG2) ldr<RV>(bev ? bev + th * DV + ev : be + th * DK + ev, bs);
    if (last) ldr<RV>(d_o + th * DV + ev, dd);
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      w[r] = var == GDN_VARIANT_FG2 ? vc[r] * sqrtf(bs[r]) : sc * vc[r];
      if (!last) dd[r] = 0.0f;
    }
    str<RV>(cl + ev, w);
    str<RV>(cl + DV + ev, dd);
  }
}

// ---- 2. record kernel -------------------------------------------------------------
// One wave per (batch*head, chunk). The operands are formed in the fragment order
// (step 4g+e, channel 16t+i) and turned into the row order the Grams need through LDS.
template <int DK, int DV>
__global__ __launch_bounds__(64) void bwd_rec_kernel(Problem p, float* __restrict__ ws) {
  constexpr int KT = DK / 16, VT = DV / 16;
  using R = Rec<DK, DV>;
  __shared__ __align__(16) float Ms[256];
  __shared__ __align__(16) float Ps[256];
  __shared__ __align__(16) float Ts[256];
  const int l = threadIdx.x, i = l & 15, g = l >> 4;
  const BwdLayout L = bwd_layout(p.B, p.steps, p.H, DK, DV);
  const int64_t item = blockIdx.x;  // bh * chunks + c
  const int64_t bh = item / L.nc, c = item % L.nc;
  const float* rb = ws + L.rows + (bh * L.rs + c * kC) * 4 * DK;  // step s of the chunk at rb + s 4 DK
  const float* cb = ws + L.cols + (bh * L.rs + c * kC) * 2 * DV;
  float* rec = ws + L.rec + item * R::size;
  __shared__ __align__(16) float tr[16 * 20];  // tile transposes

  // per key tile: B+, Q+, A^ (fragment order) kept for W and Q+ - P W; the Grams
  // M = strict_tril(B~ A~^T), P = tril(Q~ A~^T) with B~ = b e^(G - G_8), Q~ = q e^(G - G_8),
  // A~ = a e^(G_8 - G) from the transposed operands
  float4v bF[KT], qF[KT];
  float4v m = zero4(), pp = zero4();
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const int ch = 16 * t + i;
    float al[4];
    float4v av, bv, qv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float* rr = rb + (4 * g + e) * 4 * DK + ch;
      av[e] = rr[0];
      bv[e] = rr[DK];
      al[e] = rr[2 * DK];
      qv[e] = rr[3 * DK];
    }
    const Decay d = chunk_decay(al, l);
    float4v bt, qt, at, aF;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bF[t][e] = bv[e] * d.eg[e];
      qF[t][e] = qv[e] * d.eg[e];
      aF[e] = av[e] * d.eh[e];
      bt[e] = bv[e] * d.up[e];
      qt[e] = qv[e] * d.up[e];
      at[e] = av[e] * d.dn[e];
    }
    const float4v btr = lds_transpose(tr, bt, l), qtr = lds_transpose(tr, qt, l), atr = lds_transpose(tr, at, l);
    m = mma4(btr, atr, m);  // M[4g+e][i] = B~[4g+e] . A~[i]
    pp = mma4(qtr, atr, pp);
    st4(rec + R::Af + t * 256 + 4 * l, aF);
    st4(rec + R::Ar + t * 256 + 4 * l, lds_transpose(tr, aF, l));  // A^ in the row order
    if (g == 0) rec[R::Gm + ch] = d.gam;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * g + e;
    Ms[r * 16 + i] = r > i ? m[e] : 0.0f;
    Ps[r * 16 + i] = r >= i ? pp[e] : 0.0f;
  }
  __syncthreads();

  // T = (I + M)^-1 by forward substitution, column i in lane i (every lane group alike)
  float tc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = r == i ? 1.0f : 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < r; ++s2) x -= Ms[r * 16 + s2] * tc[s2];
    tc[r] = x;
  }
  if (g == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) Ts[r * 16 + i] = tc[r];
  }
  __syncthreads();
  st4(rec + R::Tm + 4 * l, ld4(Ts + 4 * l));
  st4(rec + R::Pm + 4 * l, ld4(Ps + 4 * l));
  const float4v tA = ld4(Ts + i * 16 + 4 * g);  // T[i][4g+e]
  const float4v pA = ld4(Ps + i * 16 + 4 * g);  // P[i][4g+e]

#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const float4v w = mma4(tA, bF[t], zero4());   // W = T B+ (fragment order)
    const float4v wr = mma4(bF[t], tA, zero4());  // W^T: W in the row order
    const float4v pw = mma4(pA, w, zero4());      // P W (fragment order)
    st4(rec + R::Wf + t * 256 + 4 * l, w);
    st4(rec + R::Wr + t * 256 + 4 * l, wr);
    st4(rec + R::Cf + t * 256 + 4 * l, qF[t] - pw);
  }
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    float4v wF;  // w at (step 4g+e, column 16vt+i)
#pragma unroll
    for (int e = 0; e < 4; ++e) wF[e] = cb[(4 * g + e) * 2 * DV + 16 * vt + i];
    st4(rec + R::Uf + vt * 256 + 4 * l, mma4(tA, wF, zero4()));  // U~ = T W_v
    st4(rec + R::Ur + vt * 256 + 4 * l, mma4(wF, tA, zero4()));  // U~ in the row order
  }
}

// ---- 3. recursions ----------------------------------------------------------------
// Blocks [0, B*H*dv/16): the state S_{c+1} = Gamma S_c + A^^T (U~ - W S_c), storing S_c
// for even c. Blocks [B*H*dv/16, 2 B*H*dv/16): its gradient D_{c-1} = Gamma D_c -
// W^T (A^ D_c) + (Q+ - P W)^T dO_c from D = dL/dS_final, storing D_c for odd c; D_{-1}
// is dL/dS_0. (The intra-chunk kernel rebuilds the other halves; the stores are what
// the recursions' time depends on most.)
// A block holds one 16-column slice (dk x 16) in accumulator tiles, its key tiles split
// over up to four waves; the 16 x 16 products summed over the key channels (W S, A^ D)
// are added up through LDS in wave order, one barrier a chunk. Each wave loads the next
// chunk's record while it applies the current one.
__host__ __device__ constexpr int chain_waves(int dk) { return dk / 16 < 4 ? dk / 16 : 4; }

template <int TW>
struct SOps {
  float4v wr[TW], af[TW], gm[TW], uf;
};
template <int TW>
struct GOps {
  float4v ar[TW], wf[TW], cf[TW], gm[TW], dof;
};

// Records in flight a wave (a register ring). Refills sit right after the step that
// frees their slot: a scheduling barrier keeps the compiler from moving them, and
// the refill index is hidden from the optimizer, which would otherwise turn a refill
// back into a load at the point of use. Whole ring groups run with unconditional
// refills (clamped to the last chunk), the remainder without any.
constexpr int kRing = 4;
static_assert(kRing % 2 == 0, "a ring group starts on an even chunk");

// compile-time flag: whether a recursion step stores its tile
template <bool B>
struct Keep {
  static constexpr bool value = B;
};

template <int DK, int DV>
__global__ __launch_bounds__(64 * chain_waves(DK)) void bwd_chain_kernel(Problem p, const float* __restrict__ dsf,
                                                                         float* __restrict__ ds0, float* __restrict__ ws) {
  constexpr int KT = DK / 16, VT = DV / 16, NW = chain_waves(DK), TW = KT / NW;
  using R = Rec<DK, DV>;
  __shared__ float4v xch[2][NW][64];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6, g = l >> 4, i = l & 15;
  const BwdLayout L = bwd_layout(p.B, p.steps, p.H, DK, DV);
  const int64_t nbv = p.B * p.H * VT;
  // Blocks go to the 8 XCDs in turn (block b to XCD b mod 8): with a multiple of 8
  // blocks, block b takes logical index (b mod 8) N/8 + b/8, so the slices of one
  // head, which read the same records, run on one XCD and share its L2.
  const int64_t nblk = gridDim.x, blk = blockIdx.x;
  const int64_t x = nblk % 8 == 0 ? (blk % 8) * (nblk / 8) + blk / 8 : blk;
  const bool grad = x >= nbv;
  const int64_t y = grad ? x - nbv : x;
  const int64_t bh = y / VT;
  const int vt = int(y % VT);
  const int64_t NC = L.nc;
  const int64_t full = NC - NC % kRing;  // chunks in whole ring groups
  const float* recs = ws + L.rec + bh * NC * R::size;
  // barrier for the LDS exchange only: loads in flight stay in flight
  auto lds_barrier = []() __attribute__((always_inline)) { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  float4v X[TW];  // key tiles t = w TW + j of the slice
  // element (row 16t + 4g + e, column 16vt + i) of a [dk][dv] state
  const int64_t sbase = bh * DK * DV + (4 * g) * DV + 16 * vt + i;
  if (!grad) {
    const float* s0 = p.s0;
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) X[j][e] = s0 ? s0[sbase + (16 * (w * TW + j) + e) * DV] : 0.0f;
    if (NC == 0) return;
    auto load = [&](int64_t c, SOps<TW>& o) __attribute__((always_inline)) {
      const float* r = recs + c * R::size;
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        const int t = w * TW + j;
        o.wr[j] = ld4(r + R::Wr + t * 256 + 4 * l);
        o.af[j] = ld4(r + R::Af + t * 256 + 4 * l);
        o.gm[j] = ld4(r + R::Gm + 16 * t + 4 * g);
      }
      o.uf = ld4(r + R::Uf + vt * 256 + 4 * l);
    };
    auto step = [&](int64_t c, const SOps<TW>& o, auto keep) __attribute__((always_inline)) {
      if constexpr (decltype(keep)::value) {  // c even
        float* so = ws + L.sst + (bh * NC / 2 + c / 2) * KT * VT * 256;
#pragma unroll
        for (int j = 0; j < TW; ++j) st4(so + ((w * TW + j) * VT + vt) * 256 + 4 * l, X[j]);
      }
      float4v pu = zero4();
#pragma unroll
      for (int j = 0; j < TW; ++j) pu = mma4(o.wr[j], X[j], pu);  // this wave's share of W S
      xch[c & 1][w][l] = pu;
      lds_barrier();
      float4v u = o.uf;  // U = U~ - W S
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) u -= xch[c & 1][w2][l];
#pragma unroll
      for (int j = 0; j < TW; ++j) X[j] = mma4(o.af[j], u, X[j] * o.gm[j]);
    };
    SOps<TW> ring[kRing];
#pragma unroll
    for (int k = 0; k < kRing; ++k) load(k < NC ? k : NC - 1, ring[k]);
    asm volatile("" ::: "memory");
    for (int64_t c0 = 0; c0 < full; c0 += kRing) {
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        // c0 and full are multiples of kRing: chunk c0 + k is even exactly when k is
        if (k % 2 == 0) step(c0 + k, ring[k], Keep<true>());
        else step(c0 + k, ring[k], Keep<false>());
        int64_t nb = c0 + k + kRing;
        nb = nb < NC ? nb : NC - 1;
        asm volatile("" : "+s"(nb));
        load(nb, ring[k]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      if (full + k < NC) {
        if (k % 2 == 0) step(full + k, ring[k], Keep<true>());
        else step(full + k, ring[k], Keep<false>());
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) X[j][e] = dsf ? dsf[sbase + (16 * (w * TW + j) + e) * DV] : 0.0f;
    const float* cols = ws + L.cols + bh * L.rs * 2 * DV + DV + 16 * vt + i;  // do, column 16vt + i
    auto load = [&](int64_t c, GOps<TW>& o) __attribute__((always_inline)) {
      const float* r = recs + c * R::size;
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        const int t = w * TW + j;
        o.ar[j] = ld4(r + R::Ar + t * 256 + 4 * l);
        o.wf[j] = ld4(r + R::Wf + t * 256 + 4 * l);
        o.cf[j] = ld4(r + R::Cf + t * 256 + 4 * l);
        o.gm[j] = ld4(r + R::Gm + 16 * t + 4 * g);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) o.dof[e] = cols[(c * kC + 4 * g + e) * 2 * DV];
    };
    auto step = [&](int64_t c, const GOps<TW>& o, auto keep) __attribute__((always_inline)) {
      if constexpr (decltype(keep)::value) {  // c odd
        float* so = ws + L.dst + (bh * NC / 2 + c / 2) * KT * VT * 256;
#pragma unroll
        for (int j = 0; j < TW; ++j) st4(so + ((w * TW + j) * VT + vt) * 256 + 4 * l, X[j]);
      }
      float4v px = zero4();
#pragma unroll
      for (int j = 0; j < TW; ++j) px = mma4(o.ar[j], X[j], px);  // this wave's share of A^ D
      xch[c & 1][w][l] = px;
      lds_barrier();
      float4v nx = -xch[c & 1][0][l];  // -A^ D
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) nx -= xch[c & 1][w2][l];
#pragma unroll
      for (int j = 0; j < TW; ++j) X[j] = mma4(o.wf[j], nx, mma4(o.cf[j], o.dof, X[j] * o.gm[j]));
    };
    if (NC > 0) {
      // chunks from the last: the k-th of a ring group is chunk NC - 1 - (c0 + k), odd
      // exactly when k is even (NC is even, c0 and full multiples of kRing)
      GOps<TW> ring[kRing];
#pragma unroll
      for (int k = 0; k < kRing; ++k) load(k < NC ? NC - 1 - k : 0, ring[k]);
      asm volatile("" ::: "memory");
      for (int64_t c0 = 0; c0 < full; c0 += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
          if (k % 2 == 0) step(NC - 1 - (c0 + k), ring[k], Keep<true>());
          else step(NC - 1 - (c0 + k), ring[k], Keep<false>());
          int64_t nb = NC - 1 - (c0 + k + kRing);
          nb = nb > 0 ? nb : 0;
          asm volatile("" : "+s"(nb));
          load(nb, ring[k]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        if (full + k < NC) {
          if (k % 2 == 0) step(NC - 1 - (full + k), ring[k], Keep<true>());
          else step(NC - 1 - (full + k), ring[k], Keep<false>());
        }
      }
    }
    if (ds0) {
#pragma unroll
      for (int j = 0; j < TW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) ds0[sbase + (16 * (w * TW + j) + e) * DV] = X[j][e];
    }
  }
}

// ---- 4. intra-chunk gradients -------------------------------------------------------
// One two-wave workgroup per (batch*head, chunk pair): wave w takes chunk c = 2m + w,
// with S (state before it) and D (dL/dS after it), its record and operands, and writes
// every step's dq, da, db, dalpha and dw. The value columns are taken 16 at a time.
// The recursions stored S before chunk 2m and D after chunk 2m + 1 only; per value
// tile, wave 0 forms S before chunk 2m + 1 = Gamma S + A^^T U from the U of its chunk,
// wave 1 forms D after chunk 2m = Gamma D - W^T (A^ D) + (Q+ - P W)^T dO from the A^ D of
// its chunk (both products it needs anyway), and the two tiles cross through LDS. Each
// S and D tile is used in the fragment order for U and A^ D (sums over key channels)
// and transposed through LDS for dO S^T, dR S^T and U D^T (sums over value channels).
template <int DK, int DV>
__global__ __launch_bounds__(128) void bwd_intra_kernel(Problem p, float* __restrict__ ws) {
  constexpr int KT = DK / 16, VT = DV / 16;
  using R = Rec<DK, DV>;
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: the branches on it are too
  const BwdLayout L = bwd_layout(p.B, p.steps, p.H, DK, DV);
  const int64_t NS = p.steps;
  const int64_t np = L.nc / 2, pair = blockIdx.x;
  const int64_t bh = pair / np, c = 2 * (pair % np) + w;
  const int64_t item = bh * L.nc + c;
  const float* rb = ws + L.rows + (bh * L.rs + c * kC) * 4 * DK;
  const float* cb = ws + L.cols + (bh * L.rs + c * kC) * 2 * DV;
  const float* rec = ws + L.rec + item * R::size;
  // the stored tiles this wave reads: S before chunk 2m (wave 0), D after chunk 2m + 1 (wave 1)
  const float* sX = ws + (w == 0 ? L.sst : L.dst) + pair * KT * VT * 256;
  // LDS-only barrier of the two waves: global loads in flight stay in flight
  auto lds_barrier = []() __attribute__((always_inline)) { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // Operands that are the same for every value tile: W and A^ in the row order and Gamma,
  // parked in LDS; those of the rebuilt tiles in registers, A^ (fragment order) for
  // wave 0, W and Q+ - P W (fragment order) for wave 1.
  __shared__ float4v lw[2][KT][64], la[2][KT][64];
  __shared__ float4v xs[2][KT][64], xd[2][KT][64];  // the rebuilt S and D tiles, two value tiles deep
  __shared__ __align__(16) float lg[2][DK];
  __shared__ __align__(16) float tr[2][2][16 * 20];  // transposes of the S and D tiles
  float4v x1[KT], x2[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    lw[w][t][l] = ld4(rec + R::Wr + t * 256 + 4 * l);
    la[w][t][l] = ld4(rec + R::Ar + t * 256 + 4 * l);
    x1[t] = ld4(rec + (w == 0 ? R::Af : R::Wf) + t * 256 + 4 * l);
    x2[t] = w == 0 ? zero4() : ld4(rec + R::Cf + t * 256 + 4 * l);
  }
  for (int k = l; k < DK; k += 64) lg[w][k] = rec[R::Gm + k];
  __syncthreads();
  float4v pF, tF;  // P[4g+e][i], T[4g+e][i]
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pF[e] = rec[R::Pm + (4 * g + e) * 16 + i];
    tF[e] = rec[R::Tm + (4 * g + e) * 16 + i];
  }
  const bool row_live = c * kC + i < NS;
  // over the value tiles: dP, dM (both orientations: dp[e] = dP[4g+e][i], dpt[e] =
  // dP[i][4g+e], likewise dm, dmt) and, per key tile, dO S^T, dR S^T, U D^T at
  // (step 4g+e, channel 16t+i) and the sum over v of D . S for channel 16t+i
  float4v dp = zero4(), dpt = zero4(), dm = zero4(), dmt = zero4();
  float4v qs[KT], rs[KT], ud[KT];
  float rsum[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) qs[t] = rs[t] = ud[t] = zero4(), rsum[t] = 0.0f;
  // a value tile's loads, issued one tile ahead: the stored tiles, dO in both orders, U~
  struct VOps {
    float4v st[KT], dF, doA, ur;
  };
  auto vload = [&](int vt, VOps& o) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < KT; ++t) o.st[t] = ld4(sX + (t * VT + vt) * 256 + 4 * l);
#pragma unroll
    for (int e = 0; e < 4; ++e) o.dF[e] = cb[(4 * g + e) * 2 * DV + DV + 16 * vt + i];  // dO[4g+e][16vt+i]
    o.doA = ld4(cb + i * 2 * DV + DV + 16 * vt + 4 * g);                                // dO[i][16vt+4g+e]
    o.ur = ld4(rec + R::Ur + vt * 256 + 4 * l);
  };
  VOps vn;
  vload(0, vn);
#pragma unroll 1
  for (int vt = 0; vt < VT; ++vt) {
    const VOps vc = vn;
    if (vt + 1 < VT) vload(vt + 1, vn);
    float4v sf[KT], df[KT];  // S[16t+4g+e][16vt+i], D likewise
    // U in the row order: ut[e] = U[i][16vt+4g+e]  (U^T = U~^T - S^T W^T)
    auto u_rows = [&]() __attribute__((always_inline)) {
      float4v ut = -vc.ur;
#pragma unroll
      for (int t = 0; t < KT; ++t) ut = mma4(sf[t], lw[w][t][l], ut);
      return -ut;
    };
    float4v ut, x = zero4();  // x: A^ D, then dU = A^ D + P^T dO (fragment order)
    const float4v dF = vc.dF, doA = vc.doA;
    if (w == 0) {
#pragma unroll
      for (int t = 0; t < KT; ++t) sf[t] = vc.st[t];
      ut = u_rows();
      const float4v uF = lds_transpose(tr[w][0], ut, l);  // U[4g+e][16vt+i]
#pragma unroll
      for (int t = 0; t < KT; ++t)
        xs[vt & 1][t][l] = mma4(x1[t], uF, sf[t] * *reinterpret_cast<const float4v*>(&lg[0][16 * t + 4 * g]));
    } else {
#pragma unroll
      for (int t = 0; t < KT; ++t) df[t] = vc.st[t];
#pragma unroll
      for (int t = 0; t < KT; ++t) x = mma4(la[w][t][l], df[t], x);
#pragma unroll
      for (int t = 0; t < KT; ++t)
        xd[vt & 1][t][l] = mma4(x1[t], -x, mma4(x2[t], dF, df[t] * *reinterpret_cast<const float4v*>(&lg[1][16 * t + 4 * g])));
    }
    // one barrier a value tile: a buffer is written again two tiles later, after both
    // waves have passed the next tile's barrier and so have read it
    lds_barrier();
    if (w == 0) {
#pragma unroll
      for (int t = 0; t < KT; ++t) df[t] = xd[vt & 1][t][l];
#pragma unroll
      for (int t = 0; t < KT; ++t) x = mma4(la[w][t][l], df[t], x);
    } else {
#pragma unroll
      for (int t = 0; t < KT; ++t) sf[t] = xs[vt & 1][t][l];
      ut = u_rows();
    }
    // dR^T = dU^T T: rt[e] = dR[i][16vt+4g+e]
    x = mma4(pF, dF, x);
    const float4v rt = mma4(x, tF, zero4());
    if (row_live) st4(ws + L.dw + (bh * NS + c * kC + i) * DV + 16 * vt + 4 * g, rt);
    dp = mma4(doA, ut, dp);
    dpt = mma4(ut, doA, dpt);
    dm = mma4(rt, ut, dm);
    dmt = mma4(ut, rt, dmt);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const float4v sT = lds_transpose(tr[w][0], sf[t], l);  // S[16t+i][16vt+4g+e]
      const float4v dT = lds_transpose(tr[w][1], df[t], l);
      qs[t] = mma4(doA, sT, qs[t]);
      rs[t] = mma4(rt, sT, rs[t]);
      ud[t] = mma4(ut, dT, ud[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) rsum[t] += sT[e] * dT[e];
    }
  }
  // Pairs of steps of one token (one step, or a DeltaProduct token's sub-steps) have no
  // decay between them: their terms reach dq, db and da but add exactly nothing to dG
  // (each enters it twice with opposite signs). They are kept apart (the *w products),
  // since under strong decay such an exact zero, summed from its two halves, would be
  // far larger than dG itself.
  int64_t tk[4];  // tokens of steps 4g+e
#pragma unroll
  for (int e = 0; e < 4; ++e) tk[e] = (c * kC + 4 * g + e) / p.n_h;
  const int64_t tki = (c * kC + i) / p.n_h, tkl = (c * kC + kC - 1) / p.n_h;
  float4v dpw, dptw, dmw, dmtw;  // the within-token parts (dP with its diagonal)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * g + e;
    const bool same = tk[e] == tki;
    dpw[e] = r >= i && same ? dp[e] : 0.0f;
    dptw[e] = i >= r && same ? dpt[e] : 0.0f;
    dmw[e] = r > i && same ? -dm[e] : 0.0f;
    dmtw[e] = i > r && same ? -dmt[e] : 0.0f;
    dp[e] = r > i && !same ? dp[e] : 0.0f;
    dpt[e] = i > r && !same ? dpt[e] : 0.0f;
    dm[e] = r > i && !same ? -dm[e] : 0.0f;
    dmt[e] = i > r && !same ? -dmt[e] : 0.0f;
  }

  // per key tile: the operands at (step 4g+e, channel 16t+i), the next tile's loaded
  // while this one is assembled
  struct EOps {
    float av[4], bv[4], alv[4], qv[4];
  };
  auto eload = [&](int t, EOps& o) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float* rr = rb + (4 * g + e) * 4 * DK + 16 * t + i;
      o.av[e] = rr[0];
      o.bv[e] = rr[DK];
      o.alv[e] = rr[2 * DK];
      o.qv[e] = rr[3 * DK];
    }
  };
  float* part = ws + L.part;
  EOps cur, nxt;
  eload(0, cur);
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (t + 1 < KT) {
      eload(t + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int ch = 16 * t + i;
    const float rs_t = sum_over_groups(rsum[t]);
    const Decay dc = chunk_decay(cur.alv, l);
    float4v eg, eu, ed, eh, at, bt, qt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      eg[e] = dc.eg[e];
      eu[e] = dc.up[e];
      ed[e] = dc.dn[e];
      eh[e] = dc.eh[e];
      at[e] = cur.av[e] * ed[e];
      bt[e] = cur.bv[e] * eu[e];
      qt[e] = cur.qv[e] * eu[e];
    }
    const float4v pa = mma4(dpt, at, zero4());                  // dP A~
    const float4v ma = mma4(dmt, at, zero4());                  // dM A~
    const float4v aa = mma4(dm, bt, mma4(dp, qt, zero4()));     // dP^T Q~ + dM^T B~
    const float4v paw = mma4(dptw, at, zero4());                // the same within tokens
    const float4v maw = mma4(dmtw, at, zero4());
    const float4v aaw = mma4(dmw, bt, mma4(dpw, qt, zero4()));
    // d log alpha_s = (suffix sum over s' >= s of dG_s') + (prefix sum over j < s of
    // a_j . dh_j): the A^ terms enter dG_j with a minus and G_C with a plus, so their net
    // share is that prefix sum, formed directly; the Gamma term enters at G_C.
    float4v dq, da, db, dG, ah;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dqo = qs[t][e] * eg[e] + pa[e] * eu[e];
      const float dbo = ma[e] * eu[e] - rs[t][e] * eg[e];
      const float dao = aa[e] * ed[e];
      const float dh = ud[t][e] * eh[e];
      dq[e] = dqo + paw[e] * eu[e];
      db[e] = dbo + maw[e] * eu[e];
      da[e] = dao + aaw[e] * ed[e] + dh;
      // an A^ term of a step in the chunk's last token has no decay up to the chunk's
      // end and adds nothing: left out
      ah[e] = tk[e] == tkl ? 0.0f : cur.av[e] * dh;
      dG[e] = cur.qv[e] * dqo + cur.bv[e] * dbo - cur.av[e] * dao;
    }
    dG[3] += g == 3 ? dc.gam * rs_t : 0.0f;  // G_C: the Gamma term
    float suf[4], pre[4];
    suf[3] = dG[3];
#pragma unroll
    for (int e = 2; e >= 0; --e) suf[e] = dG[e] + suf[e + 1];
    pre[0] = 0.0f;
#pragma unroll
    for (int e = 1; e < 4; ++e) pre[e] = pre[e - 1] + ah[e - 1];
    const float later = group_suffix(suf[0], l);
    const float earlier = group_prefix(pre[3] + ah[3], l);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t s = c * kC + 4 * g + e;
      if (s < NS) {
        float* pr = part + (bh * NS + s) * 4 * DK + ch;
        pr[0] = dq[e];
        pr[DK] = da[e];
        pr[2 * DK] = db[e];
        pr[3 * DK] = ((suf[e] + later) + (pre[e] + earlier)) / cur.alv[e];
      }
    }
    if (t + 1 < KT) cur = nxt;
  }
}

// ---- 5. reduce kernel -------------------------------------------------------------
// One wave per step row: the variant's chain rule (a lane takes dk / 64 consecutive
// channels and dv / 64 consecutive columns).
template <typename In, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(Problem p, GradPtrs g, const float* __restrict__ ws) {
  constexpr int RK = lane_run(DK), RV = lane_run(DV);
  const int lane = threadIdx.x & 63;
  const int64_t T = p.T, H = p.H;
  const int nh = p.n_h;
  const int64_t bth = p.B * T * H * nh;  // step rows
  const BwdLayout L = bwd_layout(p.B, p.steps, H, DK, DV);
  const float* part = ws + L.part;
  const float* dwg = ws + L.dw;
  const In* k = static_cast<const In*>(p.k);
  const In* v = static_cast<const In*>(p.v);
  const In* be = static_cast<const In*>(p.beta);
  const In* bev = static_cast<const In*>(p.beta_v);
  const In* jv = static_cast<const In*>(p.j);
  const In* et = static_cast<const In*>(p.eta);
  auto ld = [](const In* x) { return IO<In>::ld(x); };
  const int ek = lane * RK, ev = lane * RV;
  const bool kl = ek < DK, vl = ev < DV;
  const int var = p.variant;
  const int64_t stride = int64_t(gridDim.x) * (blockDim.x / 64);
  for (int64_t th = int64_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6); th < bth; th += stride) {
    // the gradients of step row th = ((b T + t) H + h) n_h + sub sit at head b H + h, step t n_h + sub
    const int64_t tok = th / nh;
    const int64_t bt = tok / H;
    const int64_t prow = ((bt / T) * H + tok % H) * p.steps + (bt % T) * nh + (th - tok * nh);
    const float* pr = part + prow * 4 * DK;
    float dq[RK], da[RK], db[RK], dal[RK], dw[RV];
    if (kl) {
      ldr<RK>(pr + ek, dq);
      ldr<RK>(pr + DK + ek, da);
      ldr<RK>(pr + 2 * DK + ek, db);
      ldr<RK>(pr + 3 * DK + ek, dal);
    }
    if (vl) ldr<RV>(dwg + prow * DV + ev, dw);
    if (var == GDN_VARIANT_DELTAPRODUCT) {  // th is a step row (token x n_h + step)
      const int sub = int(th - tok * nh);
      const float bt2 = ld(be + th);
      float sb = 0.0f, sal = 0.0f;
      if (kl) {
        float kr[RK], dk[RK];
        ldr<RK>(k + th * DK + ek, kr);
#pragma unroll
        for (int r = 0; r < RK; ++r) {
          dk[r] = da[r] + bt2 * db[r];
          sb += kr[r] * db[r];
          sal += dal[r];
        }
        str<RK>(g.dk + th * DK + ek, dk);
        if (sub == nh - 1) str<RK>(g.dq + tok * DK + ek, dq);
      }
      if (vl) {
        float vc[RV], dvo[RV];
        ldr<RV>(v + th * DV + ev, vc);
#pragma unroll
        for (int r = 0; r < RV; ++r) {
          dvo[r] = bt2 * dw[r];
          sb += vc[r] * dw[r];
        }
        str<RV>(g.dv + th * DV + ev, dvo);
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
    const float sbeta = (var == GDN_VARIANT_KDA || var == GDN_VARIANT_GDN) ? sqrtf(ld(be + th)) : 1.0f;
    const float e = var == GDN_VARIANT_ASYM ? ld(et + th) : 0.0f;
    if (kl) {
      const int64_t ir = th * DK + ek;
      float kr[RK], x[RK], dk[RK], o1[RK], o2[RK];
      ldr<RK>(k + ir, kr);
      str<RK>(g.dq + ir, dq);
      if (var == GDN_VARIANT_FG2) {
        ldr<RK>(be + ir, x);
        float vc[RK], dwk[RK];
        if (!bev) {  // shared beta (dk == dv): the value side of channel c as well
          ldr<RK>(v + th * DV + ek, vc);
          ldr<RK>(dwg + prow * DV + ek, dwk);
        }
#pragma unroll
        for (int r = 0; r < RK; ++r) {
          const float sq = sqrtf(x[r]), dab = da[r] + db[r];
          dk[r] = sq * dab;
          float d2 = kr[r] * dab;
          if (!bev) d2 += vc[r] * dwk[r];
          o1[r] = d2 / (2.0f * sq);
        }
        str<RK>(g.dk + ir, dk);
        str<RK>(g.dalpha + ir, dal);
        str<RK>(g.dbeta + ir, o1);
      } else if (var == GDN_VARIANT_ASYM) {
        ldr<RK>(jv + ir, x);
#pragma unroll
        for (int r = 0; r < RK; ++r) {
          o2[r] = e * db[r];
          sj += x[r] * db[r];
        }
        str<RK>(g.dk + ir, da);
        str<RK>(g.dj + ir, o2);
        str<RK>(g.dalpha + ir, dal);
      } else {
#pragma unroll
        for (int r = 0; r < RK; ++r) {
          const float dab = da[r] + db[r];
          dk[r] = sbeta * dab;
          sk += kr[r] * dab;
          sal += dal[r];
        }
        str<RK>(g.dk + ir, dk);
        if (var == GDN_VARIANT_KDA) str<RK>(g.dalpha + ir, dal);
      }
    }
    if (vl) {
      const int64_t ic = th * DV + ev;
      float vc[RV], dvo[RV], o3[RV];
      ldr<RV>(v + ic, vc);
      if (var == GDN_VARIANT_FG2) {
        float bs[RV];
        ldr<RV>(bev ? bev + ic : be + th * DK + ev, bs);
#pragma unroll
        for (int r = 0; r < RV; ++r) {
          const float sq = sqrtf(bs[r]);
          dvo[r] = sq * dw[r];
          o3[r] = vc[r] * dw[r] / (2.0f * sq);
        }
        if (bev) str<RV>(g.dbeta_v + ic, o3);
      } else {
        const float sc = var == GDN_VARIANT_ASYM ? e : sbeta;
#pragma unroll
        for (int r = 0; r < RV; ++r) {
          dvo[r] = sc * dw[r];
          sv += vc[r] * dw[r];
        }
      }
      str<RV>(g.dv + ic, dvo);
    }
    if (var == GDN_VARIANT_KDA || var == GDN_VARIANT_GDN) {
      const float tot = wave_sum(sk + sv);
      if (lane == 0) g.dbeta[th] = tot / (2.0f * sbeta);
      if (var == GDN_VARIANT_GDN) {
        const float ta = wave_sum(sal);
        if (lane == 0) g.dalpha[th] = ta;
      }
    } else if (var == GDN_VARIANT_ASYM) {
      const float tot = wave_sum(sj + sv);
      if (lane == 0) g.deta[th] = tot;
    }
  }
}

template <typename In, int DK, int DV>
int launch_shape(const Problem& p, const In* dO, const float* dsf, const GradPtrs& g, float* ws, hipStream_t s) {
  const BwdLayout L = bwd_layout(p.B, p.steps, p.H, DK, DV);
  const int64_t bh = p.B * p.H;
  const int64_t items = bh * L.nc;  // (batch*head, chunk) pairs
  // grids: B*H*steps <= 2^33 (checked by the caller), so every one fits 32 bits
  if (items > 0) {
    bwd_ops_kernel<In, DK, DV><<<dim3(unsigned((items * kC + 3) / 4)), dim3(256), 0, s>>>(p, dO, ws);
    bwd_rec_kernel<DK, DV><<<dim3(unsigned(items)), dim3(64), 0, s>>>(p, ws);
  }
  bwd_chain_kernel<DK, DV><<<dim3(unsigned(2 * bh * (DV / 16))), dim3(64 * chain_waves(DK)), 0, s>>>(p, dsf, g.ds0, ws);
  if (items == 0) return int(hipGetLastError());
  bwd_intra_kernel<DK, DV><<<dim3(unsigned(items / 2)), dim3(128), 0, s>>>(p, ws);  // chunk pairs
  const int64_t waves = p.B * p.T * p.H * p.n_h;
  const int64_t blocks = (waves + 3) / 4;
  bwd_reduce_kernel<In, DK, DV><<<dim3(unsigned(blocks < (int64_t(1) << 20) ? blocks : (int64_t(1) << 20))), dim3(256), 0, s>>>(p, g, ws);
  return int(hipGetLastError());
}

template <typename In, int DK>
int launch_dk(const Problem& p, const In* dO, const float* dsf, const GradPtrs& g, float* ws, hipStream_t s) {
  switch (p.dv) {
    case 16: return launch_shape<In, DK, 16>(p, dO, dsf, g, ws, s);
    case 32: return launch_shape<In, DK, 32>(p, dO, dsf, g, ws, s);
    case 64: return launch_shape<In, DK, 64>(p, dO, dsf, g, ws, s);
    case 128: return launch_shape<In, DK, 128>(p, dO, dsf, g, ws, s);
    default: return int(hipErrorInvalidValue);
  }
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
