// Chunkwise-parallel forward pass (WY / UT form): device code shared by the
// per-variant preparation units (gdn_prep_*.hip) and the scan unit (gdn_chunk.hip).
//
// Unified step (gdn.h): S_t = (I - a_t b_t^T) Diag(alpha_t) S_{t-1} + a_t w_t^T,
// o_t = S_t^T q_t. Take a chunk of C steps with start state S and inclusive
// cumulative log-decay G_r = sum_{s<=r} log alpha_s (per key channel). Writing
// u_r for the correction of step r (S_r = Diag(alpha_r) S_{r-1} + a_r u_r^T),
//   u_r = w_r - S^T (b_r . e^{G_r}) - sum_{s<r} <b_r . e^{G_r}, a_s . e^{-G_s}> u_s,
// so with B+ = B . e^G, A- = A . e^{-G}, M = strict_tril(B+ A-^T) and
// T = (I + M)^{-1} (unit lower triangular):
//   U = U~ - W S,   U~ = T Wv,   W = T B+
//   S' = Diag(e^{G_C}) S + A^^T U,          A^ = A . e^{G_C - G}
//   O  = Q+ S + P U,  Q+ = Q . e^{G},  P = tril_incl(Q+ A-^T)
// This is the diagonal-plus-rank-1 chunk recursion that the FG2-GDN reading
// notes (section 2.4) inherit from KDA's WY/UT algorithm, written out for the
// unified step. No factor e^{G_i - G_j} is formed whole: with one decay per step
// (GDN, DeltaProduct) the Gram products carry no decay and their entries are
// multiplied by e^{G_i - G_j} <= 1 afterwards; with per-channel decay every factor
// is split at a reference point inside the chunk's 16-step tiles (the first and
// last rows of a tile for its off-diagonal blocks, its row 7 for the diagonal
// block), so that none exceeds the decay of 8 steps.
//
// Kernel 1 (chunk_prep): persistent; each workgroup walks chunks. Wave w owns
// rows 16w..16w+15 of the chunk: it loads them straight into registers (16-byte
// fragments, the next chunk's rows in flight while the current one is processed),
// scans the log decay over its rows with DPP row shifts, and forms the decayed
// operands. LDS carries only what crosses waves (per-channel decay constants, A-
// for the Grams, B+ and Wv transposed, then M and T). It writes one record per
// chunk (gdn_internal.h). The variant is a template parameter: one translation
// unit per variant.
// Kernel 2 (chunk_scan): one workgroup per (batch*head, 64 value columns); each
// wave owns 16 value columns and carries its dk x 16 fp32 state slice in MFMA
// accumulator registers across all chunks. The next chunk's record is copied
// into LDS (a flat image) while the current one is processed.
//
// Precision (bf16 inputs): the Gram products run as bf16 hi/lo splits (three
// bf16 MFMAs, about 16 mantissa bits, full fp32 range); every other product runs
// on fp16 MFMA with fp32 accumulation. Quantities whose scale follows the
// caller's values (v, q, the state, U) are multiplied by exact powers of two
// before the fp16 conversion and divided back after the product, so fp16's
// range never clips them. fp32 inputs use fp32 MFMA throughout.
#pragma once

#include <algorithm>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// The state and U enter fp16 MFMAs with their per-column maximum scaled into
// [2^12, 2^13): far below fp16's 65504 and well above its subnormal range.
constexpr int kStateScaleExp = 12;

union H8 {
  half8 h;
  bhalf8 b;
  uint2 u[2];
  uint4 q;
};

// ---- lane channel maps -------------------------------------------------------------
// A lane (i = lane % 16, g = lane / 16) of the wave that owns a 16-row tile holds
// NX = D / 4 channels of its row, in 16-byte groups:
//   bf16 rows:  UW = min(8, D/4) consecutive channels per group, channel of value x
//               = (x / UW) * 4 UW + UW g + x % UW  (the natural k order of the
//               16x16x32 MFMA: slot s of k-block u is channel 32 u + 8 g + s)
//   fp32 rows:  4 consecutive channels per group, channel = (x / 4) 16 + 4 g + x % 4
//               (slot g of the e-th 16x16x4 MFMA of slice t is channel 16 t + 4 g + e)
template <bool F16, int D>
struct ChanMap {
  static constexpr int NX = D / 4;
  static constexpr int UW = F16 ? (NX < 8 ? NX : 8) : 4;
  static constexpr int NU = NX / UW;
  __device__ static constexpr int chan(int g, int x) {
    return (x / UW) * 4 * UW + UW * g + (x % UW);
  }
};

// Load group u (UW consecutive channels) of the lane's channels of a row (fp32 out).
template <bool F16, int D, typename In>
__device__ __forceinline__ void load_unit(const In* row, int g, int u, float* out) {
  using M = ChanMap<F16, D>;
  const In* p = row + u * 4 * M::UW + M::UW * g;
  if constexpr (std::is_same<In, float>::value) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    out[0] = x.x;
    out[1] = x.y;
    out[2] = x.z;
    out[3] = x.w;
  } else if constexpr (M::UW == 8) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = __uint_as_float(w[e] << 16);
      out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    out[0] = __uint_as_float(x.x << 16);
    out[1] = __uint_as_float(x.x & 0xffff0000u);
    out[2] = __uint_as_float(x.y << 16);
    out[3] = __uint_as_float(x.y & 0xffff0000u);
  }
}

// All NX channels of the lane's row.
template <bool F16, int D, typename In>
__device__ __forceinline__ void load_row(const In* row, int g, float* out) {
  using M = ChanMap<F16, D>;
#pragma unroll
  for (int u = 0; u < M::NU; ++u) load_unit<F16, D>(row, g, u, out + u * M::UW);
}

// Written values w of one row (the lane's DV/4 value channels), vector loads.
// Returns max |w| (pass 0) or stores fp16/fp32 w * scale transposed into wvt
// (pass 1).
template <bool F16, int DVT, typename In, typename Op, int LDC>
__device__ __forceinline__ float row_values(int variant, const In* vrow, const In* brow, int bstride_dk,
                                            const In* bvrow, float wscal, bool valid, int g, int r,
                                            float scale, Op (*wvt)[LDC], bool store) {
  using M = ChanMap<F16, DVT>;
  float w[M::NX];
#pragma unroll
  for (int x = 0; x < M::NX; ++x) w[x] = 0.0f;
  if (valid) {
    load_row<F16, DVT>(vrow, g, w);
    if (variant == GDN_VARIANT_FG2) {
      float bq[M::NX];
      load_row<F16, DVT>(bvrow ? bvrow : brow, g, bq);
#pragma unroll
      for (int x = 0; x < M::NX; ++x) w[x] *= sqrtf(bq[x]);
    } else {
#pragma unroll
      for (int x = 0; x < M::NX; ++x) w[x] *= wscal;
    }
  }
  (void)bstride_dk;
  float mx = 0.0f;
#pragma unroll
  for (int x = 0; x < M::NX; ++x) {
    mx = fmaxf(mx, fabsf(w[x]));
    if (store) wvt[M::chan(g, x)][r] = (Op)(w[x] * scale);
  }
  return mx;
}

__device__ __forceinline__ void quad(const float* p, float out[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  out[0] = x.x;
  out[1] = x.y;
  out[2] = x.z;
  out[3] = x.w;
}

// Eight 16-bit operand values: 4 at p0 and 4 at p1 (or zeros).
__device__ __forceinline__ H8 pair4(const void* p0, const void* p1) {
  H8 r;
  r.u[0] = *reinterpret_cast<const uint2*>(p0);
  r.u[1] = p1 ? *reinterpret_cast<const uint2*>(p1) : make_uint2(0u, 0u);
  return r;
}

// DPP lane permutation CTRL of a float (every lane reads a lane of its own row).
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Maximum over the wave: within each 16-lane row by DPP lane swaps (quads, then
// half-row and row mirrors), across rows by the lane-swap instructions.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_perm<0xb1>(x));   // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_perm<0x4e>(x));   // quad_perm 2,3,0,1
  x = fmaxf(x, dpp_perm<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_perm<0x140>(x));  // row_mirror
  return max_over_groups(x);
}

// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16 g .. 16 g + 15,
// the rows of a tile): four row-shift adds; lanes shifted in from outside the row
// read zero (bound control).
__device__ __forceinline__ float scan16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
  return x;
}

inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// ---- kernel 1: chunk-local preparation -----------------------------------------------

// The log decay is kept in base 2 on the bf16 path (hardware log2 / exp2 / rcp /
// sqrt: one instruction each, about 1 ulp) and in base e with the accurate library
// calls on the fp32 path.
template <bool F16>
__device__ __forceinline__ float path_log(float x) {
  if constexpr (F16) return __builtin_amdgcn_logf(x);
  else return logf(x);
}
template <bool F16>
__device__ __forceinline__ float path_exp(float x) {
  if constexpr (F16) return __builtin_amdgcn_exp2f(x);
  else return expf(x);
}
template <bool F16>
__device__ __forceinline__ float path_sqrt(float x) {
  if constexpr (F16) return __builtin_amdgcn_sqrtf(x);
  else return sqrtf(x);
}

// Value x (compile-time after unrolling) of bf16 groups held as uint4 (8 per group).
__device__ __forceinline__ float bf16_at(const uint4* v, int x) {
  const uint4 w = v[x / 8];
  const uint32_t word = (x % 8) / 2 == 0 ? w.x : (x % 8) / 2 == 1 ? w.y : (x % 8) / 2 == 2 ? w.z : w.w;
  return __uint_as_float((x & 1) ? (word & 0xffff0000u) : (word << 16));
}

// Raw bf16 inputs of one step row, loaded one chunk ahead of use.
template <int DK>
struct RawRow {
  using KM = ChanMap<true, DK>;
  static constexpr int KU = KM::UW == 8 ? KM::NU : 1;  // uint4 groups per key row
  uint4 k[KU], a[KU], bj[KU], q[KU];
  uint4 v[4], bv[4];
  float s_alpha, s_beta, s_eta;
};

template <bool F16, int DK, int C, bool DPV>
struct alignas(16) PrepLds {
  using Op = std::conditional_t<F16, _Float16, float>;
  using Am = std::conditional_t<F16, __bf16, float>;
  static constexpr int NT = C / 16;
  static constexpr int LDA = F16 ? DK + 8 : DK + 4;  // rows of the A sides (16-byte aligned)
  static constexpr int LDC = C + 4;
  static constexpr int QR = DPV ? C / 2 : 1;         // output rows kept in LDS (n_h >= 2)
  union RA {
    struct {
      float L[NT][DK];         // tile totals of the log decay, per channel
      float m[NT][DK];         // in-tile prefix at each tile's row 7
    } stg;                     // decay staging, read by the per-channel pass
    struct {
      Am hi[C][LDA];
      Am lo[F16 ? C : 1][LDA];
    } am;                      // A sides of the Gram blocks, one 16-row slot per tile
    struct {
      float m[C][LDC];         // strictly lower Gram M; T in fp16 after the inverse
      float t[C][LDC];         // T = (I + M)^{-1}
    } mt;
  } ra;
  Op bt[DK][LDC];              // B+ (chunk-start reference), transposed
  Op wvt[128][LDC];            // written values (scaled), transposed
  Op at[F16 ? 1 : DK][LDC];    // A^ transposed, staged for a coalesced copy (fp32 path)
  Am qmh[QR][LDA];             // Q of output rows (no decay), DeltaProduct only
  Am qml[(DPV && F16) ? QR : 1][LDA];
  union CU {
    struct {
      // per tile t and channel: [0] m_t, [1] e^m_t, [2] e^(L_t - m_t), [3] e^(sum of
      // L before t), [4] e^(sum of L after t) (base 2 on the bf16 path)
      float cst[NT][5][DK];
      float dfac[NT == 4 ? 2 : 1][DK];  // e^L_1 and e^L_2 (chunk 64)
    } v;                       // per-channel decay
    struct {
      float ltot[4];           // tile totals of the scalar log decay
      float grow[C];           // log decay from the chunk start through each row
    } s;                       // scalar decay
  } cu;
  float qs[C];                 // per output row q scale
  float red[kWaves];
};

// Waves per SIMD (= workgroups per CU) chunk_prep_kernel is compiled for: three for
// fp32 rows of 64 channels in chunks of up to 32 steps (at most 168 registers a lane,
// 48 KB of LDS a workgroup), which hides more of its load latency than two; one
// (no register cap) otherwise.
template <typename In, int DK, int C>
constexpr int prep_occupancy() {
  return (std::is_same<In, float>::value && DK == 64 && C <= 32) ? 3 : 1;
}

// V: the variant (gdn_variant); DPV: DeltaProduct with n_h >= 2 (output rows are
// every n_h-th step row).
template <typename In, int DK, int C, int V, bool DPV>
__global__ __launch_bounds__(kThreads, (prep_occupancy<In, DK, C>())) void chunk_prep_kernel(Problem p, unsigned char* __restrict__ ws,
                                                              ChunkLayout L, int want_out) {
  constexpr bool F16 = std::is_same<In, uint16_t>::value;
  constexpr bool DP = V == GDN_VARIANT_DELTAPRODUCT;
  static_assert(!DPV || DP, "multi-step rows are DeltaProduct only");
  constexpr bool CH_ALPHA = V == GDN_VARIANT_FG2 || V == GDN_VARIANT_KDA || V == GDN_VARIANT_ASYM;
  constexpr bool CH_BJ = V == GDN_VARIANT_FG2 || V == GDN_VARIANT_ASYM;  // per-channel beta / j
  constexpr bool SCALAR = !CH_ALPHA;  // one log decay per row (GDN, DeltaProduct)
  using Sm = PrepLds<F16, DK, C, DPV>;
  using Op = typename Sm::Op;
  using KM = ChanMap<F16, DK>;
  using Raw = RawRow<DK>;
  constexpr int NX = KM::NX;
  constexpr int UW = KM::UW;
  constexpr int NT = C / 16;
  constexpr int KB = F16 ? (DK + 31) / 32 : DK / 16;  // k-blocks (F16) or slices (F32) of a key row
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  static_assert(NT <= kWaves, "one wave per 16-row tile");
  static_assert(DK <= kThreads, "one thread per channel for the decay constants");
  // fragment-ordered record (the row-split scan's operand order)
  constexpr bool FRAG = frag_layout(sizeof(Op), DK, C);
  constexpr int CK = C / 32;  // k-blocks of 32 steps (fragment format)
  __shared__ Sm sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n_h = DPV ? p.n_step : 1;  // steps a token takes in the chunk
  const int R = p.rows_out, RT = (R + 15) / 16;  // output rows, 16-row tiles (R = 8: one)
  const int dv = int(p.dv);
  const int NC = int(p.nchunks);
  const int H = int(p.H);
  const int BH = int(p.B) * H;
  const int total = NC * BH;  // < 2^31 (checked on the host)
  const In* qg = static_cast<const In*>(p.q);
  const In* kg = static_cast<const In*>(p.k);
  const In* vg = static_cast<const In*>(p.v);
  const In* alg = static_cast<const In*>(p.alpha);
  const In* beg = static_cast<const In*>(p.beta);
  const In* bvg = static_cast<const In*>(p.beta_v);
  const In* jg = static_cast<const In*>(p.j);
  const In* etg = static_cast<const In*>(p.eta);
  const bool owner = wave < NT;
  const int r = 16 * wave + li;  // virtual row (step) in the chunk owned by this lane
  // FG2 with its own value-side beta; otherwise (dk == dv) the key-side sqrt(beta)
  // of the same channel scales the value
  const bool bv_sep = V == GDN_VARIANT_FG2 && bvg != nullptr;
  // value-row groups: 8 bf16 channels (32 u + 8 g + s) per uint4, or 4 (4 g + s) when dv == 16
  const int vuw = (F16 && dv == 16) ? 4 : 8;
  const int vnu = F16 ? (dv == 16 ? 1 : dv / 32) : 0;
  auto ld = [](const In* x) { return IO<In>::ld(x); };

  struct Where {
    bool valid, out_row;
    int64_t th, vrow;
    int sub, ro;
    bool pad;  // identity step of a padded token (beta = 0)
  };
  auto where = [&](int item) __attribute__((always_inline)) -> Where {
    Where w;
    // chunk-major order: the workgroups in flight read the same tokens of every
    // head, i.e. contiguous memory ([B, T, H, d] rows of one token are adjacent)
    const int n = item / BH, bh = item - n * BH;  // chunk n of the launch
    const int b = bh / H, h = bh - b * H;
    const int64_t vs = (p.c0 + n) * C + r;
    w.valid = owner && vs < p.steps;
    int64_t tok = vs;
    w.sub = 0;
    if constexpr (DPV) {
      tok = vs / n_h;
      w.sub = int(vs - tok * n_h);
    }
    w.th = (int64_t(b) * p.T + tok) * H + h;
    w.pad = w.sub >= p.n_h;
    w.vrow = DP ? w.th * p.n_h + (w.pad ? p.n_h - 1 : w.sub) : w.th;
    w.out_row = want_out && owner && w.sub == n_h - 1;
    w.ro = DPV ? r / n_h : r;
    return w;
  };
  // Issue the loads of this lane's row of the item at `w` (bf16 rows only; fp32 rows
  // are read where they are used): part 0 key, 1 decay, 2 beta / j, 3 query,
  // 4 values, -1 all. Spreading the parts over the iteration keeps the memory
  // pipeline busy without stalling the issuing wave on a burst of requests.
  auto prefetch = [&](const Where& w, Raw& raw, int part) __attribute__((always_inline)) {
    if constexpr (F16) {
      if (!w.valid) return;
      const bool all = part < 0;
      auto ld_row = [&](const In* row, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < Raw::KU; ++u) {
          if constexpr (UW == 8) {
            dst[u] = *reinterpret_cast<const uint4*>(row + u * 32 + 8 * lg);
          } else {
            const uint2 x = *reinterpret_cast<const uint2*>(row + 4 * lg);
            dst[u] = make_uint4(x.x, x.y, 0u, 0u);
          }
        }
      };
      if (all || part == 0) ld_row(kg + w.vrow * DK, raw.k);
      if (all || part == 1) {
        if constexpr (CH_ALPHA) ld_row(alg + w.th * DK, raw.a);
        else raw.s_alpha = ld(alg + w.th);
      }
      if (all || part == 2) {
        if constexpr (V == GDN_VARIANT_FG2) ld_row(beg + w.th * DK, raw.bj);
        if constexpr (V == GDN_VARIANT_ASYM) {
          ld_row(jg + w.th * DK, raw.bj);
          raw.s_eta = ld(etg + w.th);
        }
        if constexpr (V == GDN_VARIANT_KDA || V == GDN_VARIANT_GDN) raw.s_beta = ld(beg + w.th);
        if constexpr (DP) raw.s_beta = w.pad ? 0.0f : ld(beg + w.vrow);
      }
      if ((all || part == 3) && w.out_row) ld_row(qg + w.th * DK, raw.q);
      const In* vrow = vg + w.vrow * dv;
      const In* bvrow = bvg + w.th * dv;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if ((all || part == 4) && u < vnu) {
          if (vuw == 8) {
            raw.v[u] = *reinterpret_cast<const uint4*>(vrow + u * 32 + 8 * lg);
            if (bv_sep) raw.bv[u] = *reinterpret_cast<const uint4*>(bvrow + u * 32 + 8 * lg);
          } else {
            const uint2 x = *reinterpret_cast<const uint2*>(vrow + 4 * lg);
            raw.v[u] = make_uint4(x.x, x.y, 0u, 0u);
            if (bv_sep) {
              const uint2 y = *reinterpret_cast<const uint2*>(bvrow + 4 * lg);
              raw.bv[u] = make_uint4(y.x, y.y, 0u, 0u);
            }
          }
        }
      }
    }
  };

  // fragment-format offsets (elements) of this lane's 4 consecutive values of an
  // accumulator tile: P row ro, steps 16 J + 4 lg ..; W row 16 I + li, channels
  // 16 ct + 4 lg ..; U~ steps 16 I + 4 lg .., value column 16 ct + li.
  auto p_frag = [&](int ro, int J) -> size_t {
    return size_t((((ro >> 4) * CK + (J >> 1)) * 64 + (ro & 15) + 16 * (2 * (J & 1) + (lg >> 1))) * 8 + 4 * (lg & 1));
  };
  auto w_frag = [&](int I, int ct) -> size_t {
    return size_t(((I * KB + (ct >> 1)) * 64 + li + 16 * (2 * (ct & 1) + (lg >> 1))) * 8 + 4 * (lg & 1));
  };
  auto u_frag = [&](int I, int ct) -> size_t { return size_t(((I * (dv / 16) + ct) * 64 + lane) * 4); };

  // 0/1 selection fragments (B operand of a 16x16x32 MFMA) that move the k-slot of
  // relative channel 16 h + n to column n: with an A operand holding one row group
  // (lane (i, g): channels of slots 8 g + s), the product is that group transposed.
  half8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const bool hit = UW == 8 ? (8 * lg + s2 == li + 16 * hh) : (s2 < UW && UW * lg + s2 == li + 16 * hh);
      sel[hh][s2] = hit ? (_Float16)1.0f : (_Float16)0.0f;
    }

  Raw raw;
  if (int(blockIdx.x) < total) prefetch(where(blockIdx.x), raw, -1);

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const Where w = where(item);
    const bool has_next = item + int(gridDim.x) < total;
    const Where wn = where(has_next ? item + int(gridDim.x) : item);
    const int item_n = item / BH;
    unsigned char* rec = ws + (size_t(item - item_n * BH) * size_t(NC) + size_t(item_n)) * L.bytes;
    Op* W_g = reinterpret_cast<Op*>(rec + L.off_W);
    Op* AT_g = reinterpret_cast<Op*>(rec + L.off_AT);
    Op* Q_g = reinterpret_cast<Op*>(rec + L.off_Q);
    Op* P_g = reinterpret_cast<Op*>(rec + L.off_P);
    Op* UT_g = reinterpret_cast<Op*>(rec + L.off_UT);
    float* gam_g = reinterpret_cast<float*>(rec + L.off_gamma);
    float* winv_g = reinterpret_cast<float*>(rec + L.off_winv);
    float* qinv_g = reinterpret_cast<float*>(rec + L.off_qinv);

    // ---- this lane's row: write key a, erase key bb, log decay G, query, values ----
    float a[NX], bb[NX], G[NX], qv[NX];
    float wv[32];  // written values (bf16 path; the fp32 path reads them later)
#pragma unroll
    for (int x = 0; x < NX; ++x) a[x] = bb[x] = G[x] = qv[x] = 0.0f;
#pragma unroll
    for (int x = 0; x < 32; ++x) wv[x] = 0.0f;
    float wscal = 0.0f;
    if (w.valid) {
      float kf[NX], af[NX], bf[NX];
      float sa = 0.0f, sbt = 0.0f, seta = 0.0f;
      if constexpr (F16) {
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          kf[x] = bf16_at(raw.k, x);
          af[x] = CH_ALPHA ? bf16_at(raw.a, x) : 0.0f;
          bf[x] = CH_BJ ? bf16_at(raw.bj, x) : 0.0f;
        }
        sa = raw.s_alpha;
        sbt = raw.s_beta;
        seta = raw.s_eta;
        if (w.out_row) {
#pragma unroll
          for (int x = 0; x < NX; ++x) qv[x] = bf16_at(raw.q, x);
        }
      } else {
        load_row<F16, DK>(kg + w.vrow * DK, lg, kf);
        if constexpr (CH_ALPHA) load_row<F16, DK>(alg + w.th * DK, lg, af);
        else sa = ld(alg + w.th);
        if constexpr (V == GDN_VARIANT_FG2) load_row<F16, DK>(beg + w.th * DK, lg, bf);
        if constexpr (V == GDN_VARIANT_ASYM) {
          load_row<F16, DK>(jg + w.th * DK, lg, bf);
          seta = ld(etg + w.th);
        }
        if constexpr (V == GDN_VARIANT_KDA || V == GDN_VARIANT_GDN) sbt = ld(beg + w.th);
        if constexpr (DP) sbt = w.pad ? 0.0f : ld(beg + w.vrow);
        if (w.out_row) load_row<F16, DK>(qg + w.th * DK, lg, qv);
      }
      if constexpr (V == GDN_VARIANT_ASYM) {
        if (p.stabilize) {  // GDN2 stabiliser on this row's D or j (row = 4 lane groups)
          const StabCoef sc = stab_coef<NX>(
              p.stabilize, seta, [&](int i) { return KJD{kf[i], bf[i], af[i]}; },
              [](float x) { return sum_over_groups(x); }, [](float x) { return max_over_groups(x); });
#pragma unroll
          for (int x = 0; x < NX; ++x) {
            af[x] = stab_decay(sc, af[x]);
            bf[x] = stab_j(sc, kf[x], bf[x]);
          }
        }
      }
      float sbk[NX];  // FG2: sqrt(beta) per key channel
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        if constexpr (V == GDN_VARIANT_FG2) {
          sbk[x] = path_sqrt<F16>(bf[x]);
          a[x] = sbk[x] * kf[x];
          bb[x] = a[x];
          G[x] = path_log<F16>(af[x]);
        } else if constexpr (V == GDN_VARIANT_KDA || V == GDN_VARIANT_GDN) {
          a[x] = kf[x];  // scaled by sqrt(beta) below
          G[x] = V == GDN_VARIANT_KDA ? path_log<F16>(af[x]) : 0.0f;
        } else if constexpr (DP) {
          a[x] = kf[x];
          bb[x] = sbt * kf[x];
        } else {  // ASYM
          a[x] = kf[x];
          bb[x] = seta * bf[x];
          G[x] = path_log<F16>(af[x]);
        }
      }
      if constexpr (V == GDN_VARIANT_KDA || V == GDN_VARIANT_GDN) {
        const float sb = path_sqrt<F16>(sbt);
        const float lga = V == GDN_VARIANT_GDN ? path_log<F16>(sa) : 0.0f;
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          a[x] *= sb;
          bb[x] = a[x];
          if constexpr (V == GDN_VARIANT_GDN) G[x] = lga;
        }
        wscal = sb;
      } else if constexpr (DP) {
        const float lgate = w.sub == 0 ? path_log<F16>(sa) : 0.0f;
#pragma unroll
        for (int x = 0; x < NX; ++x) G[x] = lgate;
        wscal = sbt;
      } else if constexpr (V == GDN_VARIANT_ASYM) {
        wscal = seta;
      }
      if constexpr (F16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (u < vnu) {
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
              const int y = 8 * u + s2;
              float f = wscal;
              if constexpr (V == GDN_VARIANT_FG2)
                f = bv_sep ? path_sqrt<F16>(bf16_at(raw.bv, y)) : sbk[y < NX ? y : 0];
              wv[y] = (vuw == 8 || s2 < 4) ? bf16_at(raw.v, y) * f : 0.0f;
            }
          }
        }
      }
    }

    // The raw rows are consumed: the next item's loads go out part by part.
    if (has_next) prefetch(wn, raw, 0);
    // inclusive scan of the log decay over each 16-row tile; the tile totals (row
    // 15) and the prefixes at row 7 go to LDS
    if constexpr (SCALAR) {
      G[0] = scan16(G[0]);
      if (owner && li == 15 && lg == 0) sm.cu.s.ltot[wave] = G[0];
    } else {
#pragma unroll
      for (int x = 0; x < NX; ++x) G[x] = scan16(G[x]);
      if (owner && (li == 15 || li == 7)) {
        float* dst = li == 15 ? &sm.ra.stg.L[wave][0] : &sm.ra.stg.m[wave][0];
#pragma unroll
        for (int x = 0; x < NX; ++x) dst[KM::chan(lg, x)] = G[x];
      }
    }
    // power-of-two scales: per output row for q, per chunk for the written values
    float qsc = 1.0f;
    float wmax = 0.0f;
    if constexpr (F16) {
      if (owner && want_out) {
        float mx = 0.0f;
#pragma unroll
        for (int x = 0; x < NX; ++x) mx = fmaxf(mx, fabsf(qv[x]));
        qsc = pow2_scale_for(max_over_groups(mx));
      }
#pragma unroll
      for (int x = 0; x < 32; ++x) wmax = fmaxf(wmax, fabsf(wv[x]));
      wmax = wave_max(wmax);
      if (lane == 0) sm.red[wave] = wmax;
    }
    __syncthreads();

    // ---- decay constants (the reference points of chunk_prep2_kernel; base e on
    // the fp32 path): scalar decay per row, per-channel decay per tile ----
    float gabs = 0.0f, eg_row = 1.0f, eat_row = 1.0f;
    if constexpr (SCALAR) {
      float pre = 0.0f, gc = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float lt = sm.cu.s.ltot[t];
        if (t < wave) pre += lt;
        gc += lt;
      }
      gabs = pre + G[0];                                       // G of this row
      eg_row = path_exp<F16>(gabs);                            // e^{G}
      eat_row = path_exp<F16>(fminf(gc - gabs, 0.0f));         // e^{G_C - G}
      if (owner && lg == 0) sm.cu.s.grow[r] = gabs;
      if (tid < DK) gam_g[tid] = path_exp<F16>(gc);
    } else if (tid < DK) {
      const int c = tid;
      float Lt[NT], mt[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        Lt[t] = sm.ra.stg.L[t][c];
        mt[t] = sm.ra.stg.m[t][c];
      }
      float pre = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float suf = 0.0f;
#pragma unroll
        for (int t2 = t + 1; t2 < NT; ++t2) suf += Lt[t2];
        sm.cu.v.cst[t][0][c] = mt[t];
        sm.cu.v.cst[t][1][c] = path_exp<F16>(mt[t]);          // e^{G_7 - G_start}
        sm.cu.v.cst[t][2][c] = path_exp<F16>(Lt[t] - mt[t]);  // e^{G_end - G_7}
        sm.cu.v.cst[t][3][c] = path_exp<F16>(pre);            // e^{G_start}
        sm.cu.v.cst[t][4][c] = path_exp<F16>(suf);            // e^{G_C - G_end}
        pre += Lt[t];
      }
      if constexpr (NT == 4) {
        sm.cu.v.dfac[0][c] = path_exp<F16>(Lt[1]);
        sm.cu.v.dfac[1][c] = path_exp<F16>(Lt[2]);
      }
      gam_g[c] = path_exp<F16>(pre);
    }
    float wsc = 1.0f;
    if constexpr (F16) {
      float m = sm.red[0];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) m = fmaxf(m, sm.red[w2]);
      wsc = pow2_scale_for(m);
    }
    if (tid == 0) winv_g[0] = 1.0f / wsc;
    __syncthreads();

    // ---- decayed operands of this wave's rows ----
    // Per-channel decay (reference points as in chunk_prep2_kernel): B and Q sides of
    // the off-diagonal Gram blocks at the tile's first row (registers), A side at its
    // last row (LDS slot = tile; the last tile's A side is never an off-diagonal
    // operand, and with chunk 64 slot 3 holds tile 0's A side at the reference
    // between tiles 1 and 2), the diagonal blocks at the tile's row 7, on fp32 MFMA
    // from registers. Scalar decay: the Gram operands carry no decay.
    float bm[NX];  // B side of the off-diagonal (scalar decay: every) Gram block
    float qm[NX];  // Q side likewise
#pragma unroll
    for (int x = 0; x < NX; ++x) bm[x] = qm[x] = 0.0f;
    float4v mdg = {0.0f, 0.0f, 0.0f, 0.0f}, pdg = {0.0f, 0.0f, 0.0f, 0.0f};  // diagonal M^T, P^T
    if (owner) {
#pragma unroll
      for (int u = 0; u < NX / UW; ++u) {
        const int c0 = KM::chan(lg, u * UW);  // UW consecutive channels
        float cm[UW], c7[UW], c157[UW], cP[UW], cQ[UW];
        if constexpr (!SCALAR) {
#pragma unroll
          for (int e = 0; e < UW; e += 4) {
            float* dsts[5] = {cm, c7, c157, cP, cQ};
#pragma unroll
            for (int k5 = 0; k5 < 5; ++k5) {
              const float4 x = *reinterpret_cast<const float4*>(&sm.cu.v.cst[wave][k5][c0 + e]);
              dsts[k5][e] = x.x, dsts[k5][e + 1] = x.y, dsts[k5][e + 2] = x.z, dsts[k5][e + 3] = x.w;
            }
          }
        }
        float amv[UW];
        half8 xbt = {}, xat = {};  // fp16 B+ and A^ of the group (bf16 path)
#pragma unroll
        for (int e = 0; e < UW; ++e) {
          const int x = u * UW + e, c = c0 + e;
          float bplus, ahat, qplus;
          if constexpr (SCALAR) {
            amv[e] = a[x];
            bm[x] = bb[x];
            qm[x] = qv[x];
            bplus = bb[x] * eg_row;
            ahat = a[x] * eat_row;
            qplus = qv[x] * eg_row;
          } else {
            float fup, eam;  // e^{G - G_7}, e^{G_7 - G}
            if constexpr (F16) {
              fup = path_exp<F16>(G[x] - cm[e]);
              eam = __builtin_amdgcn_rcpf(fup);
            } else {
              fup = expf(G[x] - cm[e]);
              eam = expf(cm[e] - G[x]);
            }
            const float st = fup * c7[e];    // e^{G - G_start}
            const float te = eam * c157[e];  // e^{G_end - G}
            amv[e] = a[x] * te;
            bm[x] = bb[x] * st;
            qm[x] = qv[x] * st;
            bplus = bm[x] * cP[e];
            ahat = amv[e] * cQ[e];
            qplus = qm[x] * cP[e];
            const float ad = a[x] * eam;
            mdg = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, bb[x] * fup, mdg, 0, 0, 0);
            pdg = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, qv[x] * fup, pdg, 0, 0, 0);
          }
          if constexpr (F16) {
            xbt[e] = (_Float16)bplus;
            xat[e] = (_Float16)ahat;
          } else {
            sm.bt[c][r] = (Op)bplus;
            sm.at[c][r] = (Op)ahat;
          }
          qv[x] = qplus * qsc;  // Q+ (chunk-start reference), scaled
        }
        if constexpr (F16) {
          // B+ and A^ of this row group transposed by MFMA (product with a 0/1
          // selection matrix: exact): lane (li, lg) then holds 4 consecutive steps
          // 16 w + 4 lg .. of channel ch0 + 16 h + li
          const int ch0 = u * 4 * UW;
#pragma unroll
          for (int hh = 0; hh < UW / 4; ++hh) {
            const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
            const float4v tb = mma_pair_f16(xbt, sel[hh], zero);
            const float4v ta = mma_pair_f16(xat, sel[hh], zero);
            const int c = ch0 + 16 * hh + li;
            H8 pb, pa;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pb.h[e] = (_Float16)tb[e];
              pa.h[e] = (_Float16)ta[e];
            }
            *reinterpret_cast<uint2*>(&sm.bt[c][16 * wave + 4 * lg]) = pb.u[0];
            Op* adst = FRAG ? AT_g + size_t((((c >> 4) * CK + (wave >> 1)) * 64 + li + 16 * (2 * (wave & 1) + (lg >> 1))) * 8 +
                                            4 * (lg & 1))
                            : AT_g + size_t(c) * L.ldc + 16 * wave + 4 * lg;
            *reinterpret_cast<uint2*>(adst) = pa.u[0];
          }
        }
        // A side: bf16 hi / lo (or fp32), one vector store each, to slot `row`
        auto store_a = [&](int row, const float* v8) __attribute__((always_inline)) {
          if constexpr (F16) {
            H8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = e < UW ? v8[e < UW ? e : 0] : 0.0f;
              hi.b[e] = (__bf16)v;
              lo.b[e] = (__bf16)(v - (float)hi.b[e]);
            }
            if constexpr (UW == 8) {
              *reinterpret_cast<uint4*>(&sm.ra.am.hi[row][c0]) = hi.q;
              *reinterpret_cast<uint4*>(&sm.ra.am.lo[row][c0]) = lo.q;
            } else {
              *reinterpret_cast<uint2*>(&sm.ra.am.hi[row][c0]) = hi.u[0];
              *reinterpret_cast<uint2*>(&sm.ra.am.lo[row][c0]) = lo.u[0];
            }
          } else {
            *reinterpret_cast<float4*>(&sm.ra.am.hi[row][c0]) = make_float4(v8[0], v8[1], v8[2], v8[3]);
          }
        };
        if (SCALAR || wave < NT - 1) store_a(r, amv);
        if constexpr (!SCALAR && NT == 4) {
          if (wave == 0) {  // tile 0's A side at the reference between tiles 1 and 2
            float mv[UW];
#pragma unroll
            for (int e = 0; e < UW; ++e) mv[e] = amv[e] * sm.cu.v.dfac[0][c0 + e];
            store_a(48 + li, mv);
          }
        }
        if constexpr (DPV) {
          if (w.out_row) {
#pragma unroll
            for (int e = 0; e < UW; ++e) {
              const float v = qm[u * UW + e];
              if constexpr (F16) {
                const __bf16 hi = (__bf16)v;
                sm.qmh[w.ro][c0 + e] = hi;
                sm.qml[w.ro][c0 + e] = (__bf16)(v - (float)hi);
              } else {
                sm.qmh[w.ro][c0 + e] = v;
              }
            }
          }
        }
      }
      if (w.out_row) {
        Op* qrow = Q_g + size_t(w.ro) * L.ldk;
        if constexpr (FRAG) {
#pragma unroll
          for (int u = 0; u < KB; ++u) {
            H8 h8;
#pragma unroll
            for (int e = 0; e < 8; ++e) h8.h[e] = (_Float16)qv[u * 8 + e];
            *reinterpret_cast<uint4*>(Q_g + ((((w.ro >> 4) * KB + u) * 64 + (w.ro & 15) + 16 * lg) * 8)) = h8.q;
          }
        } else if constexpr (F16) {
#pragma unroll
          for (int u = 0; u < NX / UW; ++u) {
            H8 h8;
#pragma unroll
            for (int e = 0; e < 8; ++e) h8.h[e] = (_Float16)(e < UW ? qv[u * UW + (e < UW ? e : 0)] : 0.0f);
            // the row pitch (dk + 4 halves) keeps rows 8-byte aligned
            uint2* q2 = reinterpret_cast<uint2*>(qrow + KM::chan(lg, u * UW));
            q2[0] = h8.u[0];
            if constexpr (UW == 8) q2[1] = h8.u[1];
          }
        } else {
#pragma unroll
          for (int x = 0; x < NX; x += 4)
            *reinterpret_cast<float4*>(qrow + KM::chan(lg, x)) = make_float4(qv[x], qv[x + 1], qv[x + 2], qv[x + 3]);
        }
        if (lg == 0) {
          sm.qs[w.ro] = qsc;
          qinv_g[w.ro] = 1.0f / qsc;
        }
      }
      // written values, scaled, transposed into LDS (bf16 path: by MFMA, as above)
      if constexpr (F16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (u < vnu) {
            half8 xv;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) xv[s2] = (vuw == 8 || s2 < 4) ? (_Float16)(wv[8 * u + s2] * wsc) : (_Float16)0.0f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              if (vuw == 8 || hh == 0) {
                half8 sv;
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) {
                  const bool hit = vuw == 8 ? (8 * lg + s2 == li + 16 * hh) : (s2 < 4 && 4 * lg + s2 == li);
                  sv[s2] = hit ? (_Float16)1.0f : (_Float16)0.0f;
                }
                const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const float4v tv = mma_pair_f16(xv, sv, zero);
                H8 pv;
#pragma unroll
                for (int e = 0; e < 4; ++e) pv.h[e] = (_Float16)tv[e];
                *reinterpret_cast<uint2*>(&sm.wvt[32 * u + 16 * hh + li][16 * wave + 4 * lg]) = pv.u[0];
              }
            }
          }
        }
      } else {
        const In* vrow = vg + w.vrow * dv;
        const In* brow_v = beg + w.th * DK;
        const In* bvrow = bvg ? bvg + w.th * dv : nullptr;
        switch (dv) {
          case 16: row_values<F16, 16>(V, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
          case 32: row_values<F16, 32>(V, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
          case 64: row_values<F16, 64>(V, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
          default: row_values<F16, 128>(V, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
        }
      }
    }
    __syncthreads();
    if (has_next) prefetch(wn, raw, 1);

    // A^ transposed (fp32 path): the LDS tile has the record's row pitch (C + 4),
    // so the copy is flat and coalesced (the pad columns are never read as
    // operands). The bf16 path stored it from the MFMA transposes above.
    if constexpr (!F16) {
      constexpr int UNITS = DK * Sm::LDC * int(sizeof(Op)) / 16;
      static_assert(DK * Sm::LDC * sizeof(Op) % 16 == 0, "flat copy in 16-byte units");
      const uint4* src = reinterpret_cast<const uint4*>(&sm.at[0][0]);
      uint4* dst = reinterpret_cast<uint4*>(AT_g);
      for (int u = tid; u < UNITS; u += kThreads) dst[u] = src[u];
    }

    // ---- Gram tiles: M^T(J, I) = A(J) B(I)^T and P^T(J, I) = A(J) Q(I)^T ----
    // (MFMA phases run at raised wave priority, as in chunk_prep2_kernel.)
    __builtin_amdgcn_s_setprio(1);
    // Block k of a wave pairs LDS slot slot_of(k) with this wave's B / Q side; with
    // per-channel decay and chunk 64, tile 3 multiplies its sides by e^{L_2} for
    // blocks 0 and 1 (the reference between tiles 1 and 2).
    constexpr bool MOVE = !SCALAR && NT == 4;
    float fxv[MOVE ? NX : 1];
#pragma unroll
    for (int x = 0; x < (MOVE ? NX : 1); ++x) fxv[x] = 1.0f;
    if constexpr (MOVE) {
      if (wave == 3) {
#pragma unroll
        for (int x = 0; x < NX; ++x) fxv[x] = sm.cu.v.dfac[1][KM::chan(lg, x)];
      }
    }
    auto slot_of = [&](int k) -> int { return (MOVE && k == 0 && wave >= 2) ? 3 : k; };
    // B side from registers (times fxv when `moved`)
    auto gram = [&](int slot, const float* xb, bool moved) __attribute__((always_inline)) -> float4v {
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (F16) {
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int c0 = u * 4 * UW + UW * lg;
          H8 ah, al, bh, bl;
          if constexpr (UW == 8) {
            ah.q = *reinterpret_cast<const uint4*>(&sm.ra.am.hi[16 * slot + li][c0]);
            al.q = *reinterpret_cast<const uint4*>(&sm.ra.am.lo[16 * slot + li][c0]);
          } else {
            ah = pair4(&sm.ra.am.hi[16 * slot + li][c0], nullptr);
            al = pair4(&sm.ra.am.lo[16 * slot + li][c0], nullptr);
          }
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2) {
            const int x = u * UW + (s2 < UW ? s2 : 0);
            const float v = s2 < UW ? xb[x] * (MOVE && moved ? fxv[MOVE ? x : 0] : 1.0f) : 0.0f;
            bh.b[s2] = (__bf16)v;
            bl.b[s2] = (__bf16)(v - (float)bh.b[s2]);
          }
          acc = mma_pair_bf16(ah.b, bh.b, acc);
          acc = mma_pair_bf16(ah.b, bl.b, acc);
          acc = mma_pair_bf16(al.b, bh.b, acc);
        }
      } else {
#pragma unroll
        for (int t = 0; t < KB; ++t) {
          float a4[4], b4[4];
          quad(&sm.ra.am.hi[16 * slot + li][16 * t + 4 * lg], a4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int x = 4 * t + e;
            b4[e] = xb[x] * (MOVE && moved ? fxv[MOVE ? x : 0] : 1.0f);
          }
          acc = mma_slice_f32(a4, b4, acc);
        }
      }
      return acc;
    };
    // B side from the LDS copy of output row qrow (DeltaProduct's output rows)
    auto gram_q = [&](int slot, int qrow) __attribute__((always_inline)) -> float4v {
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (DPV) {
        if constexpr (F16) {
#pragma unroll
          for (int u = 0; u < KB; ++u) {
            const int c0 = u * 4 * UW + UW * lg;
            H8 ah, al, bh, bl;
            if constexpr (UW == 8) {
              ah.q = *reinterpret_cast<const uint4*>(&sm.ra.am.hi[16 * slot + li][c0]);
              al.q = *reinterpret_cast<const uint4*>(&sm.ra.am.lo[16 * slot + li][c0]);
              bh.q = *reinterpret_cast<const uint4*>(&sm.qmh[qrow][c0]);
              bl.q = *reinterpret_cast<const uint4*>(&sm.qml[qrow][c0]);
            } else {
              ah = pair4(&sm.ra.am.hi[16 * slot + li][c0], nullptr);
              al = pair4(&sm.ra.am.lo[16 * slot + li][c0], nullptr);
              bh = pair4(&sm.qmh[qrow][c0], nullptr);
              bl = pair4(&sm.qml[qrow][c0], nullptr);
            }
            acc = mma_pair_bf16(ah.b, bh.b, acc);
            acc = mma_pair_bf16(ah.b, bl.b, acc);
            acc = mma_pair_bf16(al.b, bh.b, acc);
          }
        } else {
#pragma unroll
          for (int t = 0; t < KB; ++t) {
            float a4[4], b4[4];
            quad(&sm.ra.am.hi[16 * slot + li][16 * t + 4 * lg], a4);
            quad(&sm.qmh[qrow][16 * t + 4 * lg], b4);
            acc = mma_slice_f32(a4, b4, acc);
          }
        }
      }
      return acc;
    };
    // scalar decay: e^{G_i - G_j} of the entries j = 16 J + 4 lg + e of row i (G_i = gi)
    auto decay4 = [&](int J, float gi, float f[4]) __attribute__((always_inline)) {
      if constexpr (SCALAR) {
        const float4 gj = *reinterpret_cast<const float4*>(&sm.cu.s.grow[16 * J + 4 * lg]);
        f[0] = path_exp<F16>(fminf(gi - gj.x, 0.0f));
        f[1] = path_exp<F16>(fminf(gi - gj.y, 0.0f));
        f[2] = path_exp<F16>(fminf(gi - gj.z, 0.0f));
        f[3] = path_exp<F16>(fminf(gi - gj.w, 0.0f));
      } else {
        f[0] = f[1] = f[2] = f[3] = 1.0f;
      }
    };

    float4v mreg[NT];  // M^T(J, wave): every J <= wave (scalar decay) or J < wave
#pragma unroll
    for (int J = 0; J < NT; ++J) mreg[J] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    if (owner) {
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (SCALAR ? J <= wave : J < wave) mreg[J] = gram(slot_of(J), bm, J < 2);
      }
    }
    if (want_out) {
      if constexpr (!DPV) {
        if (owner) {  // output rows are this wave's own rows
          const int ro = 16 * wave + li;
          const float qsl = sm.qs[ro];
#pragma unroll
          for (int J = 0; J < NT; ++J) {
            float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
            if (SCALAR ? J <= wave : J < wave) acc = gram(slot_of(J), qm, J < 2);
            if (!SCALAR && J == wave) acc = pdg;
            float f[4];
            decay4(J, gabs, f);
            const int s0 = 16 * J + 4 * lg;
            Op* dst = FRAG ? P_g + p_frag(ro, J) : P_g + size_t(ro) * L.ldc + s0;
            if constexpr (F16) {
              H8 h8;
#pragma unroll
              for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)((s0 + e <= ro) ? acc[e] * f[e] * qsl : 0.0f);
              *reinterpret_cast<uint2*>(dst) = h8.u[0];
            } else {
              *reinterpret_cast<float4*>(dst) =
                  make_float4((s0 + 0 <= ro) ? acc[0] * f[0] : 0.0f, (s0 + 1 <= ro) ? acc[1] * f[1] : 0.0f,
                              (s0 + 2 <= ro) ? acc[2] * f[2] : 0.0f, (s0 + 3 <= ro) ? acc[3] * f[3] : 0.0f);
            }
          }
        }
      } else {
        // DeltaProduct (scalar decay): output row ro reads the state after step tau
        if (wave < RT) {
          // With 8 output rows (R = 8) lanes 8..15 of the tile have no row: they run
          // the products on row R - 1 (the MFMAs take every lane) and store nothing.
          const int ro = 16 * wave + li;
          const bool live = ro < R;
          const int rq = live ? ro : R - 1;
          const int tau = rq * n_h + n_h - 1;
          const int jmax = min(NT - 1, ((16 * wave + 15) * n_h + n_h - 1) / 16);
          const float qsl = sm.qs[rq];
          const float gtau = sm.cu.s.grow[tau];
          for (int J = 0; J < NT; ++J) {
            float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
            if (J <= jmax) acc = gram_q(J, rq);
            float f[4];
            decay4(J, gtau, f);
            const int s0 = 16 * J + 4 * lg;
            Op* dst = FRAG ? P_g + p_frag(ro, J) : P_g + size_t(ro) * L.ldc + s0;
            if (live) {
#pragma unroll
              for (int e = 0; e < 4; ++e) dst[e] = (Op)((s0 + e <= tau) ? acc[e] * f[e] * qsl : 0.0f);
            }
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (has_next) prefetch(wn, raw, 2);
    __syncthreads();  // the A sides are dead: their space now holds M and T
    if (owner) {
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (J <= wave) {
          const float4v src = (!SCALAR && J == wave) ? mdg : mreg[J];
          float f[4];
          decay4(J, gabs, f);
          const int s0 = 16 * J + 4 * lg;
          float4 m4;
          m4.x = (s0 + 0 < r) ? src[0] * f[0] : 0.0f;
          m4.y = (s0 + 1 < r) ? src[1] * f[1] : 0.0f;
          m4.z = (s0 + 2 < r) ? src[2] * f[2] : 0.0f;
          m4.w = (s0 + 3 < r) ? src[3] * f[3] : 0.0f;
          *reinterpret_cast<float4*>(&sm.ra.mt.m[r][s0]) = m4;
        }
      }
    }
    __syncthreads();

    // ---- T = (I + M)^{-1}: diagonal 16x16 blocks by forward substitution ----
    // The waves of the inverse raise their priority while the rest of the workgroup
    // waits at its barriers, so that the other workgroup on the CU does not hold
    // this serial phase back; they drop it again before the parallel phases.
    if (wave == 0) {
      __builtin_amdgcn_s_setprio(2);
      const int bI = lane >> 4, c = lane & 15;
      if (bI < NT) {
        float xcol[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          // four partial sums shorten the dependent chain
          float s4[4] = {(rr == c) ? 1.0f : 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s2 = 0; s2 < rr; ++s2) s4[s2 & 3] -= sm.ra.mt.m[16 * bI + rr][16 * bI + s2] * xcol[s2];
          xcol[rr] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sm.ra.mt.t[16 * bI + rr][16 * bI + c] = xcol[rr];
      }
    }
    // off-diagonal blocks: T_IJ = -T_II sum_{K=J}^{I-1} M_IK T_KJ, one level per I
#pragma unroll
    for (int I = 1; I < NT; ++I) {
      __syncthreads();
      if (wave < I) {
        __builtin_amdgcn_s_setprio(2);
        const int J = wave;
        float4v xa = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int K = J; K < I; ++K) {
          float a4[4], b4[4];
          quad(&sm.ra.mt.m[16 * I + li][16 * K + 4 * lg], a4);
#pragma unroll
          for (int e = 0; e < 4; ++e) b4[e] = sm.ra.mt.t[16 * K + 4 * lg + e][16 * J + li];
          xa = mma_slice_f32(a4, b4, xa);
        }
        float a4[4], xb[4] = {xa[0], xa[1], xa[2], xa[3]};
        quad(&sm.ra.mt.t[16 * I + li][16 * I + 4 * lg], a4);
        const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
        const float4v y = mma_slice_f32(a4, xb, zero);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.ra.mt.t[16 * I + 4 * lg + e][16 * J + li] = -y[e];
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    if (has_next) prefetch(wn, raw, 3);
    // operand copy of T with a zero upper triangle (fp16 over the dead M; fp32 in place)
    Op* top = F16 ? reinterpret_cast<Op*>(&sm.ra.mt.m[0][0]) : reinterpret_cast<Op*>(&sm.ra.mt.t[0][0]);
    constexpr int LDT = F16 ? 2 * Sm::LDC : Sm::LDC;  // fp16 rows over fp32 rows: twice the elements
    for (int u = tid; u < C * C / 4; u += kThreads) {  // four values a thread
      const int rr = u / (C / 4), s0 = 4 * (u % (C / 4));
      const float4 tv = *reinterpret_cast<const float4*>(&sm.ra.mt.t[rr][s0]);
      if constexpr (F16) {
        H8 h8;
        h8.h[0] = (s0 + 0 <= rr) ? (Op)tv.x : (Op)0.0f;
        h8.h[1] = (s0 + 1 <= rr) ? (Op)tv.y : (Op)0.0f;
        h8.h[2] = (s0 + 2 <= rr) ? (Op)tv.z : (Op)0.0f;
        h8.h[3] = (s0 + 3 <= rr) ? (Op)tv.w : (Op)0.0f;
        *reinterpret_cast<uint2*>(top + rr * LDT + s0) = h8.u[0];
      } else {
        *reinterpret_cast<float4*>(&sm.ra.mt.t[rr][s0]) =
            make_float4((s0 + 0 <= rr) ? tv.x : 0.0f, (s0 + 1 <= rr) ? tv.y : 0.0f, (s0 + 2 <= rr) ? tv.z : 0.0f,
                        (s0 + 3 <= rr) ? tv.w : 0.0f);
      }
    }
    __syncthreads();

    // ---- W^T = B+^T T^T (stored as W rows) and U~ = T Wv (stored transposed) ----
    __builtin_amdgcn_s_setprio(1);
    auto tprod = [&](const Op* arow, const Op* brow, int I) __attribute__((always_inline)) -> float4v {
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (F16) {
        for (int u = 0; 2 * u <= I; ++u) {
          const bool two = 2 * u + 1 < NT;
          const H8 a8 = pair4(arow + 32 * u + 4 * lg, two ? arow + 32 * u + 16 + 4 * lg : nullptr);
          const H8 b8 = pair4(brow + 32 * u + 4 * lg, two ? brow + 32 * u + 16 + 4 * lg : nullptr);
          acc = mma_pair_f16(a8.h, b8.h, acc);
        }
      } else {
        for (int t = 0; t <= I; ++t) {
          float a4[4], b4[4];
          quad(arow + 16 * t + 4 * lg, a4);
          quad(brow + 16 * t + 4 * lg, b4);
          acc = mma_slice_f32(a4, b4, acc);
        }
      }
      return acc;
    };
    const int VT = dv / 16;
    if constexpr (F16 && NT == kWaves) {
      // chunk 64: wave w computes the W and U~ tiles of step rows 16 w .. 16 w + 15,
      // every k-block (T's upper triangle is zero), independent chains interleaved
      H8 ta[2];  // T rows 16 w + li (A of U~; B of W^T), steps 32 u + 4 lg .. (+16)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Op* trow = top + (16 * wave + li) * LDT + 32 * u + 4 * lg;
        ta[u] = pair4(trow, trow + 16);
      }
      constexpr int CT = DK / 16;
      float4v wacc[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) wacc[ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const Op* brow = &sm.bt[16 * ct + li][32 * u + 4 * lg];
          const H8 b8 = pair4(brow, brow + 16);
          wacc[ct] = mma_pair_f16(b8.h, ta[u].h, wacc[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        Op* dst = FRAG ? W_g + w_frag(wave, ct) : W_g + size_t(16 * wave + li) * L.ldk + 16 * ct + 4 * lg;
        H8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)wacc[ct][e];
        *reinterpret_cast<uint2*>(dst) = h8.u[0];
      }
      for (int c0 = 0; c0 < VT; c0 += 4) {
        float4v uacc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) uacc[j] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ct = min(c0 + j, VT - 1);  // tail tiles repeat the last one (not stored)
            const Op* brow = &sm.wvt[16 * ct + li][32 * u + 4 * lg];
            const H8 b8 = pair4(brow, brow + 16);
            uacc[j] = mma_pair_f16(ta[u].h, b8.h, uacc[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (c0 + j < VT) {
            const int ct = c0 + j;
            Op* dst = FRAG ? UT_g + u_frag(wave, ct) : UT_g + size_t(16 * ct + li) * C + 16 * wave + 4 * lg;
            H8 h8;
#pragma unroll
            for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)uacc[j][e];
            *reinterpret_cast<uint2*>(dst) = h8.u[0];
          }
        }
      }
    } else {
    constexpr int NWT = (DK / 16) * NT;
    for (int x = wave; x < NWT; x += kWaves) {
      const int ct = x / NT, I = x % NT;
      const float4v acc = tprod(&sm.bt[16 * ct + li][0], top + (16 * I + li) * LDT, I);
      Op* dst = FRAG ? W_g + w_frag(I, ct) : W_g + size_t(16 * I + li) * L.ldk + 16 * ct + 4 * lg;
      if constexpr (F16) {
        H8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)acc[e];
        *reinterpret_cast<uint2*>(dst) = h8.u[0];
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    for (int x = wave; x < NT * VT; x += kWaves) {
      const int I = x / VT, ct = x % VT;
      const float4v acc = tprod(top + (16 * I + li) * LDT, &sm.wvt[16 * ct + li][0], I);
      Op* dst = FRAG ? UT_g + u_frag(I, ct) : UT_g + size_t(16 * ct + li) * C + 16 * I + 4 * lg;
      if constexpr (F16) {
        H8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)acc[e];
        *reinterpret_cast<uint2*>(dst) = h8.u[0];
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    }  // generic W / U~ path
    __builtin_amdgcn_s_setprio(0);
    if (has_next) prefetch(wn, raw, 4);
    __syncthreads();  // LDS is reused by the next chunk
  }
}

// ---- kernel 1b: chunk preparation, two workgroups per CU ----------------------------
//
// bf16 inputs, dk = dv = 128, chunk 64, one step per token (every variant but
// DeltaProduct with n_h >= 2, and FG2 with its own value-side beta). Same
// computation and record as chunk_prep_kernel, arranged so that two workgroups fit
// on a CU (under 80 KB of LDS, at most 256 registers a lane) and one hides the
// other's latencies: each lane loads its row of the next chunk into registers
// while W and U~ of the current one are computed, decodes values where they are
// used, keeps only the decay logs across the first barriers, and takes the scale
// maxima on bf16 bit patterns. Barriers wait for LDS traffic only. Rows past the
// end of the sequence are loaded from its last row (finite values) and masked.
struct alignas(16) PrepLds2 {
  union RA {
    struct {
      float L[4][128];      // tile totals of the log decay (base 2), per channel
      float m[4][128];      // in-tile prefix at each tile's row 7
    } stg;                  // decay staging, read by the per-channel pass
    struct {
      __bf16 hi[64][136];
      __bf16 lo[64][136];
    } am;                   // A side of the off-diagonal Gram blocks, four 16-row slots
    struct {
      float m[64][68];      // strictly lower Gram M; T in fp16 after the inverse
      float t[64][68];      // T = (I + M)^{-1}
    } mt;
  } ra;
  _Float16 bt[128][68];     // B+ (chunk-start reference), transposed
  _Float16 wvt[128][68];    // written values (scaled), transposed
  union CU {
    struct {
      // per tile t and channel: [0] m_t, [1] 2^m_t, [2] 2^(L_t - m_t), [3] 2^(sum of
      // L before t), [4] 2^(sum of L after t)
      float cst[4][5][128];
      float dfac[2][128];   // 2^L_1 and 2^L_2 (decay across tiles 1 and 2)
    } v;                    // per-channel decay
    struct {
      float ltot[4];        // tile totals of the scalar log decay
      float grow[64];       // log decay from the chunk start through each row
    } s;                    // scalar decay
    struct {
      // [t] G_31 - (sum of L before tile t), [4] 2^G_31, [5] 2^(G_C - G_31)
      float chv[6][128];
    } o;                    // per-channel decay, every factor referenced to row 31
  } cu;
  float red[kWaves];
  float tdec[kWaves];       // largest decay of any channel over each 16-step tile (log2)
};

// Whether chunk_prep2_kernel covers a problem (bf16, dk = dv = 128, chunk 64;
// DeltaProduct with n_h = 1, 2 or 4, the step counts a 64-step chunk with at least
// 16 output rows allows).
inline bool prep2_covers(const Problem& p) {
  return p.dtype == GDN_DTYPE_BF16 && p.dk == 128 && p.dv == 128 && p.chunk == 64 &&
         (p.n_step == 1 || p.n_step == 2 || p.n_step == 4);
}

// STAB: the GDN2 stabiliser mode applied to the rows (ASYM only; a template
// parameter so that the other instantiations carry none of its registers).
// NH: steps per token (DeltaProduct's n_h; 1 otherwise). With NH > 1 the rows are
// Householder sub-steps: k, v and beta come from the step, the gate from the token
// at its first step, and every NH-th row (the token's last step) is an output row.
// MODE (per-channel decay only): 1 = chunks of mild decay on the path referenced
// to the chunk's middle; every other chunk is only flagged (flags[item] = 1, else
// 0); 2 = the flagged chunks, on the tile-referenced path. 0 = every chunk on the
// tile-referenced path (scalar decay).
template <int V, int STAB, int NH, int MODE, bool PLUS = false>
__global__ __launch_bounds__(kThreads, 2) void chunk_prep2_kernel(Problem p, unsigned char* __restrict__ ws,
                                                                     unsigned char* __restrict__ flags,
                                                                     ChunkLayout L, int want_out) {
  using In = uint16_t;
  constexpr int DK = 128, C = 64, NT = 4, KB = 4, CK = 2, CT = 8, VT = 8;
  constexpr bool DP = V == GDN_VARIANT_DELTAPRODUCT;
  static_assert(NH == 1 || DP, "several steps per token: DeltaProduct only");
  constexpr int TPC = C / NH;  // tokens per chunk
  constexpr bool CH_ALPHA = V == GDN_VARIANT_FG2 || V == GDN_VARIANT_KDA || V == GDN_VARIANT_ASYM;
  constexpr bool CH_BJ = V == GDN_VARIANT_FG2 || V == GDN_VARIANT_ASYM;  // per-channel beta / j
  constexpr bool SCALAR = !CH_ALPHA;  // one log decay per row (GDN, DeltaProduct)
  static_assert(SCALAR ? MODE == 0 : MODE != 0, "mild / flagged passes for per-channel decay");
  static_assert(!PLUS || V == GDN_VARIANT_FG2, "a value-side beta is FG2-GDN+ only");
  using Sm = PrepLds2;
  static_assert(sizeof(Sm) <= 80 * 1024, "two workgroups per CU");
  __shared__ Sm sm;

  // Lane indices are re-derived at the top of every item from an opaque copy of
  // the thread id: otherwise the compiler keeps every lane-dependent address of
  // the loop body live across it, more registers than two waves per SIMD allow.
  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int li = lane & 15, lg = lane >> 4;
  int r = 16 * wave + li;  // step row of this lane
  auto lane_ids = [&]() __attribute__((always_inline)) {
    int t = int(threadIdx.x);
    asm volatile("" : "+v"(t));
    tid = t;
    lane = t & 63;
    li = lane & 15;
    lg = lane >> 4;
    r = 16 * wave + li;
  };
  const int NC = int(p.nchunks);
  const int H = int(p.H);
  const int BH = int(p.B) * H;
  const int total = NC * BH;  // < 2^31 (checked on the host)
  const int64_t T = p.T;
  const In* qg = static_cast<const In*>(p.q);
  const In* kg = static_cast<const In*>(p.k);
  const In* vg = static_cast<const In*>(p.v);
  const In* alg = static_cast<const In*>(p.alpha);
  const In* beg = static_cast<const In*>(p.beta);
  const In* jg = static_cast<const In*>(p.j);
  const In* etg = static_cast<const In*>(p.eta);
  auto ld = [](const In* x) { return IO<In>::ld(x); };

  // first token-head row (b, token n TPC, h) of an item, chunk-major order
  struct Item {
    int nl, bh;   // chunk of the launch, (batch, head)
    int n;        // chunk of the sequence
    int64_t th0;  // (b T + n TPC) H + h
  };
  auto item_of = [&](int item) __attribute__((always_inline)) -> Item {
    Item it;
    it.nl = item / BH;
    it.bh = item - it.nl * BH;
    it.n = int(p.c0) + it.nl;
    const int b = it.bh / H, h = it.bh - b * H;
    it.th0 = (int64_t(b) * T + int64_t(it.n) * TPC) * H + h;
    return it;
  };
  // token-head row of step row rr (clamped to the sequence's last token)
  auto th_of = [&](const Item& it, int rr) __attribute__((always_inline)) -> int64_t {
    const int64_t last = T - 1 - int64_t(it.n) * TPC;  // >= 0
    return it.th0 + min(int64_t(rr / NH), last) * H;
  };
  // row of step rr in the per-step arrays ([B, T, H, n_h, ...]; clamped to the last
  // step; the identity step of a padded token reads the token's last real step)
  auto step_of = [&](const Item& it, int rr) __attribute__((always_inline)) -> int64_t {
    if constexpr (NH == 1) {
      return th_of(it, rr);
    } else {
      const int64_t rel = min(int64_t(rr), p.steps - 1 - int64_t(it.n) * C);  // >= 0
      return (it.th0 + (rel / NH) * H) * p.n_h + min(int(rel % NH), p.n_h - 1);
    }
  };

  // This lane's row of an item's inputs in 16-byte groups (group u: channels
  // 32 u + 8 lg ..), loaded into registers one item ahead.
  struct Raw {
    uint4 k[4], a[4], b[4], q[4], v[4];
  };
  // parts: 1 key, 2 values, 4 query, 8 decay, 16 beta / j
  auto load_raw = [&](const Item& it, Raw& x, int parts) __attribute__((always_inline)) {
    const int64_t off = th_of(it, r) * DK + 8 * lg;                       // token rows
    const int64_t offs = NH == 1 ? off : step_of(it, r) * DK + 8 * lg;   // step rows
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      auto ld16 = [&](const In* base) { return *reinterpret_cast<const uint4*>(base + off + 32 * u); };
      auto ld16s = [&](const In* base) { return *reinterpret_cast<const uint4*>(base + offs + 32 * u); };
      if (parts & 1) x.k[u] = ld16s(kg);
      if (parts & 2) x.v[u] = ld16s(vg);
      if ((parts & 4) && want_out && (NH == 1 || r % NH == NH - 1)) x.q[u] = ld16(qg);  // output rows
      if constexpr (CH_ALPHA)
        if (parts & 8) x.a[u] = ld16(alg);
      if constexpr (V == GDN_VARIANT_FG2)
        if (parts & 16) x.b[u] = ld16(beg);
      if constexpr (V == GDN_VARIANT_ASYM)
        if (parts & 16) x.b[u] = ld16(jg);
    }
  };
  auto bf = [](const uint4& v, int s) __attribute__((always_inline)) -> float {
    const uint32_t w = s / 2 == 0 ? v.x : s / 2 == 1 ? v.y : s / 2 == 2 ? v.z : v.w;
    return __uint_as_float((s & 1) ? (w & 0xffff0000u) : (w << 16));
  };
  // per-row scalars (gates of the scalar-gated variants), loaded with the stage
  struct Scal {
    float alpha, beta, eta;
  };
  auto load_scal = [&](const Item& it) __attribute__((always_inline)) -> Scal {
    Scal s{1.0f, 0.0f, 0.0f};
    const int64_t th = th_of(it, r);
    if constexpr (!CH_ALPHA) s.alpha = ld(alg + th);
    if constexpr (V == GDN_VARIANT_KDA || V == GDN_VARIANT_GDN) s.beta = ld(beg + th);
    if constexpr (DP) s.beta = (NH > 1 && r % NH >= p.n_h) ? 0.0f : ld(beg + step_of(it, r));  // padding: identity
    if constexpr (V == GDN_VARIANT_ASYM) s.eta = ld(etg + th);
    return s;
  };
  // Workgroup barrier for LDS traffic only. The waves exchange data through LDS
  // alone, so the barrier waits for this wave's LDS operations but not for its
  // outstanding global loads and stores, which a fenced barrier would drain.
  auto wg_barrier = []() __attribute__((always_inline)) { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // fragment-format offsets (elements): P row ro, steps 16 J + 4 lg ..; W row
  // 16 I + li, channels 16 ct + 4 lg ..; U~ steps 16 I + 4 lg .., column 16 ct + li
  auto p_frag = [&](int ro, int J) -> size_t {
    return size_t((((ro >> 4) * CK + (J >> 1)) * 64 + (ro & 15) + 16 * (2 * (J & 1) + (lg >> 1))) * 8 + 4 * (lg & 1));
  };
  auto w_frag = [&](int I, int ct) -> size_t {
    return size_t(((I * KB + (ct >> 1)) * 64 + li + 16 * (2 * (ct & 1) + (lg >> 1))) * 8 + 4 * (lg & 1));
  };
  auto u_frag = [&](int I, int ct) -> size_t { return size_t(((I * VT + ct) * 64 + lane) * 4); };

  // 0/1 selection fragments (B operand of a 16x16x32 MFMA) that move the k-slot of
  // relative channel 16 h + n to column n (an exact transpose of a row group)
  half8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) sel[hh][s2] = (8 * lg + s2 == li + 16 * hh) ? (_Float16)1.0f : (_Float16)0.0f;

  // the first item's inputs; later items load during the one before
  Scal scal{1.0f, 0.0f, 0.0f};
  Raw raw;
  if constexpr (NH > 1) {  // only output rows load q
#pragma unroll
    for (int u = 0; u < 4; ++u) raw.q[u] = make_uint4(0u, 0u, 0u, 0u);
  }
  // items of this workgroup: every gridDim-th one; the flagged pass skips the others
  auto next_item = [&](int item) __attribute__((always_inline)) -> int {
    if constexpr (MODE == 2) {
      // 64 of this workgroup's items per wave-wide load, the first flagged one by ballot
      const int l = int(threadIdx.x & 63);
      for (; item < total; item += 64 * int(gridDim.x)) {
        const int x = item + l * int(gridDim.x);
        const uint64_t hit = __ballot(x < total && flags[x] != 0);
        if (hit) return item + int(__builtin_ctzll(hit)) * int(gridDim.x);
      }
      return total;
    }
    return item;
  };
  const int first = next_item(blockIdx.x);
  if (first < total) {
    const Item it = item_of(first);
    load_raw(it, raw, 31);
    scal = load_scal(it);
  }

  for (int item = first, after; item < total; item = after) {
    lane_ids();
    after = next_item(item + int(gridDim.x));
    const Item it = item_of(item);
    const bool has_next = after < total;
    const Item nx = item_of(has_next ? after : item);
    const bool valid = int64_t(it.n) * C + r < p.steps;
    const bool orow = NH == 1 || r % NH == NH - 1;  // the token's last step: an output row
    const int ro = r / NH;                           // its output row
    unsigned char* rec = ws + (size_t(it.bh) * size_t(NC) + size_t(it.nl)) * L.bytes;
    _Float16* W_g = reinterpret_cast<_Float16*>(rec + L.off_W);
    _Float16* AT_g = reinterpret_cast<_Float16*>(rec + L.off_AT);
    _Float16* Q_g = reinterpret_cast<_Float16*>(rec + L.off_Q);
    _Float16* P_g = reinterpret_cast<_Float16*>(rec + L.off_P);
    _Float16* UT_g = reinterpret_cast<_Float16*>(rec + L.off_UT);
    float* gam_g = reinterpret_cast<float*>(rec + L.off_gamma);
    float* winv_g = reinterpret_cast<float*>(rec + L.off_winv);
    float* qinv_g = reinterpret_cast<float*>(rec + L.off_qinv);

    // ---- per-row factors of the variant: key side sqrt(beta) (scalar variants),
    // written-value scale, scalar log decay; invalid rows get zero weights ----
    const Scal sc = scal;
    float kscal = 1.0f, wscal = 0.0f, bscal = 1.0f, glog = 0.0f;
    if constexpr (V == GDN_VARIANT_KDA || V == GDN_VARIANT_GDN) {
      kscal = __builtin_amdgcn_sqrtf(sc.beta);
      wscal = kscal;
      if constexpr (V == GDN_VARIANT_GDN) glog = __builtin_amdgcn_logf(sc.alpha);
    } else if constexpr (DP) {
      bscal = sc.beta;
      wscal = sc.beta;
      glog = (NH == 1 || r % NH == 0) ? __builtin_amdgcn_logf(sc.alpha) : 0.0f;  // gate at the first step
    } else if constexpr (V == GDN_VARIANT_ASYM) {
      bscal = sc.eta;
      wscal = sc.eta;
    }
    if (!valid) kscal = wscal = bscal = glog = 0.0f;
    // GDN2 stabiliser coefficients of this row (identity unless asked for); rows past
    // the sequence end read the last token and are zeroed below
    StabCoef stc{__builtin_inff(), 0.0f, 1.0f};
    if constexpr (STAB != 0) {
      static_assert(V == GDN_VARIANT_ASYM, "stabilisers act on the asymmetric variant");
      // Each call unpacks afresh from the packed rows (the empty asm hides that the
      // two passes read the same words), so the unpacked row is never held whole.
      auto unpack = [&](const uint4& v, int s2) __attribute__((always_inline)) {
        uint32_t w = s2 / 2 == 0 ? v.x : s2 / 2 == 1 ? v.y : s2 / 2 == 2 ? v.z : v.w;
        asm volatile("" : "+v"(w));
        return __uint_as_float((s2 & 1) ? (w & 0xffff0000u) : (w << 16));
      };
      stc = stab_coef<32>(
          STAB, sc.eta,
          [&](int i) { return KJD{unpack(raw.k[i / 8], i % 8), unpack(raw.b[i / 8], i % 8), unpack(raw.a[i / 8], i % 8)}; },
          [](float x) { return sum_over_groups(x); }, [](float x) { return max_over_groups(x); });
    }

    // ---- phase 1: log decay and row maxima ----
    // The maxima only set power-of-two scales. They are taken on the bf16 bit
    // patterns (for non-negative values the order of the patterns is the order of
    // the values), two at a time; the written values' scale uses the bound
    // max |v| max sqrt(beta) of the row, which keeps the scaled values below 2^13.
    float G[SCALAR ? 1 : 32];
    ushort2v qm2 = {0, 0}, vm2 = {0, 0}, bm2 = {0, 0};
    // FG2-GDN+: this row's value-side beta (dv = dk channels, the lane's 32), read
    // here for the written values' bound and kept for phase 2
    // (the flagged pass, short of registers, reads it again there)
    uint4 bvr[PLUS ? 4 : 1];
    const In* bvg = static_cast<const In*>(p.beta_v);
    const int64_t offv = th_of(it, r) * DK + 8 * lg;
    if constexpr (PLUS) {
#pragma unroll
      for (int u = 0; u < 4; ++u) bvr[u] = *reinterpret_cast<const uint4*>(bvg + offv + 32 * u);
    }
    auto bv_at = [&](int u) __attribute__((always_inline)) -> uint4 {
      if constexpr (MODE == 2) return *reinterpret_cast<const uint4*>(bvg + offv + 32 * u);
      else return bvr[PLUS ? u : 0];
    };
    auto absmax2 = [](ushort2v m, uint32_t w) __attribute__((always_inline)) {
      return __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, w & 0x7fff7fffu));
    };
    auto absmax8 = [&](ushort2v m, const uint4& x) __attribute__((always_inline)) {
      return absmax2(absmax2(absmax2(absmax2(m, x.x), x.y), x.z), x.w);
    };
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (!SCALAR) {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const int x = 8 * u + s2;
          if constexpr (STAB == 1) G[x] = valid ? __builtin_amdgcn_logf(stab_decay(stc, bf(raw.a[u], s2))) : 0.0f;
          else G[x] = valid ? __builtin_amdgcn_logf(bf(raw.a[u], s2)) : 0.0f;
        }
      }
      vm2 = absmax8(vm2, raw.v[u]);
      if (want_out) qm2 = absmax8(qm2, raw.q[u]);
      if constexpr (V == GDN_VARIANT_FG2) {
        if constexpr (PLUS) bm2 = absmax8(bm2, bvr[u]);  // the written values' beta
        else bm2 = absmax8(bm2, raw.b[u]);
      }
    }
    if constexpr (SCALAR) G[0] = glog;
    auto bits_max = [](ushort2v m) __attribute__((always_inline)) {
      return __uint_as_float(uint32_t(m.x > m.y ? m.x : m.y) << 16);
    };
    const float qmax = (valid && orow) ? bits_max(qm2) : 0.0f;
    float wmax = bits_max(vm2) * (V == GDN_VARIANT_FG2 ? (valid ? __builtin_amdgcn_sqrtf(bits_max(bm2)) : 0.0f)
                                                         : fabsf(wscal));
    // inclusive scan of the log decay over each 16-row tile; the tile totals (row
    // 15) and the prefixes at row 7 go to LDS
    if constexpr (SCALAR) {
      G[0] = scan16(G[0]);
      if (li == 15 && lg == 0) sm.cu.s.ltot[wave] = G[0];
    } else {
#pragma unroll
      for (int x = 0; x < 32; ++x) G[x] = scan16(G[x]);
      if (li == 15 || (MODE != 1 && li == 7)) {  // the mild pass needs the totals only
        float* dst = li == 15 ? &sm.ra.stg.L[wave][0] : &sm.ra.stg.m[wave][0];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; e += 4)
            *reinterpret_cast<float4*>(dst + 32 * u + 8 * lg + e) =
                make_float4(G[8 * u + e], G[8 * u + e + 1], G[8 * u + e + 2], G[8 * u + e + 3]);
      }
    }
    // largest decay over this wave's tile (row 15 holds the tile totals)
    float tdmax = 0.0f;
    if constexpr (!SCALAR) {
      if (li == 15) {
#pragma unroll
        for (int x = 0; x < 32; ++x) tdmax = fmaxf(tdmax, -G[x]);
      }
      tdmax = wave_max(tdmax);
    }
    // power-of-two scales: per output row for q, per chunk for the written values
    const float qsc = want_out ? pow2_scale_for(max_over_groups(qmax)) : 1.0f;
    wmax = wave_max(wmax);
    if (lane == 0) {
      sm.red[wave] = wmax;
      sm.tdec[wave] = tdmax;
    }
    wg_barrier();

    // Mild decay (every channel decays by less than 2^-55 over each 16-step tile, so
    // by less than 2^-110 over either half of the chunk): one reference point in the
    // middle of the chunk keeps every factor in range, and the chunk takes the
    // shorter path that forms every Gram block from it. Otherwise the tile
    // references below.
    if constexpr (MODE == 1) {
      float td = sm.tdec[0];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) td = fmaxf(td, sm.tdec[w2]);
      const bool mild = td < 55.0f;
      if (tid == 0 && mild) flags[item] = 0;
      if (!mild) {
        // this chunk and every later one of the workgroup go to the flagged pass
        for (int x = item + tid * int(gridDim.x); x < total; x += kThreads * int(gridDim.x)) flags[x] = 1;
        break;
      }
    }

    // ---- decay constants ----
    // Scalar decay: every factor is a function of the row alone; the Gram entries
    // take e^{G_i - G_j} after the product. Per-channel decay: one thread per key
    // channel writes the constants of every 16-row tile t (reference points: the
    // tile's first row for the B and Q sides, its last row for the A side, its row
    // 7 for the diagonal block), so that no factor exceeds the decay of the eight
    // steps around row 7, and none of the cross-tile factors exceeds 1.
    float gabs = 0.0f, eg_row = 1.0f, eat_row = 1.0f;
    if constexpr (SCALAR) {
      float pre = 0.0f, gc = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float lt = sm.cu.s.ltot[t];
        if (t < wave) pre += lt;
        gc += lt;
      }
      gabs = pre + G[0];                                         // G of this row
      eg_row = __builtin_amdgcn_exp2f(gabs);                     // e^{G}
      eat_row = __builtin_amdgcn_exp2f(fminf(gc - gabs, 0.0f));  // e^{G_C - G}
      if (lg == 0) sm.cu.s.grow[r] = gabs;
      if (tid < DK) gam_g[tid] = __builtin_amdgcn_exp2f(gc);
    } else if (MODE == 1) {
      if (tid < DK) {  // one thread per key channel
        const int c = tid;
        float Lt[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) Lt[t] = sm.ra.stg.L[t][c];
        const float gm = Lt[0] + Lt[1];  // G at row 31
        float pre = 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          sm.cu.o.chv[t][c] = gm - pre;
          pre += Lt[t];
        }
        sm.cu.o.chv[NT][c] = __builtin_amdgcn_exp2f(gm);
        sm.cu.o.chv[NT + 1][c] = __builtin_amdgcn_exp2f(pre - gm);
        gam_g[c] = __builtin_amdgcn_exp2f(pre);
      }
    } else {
      // thread (c, half): channel c, tiles 2 half and 2 half + 1
      const int c = tid & (DK - 1), half = tid >> 7;
      float Lt[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) Lt[t] = sm.ra.stg.L[t][c];
      const float gc = (Lt[0] + Lt[1]) + (Lt[2] + Lt[3]);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = 2 * half + k;
        const float mt = sm.ra.stg.m[t][c];
        const float pre = t == 0 ? 0.0f : t == 1 ? Lt[0] : t == 2 ? Lt[0] + Lt[1] : Lt[0] + Lt[1] + Lt[2];
        const float suf = t == 3 ? 0.0f : t == 2 ? Lt[3] : t == 1 ? Lt[2] + Lt[3] : Lt[1] + Lt[2] + Lt[3];
        sm.cu.v.cst[t][0][c] = mt;
        sm.cu.v.cst[t][1][c] = __builtin_amdgcn_exp2f(mt);          // e^{G_7 - G_start}
        sm.cu.v.cst[t][2][c] = __builtin_amdgcn_exp2f(Lt[t] - mt);  // e^{G_end - G_7}
        sm.cu.v.cst[t][3][c] = __builtin_amdgcn_exp2f(pre);         // e^{G_start}
        sm.cu.v.cst[t][4][c] = __builtin_amdgcn_exp2f(suf);         // e^{G_C - G_end}
      }
      sm.cu.v.dfac[half][c] = __builtin_amdgcn_exp2f(Lt[1 + half]);
      if (half == 0) gam_g[c] = __builtin_amdgcn_exp2f(gc);
    }
    float wsc;
    {
      float m = sm.red[0];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) m = fmaxf(m, sm.red[w2]);
      wsc = pow2_scale_for(m);
    }
    if (tid == 0) winv_g[0] = 1.0f / wsc;
    if (want_out && orow && lg == 0) qinv_g[ro] = 1.0f / qsc;
    wg_barrier();

    if constexpr (MODE == 1) {
      // ---- phase 2 (mild decay): decayed operands and written values of this wave's
      // rows, one channel group at a time, every factor referenced to the chunk's
      // middle (row 31) ----
      const float wrow = (V == GDN_VARIANT_FG2 ? 1.0f : wscal) * wsc;  // written-value factor of the row
      H8 bmh[KB], bml[KB], qmh8[KB], qml8[KB];  // B sides of the Grams (bf16 hi / lo)
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int c0 = 32 * u + 8 * lg;  // 8 consecutive channels
        float cof[8], cp[8], cq[8];
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          const float4 x0 = *reinterpret_cast<const float4*>(&sm.cu.o.chv[wave][c0 + e]);
          const float4 x1 = *reinterpret_cast<const float4*>(&sm.cu.o.chv[NT][c0 + e]);
          const float4 x2 = *reinterpret_cast<const float4*>(&sm.cu.o.chv[NT + 1][c0 + e]);
          cof[e] = x0.x, cof[e + 1] = x0.y, cof[e + 2] = x0.z, cof[e + 3] = x0.w;
          cp[e] = x1.x, cp[e + 1] = x1.y, cp[e + 2] = x1.z, cp[e + 3] = x1.w;
          cq[e] = x2.x, cq[e + 1] = x2.y, cq[e + 2] = x2.z, cq[e + 3] = x2.w;
        }
        const uint4 kr = raw.k[u], vr = raw.v[u];
        uint4 br = {}, qr = {};
        if constexpr (CH_BJ) br = raw.b[u];
        uint4 bvu = {};
        if constexpr (PLUS) bvu = bv_at(u);
        if (want_out && valid && orow) qr = raw.q[u];
        half8 xbt, xat, xv;
        H8 hi, lo, qp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kf = bf(kr, e);
          float a, bb;
          if constexpr (V == GDN_VARIANT_FG2) {
            const float sb = valid ? __builtin_amdgcn_sqrtf(bf(br, e)) : 0.0f;
            a = sb * kf;
            bb = a;
            const float sbv = PLUS ? (valid ? __builtin_amdgcn_sqrtf(bf(bvu, e)) : 0.0f) : sb;
            xv[e] = (_Float16)(bf(vr, e) * sbv * wsc);
          } else if constexpr (V == GDN_VARIANT_ASYM) {
            a = valid ? kf : 0.0f;
            bb = bscal * (STAB == 2 ? stab_j(stc, kf, bf(br, e)) : bf(br, e));
          } else {  // KDA, GDN (kscal = sqrt(beta)); DeltaProduct (bscal = beta)
            a = kscal * kf;
            bb = bscal * a;
          }
          if constexpr (V != GDN_VARIANT_FG2) xv[e] = (_Float16)(bf(vr, e) * wrow);
          const float fup = __builtin_amdgcn_exp2f(G[8 * u + e] - cof[e]);  // e^{G - G_mid}
          const float eam = __builtin_amdgcn_rcpf(fup);                     // e^{G_mid - G}
          const float eg = cp[e] * fup;                                     // e^{G}
          const float eat = cq[e] * eam;                                    // e^{G_C - G}
          xbt[e] = (_Float16)(bb * eg);
          xat[e] = (_Float16)(a * eat);
          const float am = a * eam;
          hi.b[e] = (__bf16)am;
          lo.b[e] = (__bf16)(am - (float)hi.b[e]);
          const float bm = bb * fup;
          bmh[u].b[e] = (__bf16)bm;
          bml[u].b[e] = (__bf16)(bm - (float)bmh[u].b[e]);
          const float qf = bf(qr, e);
          const float qm = qf * fup;
          qmh8[u].b[e] = (__bf16)qm;
          qml8[u].b[e] = (__bf16)(qm - (float)qmh8[u].b[e]);
          qp.h[e] = (_Float16)(qf * eg * qsc);
        }
        *reinterpret_cast<uint4*>(&sm.ra.am.hi[r][c0]) = hi.q;
        *reinterpret_cast<uint4*>(&sm.ra.am.lo[r][c0]) = lo.q;
        if (want_out && orow)
          *reinterpret_cast<uint4*>(Q_g + ((((ro >> 4) * KB + u) * 64 + (ro & 15) + 16 * lg) * 8)) = qp.q;
        // B+ and A^ of the group transposed by MFMA: lane (li, lg) then holds steps
        // 16 wave + 4 lg .. of channel 32 u + 16 h + li
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
          const float4v tb = mma_pair_f16(xbt, sel[hh], zero);
          const float4v ta = mma_pair_f16(xat, sel[hh], zero);
          const int c = 32 * u + 16 * hh + li;
          H8 pb, pa;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb.h[e] = (_Float16)tb[e];
            pa.h[e] = (_Float16)ta[e];
          }
          *reinterpret_cast<uint2*>(&sm.bt[c][16 * wave + 4 * lg]) = pb.u[0];
          const float4v tv = mma_pair_f16(xv, sel[hh], zero);
          H8 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) pv.h[e] = (_Float16)tv[e];
          *reinterpret_cast<uint2*>(&sm.wvt[c][16 * wave + 4 * lg]) = pv.u[0];
          *reinterpret_cast<uint2*>(AT_g + size_t((((c >> 4) * CK + (wave >> 1)) * 64 + li + 16 * (2 * (wave & 1) + (lg >> 1))) * 8 +
                                                  4 * (lg & 1))) = pa.u[0];
        }
      }

      // The next item's inputs load in three groups, each once this item's copy is
      // consumed, so that the loads of the two workgroups on a CU do not arrive in
      // one burst: key and values here, query and beta / j after the Grams, the decay
      // before W and U~.
      if (has_next) load_raw(nx, raw, 1 | 2);
      wg_barrier();

      // ---- Gram tiles: M^T(J, I) = A-(J) B+(I)^T and P^T(J, I) = A-(J) Q+(I)^T, every J
      // together, k-block outer (tiles above the diagonal are computed and masked).
      // The MFMA phases run at raised wave priority: their MFMAs issue first and the
      // other workgroup's VALU work fills the cycles while they execute. ----
      __builtin_amdgcn_s_setprio(1);
      float4v mreg[NT], preg[NT];
#pragma unroll
      for (int J = 0; J < NT; ++J) mreg[J] = preg[J] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int c0 = 32 * u + 8 * lg;
        H8 ah[NT], al[NT];
#pragma unroll
        for (int J = 0; J < NT; ++J) {
          ah[J].q = *reinterpret_cast<const uint4*>(&sm.ra.am.hi[16 * J + li][c0]);
          al[J].q = *reinterpret_cast<const uint4*>(&sm.ra.am.lo[16 * J + li][c0]);
        }
#pragma unroll
        for (int J = 0; J < NT; ++J) mreg[J] = mma_pair_bf16(ah[J].b, bmh[u].b, mreg[J]);
#pragma unroll
        for (int J = 0; J < NT; ++J) preg[J] = mma_pair_bf16(ah[J].b, qmh8[u].b, preg[J]);
#pragma unroll
        for (int J = 0; J < NT; ++J) mreg[J] = mma_pair_bf16(ah[J].b, bml[u].b, mreg[J]);
#pragma unroll
        for (int J = 0; J < NT; ++J) preg[J] = mma_pair_bf16(ah[J].b, qml8[u].b, preg[J]);
#pragma unroll
        for (int J = 0; J < NT; ++J) mreg[J] = mma_pair_bf16(al[J].b, bmh[u].b, mreg[J]);
#pragma unroll
        for (int J = 0; J < NT; ++J) preg[J] = mma_pair_bf16(al[J].b, qmh8[u].b, preg[J]);
      }
      if (want_out && orow) {  // output rows are this wave's own rows (q scale qsc)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
          const int s0 = 16 * J + 4 * lg;
          H8 h8;
#pragma unroll
          for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)((s0 + e <= r) ? preg[J][e] * qsc : 0.0f);
          *reinterpret_cast<uint2*>(P_g + p_frag(ro, J)) = h8.u[0];
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (has_next) load_raw(nx, raw, 4 | 16);
      wg_barrier();  // A- is dead: its space now holds M and T
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (J <= wave) {
          const int s0 = 16 * J + 4 * lg;
          float4 m4;
          m4.x = (s0 + 0 < r) ? mreg[J][0] : 0.0f;
          m4.y = (s0 + 1 < r) ? mreg[J][1] : 0.0f;
          m4.z = (s0 + 2 < r) ? mreg[J][2] : 0.0f;
          m4.w = (s0 + 3 < r) ? mreg[J][3] : 0.0f;
          *reinterpret_cast<float4*>(&sm.ra.mt.m[r][s0]) = m4;
        }
      }
      wg_barrier();

    } else {
      // ---- phase 2: decayed operands and written values of this wave's rows, one
      // channel group at a time ----
      // Off-diagonal Gram blocks M(I, J), P(I, J), J < I, with per-channel decay: B and
      // Q sides of tile I referenced to its first row (kept in fp32 until the Gram
      // phase), A side of tile J to its last row (LDS slot J); block (3, 2) pairs
      // them directly, blocks (I, 0..1) of the lower half pair them through the
      // reference between tiles 1 and 2: slot 3 holds tile 0's A side moved there
      // (times e^{L_1}), and tile 3's B and Q sides move back to it (times e^{L_2}) in
      // the Gram phase. Tile 3's own A side is never an off-diagonal operand. The
      // diagonal blocks use row 7 of the tile on both sides and run here, on fp32
      // MFMA straight from registers (the A and B operand layouts of a 16-row tile
      // are the same).
      const float wrow = (V == GDN_VARIANT_FG2 ? 1.0f : wscal) * wsc;  // written-value factor of the row
      float bsv[SCALAR ? 1 : 32], qsv[SCALAR ? 1 : 32];                // B and Q sides (per-channel decay)
      H8 bmh[SCALAR ? KB : 1], bml[SCALAR ? KB : 1], qmh8[SCALAR ? KB : 1], qml8[SCALAR ? KB : 1];  // (scalar)
      float4v mdg = {0.0f, 0.0f, 0.0f, 0.0f}, pdg = {0.0f, 0.0f, 0.0f, 0.0f};  // diagonal blocks M^T, P^T
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int c0 = 32 * u + 8 * lg;  // 8 consecutive channels
        float cm[8], c7[8], c157[8], cP[8], cQ[8];
        if constexpr (!SCALAR) {
          auto ld8 = [&](const float* src, float* d) __attribute__((always_inline)) {
            const float4 x0 = *reinterpret_cast<const float4*>(src);
            const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
            d[0] = x0.x, d[1] = x0.y, d[2] = x0.z, d[3] = x0.w, d[4] = x1.x, d[5] = x1.y, d[6] = x1.z, d[7] = x1.w;
          };
          ld8(&sm.cu.v.cst[wave][0][c0], cm);
          ld8(&sm.cu.v.cst[wave][1][c0], c7);
          ld8(&sm.cu.v.cst[wave][2][c0], c157);
          ld8(&sm.cu.v.cst[wave][3][c0], cP);
          ld8(&sm.cu.v.cst[wave][4][c0], cQ);
        }
        const uint4 kr = raw.k[u], vr = raw.v[u];
        uint4 br = {}, qr = {};
        if constexpr (CH_BJ) br = raw.b[u];
        uint4 bvu = {};
        if constexpr (PLUS) bvu = bv_at(u);
        if (want_out && valid && orow) qr = raw.q[u];
        half8 xbt, xat, xv;
        H8 hi, lo, qp;
        float aev[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kf = bf(kr, e);
          float a, bb;
          if constexpr (V == GDN_VARIANT_FG2) {
            const float sb = valid ? __builtin_amdgcn_sqrtf(bf(br, e)) : 0.0f;
            a = sb * kf;
            bb = a;
            const float sbv = PLUS ? (valid ? __builtin_amdgcn_sqrtf(bf(bvu, e)) : 0.0f) : sb;
            xv[e] = (_Float16)(bf(vr, e) * sbv * wsc);
          } else if constexpr (V == GDN_VARIANT_ASYM) {
            a = valid ? kf : 0.0f;
            bb = bscal * (STAB == 2 ? stab_j(stc, kf, bf(br, e)) : bf(br, e));
          } else {  // KDA, GDN (kscal = sqrt(beta)); DeltaProduct (bscal = beta)
            a = kscal * kf;
            bb = bscal * a;
          }
          if constexpr (V != GDN_VARIANT_FG2) xv[e] = (_Float16)(bf(vr, e) * wrow);
          const float qf = bf(qr, e);
          if constexpr (SCALAR) {
            hi.b[e] = (__bf16)a;
            lo.b[e] = (__bf16)(a - (float)hi.b[e]);
            bmh[u].b[e] = (__bf16)bb;
            bml[u].b[e] = (__bf16)(bb - (float)bmh[u].b[e]);
            qmh8[u].b[e] = (__bf16)qf;
            qml8[u].b[e] = (__bf16)(qf - (float)qmh8[u].b[e]);
            xbt[e] = (_Float16)(bb * eg_row);
            xat[e] = (_Float16)(a * eat_row);
            qp.h[e] = (_Float16)(qf * eg_row * qsc);
          } else {
            const int x = 8 * u + e;
            const float fup = __builtin_amdgcn_exp2f(G[x] - cm[e]);  // e^{G - G_7}
            const float eam = __builtin_amdgcn_rcpf(fup);            // e^{G_7 - G}
            const float st = fup * c7[e];                            // e^{G - G_start}
            const float te = eam * c157[e];                          // e^{G_end - G}
            const float ae = a * te;
            aev[e] = ae;
            bsv[x] = bb * st;
            qsv[x] = qf * st;
            xbt[e] = (_Float16)(bsv[x] * cP[e]);                     // B e^{G}
            xat[e] = (_Float16)(ae * cQ[e]);                         // A e^{G_C - G}
            qp.h[e] = (_Float16)(qsv[x] * cP[e] * qsc);              // Q e^{G}, scaled
            const float ad = a * eam;
            mdg = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, bb * fup, mdg, 0, 0, 0);
            pdg = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, qf * fup, pdg, 0, 0, 0);
          }
        }
        if (SCALAR || wave < 3) {
          if constexpr (!SCALAR) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              hi.b[e] = (__bf16)aev[e];
              lo.b[e] = (__bf16)(aev[e] - (float)hi.b[e]);
            }
          }
          *reinterpret_cast<uint4*>(&sm.ra.am.hi[r][c0]) = hi.q;
          *reinterpret_cast<uint4*>(&sm.ra.am.lo[r][c0]) = lo.q;
        }
        if constexpr (!SCALAR) {
          if (wave == 0) {  // tile 0's A side at the reference between tiles 1 and 2 (slot 3)
            const float4 d0 = *reinterpret_cast<const float4*>(&sm.cu.v.dfac[0][c0]);
            const float4 d1 = *reinterpret_cast<const float4*>(&sm.cu.v.dfac[0][c0 + 4]);
            const float df[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            H8 mh, ml;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float am = aev[e] * df[e];
              mh.b[e] = (__bf16)am;
              ml.b[e] = (__bf16)(am - (float)mh.b[e]);
            }
            *reinterpret_cast<uint4*>(&sm.ra.am.hi[48 + li][c0]) = mh.q;
            *reinterpret_cast<uint4*>(&sm.ra.am.lo[48 + li][c0]) = ml.q;
          }
        }
        if (want_out && orow)
          *reinterpret_cast<uint4*>(Q_g + ((((ro >> 4) * KB + u) * 64 + (ro & 15) + 16 * lg) * 8)) = qp.q;
        // B+ and A^ of the group transposed by MFMA: lane (li, lg) then holds steps
        // 16 wave + 4 lg .. of channel 32 u + 16 h + li
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
          const float4v tb = mma_pair_f16(xbt, sel[hh], zero);
          const float4v ta = mma_pair_f16(xat, sel[hh], zero);
          const int c = 32 * u + 16 * hh + li;
          H8 pb, pa;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb.h[e] = (_Float16)tb[e];
            pa.h[e] = (_Float16)ta[e];
          }
          *reinterpret_cast<uint2*>(&sm.bt[c][16 * wave + 4 * lg]) = pb.u[0];
          const float4v tv = mma_pair_f16(xv, sel[hh], zero);
          H8 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) pv.h[e] = (_Float16)tv[e];
          *reinterpret_cast<uint2*>(&sm.wvt[c][16 * wave + 4 * lg]) = pv.u[0];
          *reinterpret_cast<uint2*>(AT_g + size_t((((c >> 4) * CK + (wave >> 1)) * 64 + li + 16 * (2 * (wave & 1) + (lg >> 1))) * 8 +
                                                  4 * (lg & 1))) = pa.u[0];
        }
      }

      // The next item's inputs load in three groups, each once this item's copy is
      // consumed, so that the loads of the two workgroups on a CU do not arrive in
      // one burst: key and values here, query and beta / j after the Grams, the decay
      // before W and U~.
      if (has_next) load_raw(nx, raw, 1 | 2);
      wg_barrier();

      // ---- Gram tiles: M^T(J, I) = A(J) B(I)^T and P^T(J, I) = A(J) Q(I)^T, k-block
      // outer, independent accumulator chains interleaved. Scalar decay: every J
      // (blocks above the diagonal are computed and masked), the decay applied to the
      // entries afterwards. Per-channel decay: the three off-diagonal blocks J = 0, 1, 2
      // (those with J >= I are computed and masked). ----
      constexpr int NGB = SCALAR ? NT : NT - 1;
      __builtin_amdgcn_s_setprio(1);  // MFMA phase (as in the mild pass)
      float4v mreg[NGB], preg[NGB];
#pragma unroll
      for (int J = 0; J < NGB; ++J) mreg[J] = preg[J] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int c0 = 32 * u + 8 * lg;
        if constexpr (SCALAR) {
          H8 ah[NT], al[NT];
#pragma unroll
          for (int J = 0; J < NT; ++J) {
            ah[J].q = *reinterpret_cast<const uint4*>(&sm.ra.am.hi[16 * J + li][c0]);
            al[J].q = *reinterpret_cast<const uint4*>(&sm.ra.am.lo[16 * J + li][c0]);
          }
#pragma unroll
          for (int J = 0; J < NT; ++J) mreg[J] = mma_pair_bf16(ah[J].b, bmh[u].b, mreg[J]);
#pragma unroll
          for (int J = 0; J < NT; ++J) preg[J] = mma_pair_bf16(ah[J].b, qmh8[u].b, preg[J]);
#pragma unroll
          for (int J = 0; J < NT; ++J) mreg[J] = mma_pair_bf16(ah[J].b, bml[u].b, mreg[J]);
#pragma unroll
          for (int J = 0; J < NT; ++J) preg[J] = mma_pair_bf16(ah[J].b, qml8[u].b, preg[J]);
#pragma unroll
          for (int J = 0; J < NT; ++J) mreg[J] = mma_pair_bf16(al[J].b, bmh[u].b, mreg[J]);
#pragma unroll
          for (int J = 0; J < NT; ++J) preg[J] = mma_pair_bf16(al[J].b, qmh8[u].b, preg[J]);
        } else {
          // A sides: block 0 from slot 3 for tiles 2 and 3 (slot 0 for tile 1), blocks
          // 1 and 2 from slots 1 and 2
          const int row0 = (wave >= 2 ? 48 : 0) + li;
          H8 ah[3], al[3];
          ah[0].q = *reinterpret_cast<const uint4*>(&sm.ra.am.hi[row0][c0]);
          al[0].q = *reinterpret_cast<const uint4*>(&sm.ra.am.lo[row0][c0]);
#pragma unroll
          for (int J = 1; J < 3; ++J) {
            ah[J].q = *reinterpret_cast<const uint4*>(&sm.ra.am.hi[16 * J + li][c0]);
            al[J].q = *reinterpret_cast<const uint4*>(&sm.ra.am.lo[16 * J + li][c0]);
          }
          H8 bsh, bsl, qsh, qsl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float b0 = bsv[8 * u + e], q0 = qsv[8 * u + e];
            bsh.b[e] = (__bf16)b0;
            bsl.b[e] = (__bf16)(b0 - (float)bsh.b[e]);
            qsh.b[e] = (__bf16)q0;
            qsl.b[e] = (__bf16)(q0 - (float)qsh.b[e]);
          }
          // blocks 0 and 1 of tile 3: its B and Q sides moved to the reference between
          // tiles 1 and 2 (times e^{L_2}, at most 1)
          H8 bxh = bsh, bxl = bsl, qxh = qsh, qxl = qsl;
          if (wave == 3) {
            const float4 d0 = *reinterpret_cast<const float4*>(&sm.cu.v.dfac[1][c0]);
            const float4 d1 = *reinterpret_cast<const float4*>(&sm.cu.v.dfac[1][c0 + 4]);
            const float df[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float b0 = bsv[8 * u + e] * df[e], q0 = qsv[8 * u + e] * df[e];
              bxh.b[e] = (__bf16)b0;
              bxl.b[e] = (__bf16)(b0 - (float)bxh.b[e]);
              qxh.b[e] = (__bf16)q0;
              qxl.b[e] = (__bf16)(q0 - (float)qxh.b[e]);
            }
          }
          mreg[0] = mma_pair_bf16(ah[0].b, bxh.b, mreg[0]);
          mreg[1] = mma_pair_bf16(ah[1].b, bxh.b, mreg[1]);
          mreg[2] = mma_pair_bf16(ah[2].b, bsh.b, mreg[2]);
          preg[0] = mma_pair_bf16(ah[0].b, qxh.b, preg[0]);
          preg[1] = mma_pair_bf16(ah[1].b, qxh.b, preg[1]);
          preg[2] = mma_pair_bf16(ah[2].b, qsh.b, preg[2]);
          mreg[0] = mma_pair_bf16(ah[0].b, bxl.b, mreg[0]);
          mreg[1] = mma_pair_bf16(ah[1].b, bxl.b, mreg[1]);
          mreg[2] = mma_pair_bf16(ah[2].b, bsl.b, mreg[2]);
          preg[0] = mma_pair_bf16(ah[0].b, qxl.b, preg[0]);
          preg[1] = mma_pair_bf16(ah[1].b, qxl.b, preg[1]);
          preg[2] = mma_pair_bf16(ah[2].b, qsl.b, preg[2]);
          mreg[0] = mma_pair_bf16(al[0].b, bxh.b, mreg[0]);
          mreg[1] = mma_pair_bf16(al[1].b, bxh.b, mreg[1]);
          mreg[2] = mma_pair_bf16(al[2].b, bsh.b, mreg[2]);
          preg[0] = mma_pair_bf16(al[0].b, qxh.b, preg[0]);
          preg[1] = mma_pair_bf16(al[1].b, qxh.b, preg[1]);
          preg[2] = mma_pair_bf16(al[2].b, qsh.b, preg[2]);
        }
      }
      // Gram block of tile J as seen by this wave: accumulator and, for scalar decay,
      // the factors e^{G_i - G_j} of its entries (j = 16 J + 4 lg + e, i = r)
      float fdec[NT][4];
#pragma unroll
      for (int J = 0; J < NT; ++J)
#pragma unroll
        for (int e = 0; e < 4; ++e) fdec[J][e] = 1.0f;
      if constexpr (SCALAR) {
#pragma unroll
        for (int J = 0; J < NT; ++J) {
          const float4 gj = *reinterpret_cast<const float4*>(&sm.cu.s.grow[16 * J + 4 * lg]);
          const float g4[4] = {gj.x, gj.y, gj.z, gj.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) fdec[J][e] = __builtin_amdgcn_exp2f(fminf(gabs - g4[e], 0.0f));
        }
      }
      auto mblk = [&](int J) __attribute__((always_inline)) -> float4v {
        if constexpr (SCALAR) return mreg[J];
        else return J < wave ? mreg[J < 2 ? J : 2] : mdg;
      };
      auto pblk = [&](int J) __attribute__((always_inline)) -> float4v {
        if constexpr (SCALAR) return preg[J];
        else return J < wave ? preg[J < 2 ? J : 2] : pdg;
      };
      if (want_out && orow) {  // output rows are this wave's own rows (q scale qsc)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
          const int s0 = 16 * J + 4 * lg;
          const float4v src = pblk(J);
          H8 h8;
#pragma unroll
          for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)((s0 + e <= r) ? src[e] * fdec[J][e] * qsc : 0.0f);
          *reinterpret_cast<uint2*>(P_g + p_frag(ro, J)) = h8.u[0];
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (has_next) load_raw(nx, raw, 4 | 16);
      wg_barrier();  // the A sides are dead: their space now holds M and T
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (J <= wave) {
          const int s0 = 16 * J + 4 * lg;
          const float4v src = mblk(J);
          float4 m4;
          m4.x = (s0 + 0 < r) ? src[0] * fdec[J][0] : 0.0f;
          m4.y = (s0 + 1 < r) ? src[1] * fdec[J][1] : 0.0f;
          m4.z = (s0 + 2 < r) ? src[2] * fdec[J][2] : 0.0f;
          m4.w = (s0 + 3 < r) ? src[3] * fdec[J][3] : 0.0f;
          *reinterpret_cast<float4*>(&sm.ra.mt.m[r][s0]) = m4;
        }
      }
      wg_barrier();

    }

    // ---- T = (I + M)^{-1}: diagonal 16x16 blocks by forward substitution ----
    // (at raised wave priority, as in chunk_prep_kernel)
    if (wave == 0) {
      __builtin_amdgcn_s_setprio(2);
      const int bI = lane >> 4, c = lane & 15;
      float xcol[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float s4[4] = {(rr == c) ? 1.0f : 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < rr; ++s2) s4[s2 & 3] -= sm.ra.mt.m[16 * bI + rr][16 * bI + s2] * xcol[s2];
        xcol[rr] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.ra.mt.t[16 * bI + rr][16 * bI + c] = xcol[rr];
    }
    // off-diagonal blocks: T_IJ = -T_II sum_{K=J}^{I-1} M_IK T_KJ, one level per I
#pragma unroll
    for (int I = 1; I < NT; ++I) {
      wg_barrier();
      if (wave < I) {
        __builtin_amdgcn_s_setprio(2);
        const int J = wave;
        float4v xa = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int K = J; K < I; ++K) {
          float a4[4], b4[4];
          quad(&sm.ra.mt.m[16 * I + li][16 * K + 4 * lg], a4);
#pragma unroll
          for (int e = 0; e < 4; ++e) b4[e] = sm.ra.mt.t[16 * K + 4 * lg + e][16 * J + li];
          xa = mma_slice_f32(a4, b4, xa);
        }
        float a4[4], xb[4] = {xa[0], xa[1], xa[2], xa[3]};
        quad(&sm.ra.mt.t[16 * I + li][16 * I + 4 * lg], a4);
        const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
        const float4v y = mma_slice_f32(a4, xb, zero);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.ra.mt.t[16 * I + 4 * lg + e][16 * J + li] = -y[e];
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wg_barrier();
    // operand copy of T in fp16 with a zero upper triangle, over the dead M
    _Float16* top = reinterpret_cast<_Float16*>(&sm.ra.mt.m[0][0]);
    constexpr int LDT = 2 * 68;
    for (int u = tid; u < C * C / 4; u += kThreads) {
      const int rr = u / (C / 4), s0 = 4 * (u % (C / 4));
      const float4 tv = *reinterpret_cast<const float4*>(&sm.ra.mt.t[rr][s0]);
      H8 h8;
      h8.h[0] = (s0 + 0 <= rr) ? (_Float16)tv.x : (_Float16)0.0f;
      h8.h[1] = (s0 + 1 <= rr) ? (_Float16)tv.y : (_Float16)0.0f;
      h8.h[2] = (s0 + 2 <= rr) ? (_Float16)tv.z : (_Float16)0.0f;
      h8.h[3] = (s0 + 3 <= rr) ? (_Float16)tv.w : (_Float16)0.0f;
      *reinterpret_cast<uint2*>(top + rr * LDT + s0) = h8.u[0];
    }
    wg_barrier();

    if (has_next) {
      load_raw(nx, raw, 8);
      scal = load_scal(nx);
    }
    // ---- W^T = B+^T T^T (stored as W rows) and U~ = T Wv (stored transposed): wave w
    // computes the tiles of step rows 16 w .., independent chains interleaved (an
    // MFMA phase: raised wave priority) ----
    __builtin_amdgcn_s_setprio(1);
    H8 ta[2];  // T rows 16 w + li, steps 32 u + 4 lg .. (+16)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const _Float16* trow = top + (16 * wave + li) * LDT + 32 * u + 4 * lg;
      ta[u] = pair4(trow, trow + 16);
    }
    {
      float4v wacc[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) wacc[ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const _Float16* brow = &sm.bt[16 * ct + li][32 * u + 4 * lg];
          wacc[ct] = mma_pair_f16(pair4(brow, brow + 16).h, ta[u].h, wacc[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        H8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)wacc[ct][e];
        *reinterpret_cast<uint2*>(W_g + w_frag(wave, ct)) = h8.u[0];
      }
    }
    {
      float4v uacc[VT];
#pragma unroll
      for (int ct = 0; ct < VT; ++ct) uacc[ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int ct = 0; ct < VT; ++ct) {
          const _Float16* brow = &sm.wvt[16 * ct + li][32 * u + 4 * lg];
          uacc[ct] = mma_pair_f16(ta[u].h, pair4(brow, brow + 16).h, uacc[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < VT; ++ct) {
        H8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)uacc[ct][e];
        *reinterpret_cast<uint2*>(UT_g + u_frag(wave, ct)) = h8.u[0];
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wg_barrier();  // LDS is reused by the next chunk
  }
}

template <typename In, int DK, int C, int V, bool DPV>
int launch_prep_t(const Problem& p, void* ws, bool want_out, hipStream_t s) {
  const ChunkLayout L = chunk_layout(p);
  const int64_t items = p.nchunks * p.B * p.H;
  if constexpr (std::is_same<In, uint16_t>::value && DK == 128 && C == 64) {
    if (prep2_covers(p)) {  // two workgroups per CU
      const int64_t grid = std::min<int64_t>(items, 2 * int64_t(device_cus()));
      unsigned char* w = static_cast<unsigned char*>(ws);
      unsigned char* fl = w + record_bytes(p, L);  // one byte per item, after the records
      const int wo = want_out ? 1 : 0;
      const dim3 g = dim3(unsigned(grid));
      if constexpr (DPV) {
        if (p.n_step == 2)
          chunk_prep2_kernel<V, 0, 2, 0><<<g, kThreads, 0, s>>>(p, w, fl, L, wo);
        else
          chunk_prep2_kernel<V, 0, 4, 0><<<g, kThreads, 0, s>>>(p, w, fl, L, wo);
      } else if constexpr (V == GDN_VARIANT_GDN || V == GDN_VARIANT_DELTAPRODUCT) {
        chunk_prep2_kernel<V, 0, 1, 0><<<g, kThreads, 0, s>>>(p, w, fl, L, wo);
      } else {
        // per-channel decay: chunks of mild decay first, then the flagged ones
        auto two_pass = [&](auto mild_pass, auto flagged_pass) {
          mild_pass<<<g, kThreads, 0, s>>>(p, w, fl, L, wo);
          flagged_pass<<<g, kThreads, 0, s>>>(p, w, fl, L, wo);
        };
        if constexpr (V == GDN_VARIANT_ASYM) {
          if (p.stabilize == GDN_STABILIZE_CLIP_DECAY)
            two_pass(chunk_prep2_kernel<V, 1, 1, 1>, chunk_prep2_kernel<V, 1, 1, 2>);
          else if (p.stabilize == GDN_STABILIZE_PROJECT_J)
            two_pass(chunk_prep2_kernel<V, 2, 1, 1>, chunk_prep2_kernel<V, 2, 1, 2>);
          else
            two_pass(chunk_prep2_kernel<V, 0, 1, 1>, chunk_prep2_kernel<V, 0, 1, 2>);
        } else if constexpr (V == GDN_VARIANT_FG2) {
          if (p.beta_v != nullptr)  // FG2-GDN+
            two_pass(chunk_prep2_kernel<V, 0, 1, 1, true>, chunk_prep2_kernel<V, 0, 1, 2, true>);
          else
            two_pass(chunk_prep2_kernel<V, 0, 1, 1>, chunk_prep2_kernel<V, 0, 1, 2>);
        } else {
          two_pass(chunk_prep2_kernel<V, 0, 1, 1>, chunk_prep2_kernel<V, 0, 1, 2>);
        }
      }
      return int(hipGetLastError());
    }
  }
  constexpr size_t lds = sizeof(PrepLds<std::is_same<In, uint16_t>::value, DK, C, DPV>);
  constexpr int occ = prep_occupancy<In, DK, C>();
  static_assert(occ == 1 || occ * lds <= 160 * 1024, "LDS of the intended occupancy");
  const int per_cu = occ > 1 ? occ : lds <= 40 * 1024 ? 4 : lds <= 80 * 1024 ? 2 : 1;
  const int64_t grid = std::min<int64_t>(items, int64_t(device_cus()) * per_cu);
  chunk_prep_kernel<In, DK, C, V, DPV><<<dim3(unsigned(grid)), kThreads, 0, s>>>(
      p, static_cast<unsigned char*>(ws), L, want_out ? 1 : 0);
  return int(hipGetLastError());
}

template <typename In, int DK, int V>
int launch_prep_dk(const Problem& p, void* ws, bool want_out, hipStream_t s) {
  constexpr bool DPAIR = V == GDN_VARIANT_DELTAPRODUCT;
  switch (p.chunk) {
    case 16:
      if constexpr (DPAIR)
        if (p.n_h > 1) return launch_prep_t<In, DK, 16, V, DPAIR>(p, ws, want_out, s);
      return launch_prep_t<In, DK, 16, V, false>(p, ws, want_out, s);
    case 32:
      if constexpr (DPAIR)
        if (p.n_h > 1) return launch_prep_t<In, DK, 32, V, DPAIR>(p, ws, want_out, s);
      return launch_prep_t<In, DK, 32, V, false>(p, ws, want_out, s);
    case 64:
      if constexpr (std::is_same<In, float>::value && DK == 128) {
        return int(hipErrorInvalidValue);
      } else {
        if constexpr (DPAIR)
          if (p.n_h > 1) return launch_prep_t<In, DK, 64, V, DPAIR>(p, ws, want_out, s);
        return launch_prep_t<In, DK, 64, V, false>(p, ws, want_out, s);
      }
    default: return int(hipErrorInvalidValue);
  }
}

template <typename In, int V>
int launch_prep_in(const Problem& p, void* ws, bool want_out, hipStream_t s) {
  switch (p.dk) {
    case 16: return launch_prep_dk<In, 16, V>(p, ws, want_out, s);
    case 32: return launch_prep_dk<In, 32, V>(p, ws, want_out, s);
    case 64: return launch_prep_dk<In, 64, V>(p, ws, want_out, s);
    case 128: return launch_prep_dk<In, 128, V>(p, ws, want_out, s);
    default: return int(hipErrorInvalidValue);
  }
}

template <int V>
int launch_prep_variant(const Problem& p, void* ws, bool want_out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.dtype == GDN_DTYPE_BF16 ? launch_prep_in<uint16_t, V>(p, ws, want_out, s)
                                   : launch_prep_in<float, V>(p, ws, want_out, s);
}

}  // namespace
}  // namespace gdn
