// Chunkwise-parallel forward pass (WY / UT form), two kernels per call.
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
// unified step. The Gram factors use a reference point in the middle of the
// chunk (e^{G - G_mid}, e^{G_mid - G}) so that no factor exceeds the decay
// accumulated over half a chunk.
//
// Kernel 1 (chunk_prep): persistent; each workgroup walks chunks. Wave w owns
// rows 16w..16w+15 of the chunk: it loads them straight into registers (16-byte
// fragments), scans the log decay over its rows with lane shuffles, and forms the
// decayed operands. LDS carries only what crosses waves (A- for the Grams, B+ and
// Wv transposed, then M and T). It writes one record per chunk (gdn_internal.h).
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Inclusive prefix sum over the 16 lanes of a lane group (rows of a tile).
__device__ __forceinline__ float scan16(float x, int i) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const float y = __shfl_up(x, d, 16);
    if (i >= d) x += y;
  }
  return x;
}

// ---- kernel 1: chunk-local preparation -----------------------------------------------

// exp / log / sqrt: the hardware instructions (one VALU op each, about 1 ulp in
// the base-2 domain) on the bf16 path, the accurate library calls on the fp32 path.
template <bool F16>
__device__ __forceinline__ float dexp(float x) {
  if constexpr (F16) return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
  else return expf(x);
}
template <bool F16>
__device__ __forceinline__ float dlog(float x) {
  if constexpr (F16) return __builtin_amdgcn_logf(x) * 0.6931471805599453f;
  else return logf(x);
}
template <bool F16>
__device__ __forceinline__ float dsqrt(float x) {
  if constexpr (F16) return __builtin_amdgcn_sqrtf(x);
  else return sqrtf(x);
}

// Value x (0 <= x < 8 * n, compile-time after unrolling) of bf16 groups held as uint4.
__device__ __forceinline__ float bf16_at(const uint4* v, int x) {
  const uint4 w = v[x / 8];
  const uint32_t word = (x % 8) / 2 == 0 ? w.x : (x % 8) / 2 == 1 ? w.y : (x % 8) / 2 == 2 ? w.z : w.w;
  return __uint_as_float((x & 1) ? (word & 0xffff0000u) : (word << 16));
}

// Raw inputs of one step row, loaded ahead of use (bf16 rows as packed groups).
template <bool F16, int DK>
struct RawRow {
  using KM = ChanMap<F16, DK>;
  static constexpr int KU = F16 ? (KM::UW == 8 ? KM::NU : 1) : 1;  // uint4 per key row (bf16)
  uint4 k[KU], a[KU], bj[KU], q[KU];
  uint4 v[4], bv[4];
  float s_alpha, s_beta, s_eta;
};

template <bool F16, int DK, int C, bool DPV>
struct PrepLds {
  using Op = std::conditional_t<F16, _Float16, float>;
  using Am = std::conditional_t<F16, __bf16, float>;
  static constexpr int LDA = F16 ? DK + 8 : DK + 4;  // rows of A- (16-byte aligned)
  static constexpr int LDC = C + 4;
  static constexpr int QR = DPV ? C / 2 : 1;         // output rows kept in LDS (n_h >= 2)
  union RA {
    struct {
      Am hi[C][LDA];
      Am lo[F16 ? C : 1][LDA];
    } am;                      // A- (mid reference), Gram phase
    struct {
      float m[C][LDC];         // strictly lower Gram M; T in fp16 after the inverse
      float t[C][LDC];         // T = (I + M)^{-1}
    } mt;
  } ra;
  Op bt[DK][LDC];              // B+ (chunk-start reference), transposed
  Op wvt[128][LDC];            // written values (scaled), transposed
  Op at[DK][LDC];              // A^ transposed, staged for a coalesced copy to the record
  Am qmh[QR][LDA];             // Q+ (mid reference) of output rows, DeltaProduct only
  Am qml[(DPV && F16) ? QR : 1][LDA];
  float tot[kWaves][DK];       // per-tile totals of the log decay
  float gmid_loc[DK];          // in-tile prefix at the middle row
  float qs[C];                 // per output row q scale
  float red[kWaves];
};

template <typename In, int DK, int C, bool DPV>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(Problem p, unsigned char* __restrict__ ws,
                                                              ChunkLayout L, int want_out) {
  constexpr bool F16 = std::is_same<In, uint16_t>::value;
  using Sm = PrepLds<F16, DK, C, DPV>;
  using Op = typename Sm::Op;
  using KM = ChanMap<F16, DK>;
  using Raw = RawRow<F16, DK>;
  constexpr int NX = KM::NX;
  constexpr int NT = C / 16;
  constexpr int KB = F16 ? (DK + 31) / 32 : DK / 16;  // k-blocks (F16) or slices (F32) of a key row
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  static_assert(NT <= kWaves, "one wave per 16-row tile");
  __shared__ Sm sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n_h = p.n_h, R = p.rows_out, RT = R / 16;
  const int dv = int(p.dv);
  const int64_t NC = p.nchunks;
  const int64_t total = NC * p.B * p.H;
  const int mid = C / 2 - 1, tile_mid = mid / 16, row_mid = mid % 16;
  const In* qg = static_cast<const In*>(p.q);
  const In* kg = static_cast<const In*>(p.k);
  const In* vg = static_cast<const In*>(p.v);
  const In* alg = static_cast<const In*>(p.alpha);
  const In* beg = static_cast<const In*>(p.beta);
  const In* bvg = static_cast<const In*>(p.beta_v);
  const In* jg = static_cast<const In*>(p.j);
  const In* etg = static_cast<const In*>(p.eta);
  const bool dp = p.variant == GDN_VARIANT_DELTAPRODUCT;
  const bool owner = wave < NT;
  const int r = 16 * wave + li;  // virtual row (step) in the chunk owned by this lane
  // value-row groups: 8 bf16 channels (32 u + 8 g + s) per uint4, or 4 (4 g + s) when dv == 16
  const int vuw = (F16 && dv == 16) ? 4 : 8;
  const int vnu = F16 ? (dv == 16 ? 1 : dv / 32) : 0;
  auto ld = [](const In* x) { return IO<In>::ld(x); };

  struct Where {
    bool valid, out_row;
    int64_t tok, th, vrow;
    int sub, ro;
  };
  auto where = [&](int64_t item) __attribute__((always_inline)) -> Where {
    Where w;
    const int64_t bh = item / NC, n = item % NC;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t vs = n * C + r;
    w.valid = owner && vs < p.steps;
    w.tok = vs / n_h;
    w.sub = int(vs % n_h);
    w.th = (b * p.T + w.tok) * p.H + h;
    w.vrow = dp ? w.th * n_h + w.sub : w.th;
    w.out_row = want_out && owner && w.sub == n_h - 1;
    w.ro = r / n_h;
    return w;
  };
  // Issue every load of this lane's row of `item` (bf16 rows only; fp32 rows are
  // read where they are used).
  auto prefetch = [&](int64_t item, Raw& raw) __attribute__((always_inline)) {
    if constexpr (F16) {
      const Where w = where(item);
      raw.s_alpha = raw.s_beta = raw.s_eta = 0.0f;
      if (!w.valid) return;
      auto ld_row = [&](const In* row, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < Raw::KU; ++u) {
          if constexpr (KM::UW == 8) {
            dst[u] = *reinterpret_cast<const uint4*>(row + u * 32 + 8 * lg);
          } else {
            const uint2 x = *reinterpret_cast<const uint2*>(row + 4 * lg);
            dst[u] = make_uint4(x.x, x.y, 0u, 0u);
          }
        }
      };
      ld_row(kg + w.vrow * DK, raw.k);
      if (dp) {
        raw.s_beta = ld(beg + w.vrow);
        raw.s_alpha = ld(alg + w.th);
      } else {
        if (p.variant == GDN_VARIANT_GDN) raw.s_alpha = ld(alg + w.th);
        else ld_row(alg + w.th * DK, raw.a);
        if (p.variant == GDN_VARIANT_FG2) ld_row(beg + w.th * DK, raw.bj);
        else if (p.variant == GDN_VARIANT_ASYM) ld_row(jg + w.th * DK, raw.bj);
        else raw.s_beta = ld(beg + w.th);
        if (p.variant == GDN_VARIANT_ASYM) raw.s_eta = ld(etg + w.th);
      }
      if (w.out_row && w.tok < p.T) ld_row(qg + w.th * DK, raw.q);
      const In* vrow = vg + w.vrow * dv;
      const In* bvrow = bvg ? bvg + w.th * dv : beg + w.th * DK;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < vnu) {
          if (vuw == 8) {
            raw.v[u] = *reinterpret_cast<const uint4*>(vrow + u * 32 + 8 * lg);
            if (p.variant == GDN_VARIANT_FG2) raw.bv[u] = *reinterpret_cast<const uint4*>(bvrow + u * 32 + 8 * lg);
          } else {
            const uint2 x = *reinterpret_cast<const uint2*>(vrow + 4 * lg);
            raw.v[u] = make_uint4(x.x, x.y, 0u, 0u);
            if (p.variant == GDN_VARIANT_FG2) {
              const uint2 y = *reinterpret_cast<const uint2*>(bvrow + 4 * lg);
              raw.bv[u] = make_uint4(y.x, y.y, 0u, 0u);
            }
          }
        }
      }
    }
  };

  Raw raw;
  if (blockIdx.x < total) prefetch(blockIdx.x, raw);

  for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
    const Where w = where(item);
    const int64_t n = item % NC;
    unsigned char* rec = ws + size_t(item) * L.bytes;
    Op* W_g = reinterpret_cast<Op*>(rec + L.off_W);
    Op* AT_g = reinterpret_cast<Op*>(rec + L.off_AT);
    Op* Q_g = reinterpret_cast<Op*>(rec + L.off_Q);
    Op* P_g = reinterpret_cast<Op*>(rec + L.off_P);
    Op* UT_g = reinterpret_cast<Op*>(rec + L.off_UT);
    float* gam_g = reinterpret_cast<float*>(rec + L.off_gamma);
    float* winv_g = reinterpret_cast<float*>(rec + L.off_winv);
    float* qinv_g = reinterpret_cast<float*>(rec + L.off_qinv);
    (void)n;

    // ---- keys, written value factor, log decay of this lane's row ----
    // a: write key, bb: erase key, G: log decay (then its scan), wscal: scalar
    // factor of the written value.
    float a[NX], bb[NX], G[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) a[x] = bb[x] = G[x] = 0.0f;
    float wscal = 0.0f;
    if (w.valid) {
      if constexpr (F16) {
        const float sa = raw.s_alpha, sbt = raw.s_beta;
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          const float kx = bf16_at(raw.k, x);
          if (dp) {
            a[x] = kx;
            bb[x] = sbt * kx;
            G[x] = w.sub == 0 ? dlog<F16>(sa) : 0.0f;
          } else {
            G[x] = dlog<F16>(p.variant == GDN_VARIANT_GDN ? sa : bf16_at(raw.a, x));
            if (p.variant == GDN_VARIANT_FG2) {
              a[x] = dsqrt<F16>(bf16_at(raw.bj, x)) * kx;
              bb[x] = a[x];
            } else if (p.variant == GDN_VARIANT_ASYM) {
              a[x] = kx;
              bb[x] = raw.s_eta * bf16_at(raw.bj, x);
            } else {
              a[x] = dsqrt<F16>(sbt) * kx;
              bb[x] = a[x];
            }
          }
        }
        wscal = dp ? sbt : p.variant == GDN_VARIANT_ASYM ? raw.s_eta : dsqrt<F16>(sbt);
      } else {
        if (dp) {
          load_row<F16, DK>(kg + w.vrow * DK, lg, a);
          const float bi = ld(beg + w.vrow);
          const float lgate = w.sub == 0 ? dlog<F16>(ld(alg + w.th)) : 0.0f;
#pragma unroll
          for (int x = 0; x < NX; ++x) {
            bb[x] = bi * a[x];
            G[x] = lgate;
          }
          wscal = bi;
        } else {
          load_row<F16, DK>(kg + w.th * DK, lg, a);
          if (p.variant == GDN_VARIANT_GDN) {
            const float lgam = dlog<F16>(ld(alg + w.th));
#pragma unroll
            for (int x = 0; x < NX; ++x) G[x] = lgam;
          } else {
            load_row<F16, DK>(alg + w.th * DK, lg, G);
#pragma unroll
            for (int x = 0; x < NX; ++x) G[x] = dlog<F16>(G[x]);
          }
          if (p.variant == GDN_VARIANT_FG2) {
            load_row<F16, DK>(beg + w.th * DK, lg, bb);
#pragma unroll
            for (int x = 0; x < NX; ++x) {
              a[x] *= dsqrt<F16>(bb[x]);
              bb[x] = a[x];
            }
          } else if (p.variant == GDN_VARIANT_ASYM) {
            load_row<F16, DK>(jg + w.th * DK, lg, bb);
            const float e = ld(etg + w.th);
#pragma unroll
            for (int x = 0; x < NX; ++x) bb[x] *= e;
            wscal = e;
          } else {
            const float sb = dsqrt<F16>(ld(beg + w.th));
#pragma unroll
            for (int x = 0; x < NX; ++x) {
              a[x] *= sb;
              bb[x] = a[x];
            }
            wscal = sb;
          }
        }
      }
    }
    // inclusive scan of the log decay over the tile's 16 rows, then tile totals
#pragma unroll
    for (int x = 0; x < NX; ++x) G[x] = scan16(G[x], li);
    if (owner && li == 15) {
#pragma unroll
      for (int x = 0; x < NX; ++x) sm.tot[wave][KM::chan(lg, x)] = G[x];
    }
    if (owner && wave == tile_mid && li == row_mid) {
#pragma unroll
      for (int x = 0; x < NX; ++x) sm.gmid_loc[KM::chan(lg, x)] = G[x];
    }
    // query row (fp32) and its power-of-two scale
    float qv[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) qv[x] = 0.0f;
    float qsc = 1.0f;
    if (owner && want_out) {
      if (w.out_row && w.valid && w.tok < p.T) {
        if constexpr (F16) {
#pragma unroll
          for (int x = 0; x < NX; ++x) qv[x] = bf16_at(raw.q, x);
        } else {
          load_row<F16, DK>(qg + w.th * DK, lg, qv);
        }
      }
      if constexpr (F16) {
        float mx = 0.0f;
#pragma unroll
        for (int x = 0; x < NX; ++x) mx = fmaxf(mx, fabsf(qv[x]));
        qsc = pow2_scale_for(max_over_groups(mx));
      }
    }
    // written values w (bf16 path: from the prefetched groups); max |w| for the
    // power-of-two scale of Wv
    float wv[32];
#pragma unroll
    for (int x = 0; x < 32; ++x) wv[x] = 0.0f;
    float wmax = 0.0f;
    if constexpr (F16) {
      if (w.valid) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (u < vnu) {
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
              const float vx = bf16_at(raw.v, 8 * u + s2);
              const float f = p.variant == GDN_VARIANT_FG2 ? dsqrt<F16>(bf16_at(raw.bv, 8 * u + s2)) : wscal;
              wv[8 * u + s2] = (vuw == 8 || s2 < 4) ? vx * f : 0.0f;
              wmax = fmaxf(wmax, fabsf(wv[8 * u + s2]));
            }
          }
        }
      }
    }
    wmax = wave_max(wmax);
    if (lane == 0) sm.red[wave] = wmax;
    __syncthreads();

    float wsc = 1.0f;
    if constexpr (F16) {
      float m = sm.red[0];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) m = fmaxf(m, sm.red[w2]);
      wsc = pow2_scale_for(m);
    }

    // ---- decayed operands of this wave's rows ----
    float bm[NX];  // B+ with the mid reference: B-side of M
    float qm[NX];  // Q+ with the mid reference: B-side of P
#pragma unroll
    for (int x = 0; x < NX; ++x) bm[x] = qm[x] = 0.0f;
    if (owner) {
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int c = KM::chan(lg, x);
        float pre = 0.0f, ge = 0.0f, gm = sm.gmid_loc[c];
#pragma unroll
        for (int I = 0; I < NT; ++I) {
          const float tv = sm.tot[I][c];
          if (I < wave) pre += tv;
          if (I < tile_mid) gm += tv;
          ge += tv;
        }
        const float g = G[x] + pre;
        const float fup = dexp<F16>(g - gm);   // e^{G - G_mid}
        const float eg = dexp<F16>(g);         // e^{G}
        bm[x] = bb[x] * fup;
        sm.bt[c][r] = (Op)(bb[x] * eg);
        sm.at[c][r] = (Op)(a[x] * dexp<F16>(ge - g));
        const float am = a[x] * dexp<F16>(gm - g);
        if constexpr (F16) {
          const __bf16 hi = (__bf16)am;
          sm.ra.am.hi[r][c] = hi;
          sm.ra.am.lo[r][c] = (__bf16)(am - (float)hi);
        } else {
          sm.ra.am.hi[r][c] = am;
        }
        if (wave == 0 && li == 0) gam_g[c] = dexp<F16>(ge);
        qm[x] = qv[x] * fup;
        qv[x] = qv[x] * eg * qsc;              // Q+ (chunk-start reference), scaled
        if constexpr (DPV) {
          if (w.out_row) {
            if constexpr (F16) {
              const __bf16 hi = (__bf16)qm[x];
              sm.qmh[w.ro][c] = hi;
              sm.qml[w.ro][c] = (__bf16)(qm[x] - (float)hi);
            } else {
              sm.qmh[w.ro][c] = qm[x];
            }
          }
        }
      }
      if (w.out_row) {
        Op* qrow = Q_g + size_t(w.ro) * L.ldk;
        if constexpr (F16) {
#pragma unroll
          for (int u = 0; u < KB; ++u) {
            if constexpr (KM::UW == 8) {
              H8 h8;
#pragma unroll
              for (int s2 = 0; s2 < 8; ++s2) h8.h[s2] = (_Float16)qv[8 * u + s2];
              // the row pitch (dk + 4 halves) keeps rows 8-byte aligned
              uint2* q2 = reinterpret_cast<uint2*>(qrow + KM::chan(lg, 8 * u));
              q2[0] = h8.u[0];
              q2[1] = h8.u[1];
            } else {
#pragma unroll
              for (int s2 = 0; s2 < KM::UW; ++s2) qrow[KM::chan(lg, s2)] = (_Float16)qv[s2];
            }
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
      // written values, scaled, transposed into LDS
      if constexpr (F16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (u < vnu) {
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
              if (vuw == 8 || s2 < 4) {
                const int c = vuw == 8 ? 32 * u + 8 * lg + s2 : 4 * lg + s2;
                sm.wvt[c][r] = (Op)(wv[8 * u + s2] * wsc);
              }
            }
          }
        }
      } else {
        const In* vrow = vg + w.vrow * dv;
        const In* brow_v = beg + w.th * DK;
        const In* bvrow = bvg ? bvg + w.th * dv : nullptr;
        switch (dv) {
          case 16: row_values<F16, 16>(p.variant, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
          case 32: row_values<F16, 32>(p.variant, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
          case 64: row_values<F16, 64>(p.variant, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
          default: row_values<F16, 128>(p.variant, vrow, brow_v, DK, bvrow, wscal, w.valid, lg, r, wsc, sm.wvt, true); break;
        }
      }
    }
    if (tid == 0) winv_g[0] = 1.0f / wsc;
    // Every raw value of this item is consumed: load the next item's rows now so
    // they arrive while the Grams, the inverse and W / U~ are computed.
    if (item + gridDim.x < total) prefetch(item + gridDim.x, raw);
    __syncthreads();

    // A^ transposed: the LDS tile has the record's row pitch (C + 4), so the copy
    // is flat and coalesced (the pad columns are never read as operands).
    {
      constexpr int UNITS = DK * Sm::LDC * int(sizeof(Op)) / 16;
      static_assert(DK * Sm::LDC * sizeof(Op) % 16 == 0, "flat copy in 16-byte units");
      const uint4* src = reinterpret_cast<const uint4*>(&sm.at[0][0]);
      uint4* dst = reinterpret_cast<uint4*>(AT_g);
      for (int u = tid; u < UNITS; u += kThreads) dst[u] = src[u];
    }

    // ---- Gram tiles: M^T(J, I) = A-(J) B+(I)^T and P^T(J, Io) = A-(J) Q+(Io)^T ----
    // The B side (own rows) is split into bf16 hi/lo once per item.
    H8 bmh[F16 ? KB : 1], bml[F16 ? KB : 1], qmh8[F16 ? KB : 1], qml8[F16 ? KB : 1];
    if constexpr (F16) {
#pragma unroll
      for (int u = 0; u < KB; ++u) {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const float v0 = s2 < KM::UW ? bm[u * KM::UW + (s2 < KM::UW ? s2 : 0)] : 0.0f;
          const float v1 = s2 < KM::UW ? qm[u * KM::UW + (s2 < KM::UW ? s2 : 0)] : 0.0f;
          const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
          bmh[u].b[s2] = h0;
          bml[u].b[s2] = (__bf16)(v0 - (float)h0);
          qmh8[u].b[s2] = h1;
          qml8[u].b[s2] = (__bf16)(v1 - (float)h1);
        }
      }
    }
    // A side from LDS rows of tile J; B side from registers (own rows) or LDS.
    auto gram = [&](int J, const H8* xh, const H8* xl, const float* xb, int qrow_lds)
        __attribute__((always_inline)) -> float4v {
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (F16) {
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int c0 = u * 4 * KM::UW + KM::UW * lg;
          H8 ah, al, bh, bl;
          if constexpr (KM::UW == 8) {
            ah.q = *reinterpret_cast<const uint4*>(&sm.ra.am.hi[16 * J + li][c0]);
            al.q = *reinterpret_cast<const uint4*>(&sm.ra.am.lo[16 * J + li][c0]);
          } else {
            ah = pair4(&sm.ra.am.hi[16 * J + li][c0], nullptr);
            al = pair4(&sm.ra.am.lo[16 * J + li][c0], nullptr);
          }
          if (qrow_lds >= 0) {
            if constexpr (DPV) {
              if constexpr (KM::UW == 8) {
                bh.q = *reinterpret_cast<const uint4*>(&sm.qmh[qrow_lds][c0]);
                bl.q = *reinterpret_cast<const uint4*>(&sm.qml[qrow_lds][c0]);
              } else {
                bh = pair4(&sm.qmh[qrow_lds][c0], nullptr);
                bl = pair4(&sm.qml[qrow_lds][c0], nullptr);
              }
            }
          } else {
            bh = xh[u];
            bl = xl[u];
          }
          acc = mma_pair_bf16(ah.b, bh.b, acc);
          acc = mma_pair_bf16(ah.b, bl.b, acc);
          acc = mma_pair_bf16(al.b, bh.b, acc);
        }
      } else {
#pragma unroll
        for (int t = 0; t < KB; ++t) {
          float a4[4], b4[4];
          quad(&sm.ra.am.hi[16 * J + li][16 * t + 4 * lg], a4);
          if (qrow_lds >= 0) {
            if constexpr (DPV) quad(&sm.qmh[qrow_lds][16 * t + 4 * lg], b4);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) b4[e] = xb[4 * t + e];
          }
          acc = mma_slice_f32(a4, b4, acc);
        }
      }
      return acc;
    };

    float4v mreg[NT];
#pragma unroll
    for (int J = 0; J < NT; ++J) mreg[J] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    if (owner) {
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (J <= wave) mreg[J] = gram(J, bmh, bml, bm, -1);
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
            if (J <= wave) acc = gram(J, qmh8, qml8, qm, -1);
            const int s0 = 16 * J + 4 * lg;
            Op* dst = P_g + size_t(ro) * L.ldc + s0;
            if constexpr (F16) {
              H8 h8;
#pragma unroll
              for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)((s0 + e <= ro) ? acc[e] * qsl : 0.0f);
              *reinterpret_cast<uint2*>(dst) = h8.u[0];
            } else {
              *reinterpret_cast<float4*>(dst) = make_float4((s0 + 0 <= ro) ? acc[0] : 0.0f, (s0 + 1 <= ro) ? acc[1] : 0.0f,
                                                            (s0 + 2 <= ro) ? acc[2] : 0.0f, (s0 + 3 <= ro) ? acc[3] : 0.0f);
            }
          }
        }
      } else {
        if (wave < RT) {
          const int ro = 16 * wave + li;
          const int tau = ro * n_h + n_h - 1;
          const int jmax = min(NT - 1, ((16 * wave + 15) * n_h + n_h - 1) / 16);
          const float qsl = sm.qs[ro];
          for (int J = 0; J < NT; ++J) {
            float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
            if (J <= jmax) acc = gram(J, qmh8, qml8, qm, ro);
            const int s0 = 16 * J + 4 * lg;
            Op* dst = P_g + size_t(ro) * L.ldc + s0;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = (Op)((s0 + e <= tau) ? acc[e] * qsl : 0.0f);
          }
        }
      }
    }
    __syncthreads();  // A- is dead: its space now holds M and T
    if (owner) {
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
    }
    __syncthreads();

    // ---- T = (I + M)^{-1}: diagonal 16x16 blocks by forward substitution ----
    if (wave == 0) {
      const int bI = lane >> 4, c = lane & 15;
      if (bI < NT) {
        float xcol[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float sacc = (rr == c) ? 1.0f : 0.0f;
#pragma unroll
          for (int s2 = 0; s2 < rr; ++s2) sacc -= sm.ra.mt.m[16 * bI + rr][16 * bI + s2] * xcol[s2];
          xcol[rr] = sacc;
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
    __syncthreads();
    // operand copy of T with a zero upper triangle (fp16 over the dead M; fp32 in place)
    Op* top = F16 ? reinterpret_cast<Op*>(&sm.ra.mt.m[0][0]) : reinterpret_cast<Op*>(&sm.ra.mt.t[0][0]);
    constexpr int LDT = F16 ? 2 * Sm::LDC : Sm::LDC;  // fp16 rows over fp32 rows: twice the elements
    for (int u = tid; u < C * C; u += kThreads) {
      const int rr = u / C, s2 = u % C;
      const float tv = sm.ra.mt.t[rr][s2];
      if constexpr (F16) top[rr * LDT + s2] = (s2 <= rr) ? (Op)tv : (Op)0.0f;
      else if (s2 > rr) sm.ra.mt.t[rr][s2] = 0.0f;
    }
    __syncthreads();

    // ---- W^T = B+^T T^T (stored as W rows) and U~ = T Wv (stored transposed) ----
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
    constexpr int NWT = (DK / 16) * NT;
    for (int x = wave; x < NWT; x += kWaves) {
      const int ct = x / NT, I = x % NT;
      const float4v acc = tprod(&sm.bt[16 * ct + li][0], top + (16 * I + li) * LDT, I);
      Op* dst = W_g + size_t(16 * I + li) * L.ldk + 16 * ct + 4 * lg;
      if constexpr (F16) {
        H8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)acc[e];
        *reinterpret_cast<uint2*>(dst) = h8.u[0];
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    const int VT = dv / 16;
    for (int x = wave; x < NT * VT; x += kWaves) {
      const int I = x / VT, ct = x % VT;
      const float4v acc = tprod(top + (16 * I + li) * LDT, &sm.wvt[16 * ct + li][0], I);
      Op* dst = UT_g + size_t(16 * ct + li) * C + 16 * I + 4 * lg;
      if constexpr (F16) {
        H8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) h8.h[e] = (_Float16)acc[e];
        *reinterpret_cast<uint2*>(dst) = h8.u[0];
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    __syncthreads();  // LDS is reused by the next chunk
  }
}

// ---- kernel 2: sequential scan over chunks ------------------------------------------

template <typename In, int DK, int C>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(Problem p, const unsigned char* __restrict__ ws,
                                                              ChunkLayout L, int want_out) {
  constexpr bool F16 = std::is_same<In, uint16_t>::value;
  using Op = std::conditional_t<F16, _Float16, float>;
  constexpr int ES = sizeof(Op);
  constexpr ChunkLayout LC = make_chunk_layout(ES, DK, 128, C);
  constexpr int IMG = int(LC.image_bytes);
  constexpr int UNITS = (IMG + 15) / 16;
  constexpr int LDK = DK + 4, LDC = C + 4;
  constexpr int NT = C / 16;
  constexpr int KS = DK / 16;
  constexpr int KP = (KS + 1) / 2;
  constexpr int NP = (NT + 1) / 2;
  // bf16 outputs are staged in LDS for 16-byte stores; fp32 outputs go out directly
  constexpr int OSR = F16 ? C : 1;
  static_assert(2 * UNITS * 16 + 2 * OSR * 64 * sizeof(In) <= 160 * 1024, "LDS budget");
  __shared__ uint4 img[2][UNITS];
  __shared__ In ostage[2][OSR][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int dv = int(p.dv);
  const int cblocks = (dv + 63) / 64;
  // Workgroups are dealt round-robin to the 8 XCDs; the column blocks of one
  // (batch, head) read the same chunk records, so they are placed 8 apart (same
  // XCD, shared L2) whenever the grid allows.
  int64_t bh;
  int cb;
  {
    const int64_t x = blockIdx.x, nbh = p.B * p.H;
    const int64_t full = (nbh / 8) * 8 * cblocks;  // part of the grid with whole groups of 8
    if (cblocks > 1 && x < full) {
      const int64_t grp = x / (8 * cblocks), rem = x % (8 * cblocks);
      bh = grp * 8 + rem % 8;
      cb = int(rem / 8);
    } else {
      bh = x / cblocks;
      cb = int(x % cblocks);
    }
  }
  const int cbase = cb * 64;
  const int col0 = cbase + 16 * wave;
  const bool active = col0 < dv;
  const int col = col0 + li;
  const int R = p.rows_out, RT = R / 16;
  const int64_t NC = p.nchunks;
  const int64_t b = bh / p.H, h = bh % p.H;
  In* o = static_cast<In*>(p.o);
  const int units = int((want_out ? L.image_bytes : L.state_bytes) + 15) / 16;

  auto rec_of = [&](int64_t n) -> const unsigned char* {
    return ws + (size_t(bh) * size_t(NC) + size_t(n)) * L.bytes;
  };

  // The record image goes global -> LDS directly (no registers): each wave copies
  // 1 KB blocks, lane l moving 16 bytes to block base + 16 l.
  constexpr int WBLK = (UNITS + 64 * kWaves - 1) / (64 * kWaves);  // blocks per wave
  using UtRaw = std::conditional_t<F16, uint2, uint4>;
  UtRaw ut_next[NT];
  auto issue_loads = [&](int64_t n, int buf) __attribute__((always_inline)) {
    const uint4* src = reinterpret_cast<const uint4*>(rec_of(n));
#pragma unroll
    for (int k = 0; k < WBLK; ++k) {
      const int u0 = (k * kWaves + wave) * 64;
      if (u0 < units) {
        const int x = u0 + lane;
        if (x < units)
          __builtin_amdgcn_global_load_lds(
              static_cast<const void*>(src + x),
              reinterpret_cast<__attribute__((address_space(3))) void*>(
                  reinterpret_cast<uintptr_t>(&img[buf][u0]) & 0xffffffffu),
              16, 0, 0);
      }
    }
    if (active) {
      const Op* ut = reinterpret_cast<const Op*>(rec_of(n) + L.off_UT) + size_t(col) * C + 4 * lg;
#pragma unroll
      for (int m = 0; m < NT; ++m) ut_next[m] = *reinterpret_cast<const UtRaw*>(ut + 16 * m);
    }
  };
  // wait for this wave's copies (all outstanding vector memory operations)
  auto land_loads = []() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0); };
  // coalesced copy of a staged output block (rows of chunk n) to o
  const int ounits_row = (min(64, dv - cbase) * int(sizeof(In))) / 16;
  auto flush_out = [&](int buf, int64_t n) __attribute__((always_inline)) {
    if constexpr (!F16) return;
    for (int x = tid; x < R * ounits_row; x += kThreads) {
      const int ro = x / ounits_row, cu = x % ounits_row;
      const int64_t t = n * R + ro;
      if (t < p.T) {
        const int c = cu * 16 / int(sizeof(In));
        const uint4 val = *reinterpret_cast<const uint4*>(&ostage[buf][ro][c]);
        *reinterpret_cast<uint4*>(o + ((b * p.T + t) * p.H + h) * dv + cbase + c) = val;
      }
    }
  };

  // state slice: S[ct][e] = S[16 ct + 4 lg + e][col]
  float S[KS][4];
  const size_t sbase = size_t(bh) * DK * size_t(dv);
#pragma unroll
  for (int ct = 0; ct < KS; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[ct][e] = (active && p.s0) ? p.s0[sbase + size_t(16 * ct + 4 * lg + e) * dv + col] : 0.0f;

  issue_loads(0, 0);
  land_loads();
  UtRaw ut_cur[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) ut_cur[m] = ut_next[m];
  __syncthreads();

  for (int64_t n = 0; n < NC; ++n) {
    const int buf = int(n & 1);
    if (n + 1 < NC) issue_loads(n + 1, buf ^ 1);
    if (want_out && n > 0) flush_out(buf ^ 1, n - 1);
    const unsigned char* base = reinterpret_cast<const unsigned char*>(&img[buf][0]);
    const Op* Wl = reinterpret_cast<const Op*>(base + LC.off_W);
    const Op* ATl = reinterpret_cast<const Op*>(base + LC.off_AT);
    const float* gaml = reinterpret_cast<const float*>(base + LC.off_gamma);
    const float* winvl = reinterpret_cast<const float*>(base + LC.off_winv);
    const Op* Ql = reinterpret_cast<const Op*>(base + LC.off_Q);
    const Op* Pl = reinterpret_cast<const Op*>(base + LC.off_P);
    const float* qinvl = reinterpret_cast<const float*>(base + LC.off_qinv);
    if (active) {
      const float winv = winvl[0];
      float ut[NT][4];
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        if constexpr (F16) {
          H8 t8;
          t8.u[0] = ut_cur[m];
          t8.u[1] = make_uint2(0u, 0u);
#pragma unroll
          for (int e = 0; e < 4; ++e) ut[m][e] = (float)t8.h[e] * winv;
        } else {
          ut[m][0] = __uint_as_float(ut_cur[m].x);
          ut[m][1] = __uint_as_float(ut_cur[m].y);
          ut[m][2] = __uint_as_float(ut_cur[m].z);
          ut[m][3] = __uint_as_float(ut_cur[m].w);
        }
      }

      // state as the B operand (power-of-two scaled fp16 when F16)
      float iS = 1.0f;
      half8 sh[KP];
      if constexpr (F16) {
        float cm = 0.0f;
#pragma unroll
        for (int ct = 0; ct < KS; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) cm = fmaxf(cm, fabsf(S[ct][e]));
        cm = max_over_groups(cm);
        const float sS = pow2_scale_for(cm, kStateScaleExp);
        iS = 1.0f / sS;
#pragma unroll
        for (int u = 0; u < KP; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sh[u][e] = (_Float16)(S[2 * u][e] * sS);
            sh[u][4 + e] = (2 * u + 1 < KS) ? (_Float16)(S[2 * u + 1][e] * sS) : (_Float16)0.0f;
          }
      }
      auto times_state = [&](const Op* arow) __attribute__((always_inline)) -> float4v {
        float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (F16) {
#pragma unroll
          for (int u = 0; u < KP; ++u) {
            const bool two = 2 * u + 1 < KS;
            const H8 a8 = pair4(arow + 32 * u + 4 * lg, two ? arow + 32 * u + 16 + 4 * lg : nullptr);
            acc = mma_pair_f16(a8.h, sh[u], acc);
          }
        } else {
#pragma unroll
          for (int t = 0; t < KS; ++t) {
            float a4[4];
            quad(arow + 16 * t + 4 * lg, a4);
            acc = mma_slice_f32(a4, S[t], acc);
          }
        }
        return acc;
      };

      // U = U~ - W S
      float Um[NT][4];
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const float4v acc = times_state(Wl + (16 * m + li) * LDK);
#pragma unroll
        for (int e = 0; e < 4; ++e) Um[m][e] = ut[m][e] - acc[e] * iS;
      }
      float iU = 1.0f;
      half8 uh[NP];
      if constexpr (F16) {
        float cm = 0.0f;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) cm = fmaxf(cm, fabsf(Um[m][e]));
        cm = max_over_groups(cm);
        const float sU = pow2_scale_for(cm, kStateScaleExp);
        iU = 1.0f / sU;
#pragma unroll
        for (int u = 0; u < NP; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uh[u][e] = (_Float16)(Um[2 * u][e] * sU);
            uh[u][4 + e] = (2 * u + 1 < NT) ? (_Float16)(Um[2 * u + 1][e] * sU) : (_Float16)0.0f;
          }
      }
      auto times_u = [&](const Op* arow) __attribute__((always_inline)) -> float4v {
        float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (F16) {
#pragma unroll
          for (int u = 0; u < NP; ++u) {
            const bool two = 2 * u + 1 < NT;
            const H8 a8 = pair4(arow + 32 * u + 4 * lg, two ? arow + 32 * u + 16 + 4 * lg : nullptr);
            acc = mma_pair_f16(a8.h, uh[u], acc);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            float a4[4];
            quad(arow + 16 * t + 4 * lg, a4);
            acc = mma_slice_f32(a4, Um[t], acc);
          }
        }
        return acc;
      };

      // O = (Q+ S + P U) / q-scale   (chunk-start state), staged in LDS
      if (want_out) {
#pragma unroll
        for (int mo = 0; mo < NT; ++mo) {
          if (mo < RT) {
            const float4v a1 = times_state(Ql + (16 * mo + li) * LDK);
            const float4v a2 = times_u(Pl + (16 * mo + li) * LDC);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int ro = 16 * mo + 4 * lg + e;
              const float ov = (a1[e] * iS + a2[e] * iU) * qinvl[ro];
              if constexpr (F16) {
                ostage[buf][ro][16 * wave + li] = f32_to_bf16(ov);
              } else {
                const int64_t t = n * R + ro;
                if (t < p.T) o[((b * p.T + t) * p.H + h) * dv + col] = ov;
              }
            }
          }
        }
      }
      // S <- Diag(gamma) S + A^^T U
#pragma unroll
      for (int ct = 0; ct < KS; ++ct) {
        const float4v acc = times_u(ATl + (16 * ct + li) * LDC);
#pragma unroll
        for (int e = 0; e < 4; ++e) S[ct][e] = gaml[16 * ct + 4 * lg + e] * S[ct][e] + acc[e] * iU;
      }
    }
    if (n + 1 < NC) {
      land_loads();
#pragma unroll
      for (int m = 0; m < NT; ++m) ut_cur[m] = ut_next[m];
    }
    __syncthreads();
  }
  if (want_out) flush_out(int((NC - 1) & 1), NC - 1);

  if (active && p.s_final) {
#pragma unroll
    for (int ct = 0; ct < KS; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) p.s_final[sbase + size_t(16 * ct + 4 * lg + e) * dv + col] = S[ct][e];
  }
}

// ---- launch ----------------------------------------------------------------------------

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// which = 1: prepare only, 2: scan only, 3: both
template <typename In, int DK, int C, bool DPV>
int launch_chunk_t(const Problem& p, void* ws, bool want_out, hipStream_t s, int which) {
  const ChunkLayout L = chunk_layout(p);
  unsigned char* w = static_cast<unsigned char*>(ws);
  if (which & 1) {
    constexpr bool F16 = std::is_same<In, uint16_t>::value;
    const int64_t items = p.nchunks * p.B * p.H;
    const int per_cu = sizeof(PrepLds<F16, DK, C, DPV>) <= 80 * 1024 ? 2 : 1;
    const int64_t grid = std::min<int64_t>(items, int64_t(device_cus()) * per_cu);
    chunk_prep_kernel<In, DK, C, DPV><<<dim3(unsigned(grid)), kThreads, 0, s>>>(p, w, L, want_out ? 1 : 0);
  }
  if (which & 2) {
    const unsigned cblocks = unsigned((p.dv + 63) / 64);
    const dim3 g2(unsigned(p.B * p.H) * cblocks);
    chunk_scan_kernel<In, DK, C><<<g2, kThreads, 0, s>>>(p, w, L, want_out ? 1 : 0);
  }
  return int(hipGetLastError());
}

template <typename In, int DK, int C>
int launch_chunk_dp(const Problem& p, void* ws, bool want_out, hipStream_t s, int which) {
  if (p.n_h > 1) return launch_chunk_t<In, DK, C, true>(p, ws, want_out, s, which);
  return launch_chunk_t<In, DK, C, false>(p, ws, want_out, s, which);
}

template <typename In, int DK>
int launch_chunk_dk(const Problem& p, void* ws, bool want_out, hipStream_t s, int which) {
  switch (p.chunk) {
    case 16: return launch_chunk_dp<In, DK, 16>(p, ws, want_out, s, which);
    case 32: return launch_chunk_dp<In, DK, 32>(p, ws, want_out, s, which);
    case 64:
      if constexpr (std::is_same<In, float>::value && DK == 128) return int(hipErrorInvalidValue);
      else return launch_chunk_dp<In, DK, 64>(p, ws, want_out, s, which);
    default: return int(hipErrorInvalidValue);
  }
}

template <typename In>
int launch_chunk_in(const Problem& p, void* ws, bool want_out, hipStream_t s, int which) {
  switch (p.dk) {
    case 16: return launch_chunk_dk<In, 16>(p, ws, want_out, s, which);
    case 32: return launch_chunk_dk<In, 32>(p, ws, want_out, s, which);
    case 64: return launch_chunk_dk<In, 64>(p, ws, want_out, s, which);
    case 128: return launch_chunk_dk<In, 128>(p, ws, want_out, s, which);
    default: return int(hipErrorInvalidValue);
  }
}

int dispatch(const Problem& p, void* ws, bool want_out, void* stream, int which) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.dtype == GDN_DTYPE_BF16 ? launch_chunk_in<uint16_t>(p, ws, want_out, s, which)
                                   : launch_chunk_in<float>(p, ws, want_out, s, which);
}

}  // namespace

int launch_chunk(const Problem& p, void* ws, bool want_out, void* stream) {
  return dispatch(p, ws, want_out, stream, 3);
}
int launch_prep(const Problem& p, void* ws, bool want_out, void* stream) {
  return dispatch(p, ws, want_out, stream, 1);
}
int launch_scan(const Problem& p, void* ws, bool want_out, void* stream) {
  return dispatch(p, ws, want_out, stream, 2);
}

}  // namespace gdn
