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
// Kernel 1 (chunk_prep): one workgroup per (chunk, batch*head); everything that
// does not depend on the carried state. Writes a per-chunk record
// {W, U~^T, A^^T, Q+, P, gamma = e^{G_C}, scales} to the workspace.
// Kernel 2 (chunk_scan): one workgroup per (batch*head, 64 value columns); each
// wave owns 16 value columns and carries its 128x16 (dk x 16) fp32 state slice in
// MFMA accumulator registers across all chunks; the chunk records are staged
// into LDS one chunk ahead (double buffer).
//
// Precision (bf16 inputs): the Gram products run as bf16 hi/lo splits (three
// bf16 MFMAs, about 16 mantissa bits, full fp32 range); every other product runs
// on fp16 MFMA with fp32 accumulation. Quantities whose scale follows the
// caller's values (v, q, the state, U) are multiplied by exact powers of two
// before the fp16 conversion and divided back after the product, so fp16's
// range never clips them. fp32 inputs use fp32 MFMA throughout.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
// The state and U enter fp16 MFMAs with their per-column maximum scaled into
// [2^12, 2^13): far below fp16's 65504 and well above its subnormal range.
constexpr int kStateScaleExp = 12;

// ---- per-variant construction of (a, b, w, log alpha, q) -----------------------

template <typename In>
struct RowSrc {
  int variant, n_h;
  int64_t T, H, dk, dv, steps, b, h, vs0, t0;
  const In *q, *k, *v, *al, *be, *bev, *jv, *et;

  __device__ __forceinline__ void init(const Problem& p, int64_t bh, int64_t n, int C) {
    variant = p.variant;
    n_h = p.n_h;
    T = p.T;
    H = p.H;
    dk = p.dk;
    dv = p.dv;
    steps = p.steps;
    b = bh / p.H;
    h = bh % p.H;
    vs0 = n * C;
    t0 = vs0 / p.n_h;
    q = static_cast<const In*>(p.q);
    k = static_cast<const In*>(p.k);
    v = static_cast<const In*>(p.v);
    al = static_cast<const In*>(p.alpha);
    be = static_cast<const In*>(p.beta);
    bev = static_cast<const In*>(p.beta_v);
    jv = static_cast<const In*>(p.j);
    et = static_cast<const In*>(p.eta);
  }
  __device__ __forceinline__ static float ld(const In* ptr) { return IO<In>::ld(ptr); }
  __device__ __forceinline__ int64_t th(int64_t t) const { return (b * T + t) * H + h; }

  // log alpha of step r (within the chunk) for key channel c; 0 past the end
  __device__ float logdecay(int r, int c) const {
    const int64_t vs = vs0 + r;
    if (vs >= steps) return 0.0f;
    if (variant == GDN_VARIANT_DELTAPRODUCT) {
      const int64_t t = vs / n_h;
      return (vs % n_h == 0) ? logf(ld(al + th(t))) : 0.0f;
    }
    const int64_t x = th(vs);
    if (variant == GDN_VARIANT_GDN) return logf(ld(al + x));
    return logf(ld(al + x * dk + c));
  }

  // write key a and erase key b of step r, key channel c
  __device__ void keys(int r, int c, float& a, float& bb) const {
    const int64_t vs = vs0 + r;
    if (vs >= steps) {
      a = 0.0f;
      bb = 0.0f;
      return;
    }
    if (variant == GDN_VARIANT_DELTAPRODUCT) {
      const int64_t ti = th(vs / n_h) * n_h + vs % n_h;
      a = ld(k + ti * dk + c);
      bb = ld(be + ti) * a;
      return;
    }
    const int64_t x = th(vs);
    if (variant == GDN_VARIANT_ASYM) {
      a = ld(k + x * dk + c);
      bb = ld(et + x) * ld(jv + x * dk + c);
      return;
    }
    const float sb = variant == GDN_VARIANT_FG2 ? sqrtf(ld(be + x * dk + c)) : sqrtf(ld(be + x));
    a = sb * ld(k + x * dk + c);
    bb = a;
  }

  // written value w of step r, value channel c
  __device__ float value(int r, int c) const {
    const int64_t vs = vs0 + r;
    if (vs >= steps) return 0.0f;
    if (variant == GDN_VARIANT_DELTAPRODUCT) {
      const int64_t ti = th(vs / n_h) * n_h + vs % n_h;
      return ld(be + ti) * ld(v + ti * dv + c);
    }
    const int64_t x = th(vs);
    const float vv = ld(v + x * dv + c);
    if (variant == GDN_VARIANT_ASYM) return ld(et + x) * vv;
    if (variant == GDN_VARIANT_FG2)
      return sqrtf(bev ? ld(bev + x * dv + c) : ld(be + x * dk + c)) * vv;
    return sqrtf(ld(be + x)) * vv;
  }

  // query of output row ro (token t0 + ro), key channel c; 0 past the end
  __device__ float query(int ro, int c) const {
    const int64_t t = t0 + ro;
    if (t >= T) return 0.0f;
    return ld(q + th(t) * dk + c);
  }
};

// ---- LDS quad / pair loads -------------------------------------------------------

// Four consecutive operand elements as fp32.
__device__ __forceinline__ void quad(const float* p, float out[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  out[0] = x.x;
  out[1] = x.y;
  out[2] = x.z;
  out[3] = x.w;
}

union H8 {
  half8 h;
  bhalf8 b;
  uint2 u[2];
};

// Eight fp16 operand values: slice s0 at p0 (4 elements), slice s1 at p1 or zeros.
__device__ __forceinline__ half8 pair16(const _Float16* p0, const _Float16* p1) {
  H8 r;
  r.u[0] = *reinterpret_cast<const uint2*>(p0);
  r.u[1] = p1 ? *reinterpret_cast<const uint2*>(p1) : make_uint2(0u, 0u);
  return r.h;
}
__device__ __forceinline__ bhalf8 pairb16(const __bf16* p0, const __bf16* p1) {
  H8 r;
  r.u[0] = *reinterpret_cast<const uint2*>(p0);
  r.u[1] = p1 ? *reinterpret_cast<const uint2*>(p1) : make_uint2(0u, 0u);
  return r.b;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// ---- kernel 1: chunk-local preparation ------------------------------------------------

template <bool F16, int DK, int C>
struct PrepSmem {
  using Op = std::conditional_t<F16, _Float16, float>;
  using Am = std::conditional_t<F16, __bf16, float>;
  static constexpr int LDK = DK + 4, LDC = C + 4;
  union {
    float G[C][DK];   // cumulative log decay (phases A-B)
    float tf[C][LDC]; // T = (I + M)^{-1} in fp32 (phases D-E)
  } u1;
  union {
    Op at[DK][LDC];   // A^ transposed, staged for a coalesced copy (phase B)
    float mf[C][LDC]; // strictly lower Gram M (phases C-D)
  } u2;
  float tot[kThreads];        // cumsum segment totals
  Am amh[C][LDK];             // A- (mid reference); hi part when F16
  Am aml[F16 ? C : 1][LDK];   // lo part (F16)
  Op bt[DK][LDC];             // B+ (chunk-start reference), transposed
  Op wvt[128][LDC];           // written values, transposed, scaled by ws
  Op top[F16 ? C : 1][LDC];   // T in fp16 (F16)
  float qs[C];                // per output row power-of-two q scale
  float red[kThreads / 64];
};

template <typename In, int DK, int C>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(Problem p, unsigned char* __restrict__ ws,
                                                              ChunkLayout L, int want_out) {
  constexpr bool F16 = std::is_same<In, uint16_t>::value;
  using Sm = PrepSmem<F16, DK, C>;
  using Op = typename Sm::Op;
  constexpr int NT = C / 16;          // 16-step tiles in a chunk
  constexpr int KS = DK / 16;         // 16-channel slices of a key row
  constexpr int KP = (KS + 1) / 2;    // slice pairs (fp16 / bf16 MFMA take two)
  constexpr int SEG = kThreads / DK;  // cumsum segments per channel
  constexpr int RPS = C / SEG;
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  static_assert(C % SEG == 0, "segments");
  __shared__ Sm sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t n = int64_t(blockIdx.x) % p.nchunks, bh = int64_t(blockIdx.x) / p.nchunks;
  const int R = p.rows_out, n_h = p.n_h;
  const int RT = R / 16;
  const int dv = int(p.dv);
  RowSrc<In> src;
  src.init(p, bh, n, C);

  unsigned char* rec = ws + (size_t(bh) * size_t(p.nchunks) + size_t(n)) * L.bytes;
  Op* W_g = reinterpret_cast<Op*>(rec + L.off_W);
  Op* UT_g = reinterpret_cast<Op*>(rec + L.off_UT);
  Op* AT_g = reinterpret_cast<Op*>(rec + L.off_AT);
  Op* Q_g = reinterpret_cast<Op*>(rec + L.off_Q);
  Op* P_g = reinterpret_cast<Op*>(rec + L.off_P);
  float* gam_g = reinterpret_cast<float*>(rec + L.off_gamma);
  float* qinv_g = reinterpret_cast<float*>(rec + L.off_qinv);
  float* winv_g = reinterpret_cast<float*>(rec + L.off_winv);

  // ---- A: cumulative log decay and the power-of-two scales ----
  {
    const int seg = tid / DK, c = tid % DK;
    float acc = 0.0f;
    for (int i = 0; i < RPS; ++i) {
      const int r = seg * RPS + i;
      acc += src.logdecay(r, c);
      sm.u1.G[r][c] = acc;
    }
    sm.tot[seg * DK + c] = acc;
  }
  float wmax = 0.0f;
  if (F16) {
    for (int u = tid; u < C * dv; u += kThreads) wmax = fmaxf(wmax, fabsf(src.value(u / dv, u % dv)));
    wmax = wave_max(wmax);
    if (lane == 0) sm.red[wave] = wmax;
    if (want_out) {
      for (int ro = wave; ro < R; ro += kThreads / 64) {
        float m = 0.0f;
        for (int c = lane; c < DK; c += 64) m = fmaxf(m, fabsf(src.query(ro, c)));
        m = wave_max(m);
        if (lane == 0) sm.qs[ro] = pow2_scale_for(m);
      }
    }
  } else {
    for (int ro = tid; ro < C; ro += kThreads) sm.qs[ro] = 1.0f;
  }
  __syncthreads();
  {
    const int seg = tid / DK, c = tid % DK;
    float off = 0.0f;
    for (int s = 0; s < seg; ++s) off += sm.tot[s * DK + c];
    if (seg > 0)
      for (int i = 0; i < RPS; ++i) sm.u1.G[seg * RPS + i][c] += off;
  }
  float wsc = 1.0f;
  if (F16) {
    float m = sm.red[0];
#pragma unroll
    for (int w2 = 1; w2 < kThreads / 64; ++w2) m = fmaxf(m, sm.red[w2]);
    wsc = pow2_scale_for(m);
  }
  __syncthreads();

  // ---- B1: decayed operands ----
  const float* Gmid = sm.u1.G[C / 2 - 1];
  const float* Gend = sm.u1.G[C - 1];
  for (int u = tid; u < C * DK; u += kThreads) {
    const int r = u / DK, c = u % DK;
    float a, bb;
    src.keys(r, c, a, bb);
    const float Gr = sm.u1.G[r][c];
    const float am = a * expf(Gmid[c] - Gr);
    if constexpr (F16) {
      const __bf16 hi = (__bf16)am;
      sm.amh[r][c] = hi;
      sm.aml[r][c] = (__bf16)(am - (float)hi);
    } else {
      sm.amh[r][c] = am;
    }
    sm.bt[c][r] = (Op)(bb * expf(Gr));
    sm.u2.at[c][r] = (Op)(a * expf(Gend[c] - Gr));
  }
  for (int u = tid; u < C * dv; u += kThreads) {
    const int r = u / dv, c = u % dv;
    sm.wvt[c][r] = (Op)(src.value(r, c) * wsc);
  }
  if (want_out) {
    for (int u = tid; u < R * DK; u += kThreads) {
      const int ro = u / DK, c = u % DK;
      const int tau = ro * n_h + n_h - 1;
      Q_g[u] = (Op)(src.query(ro, c) * expf(sm.u1.G[tau][c]) * sm.qs[ro]);
    }
    for (int ro = tid; ro < R; ro += kThreads) qinv_g[ro] = 1.0f / sm.qs[ro];
  }
  for (int c = tid; c < DK; c += kThreads) gam_g[c] = expf(Gend[c]);
  if (tid == 0) winv_g[0] = 1.0f / wsc;
  __syncthreads();

  // ---- B2: per-wave Gram fragments (own tile row), A^ copy-out ----
  for (int u = tid; u < DK * C; u += kThreads) AT_g[u] = sm.u2.at[u / C][u % C];
  // Row fragments in the slice layout: lane (li, lg) holds row 16*wave + li at
  // channels 16 t + 4 lg + e.
  float bm[KS][4], qm[KS][4];
  if (wave < NT) {
    const int r = 16 * wave + li;
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * t + 4 * lg + e;
        float a, bb;
        src.keys(r, c, a, bb);
        bm[t][e] = bb * expf(sm.u1.G[r][c] - Gmid[c]);
      }
  }
  if (want_out && wave < RT) {
    const int ro = 16 * wave + li;
    const int tau = ro * n_h + n_h - 1;
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * t + 4 * lg + e;
        qm[t][e] = src.query(ro, c) * expf(sm.u1.G[tau][c] - Gmid[c]);
      }
  }
  __syncthreads();

  // ---- C: Gram tiles M^T = A- B+^T (masked strictly lower) and P^T = A- Q+^T ----
  auto gram_tile = [&](int J, const float (&x)[KS][4]) -> float4v {
    float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (F16) {
#pragma unroll
      for (int u = 0; u < KP; ++u) {
        const bool two = 2 * u + 1 < KS;
        const __bf16* rh = &sm.amh[16 * J + li][0];
        const __bf16* rl = &sm.aml[16 * J + li][0];
        const bhalf8 ah = pairb16(rh + 32 * u + 4 * lg, two ? rh + 32 * u + 16 + 4 * lg : nullptr);
        const bhalf8 al = pairb16(rl + 32 * u + 4 * lg, two ? rl + 32 * u + 16 + 4 * lg : nullptr);
        bhalf8 bh, bl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = x[2 * u][e];
          const float x1 = two ? x[2 * u + 1][e] : 0.0f;
          const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
          bh[e] = h0;
          bh[4 + e] = h1;
          bl[e] = (__bf16)(x0 - (float)h0);
          bl[4 + e] = (__bf16)(x1 - (float)h1);
        }
        acc = mma_pair_bf16(ah, bh, acc);
        acc = mma_pair_bf16(ah, bl, acc);
        acc = mma_pair_bf16(al, bh, acc);
      }
    } else {
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        float a4[4];
        quad(&sm.amh[16 * J + li][16 * t + 4 * lg], a4);
        acc = mma_slice_f32(a4, x[t], acc);
      }
    }
    return acc;
  };
  if (wave < NT) {
    const int I = wave;
    const int r = 16 * I + li;
    for (int J = 0; J <= I; ++J) {
      const float4v acc = gram_tile(J, bm);
      float4 m4;
      const int s0 = 16 * J + 4 * lg;
      m4.x = (s0 + 0 < r) ? acc[0] : 0.0f;
      m4.y = (s0 + 1 < r) ? acc[1] : 0.0f;
      m4.z = (s0 + 2 < r) ? acc[2] : 0.0f;
      m4.w = (s0 + 3 < r) ? acc[3] : 0.0f;
      *reinterpret_cast<float4*>(&sm.u2.mf[r][s0]) = m4;
    }
  }
  if (want_out && wave < RT) {
    const int Io = wave;
    const int ro = 16 * Io + li;
    const int tau = ro * n_h + n_h - 1;
    const int jmax = min(NT - 1, ((16 * Io + 15) * n_h + n_h - 1) / 16);
    const float qsc = sm.qs[ro];
    for (int J = 0; J < NT; ++J) {
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if (J <= jmax) acc = gram_tile(J, qm);
      const int s0 = 16 * J + 4 * lg;
      Op* dst = P_g + size_t(ro) * C + s0;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = (Op)((s0 + e <= tau) ? acc[e] * qsc : 0.0f);
    }
  }
  __syncthreads();

  // ---- D: T = (I + M)^{-1}; diagonal 16x16 blocks by forward substitution ----
  if (wave == 0) {
    const int bI = lane >> 4, c = lane & 15;
    if (bI < NT) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == c) ? 1.0f : 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < r; ++s2) s -= sm.u2.mf[16 * bI + r][16 * bI + s2] * x[s2];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.u1.tf[16 * bI + r][16 * bI + c] = x[r];
    }
  }
  // off-diagonal blocks: T_IJ = -T_II sum_{K=J}^{I-1} M_IK T_KJ, one level per I
  for (int I = 1; I < NT; ++I) {
    __syncthreads();
    if (wave < I) {
      const int J = wave;
      float4v x = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int K = J; K < I; ++K) {
        float a4[4], b4[4];
        quad(&sm.u2.mf[16 * I + li][16 * K + 4 * lg], a4);
#pragma unroll
        for (int e = 0; e < 4; ++e) b4[e] = sm.u1.tf[16 * K + 4 * lg + e][16 * J + li];
        x = mma_slice_f32(a4, b4, x);
      }
      float a4[4], xb[4] = {x[0], x[1], x[2], x[3]};
      quad(&sm.u1.tf[16 * I + li][16 * I + 4 * lg], a4);
      const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const float4v y = mma_slice_f32(a4, xb, zero);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u1.tf[16 * I + 4 * lg + e][16 * J + li] = -y[e];
    }
  }
  __syncthreads();
  // operand copy of T with its upper triangle cleared
  for (int u = tid; u < C * C; u += kThreads) {
    const int r = u / C, s = u % C;
    if constexpr (F16) {
      sm.top[r][s] = (s <= r) ? (_Float16)sm.u1.tf[r][s] : (_Float16)0.0f;
    } else {
      if (s > r) sm.u1.tf[r][s] = 0.0f;
    }
  }
  __syncthreads();

  // ---- E: W^T = B+^T T^T (stored as W rows) and U~ = T Wv (stored transposed) ----
  auto trow = [&](int r) -> const Op* {
    if constexpr (F16) return &sm.top[r][0];
    else return &sm.u1.tf[r][0];
  };
  // product of a row-fragment source `arow` (A operand, 16 rows) with rows of T
  // (B operand), summed over the step index s <= 16 I + 15.
  constexpr int NWT = KS * NT;
  for (int x = wave; x < NWT; x += kThreads / 64) {
    const int ct = x / NT, I = x % NT;
    float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const Op* arow = &sm.bt[16 * ct + li][0];
    const Op* brow = trow(16 * I + li);
    if constexpr (F16) {
      for (int u = 0; 2 * u <= I; ++u) {
        const bool two = 2 * u + 1 < NT;
        const half8 a8 = pair16(arow + 32 * u + 4 * lg, two ? arow + 32 * u + 16 + 4 * lg : nullptr);
        const half8 b8 = pair16(brow + 32 * u + 4 * lg, two ? brow + 32 * u + 16 + 4 * lg : nullptr);
        acc = mma_pair_f16(a8, b8, acc);
      }
    } else {
      for (int t = 0; t <= I; ++t) {
        float a4[4], b4[4];
        quad(arow + 16 * t + 4 * lg, a4);
        quad(brow + 16 * t + 4 * lg, b4);
        acc = mma_slice_f32(a4, b4, acc);
      }
    }
    Op* dst = W_g + size_t(16 * I + li) * DK + 16 * ct + 4 * lg;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = (Op)acc[e];
  }
  const int VT = dv / 16;
  for (int x = wave; x < NT * VT; x += kThreads / 64) {
    const int I = x / VT, ct = x % VT;
    float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const Op* arow = trow(16 * I + li);
    const Op* brow = &sm.wvt[16 * ct + li][0];
    if constexpr (F16) {
      for (int u = 0; 2 * u <= I; ++u) {
        const bool two = 2 * u + 1 < NT;
        const half8 a8 = pair16(arow + 32 * u + 4 * lg, two ? arow + 32 * u + 16 + 4 * lg : nullptr);
        const half8 b8 = pair16(brow + 32 * u + 4 * lg, two ? brow + 32 * u + 16 + 4 * lg : nullptr);
        acc = mma_pair_f16(a8, b8, acc);
      }
    } else {
      for (int t = 0; t <= I; ++t) {
        float a4[4], b4[4];
        quad(arow + 16 * t + 4 * lg, a4);
        quad(brow + 16 * t + 4 * lg, b4);
        acc = mma_slice_f32(a4, b4, acc);
      }
    }
    Op* dst = UT_g + size_t(16 * ct + li) * C + 16 * I + 4 * lg;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = (Op)acc[e];
  }
}

// ---- kernel 2: sequential scan over chunks ------------------------------------------

template <bool F16, int DK, int C>
struct ScanSmem {
  using Op = std::conditional_t<F16, _Float16, float>;
  static constexpr int LDK = DK + 4, LDC = C + 4;
  Op w[2][C][LDK];
  Op at[2][DK][LDC];
  Op q[2][C][LDK];
  Op pm[2][C][LDC];
  float gam[2][DK];
  float qinv[2][C];
  float winv[2][4];
};

// 16-byte units of one chunk record, by region.
template <int ES, int DK, int C>
struct Units {
  static constexpr int W = C * DK * ES / 16;
  static constexpr int AT = DK * C * ES / 16;
  static constexpr int Q = C * DK * ES / 16;   // upper bound (R <= C)
  static constexpr int P = C * C * ES / 16;
  static constexpr int GAM = DK / 4;
  static constexpr int QI = C / 4;
  static constexpr int WI = 1;
  static constexpr int TOTAL = W + AT + Q + P + GAM + QI + WI;
  static constexpr int PER_THREAD = (TOTAL + kThreads - 1) / kThreads;
};

template <typename In, int DK, int C>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(Problem p, const unsigned char* __restrict__ ws,
                                                              ChunkLayout L, int want_out) {
  constexpr bool F16 = std::is_same<In, uint16_t>::value;
  using Sm = ScanSmem<F16, DK, C>;
  using Op = typename Sm::Op;
  constexpr int ES = sizeof(Op);
  constexpr int NT = C / 16;
  constexpr int KS = DK / 16;
  constexpr int KP = (KS + 1) / 2;
  constexpr int NP = (NT + 1) / 2;
  using U = Units<ES, DK, C>;
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  __shared__ Sm sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int dv = int(p.dv);
  const int cblocks = (dv + 63) / 64;
  const int64_t bh = blockIdx.x / cblocks;
  const int col0 = (blockIdx.x % cblocks) * 64 + 16 * wave;
  const bool active = col0 < dv;
  const int col = col0 + li;
  const int R = p.rows_out, RT = R / 16, n_h = p.n_h;
  const int64_t NC = p.nchunks;
  const int64_t b = bh / p.H, h = bh % p.H;
  In* o = static_cast<In*>(p.o);

  // unit counts of this call (Q / P / qinv only when outputs are produced)
  const int nQ = want_out ? R * DK * ES / 16 : 0;
  const int nP = want_out ? R * C * ES / 16 : 0;
  const int nQI = want_out ? R / 4 : 0;
  const int b1 = U::W, b2 = b1 + U::AT, b3 = b2 + nQ, b4 = b3 + nP, b5 = b4 + U::GAM, b6 = b5 + nQI,
            b7 = b6 + U::WI;

  auto rec_of = [&](int64_t n) -> const unsigned char* {
    return ws + (size_t(bh) * size_t(NC) + size_t(n)) * L.bytes;
  };
  // global source of unit x
  auto unit_src = [&](const unsigned char* rec, int x) -> const uint4* {
    size_t off;
    if (x < b1) off = L.off_W + size_t(x) * 16;
    else if (x < b2) off = L.off_AT + size_t(x - b1) * 16;
    else if (x < b3) off = L.off_Q + size_t(x - b2) * 16;
    else if (x < b4) off = L.off_P + size_t(x - b3) * 16;
    else if (x < b5) off = L.off_gamma + size_t(x - b4) * 16;
    else if (x < b6) off = L.off_qinv + size_t(x - b5) * 16;
    else off = L.off_winv;
    return reinterpret_cast<const uint4*>(rec + off);
  };
  // LDS destination of unit x in buffer `buf` (rows are padded, so 8-byte halves)
  auto unit_dst = [&](int buf, int x) -> unsigned char* {
    auto rowpad = [](unsigned char* base, int xr, int row_units, int ld_bytes) {
      return base + size_t(xr / row_units) * ld_bytes + size_t(xr % row_units) * 16;
    };
    if (x < b1) return rowpad(reinterpret_cast<unsigned char*>(&sm.w[buf][0][0]), x, DK * ES / 16, Sm::LDK * ES);
    if (x < b2) return rowpad(reinterpret_cast<unsigned char*>(&sm.at[buf][0][0]), x - b1, C * ES / 16, Sm::LDC * ES);
    if (x < b3) return rowpad(reinterpret_cast<unsigned char*>(&sm.q[buf][0][0]), x - b2, DK * ES / 16, Sm::LDK * ES);
    if (x < b4) return rowpad(reinterpret_cast<unsigned char*>(&sm.pm[buf][0][0]), x - b3, C * ES / 16, Sm::LDC * ES);
    if (x < b5) return reinterpret_cast<unsigned char*>(&sm.gam[buf][0]) + size_t(x - b4) * 16;
    if (x < b6) return reinterpret_cast<unsigned char*>(&sm.qinv[buf][0]) + size_t(x - b5) * 16;
    return reinterpret_cast<unsigned char*>(&sm.winv[buf][0]);
  };

  uint4 stage[U::PER_THREAD];
  using UtRaw = std::conditional_t<F16, uint2, uint4>;
  UtRaw ut_next[NT];
  auto issue_loads = [&](int64_t n) {
    const unsigned char* rec = rec_of(n);
#pragma unroll
    for (int i = 0; i < U::PER_THREAD; ++i) {
      const int x = tid + i * kThreads;
      if (x < b7) stage[i] = *unit_src(rec, x);
    }
    if (active) {
      const Op* ut = reinterpret_cast<const Op*>(rec + L.off_UT) + size_t(col) * C + 4 * lg;
#pragma unroll
      for (int m = 0; m < NT; ++m) ut_next[m] = *reinterpret_cast<const UtRaw*>(ut + 16 * m);
    }
  };
  auto commit_loads = [&](int buf) {
#pragma unroll
    for (int i = 0; i < U::PER_THREAD; ++i) {
      const int x = tid + i * kThreads;
      if (x < b7) {
        uint2* d = reinterpret_cast<uint2*>(unit_dst(buf, x));
        d[0] = make_uint2(stage[i].x, stage[i].y);
        d[1] = make_uint2(stage[i].z, stage[i].w);
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

  issue_loads(0);
  commit_loads(0);
  UtRaw ut_cur[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) ut_cur[m] = ut_next[m];
  __syncthreads();

  for (int64_t n = 0; n < NC; ++n) {
    const int buf = int(n & 1);
    if (n + 1 < NC) issue_loads(n + 1);
    if (active) {
      const float winv = sm.winv[buf][0];
      float ut[NT][4];
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        if constexpr (F16) {
          H8 t;
          t.u[0] = ut_cur[m];
          t.u[1] = make_uint2(0u, 0u);
#pragma unroll
          for (int e = 0; e < 4; ++e) ut[m][e] = (float)t.h[e] * winv;
        } else {
          ut[m][0] = __uint_as_float(ut_cur[m].x);
          ut[m][1] = __uint_as_float(ut_cur[m].y);
          ut[m][2] = __uint_as_float(ut_cur[m].z);
          ut[m][3] = __uint_as_float(ut_cur[m].w);
        }
      }

      // state as the B operand (power-of-two scaled fp16 when F16)
      float sS = 1.0f, iS = 1.0f;
      half8 sh[KP];
      if constexpr (F16) {
        float cm = 0.0f;
#pragma unroll
        for (int ct = 0; ct < KS; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) cm = fmaxf(cm, fabsf(S[ct][e]));
        cm = max_over_groups(cm);
        sS = pow2_scale_for(cm, kStateScaleExp);
        iS = 1.0f / sS;
#pragma unroll
        for (int u = 0; u < KP; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sh[u][e] = (_Float16)(S[2 * u][e] * sS);
            sh[u][4 + e] = (2 * u + 1 < KS) ? (_Float16)(S[2 * u + 1][e] * sS) : (_Float16)0.0f;
          }
      }
      // A-operand row product with the state: rows `arow` (16 rows, DK wide)
      auto times_state = [&](const Op* arow) -> float4v {
        float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (F16) {
#pragma unroll
          for (int u = 0; u < KP; ++u) {
            const bool two = 2 * u + 1 < KS;
            const half8 a8 = pair16(arow + 32 * u + 4 * lg, two ? arow + 32 * u + 16 + 4 * lg : nullptr);
            acc = mma_pair_f16(a8, sh[u], acc);
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
        const float4v acc = times_state(&sm.w[buf][16 * m + li][0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) Um[m][e] = ut[m][e] - acc[e] * iS;
      }
      float sU = 1.0f, iU = 1.0f;
      half8 uh[NP];
      if constexpr (F16) {
        float cm = 0.0f;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) cm = fmaxf(cm, fabsf(Um[m][e]));
        cm = max_over_groups(cm);
        sU = pow2_scale_for(cm, kStateScaleExp);
        iU = 1.0f / sU;
#pragma unroll
        for (int u = 0; u < NP; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uh[u][e] = (_Float16)(Um[2 * u][e] * sU);
            uh[u][4 + e] = (2 * u + 1 < NT) ? (_Float16)(Um[2 * u + 1][e] * sU) : (_Float16)0.0f;
          }
      }
      // A-operand row product with U (summed over the chunk's steps, up to slice smax)
      auto times_u = [&](const Op* arow, int smax) -> float4v {
        float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (F16) {
#pragma unroll
          for (int u = 0; u < NP; ++u) {
            if (2 * u > smax) break;
            const bool two = 2 * u + 1 < NT;
            const half8 a8 = pair16(arow + 32 * u + 4 * lg, two ? arow + 32 * u + 16 + 4 * lg : nullptr);
            acc = mma_pair_f16(a8, uh[u], acc);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t > smax) break;
            float a4[4];
            quad(arow + 16 * t + 4 * lg, a4);
            acc = mma_slice_f32(a4, Um[t], acc);
          }
        }
        return acc;
      };

      // O = (Q+ S + P U) / q-scale   (uses the chunk-start state)
      if (want_out) {
        for (int mo = 0; mo < RT; ++mo) {
          const float4v a1 = times_state(&sm.q[buf][16 * mo + li][0]);
          const int smax = min(NT - 1, ((16 * mo + 15) * n_h + n_h - 1) / 16);
          const float4v a2 = times_u(&sm.pm[buf][16 * mo + li][0], smax);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ro = 16 * mo + 4 * lg + e;
            const int64_t t = n * R + ro;
            if (t < p.T) {
              const float ov = (a1[e] * iS + a2[e] * iU) * sm.qinv[buf][ro];
              IO<In>::st(o + ((b * p.T + t) * p.H + h) * dv + col, ov);
            }
          }
        }
      }
      // S <- Diag(gamma) S + A^^T U
#pragma unroll
      for (int ct = 0; ct < KS; ++ct) {
        const float4v acc = times_u(&sm.at[buf][16 * ct + li][0], NT - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) S[ct][e] = sm.gam[buf][16 * ct + 4 * lg + e] * S[ct][e] + acc[e] * iU;
      }
    }
    if (n + 1 < NC) {
      commit_loads(buf ^ 1);
#pragma unroll
      for (int m = 0; m < NT; ++m) ut_cur[m] = ut_next[m];
    }
    __syncthreads();
  }

  if (active && p.s_final) {
#pragma unroll
    for (int ct = 0; ct < KS; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) p.s_final[sbase + size_t(16 * ct + 4 * lg + e) * dv + col] = S[ct][e];
  }
}

// which = 1: prepare only, 2: scan only, 3: both
template <typename In, int DK, int C>
int launch_chunk_t(const Problem& p, void* ws, bool want_out, hipStream_t s, int which) {
  const ChunkLayout L = chunk_layout(p);
  unsigned char* w = static_cast<unsigned char*>(ws);
  if (which & 1) {
    const dim3 g1(unsigned(p.nchunks * p.B * p.H));
    chunk_prep_kernel<In, DK, C><<<g1, kThreads, 0, s>>>(p, w, L, want_out ? 1 : 0);
  }
  if (which & 2) {
    const unsigned cblocks = unsigned((p.dv + 63) / 64);
    const dim3 g2(unsigned(p.B * p.H) * cblocks);
    chunk_scan_kernel<In, DK, C><<<g2, kThreads, 0, s>>>(p, w, L, want_out ? 1 : 0);
  }
  return int(hipGetLastError());
}

template <typename In, int DK>
int launch_chunk_dk(const Problem& p, void* ws, bool want_out, hipStream_t s, int which) {
  switch (p.chunk) {
    case 16: return launch_chunk_t<In, DK, 16>(p, ws, want_out, s, which);
    case 32: return launch_chunk_t<In, DK, 32>(p, ws, want_out, s, which);
    case 64:
      if constexpr (std::is_same<In, float>::value && DK == 128) return int(hipErrorInvalidValue);
      else return launch_chunk_t<In, DK, 64>(p, ws, want_out, s, which);
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
