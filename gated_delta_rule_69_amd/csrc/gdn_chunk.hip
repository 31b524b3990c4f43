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
#include "gdn_chunk.h"

namespace gdn {
namespace {

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
  // Outputs are staged in LDS for full-row 16-byte stores whenever the stage fits
  // beside the double-buffered image (every bf16 case; fp32 but for chunk 64 with
  // 64 key channels); otherwise they are stored from registers one step later.
  constexpr bool OSTAGE = F16 || (2 * UNITS * 16 + 2 * C * 64 * 4 <= 160 * 1024);
  constexpr int OSR = OSTAGE ? C : 1;
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
  // output rows a chunk: R = 8 fills half of one 16-row tile, whose other rows are
  // computed from unwritten record rows and never stored
  const int R = p.rows_out, RT = (R + 15) / 16;
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
    if constexpr (!OSTAGE) return;
    for (int x = tid; x < R * ounits_row; x += kThreads) {
      const int ro = x / ounits_row, cu = x % ounits_row;
      const int64_t t = (p.c0 + n) * R + ro;
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

  // unstaged fp32 outputs of a chunk stay in registers until the next chunk's copies
  // are issued: stores issued just before the end-of-step wait would hold it up
  float ohold[NT][4];
  auto store_hold = [&](int64_t n) __attribute__((always_inline)) {
    if constexpr (!OSTAGE) {
      if (!active) return;
#pragma unroll
      for (int mo = 0; mo < NT; ++mo) {
        if (mo < RT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ro = 16 * mo + 4 * lg + e;
            const int64_t t = (p.c0 + n) * R + ro;
            if (ro < R && t < p.T) o[((b * p.T + t) * p.H + h) * dv + col] = ohold[mo][e];
          }
        }
      }
    }
  };

  for (int64_t n = 0; n < NC; ++n) {
    const int buf = int(n & 1);
    if (n + 1 < NC) issue_loads(n + 1, buf ^ 1);
    if (want_out && n > 0) {
      flush_out(buf ^ 1, n - 1);
      store_hold(n - 1);
    }
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
              } else if constexpr (OSTAGE) {
                ostage[buf][ro][16 * wave + li] = ov;
              } else {
                ohold[mo][e] = ov;
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
  if (want_out) {
    flush_out(int((NC - 1) & 1), NC - 1);
    store_hold(NC - 1);
  }

  if (active && p.s_final) {
#pragma unroll
    for (int ct = 0; ct < KS; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) p.s_final[sbase + size_t(16 * ct + 4 * lg + e) * dv + col] = S[ct][e];
  }
}

// ---- kernel 2b: sequential scan, row-split waves (fragment-format records) ---------
//
// bf16 inputs, dk = 128, chunk 64. One workgroup per (batch*head, NB value
// columns). State wave w owns rows 16w..16w+15 of U and rows 32w..32w+31 of the
// workgroup's dk x NB state slice (fp32, MFMA accumulator layout); output wave w
// owns rows 16w..16w+15 of O, computed beside the state chain. A operands (a
// wave's rows of W, A^^T and its U~ tile; of Q+ and P for output waves) are read
// straight from the record into registers one chunk ahead. The B operands, the state and U in fp16,
// cross waves through LDS, transposed, each wave block with its own power-of-two
// scale per column; a fragment is brought to the column's common (smallest) scale
// by an exact power-of-two product before its MFMA. Two barriers per chunk.
// chunks of look-ahead of the scan's L2 prefetch wave
constexpr int kAhead = 2;

template <int NCT>
__global__ __launch_bounds__(2 * kThreads + 64) void chunk_scan_rows_kernel(Problem p, const unsigned char* __restrict__ ws,
                                                                   ChunkLayout L, int want_out) {
  constexpr int DK = 128, C = 64;
  constexpr int NB = 16 * NCT;
  constexpr int KU = DK / 32;             // k-blocks over dk (one per wave block of state rows)
  constexpr int CU = C / 32;              // k-blocks over the chunk (two wave blocks of U rows each)
  constexpr int SRT = DK / 16 / kWaves;   // state row tiles per wave
  static_assert(SRT * 16 * kWaves == DK && KU == kWaves, "one k-block of state rows per wave");
  __shared__ __align__(16) _Float16 st[NB][DK + 8];   // state^T, fp16, block-scaled
  __shared__ __align__(16) _Float16 ut[NB][C + 8];    // U^T, fp16, block-scaled
  __shared__ __align__(16) float ssc[NB][kWaves];     // state scale of (column, wave block)
  __shared__ __align__(16) float usc[NB][kWaves];     // U scale of (column, wave block)
  __shared__ __align__(16) uint16_t ost[C][NB + 8];   // output rows of the chunk (bf16)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar branches)
  const int li = lane & 15, lg = lane >> 4;
  const int dv = int(p.dv), dvt = dv / 16;
  const int cblocks = dv / NB;
  int bh, cb;
  {
    // column blocks of one (batch, head) read the same records: place them 8
    // workgroups apart (same XCD, shared L2) whenever the grid allows
    const int x = blockIdx.x, nbh = int(p.B * p.H);
    const int full = (nbh / 8) * 8 * cblocks;
    if (cblocks > 1 && x < full) {
      const int grp = x / (8 * cblocks), rem = x % (8 * cblocks);
      bh = grp * 8 + rem % 8;
      cb = rem / 8;
    } else {
      bh = x / cblocks;
      cb = x % cblocks;
    }
  }
  const int H = int(p.H);
  const int b = bh / H, h = bh - b * H;
  const int NC = int(p.nchunks);
  const int R = p.rows_out;
  uint16_t* o = static_cast<uint16_t*>(p.o);
  const int col_base = cb * NB;

  // A operands of one chunk, in two halves refilled for the next chunk as soon as
  // the current chunk's half is consumed (mid-step), so that one register set
  // suffices: FA for U, FB for the state update. The output waves hold FO.
  struct FragsA {
    uint4 w[KU];
    uint2 u[NCT];
    float winv;
  };
  struct FragsB {
    uint4 at[SRT][CU];
    float4 gam[SRT];
  };
  struct FragsO {
    uint4 q[KU], pp[CU];
    float4 qi;
  };
  auto rec_of = [&](int n) -> const unsigned char* { return ws + (size_t(bh) * size_t(NC) + size_t(n)) * L.bytes; };
  auto load_a = [&](int n, FragsA& f) __attribute__((always_inline)) {
    const unsigned char* rec = rec_of(n);
    const uint4* Wf = reinterpret_cast<const uint4*>(rec + L.off_W);
    const uint2* Uf = reinterpret_cast<const uint2*>(rec + L.off_UT);
#pragma unroll
    for (int u = 0; u < KU; ++u) f.w[u] = Wf[(wave * KU + u) * 64 + lane];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) f.u[ct] = Uf[(wave * dvt + cb * NCT + ct) * 64 + lane];
    f.winv = *reinterpret_cast<const float*>(rec + L.off_winv);
  };
  auto load_b = [&](int n, FragsB& f) __attribute__((always_inline)) {
    const unsigned char* rec = rec_of(n);
    const uint4* Af = reinterpret_cast<const uint4*>(rec + L.off_AT);
    const float* gam = reinterpret_cast<const float*>(rec + L.off_gamma);
#pragma unroll
    for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
      for (int u = 0; u < CU; ++u) f.at[rt][u] = Af[((wave * SRT + rt) * CU + u) * 64 + lane];
#pragma unroll
    for (int rt = 0; rt < SRT; ++rt) f.gam[rt] = *reinterpret_cast<const float4*>(gam + 32 * wave + 16 * rt + 4 * lg);
  };
  // output wave ow: its 16 output rows of Q+ and P, and their 1/qs
  auto load_o = [&](int n, int ow, FragsO& f) __attribute__((always_inline)) {
    const unsigned char* rec = rec_of(n);
    const uint4* Qf = reinterpret_cast<const uint4*>(rec + L.off_Q);
    const uint4* Pf = reinterpret_cast<const uint4*>(rec + L.off_P);
    const float* qinv = reinterpret_cast<const float*>(rec + L.off_qinv);
#pragma unroll
    for (int u = 0; u < KU; ++u) f.q[u] = Qf[(ow * KU + u) * 64 + lane];
#pragma unroll
    for (int u = 0; u < CU; ++u) f.pp[u] = Pf[(ow * CU + u) * 64 + lane];
    f.qi = *reinterpret_cast<const float4*>(qinv + 16 * ow + 4 * lg);
  };

  // ---- prefetch wave: pulls the records of chunk n + kAhead into L2 while the
  // compute waves process chunk n (one dword of every 128-byte line this
  // workgroup will read, moved to a scratch LDS word: nothing waits on it). It
  // joins every barrier of the compute waves without a memory fence.
  if (wave == kWaves) {
    __shared__ uint32_t sink[64];
    auto touch = [&](int n) __attribute__((always_inline)) {
      const unsigned char* rec = rec_of(n);
      auto line = [&](const unsigned char* a) __attribute__((always_inline)) {
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(a),
                                         reinterpret_cast<__attribute__((address_space(3))) void*>(
                                             reinterpret_cast<uintptr_t>(&sink[0]) & 0xffffffffu),
                                         4, 0, 0);
      };
      // W, Q+, A^^T, P: contiguous [0, off_UT), shared by the head's column
      // blocks (same XCD, same L2): each block touches its share of the lines
      const int main_lines = int(L.off_UT / 128);
      const int share = (main_lines + cblocks - 1) / cblocks;
      const int x0 = cb * share, x1 = min(main_lines, x0 + share);
      for (int x = x0 + lane; x < x1; x += 64) line(rec + size_t(x) * 128);
      // this workgroup's U~ tiles (NCT * 512 bytes per row block), then gamma, 1/qs, 1/ws
      constexpr int UL = 4 * NCT;  // lines per row block
      for (int x = lane; x < kWaves * UL + 7; x += 64) {
        if (x < kWaves * UL)
          line(rec + L.off_UT + size_t((x / UL) * dvt + cb * NCT) * 512 + size_t(x % UL) * 128);
        else
          line(rec + L.off_gamma + size_t(x - kWaves * UL) * 128);
      }
    };
    for (int n = 1; n < min(NC, kAhead); ++n) touch(n);
    __builtin_amdgcn_s_barrier();
    for (int n = 0; n < NC; ++n) {
      if (n + kAhead < NC) touch(n + kAhead);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);  // no LDS write may outlive the workgroup
    return;
  }

  // 1 / x for a power of two x in [2^-126, 2^126] (exact, one integer op)
  auto inv_pow2 = [](float x) { return __uint_as_float(0x7f000000u - __float_as_uint(x)); };
  // B-operand fragments of the state (k-block u) and of U (k-block u), brought to
  // the column's common (smallest) scale; *inv receives 1 / that scale
  auto state_frags = [&](half8 (&bv)[KU][NCT], float (&ics)[NCT]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float4 s4 = *reinterpret_cast<const float4*>(&ssc[16 * ct + li][0]);
      const float cs = fminf(fminf(s4.x, s4.y), fminf(s4.z, s4.w));
      const float f[4] = {cs * inv_pow2(s4.x), cs * inv_pow2(s4.y), cs * inv_pow2(s4.z), cs * inv_pow2(s4.w)};
      ics[ct] = inv_pow2(cs);
#pragma unroll
      for (int u = 0; u < KU; ++u)
        bv[u][ct] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&st[16 * ct + li][32 * u + 8 * lg])) *
                    (_Float16)f[u];
    }
  };
  // fragment u of a column holds U rows 32 u + 8 lg .. +7: wave block 2 u + lg / 2
  auto u_frags = [&](half8 (&bv)[CU][NCT], float (&icu)[NCT]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float4 s4 = *reinterpret_cast<const float4*>(&usc[16 * ct + li][0]);
      const float cu = fminf(fminf(s4.x, s4.y), fminf(s4.z, s4.w));
      icu[ct] = inv_pow2(cu);
      const float f[2] = {cu * inv_pow2((lg >> 1) ? s4.y : s4.x), cu * inv_pow2((lg >> 1) ? s4.w : s4.z)};
#pragma unroll
      for (int u = 0; u < CU; ++u)
        bv[u][ct] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&ut[16 * ct + li][32 * u + 8 * lg])) *
                    (_Float16)f[u];
    }
  };

  // ---- output waves: O = (Q+ S + P U) / qs for 16 output rows each, off the state
  // chain: the Q+ S part between the step's two barriers' first half (the state of
  // the chunk start is in st until the second barrier), P U after the first barrier
  // (U is in ut until the next step's first barrier). Rows are staged in this
  // wave's own rows of ost and written with 16-byte stores.
  if (wave > kWaves) {
    const int ow = wave - kWaves - 1;
    const bool act = want_out && ow < (R + 15) / 16;  // R = 8: half of one wave's rows
    FragsO fo;
    if (act && NC > 0) load_o(0, ow, fo);
    __syncthreads();
    for (int n = 0; n < NC; ++n) {
      float4v oa[NCT], pa[NCT];
      float ics[NCT];
      if (act) {
        half8 bv[KU][NCT];
        state_frags(bv, ics);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) oa[ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) oa[ct] = mma_pair_f16(__builtin_bit_cast(half8, fo.q[u]), bv[u][ct], oa[ct]);
      }
      __syncthreads();
      if (act) {
        half8 bu[CU][NCT];
        float icu[NCT];
        u_frags(bu, icu);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) pa[ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < CU; ++u)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) pa[ct] = mma_pair_f16(__builtin_bit_cast(half8, fo.pp[u]), bu[u][ct], pa[ct]);
        const float qi[4] = {fo.qi.x, fo.qi.y, fo.qi.z, fo.qi.w};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ov = (oa[ct][e] * ics[ct] + pa[ct][e] * icu[ct]) * qi[e];
            ost[16 * ow + 4 * lg + e][16 * ct + li] = __builtin_bit_cast(uint16_t, (__bf16)ov);
          }
        if (n + 1 < NC) load_o(n + 1, ow, fo);
        // this wave's 16 rows: NB / 8 16-byte units each (LDS order within a wave)
        constexpr int RU = NB / 8;
        for (int x = lane; x < 16 * RU; x += 64) {
          const int ro = 16 * ow + x / RU, c8 = x % RU;
          const int64_t t = (p.c0 + n) * R + ro;
          if (ro < R && t < p.T)
            *reinterpret_cast<uint4*>(o + ((int64_t(b) * p.T + t) * H + h) * dv + col_base + 8 * c8) =
                *reinterpret_cast<const uint4*>(&ost[ro][8 * c8]);
        }
      }
      __syncthreads();
    }
    return;
  }

  // ---- state waves ----
  // They carry the dependent chain, so their instructions issue ahead of the output
  // and prefetch waves' on the same SIMD (wave priority only; no memory effect).
  __builtin_amdgcn_s_setprio(3);
  // state: S[rt][ct][e] = S[32 w + 16 rt + 4 lg + e][col_base + 16 ct + li]
  float S[SRT][NCT][4];
  const size_t sbase = size_t(bh) * DK * size_t(dv);
#pragma unroll
  for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[rt][ct][e] = p.s0 ? p.s0[sbase + size_t(32 * wave + 16 * rt + 4 * lg + e) * dv + col_base + 16 * ct + li]
                            : 0.0f;
  // publish this wave's state rows: fp16 image and the block's column scales
  auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float m = 0.0f;
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(S[rt][ct][e]));
      const float sc = block_scale(max_over_groups(m), kStateScaleExp);
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt) {
        H8 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hv.h[e] = (_Float16)(S[rt][ct][e] * sc);
        *reinterpret_cast<uint2*>(&st[16 * ct + li][32 * wave + 16 * rt + 4 * lg]) = hv.u[0];
      }
      if (lg == 0) ssc[16 * ct + li][wave] = sc;
    }
  };

  auto step = [&](int n, FragsA& fa, FragsB& fb) __attribute__((always_inline)) {
    const int nn = min(n + 1, NC - 1);  // next chunk (the last one is read again at the end)
    // ---- U = U~ / ws - W S (B = state at the column's common scale) ----
    float ics[NCT];
    float4v ua[NCT];
    {
      half8 bv[KU][NCT];
      state_frags(bv, ics);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) ua[ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) ua[ct] = mma_pair_f16(__builtin_bit_cast(half8, fa.w[u]), bv[u][ct], ua[ct]);
    }
    // U rows 16 w + 4 lg + e, column 16 ct + li; fp16 U^T with this block's scale
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const half4 t4 = __builtin_bit_cast(half4, fa.u[ct]);
      float uv[4], m = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uv[e] = (float)t4[e] * fa.winv - ua[ct][e] * ics[ct];
        m = fmaxf(m, fabsf(uv[e]));
      }
      const float su = block_scale(max_over_groups(m), kStateScaleExp);
      H8 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e) hv.h[e] = (_Float16)(uv[e] * su);
      *reinterpret_cast<uint2*>(&ut[16 * ct + li][16 * wave + 4 * lg]) = hv.u[0];
      if (lg == 0) usc[16 * ct + li][wave] = su;
    }
    load_a(nn, fa);
    __syncthreads();

    // ---- S' = Diag(gamma) S + A^^T U (B = U at the column's common scale) ----
    float4v sa[SRT][NCT];
    float icu[NCT];
    {
      half8 bu[CU][NCT];
      u_frags(bu, icu);
#pragma unroll
      for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) sa[rt][ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < CU; ++u)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int rt = 0; rt < SRT; ++rt) sa[rt][ct] = mma_pair_f16(__builtin_bit_cast(half8, fb.at[rt][u]), bu[u][ct], sa[rt][ct]);
    }
    const float gm[SRT][4] = {{fb.gam[0].x, fb.gam[0].y, fb.gam[0].z, fb.gam[0].w},
                              {fb.gam[SRT - 1].x, fb.gam[SRT - 1].y, fb.gam[SRT - 1].z, fb.gam[SRT - 1].w}};
#pragma unroll
    for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[rt][ct][e] = gm[rt][e] * S[rt][ct][e] + sa[rt][ct][e] * icu[ct];
    load_b(nn, fb);
    publish_state();
    __syncthreads();
  };

  publish_state();
  __syncthreads();
  if (NC > 0) {
    FragsA fa;
    FragsB fb;
    load_a(0, fa);
    load_b(0, fb);
    for (int n = 0; n < NC; ++n) step(n, fa, fb);
  }

  if (p.s_final) {
#pragma unroll
    for (int rt = 0; rt < SRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.s_final[sbase + size_t(32 * wave + 16 * rt + 4 * lg + e) * dv + col_base + 16 * ct + li] = S[rt][ct][e];
  }
}

// ---- launch ----------------------------------------------------------------------------

template <typename In, int DK, int C>
int launch_scan_t(const Problem& p, void* ws, bool want_out, hipStream_t s) {
  const ChunkLayout L = chunk_layout(p);
  if constexpr (std::is_same<In, uint16_t>::value && DK == 128 && C == 64) {
    // fragment-format records: row-split scan, 16 value columns per workgroup
    // (one workgroup per 16 columns keeps the step latency short: the scan is a
    // chain of dependent MFMA / LDS / barrier phases, 512 steps long at 32K)
    const dim3 g(unsigned(p.B * p.H) * unsigned(p.dv / 16));
    chunk_scan_rows_kernel<1><<<g, 2 * kThreads + 64, 0, s>>>(p, static_cast<const unsigned char*>(ws), L,
                                                         want_out ? 1 : 0);
    return int(hipGetLastError());
  } else {
    const unsigned cblocks = unsigned((p.dv + 63) / 64);
    const dim3 g2(unsigned(p.B * p.H) * cblocks);
    chunk_scan_kernel<In, DK, C><<<g2, kThreads, 0, s>>>(p, static_cast<const unsigned char*>(ws), L,
                                                         want_out ? 1 : 0);
    return int(hipGetLastError());
  }
}

template <typename In, int DK>
int launch_scan_dk(const Problem& p, void* ws, bool want_out, hipStream_t s) {
  switch (p.chunk) {
    case 16: return launch_scan_t<In, DK, 16>(p, ws, want_out, s);
    case 32: return launch_scan_t<In, DK, 32>(p, ws, want_out, s);
    case 64:
      if constexpr (std::is_same<In, float>::value && DK == 128) return int(hipErrorInvalidValue);
      else return launch_scan_t<In, DK, 64>(p, ws, want_out, s);
    default: return int(hipErrorInvalidValue);
  }
}

template <typename In>
int launch_scan_in(const Problem& p, void* ws, bool want_out, hipStream_t s) {
  switch (p.dk) {
    case 16: return launch_scan_dk<In, 16>(p, ws, want_out, s);
    case 32: return launch_scan_dk<In, 32>(p, ws, want_out, s);
    case 64: return launch_scan_dk<In, 64>(p, ws, want_out, s);
    case 128: return launch_scan_dk<In, 128>(p, ws, want_out, s);
    default: return int(hipErrorInvalidValue);
  }
}

}  // namespace

int launch_prep(const Problem& p, void* ws, bool want_out, void* stream) {
  switch (p.variant) {
    case GDN_VARIANT_FG2: return launch_prep_fg2(p, ws, want_out, stream);
    case GDN_VARIANT_KDA: return launch_prep_kda(p, ws, want_out, stream);
    case GDN_VARIANT_GDN: return launch_prep_gdn(p, ws, want_out, stream);
    case GDN_VARIANT_DELTAPRODUCT: return launch_prep_dp(p, ws, want_out, stream);
    case GDN_VARIANT_ASYM: return launch_prep_asym(p, ws, want_out, stream);
    default: return int(hipErrorInvalidValue);
  }
}

int launch_scan(const Problem& p, void* ws, bool want_out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.dtype == GDN_DTYPE_BF16 ? launch_scan_in<uint16_t>(p, ws, want_out, s)
                                   : launch_scan_in<float>(p, ws, want_out, s);
}

int launch_chunk(const Problem& p, void* ws, bool want_out, void* stream) {
  const int e = launch_prep(p, ws, want_out, stream);
  if (e != 0) return e;
  return launch_scan(p, ws, want_out, stream);
}

}  // namespace gdn
