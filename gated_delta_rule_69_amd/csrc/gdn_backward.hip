// Backward pass of the token recurrence (reverse mode), every variant: FG2, FG2+, KDA,
// GDN, ASYM, and DeltaProduct as its sequence of Householder sub-steps.
//
// Per token, with X = Diag(alpha) S_{t-1}, u = w - X^T b, S_t = X + a u^T,
// o_t = S_t^T q_t and G = dL/dS_t (the later tokens' gradient plus q_t do_t^T):
//   dq = S_t do,  dw = G^T a,  da = G u,  db = -X dw,  dX = G - b dw^T,
//   dalpha = rowsum(dX . S_{t-1}),  dL/dS_{t-1} = Diag(alpha) dX,
// then the chain rule through the variant's (a, b, w, alpha) map (FG2-GDN reading
// notes, section 2.2 eq. (11) and section 2.3 eq. (13); GDN2-stability page, eq. (1)).
//
// Kernel A: one wave per (batch, head, 16-column slice of the state) (lane
// l = j + 16 g: column j, key rows g NR .. g NR + NR - 1, as in the forward recurrent
// kernel). A forward pass stores the slice state every kCB tokens; the backward sweep
// takes the chunks in reverse, recomputes the chunk's states from its checkpoint
// into the workspace, and walks the chunk backwards. Column-complete quantities
// (dw) come out of the wave directly; row quantities (da, db, dq, dalpha) are partial
// sums over the wave's 16 columns, reduced across the 16 lanes by a transposing
// butterfly and written per slice. Kernel B sums the slices in a fixed order and
// applies the variant's chain rule, one wave per token and head.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCB = 64;  // tokens per checkpoint interval

// Workspace (floats): per (batch*head, slice) the checkpoints and the current chunk's
// states, in lane order ([step][NR/4][64 lanes][4]: one 16-byte vector per lane);
// then the row partials [slice][B*T*H][4][dk] and dw [B*T*H][dv].
struct BwdLayout {
  int64_t slice_floats, part, dw, total;
};

// T counts steps here (tokens x n_h for DeltaProduct, whose rows are sub-steps).
__host__ __device__ inline BwdLayout bwd_layout(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  BwdLayout L;
  const int64_t nck = (T + kCB - 1) / kCB;
  const int64_t ns = dv / 16;
  const int64_t bth = B * T * H;
  L.slice_floats = (nck + kCB) * dk * 16;
  L.part = B * H * ns * L.slice_floats;
  L.dw = L.part + ns * bth * 4 * dk;
  L.total = L.dw + bth * dv;
  return L;
}

// Sum over the 16 lanes of a row group (lanes j = 0..15 at fixed g) of NR values per
// lane, by a butterfly that halves the value count at each exchange (transpose-
// reduce). On return lane j holds sums for M = max(NR / 16, 1) rows, out[i] for
// row i + M * (j * M * 16 / NR) ... expressed by row_of(j, i).
template <int NR>
struct RowReduce16 {
  static constexpr int M = NR >= 16 ? NR / 16 : 1;
  __device__ static __forceinline__ void run(float (&v)[NR], int j, float (&out)[M]) {
    int n = NR;
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      if (n >= 2) {
        const bool hi = (j & m) != 0;
#pragma unroll
        for (int i = 0; i < NR / 2; ++i) {
          if (i < n / 2) {
            const float lo_v = v[i], hi_v = v[i + n / 2];
            const float send = hi ? lo_v : hi_v;
            const float keep = hi ? hi_v : lo_v;
            v[i] = keep + __shfl_xor(send, m, 64);
          }
        }
        n /= 2;
      } else {
        v[0] += __shfl_xor(v[0], m, 64);
      }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) out[i] = v[i];
  }
  // row (within the group's NR rows) of out[i] in lane j
  __device__ static __forceinline__ int row_of(int j, int i) {
    if constexpr (NR >= 16) {
      return j * M + i;
    } else {
      return j / (16 / NR);  // NR < 16: lanes j .. share the row j / (16 / NR)
    }
  }
  // whether lane j writes its rows (one writer per row)
  __device__ static __forceinline__ bool writer(int j) {
    if constexpr (NR >= 16) return true;
    else return j % (16 / NR) == 0;
  }
};

// Kernel A: one wave per (batch*head, 16-column slice): forward with checkpoints,
// then the reverse sweep; writes dw (column-complete) and the row partials.
template <typename In, int DK>
__global__ __launch_bounds__(64) void bwd_slice_kernel(Problem p, const In* __restrict__ d_o,
                                                       const float* __restrict__ dsf, float* __restrict__ ds0,
                                                       float* __restrict__ ws) {
  constexpr int NR = DK / 4;
  using RR = RowReduce16<NR>;
  const int lane = threadIdx.x;
  const int j = lane & 15, gr = lane >> 4;
  const int64_t T = p.T, H = p.H, dv = p.dv;
  const int ns = int(dv / 16);
  const int64_t bh = blockIdx.x / ns;
  const int wave = int(blockIdx.x % ns);  // column slice
  const int64_t b = bh / H, h = bh % H;
  const int col = wave * 16 + j;
  const int row0 = gr * NR;
  const int nh = p.n_h;
  const int64_t NS = p.steps;  // steps: tokens x n_h
  const BwdLayout L = bwd_layout(p.B, NS, H, DK, dv);
  float* wsl = ws + int64_t(blockIdx.x) * L.slice_floats;
  const int64_t nck = (NS + kCB - 1) / kCB;
  const int64_t bth = p.B * T * H * nh;  // step rows

  const In* q = static_cast<const In*>(p.q);
  const In* k = static_cast<const In*>(p.k);
  const In* v = static_cast<const In*>(p.v);
  const In* al = static_cast<const In*>(p.alpha);
  const In* be = static_cast<const In*>(p.beta);
  const In* bev = static_cast<const In*>(p.beta_v);
  const In* jv = static_cast<const In*>(p.j);
  const In* et = static_cast<const In*>(p.eta);
  auto ld = [](const In* x) { return IO<In>::ld(x); };

  // A token's inputs as loaded (raw 16- or 8-byte vectors and scalars), so that the
  // next token's loads can be in flight while the current one is computed; finish()
  // converts them into (a, b, alpha) rows, w of this lane's column, q rows and do.
  using V4 = std::conditional_t<std::is_same<In, float>::value, float4, uint2>;
  struct Raw {
    V4 k[NR / 4], x[NR / 4], y[NR / 4], qv[NR / 4];
    In s, vc, vb, dout;
    bool first;  // DeltaProduct: the token's first step (the gate acts)
  };
  auto rows = [&](const In* base, V4 (&dst)[NR / 4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NR / 4; ++i) dst[i] = reinterpret_cast<const V4*>(base)[i];
  };
  auto cvt = [](const V4& x, float* o) __attribute__((always_inline)) {
    if constexpr (std::is_same<In, float>::value) {
      o[0] = x.x, o[1] = x.y, o[2] = x.z, o[3] = x.w;
    } else {
      o[0] = __uint_as_float(x.x << 16), o[1] = __uint_as_float(x.x & 0xffff0000u);
      o[2] = __uint_as_float(x.y << 16), o[3] = __uint_as_float(x.y & 0xffff0000u);
    }
  };
  auto load_raw = [&](int64_t vs, Raw& r, bool with_q) __attribute__((always_inline)) {
    const int64_t t = vs / nh;
    const int sub = int(vs - t * nh);
    const int64_t th = (b * T + t) * H + h;
    const int64_t sr = th * nh + sub;  // step row ([B, T, H, n_h] for DeltaProduct)
    rows(k + sr * DK + row0, r.k);
    r.vc = v[sr * dv + col];
    r.first = sub == 0;
    if (p.variant == GDN_VARIANT_DELTAPRODUCT) {
      r.s = be[sr];
      r.vb = al[th];
      if (with_q) {
        if (sub == nh - 1) {
          rows(q + th * DK + row0, r.qv);
          r.dout = d_o[th * dv + col];
        } else {  // q is read after the last step only
#pragma unroll
          for (int i = 0; i < NR / 4; ++i) r.qv[i] = V4{};
          r.dout = In(0);
        }
      }
      return;
    }
    if (p.variant == GDN_VARIANT_ASYM) {
      r.s = et[th];
      rows(jv + th * DK + row0, r.y);
      rows(al + th * DK + row0, r.x);
    } else if (p.variant == GDN_VARIANT_FG2) {
      rows(be + th * DK + row0, r.y);
      rows(al + th * DK + row0, r.x);
      r.vb = bev ? bev[th * dv + col] : be[th * DK + col];
    } else {
      r.s = be[th];
      if (p.variant == GDN_VARIANT_KDA) rows(al + th * DK + row0, r.x);
      else r.vb = al[th];
    }
    if (with_q) {
      rows(q + th * DK + row0, r.qv);
      r.dout = d_o[th * dv + col];
    }
  };
  auto finish = [&](const Raw& r, float (&a)[NR], float (&bb)[NR], float (&alpha)[NR], float& w)
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NR / 4; ++i) cvt(r.k[i], a + 4 * i);
    const float vc = ld(&r.vc);
    if (p.variant == GDN_VARIANT_DELTAPRODUCT) {
      const float bt = ld(&r.s);
      const float gm = r.first ? ld(&r.vb) : 1.0f;
#pragma unroll
      for (int q2 = 0; q2 < NR; ++q2) {
        bb[q2] = bt * a[q2];
        alpha[q2] = gm;
      }
      w = bt * vc;
    } else if (p.variant == GDN_VARIANT_ASYM) {
      const float e = ld(&r.s);
#pragma unroll
      for (int i = 0; i < NR / 4; ++i) {
        cvt(r.y[i], bb + 4 * i);
        cvt(r.x[i], alpha + 4 * i);
      }
#pragma unroll
      for (int q2 = 0; q2 < NR; ++q2) bb[q2] *= e;
      w = e * vc;
    } else if (p.variant == GDN_VARIANT_FG2) {
      float beta[NR];
#pragma unroll
      for (int i = 0; i < NR / 4; ++i) {
        cvt(r.y[i], beta + 4 * i);
        cvt(r.x[i], alpha + 4 * i);
      }
#pragma unroll
      for (int q2 = 0; q2 < NR; ++q2) {
        a[q2] *= sqrtf(beta[q2]);
        bb[q2] = a[q2];
      }
      w = vc * sqrtf(ld(&r.vb));
    } else {
      const float sb = sqrtf(ld(&r.s));
#pragma unroll
      for (int q2 = 0; q2 < NR; ++q2) {
        a[q2] *= sb;
        bb[q2] = a[q2];
      }
      if (p.variant == GDN_VARIANT_KDA) {
#pragma unroll
        for (int i = 0; i < NR / 4; ++i) cvt(r.x[i], alpha + 4 * i);
      } else {
        const float gm = ld(&r.vb);
#pragma unroll
        for (int q2 = 0; q2 < NR; ++q2) alpha[q2] = gm;
      }
      w = sb * vc;
    }
  };
  // slice state of one step in lane order: 16-byte vectors, coalesced
  auto save = [&](float* base, const float (&S)[NR]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NR / 4; ++i)
      reinterpret_cast<float4*>(base)[i * 64 + lane] = make_float4(S[4 * i], S[4 * i + 1], S[4 * i + 2], S[4 * i + 3]);
  };
  auto restore = [&](const float* base, float (&S)[NR]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NR / 4; ++i) {
      const float4 x = reinterpret_cast<const float4*>(base)[i * 64 + lane];
      S[4 * i] = x.x, S[4 * i + 1] = x.y, S[4 * i + 2] = x.z, S[4 * i + 3] = x.w;
    }
  };
  auto fwd = [&](float (&S)[NR], const Raw& raw) __attribute__((always_inline)) {
    float a[NR], bb[NR], alpha[NR], w;
    finish(raw, a, bb, alpha, w);
    float bx = 0.0f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      S[r] *= alpha[r];
      bx += bb[r] * S[r];
    }
    const float u = w - sum_over_groups(bx);
#pragma unroll
    for (int r = 0; r < NR; ++r) S[r] += a[r] * u;
  };

  float* ck = wsl;                  // [nck][DK * 16]
  float* cs = wsl + nck * DK * 16;  // [kCB][DK * 16]
  float S[NR];
  const size_t sbase = size_t(bh) * DK * size_t(dv);
#pragma unroll
  for (int r = 0; r < NR; ++r) S[r] = p.s0 ? p.s0[sbase + size_t(row0 + r) * dv + col] : 0.0f;
  Raw cur, nxt;
  if (NS > 0) load_raw(0, cur, false);
  nxt = cur;
  for (int64_t t = 0; t < NS; ++t) {
    if (t + 1 < NS) load_raw(t + 1, nxt, false);  // in flight during this step
    if (t % kCB == 0) save(ck + (t / kCB) * DK * 16, S);
    fwd(S, cur);
    cur = nxt;
  }

  float G[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) G[r] = dsf ? dsf[sbase + size_t(row0 + r) * dv + col] : 0.0f;
  float* part = ws + L.part;
  float* dwg = ws + L.dw;
  for (int64_t c = nck - 1; c >= 0; --c) {
    const int64_t t0 = c * kCB, t1 = min(NS, t0 + kCB);
    restore(ck + c * DK * 16, S);
    load_raw(t0, cur, false);
    nxt = cur;
    for (int64_t t = t0; t < t1; ++t) {  // the states before each token of the chunk
      if (t + 1 < t1) load_raw(t + 1, nxt, false);
      save(cs + (t - t0) * DK * 16, S);
      fwd(S, cur);
      cur = nxt;
    }
    load_raw(t1 - 1, cur, true);
    nxt = cur;
    for (int64_t t = t1 - 1; t >= t0; --t) {
      if (t > t0) load_raw(t - 1, nxt, true);  // in flight during this token
      float a[NR], bb[NR], alpha[NR], w, qv[NR];
      finish(cur, a, bb, alpha, w);
      const int64_t th = ((b * T + t / nh) * H + h) * nh + t % nh;  // step row
#pragma unroll
      for (int i = 0; i < NR / 4; ++i) cvt(cur.qv[i], qv + 4 * i);
      const float doc = ld(&cur.dout);
      float Sp[NR], X[NR];
      restore(cs + (t - t0) * DK * 16, Sp);
      float bx = 0.0f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        X[r] = alpha[r] * Sp[r];
        bx += bb[r] * X[r];
      }
      const float u = w - sum_over_groups(bx);
      float dq[NR], da[NR], db[NR], dal[NR];
      float gw = 0.0f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        dq[r] = (X[r] + a[r] * u) * doc;  // S_t do, this column's term
        G[r] += qv[r] * doc;
        gw += G[r] * a[r];
      }
      const float dw = sum_over_groups(gw);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        da[r] = G[r] * u;
        db[r] = -X[r] * dw;
        const float dX = G[r] - bb[r] * dw;
        dal[r] = dX * Sp[r];
        G[r] = alpha[r] * dX;
      }
      if (gr == 0) dwg[th * dv + col] = dw;
      float* pw = part + (int64_t(wave) * bth + th) * 4 * DK;
      float o4[4][RR::M];
      RR::run(dq, j, o4[0]);
      RR::run(da, j, o4[1]);
      RR::run(db, j, o4[2]);
      RR::run(dal, j, o4[3]);
      if (RR::writer(j)) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
#pragma unroll
          for (int i = 0; i < RR::M; ++i) pw[qd * DK + row0 + RR::row_of(j, i)] = o4[qd][i];
      }
      cur = nxt;
    }
  }
  if (ds0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) ds0[sbase + size_t(row0 + r) * dv + col] = G[r];
  }
}

// Kernel B: one wave per token-head: the partials summed over the slices in order,
// then the variant's chain rule.
template <typename In, int DK>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(Problem p, GradPtrs g, const float* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const int64_t T = p.T, H = p.H, dv = p.dv;
  const int ns = int(dv / 16);
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
    if (p.variant == GDN_VARIANT_DELTAPRODUCT) {  // th is a step row (token x n_h + step)
      const int64_t tok = th / nh;
      const int sub = int(th - tok * nh);
      const float bt = ld(be + th);
      float sb = 0.0f, sal = 0.0f;
      for (int r = lane; r < DK; r += 64) {
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int w2 = 0; w2 < ns; ++w2) {
          const float* pr = part + (int64_t(w2) * bth + th) * 4 * DK;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) s4[qd] += pr[qd * DK + r];
        }
        g.dk[th * DK + r] = s4[1] + bt * s4[2];
        sb += ld(k + th * DK + r) * s4[2];
        sal += s4[3];
        if (sub == nh - 1) g.dq[tok * DK + r] = s4[0];
      }
      for (int cc = lane; cc < dv; cc += 64) {
        const float dw = dwg[th * dv + cc];
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
        const float* pr = part + (int64_t(w2) * bth + th) * 4 * DK;
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
        if (!bev) db += ld(v + th * dv + r) * dwg[th * dv + r];  // shared beta (dk == dv)
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
      const float dw = dwg[th * dv + cc];
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
  const unsigned slices = unsigned(p.B * p.H * (p.dv / 16));
  bwd_slice_kernel<In, DK><<<dim3(slices), dim3(64), 0, s>>>(p, dO, dsf, g.ds0, ws);
  int e = int(hipGetLastError());
  if (e != 0 || p.T == 0) return e;
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
