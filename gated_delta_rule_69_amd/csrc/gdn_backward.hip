// Backward pass of the token recurrence (reverse mode), every variant with one step a
// token (FG2, FG2+, KDA, GDN, ASYM).
//
// Per token, with X = Diag(alpha) S_{t-1}, u = w - X^T b, S_t = X + a u^T,
// o_t = S_t^T q_t and G = dL/dS_t (the later tokens' gradient plus q_t do_t^T):
//   dq = S_t do,  dw = G^T a,  da = G u,  db = -X dw,  dX = G - b dw^T,
//   dalpha = rowsum(dX . S_{t-1}),  dL/dS_{t-1} = Diag(alpha) dX,
// then the chain rule through the variant's (a, b, w, alpha) map (FG2-GDN reading
// notes, section 2.2 eq. (11) and section 2.3 eq. (13); GDN2-stability page, eq. (1)).
//
// One workgroup per (batch, head), one wave per 16-column slice of the state (lane
// l = j + 16 g: column j, key rows g NR .. g NR + NR - 1, as in the forward recurrent
// kernel). A forward pass stores the slice state every CB tokens; the backward sweep
// takes the chunks in reverse, recomputes the chunk's states from its checkpoint
// into the workspace, and walks the chunk backwards. Column-complete quantities
// (dw) come out of the wave directly; row quantities (da, db, dq, dalpha) are partial
// sums over the wave's 16 columns, reduced across the 16 lanes by a transposing
// butterfly and across the slices, in a fixed order, after each chunk.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCB = 64;  // tokens per checkpoint interval

struct BwdLayout {
  int64_t ckpt, cs, part, dw, per_head;  // float offsets within a head's area
};

__host__ __device__ inline BwdLayout bwd_layout(int64_t T, int64_t dk, int64_t dv) {
  BwdLayout L;
  const int64_t nck = (T + kCB - 1) / kCB;
  const int64_t ns = dv / 16;
  L.ckpt = 0;
  L.cs = L.ckpt + nck * dk * dv;
  L.part = L.cs + int64_t(kCB) * dk * dv;
  L.dw = L.part + ns * kCB * 4 * dk;
  L.per_head = L.dw + int64_t(kCB) * dv;
  L.per_head = (L.per_head + 63) / 64 * 64;
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

template <typename In, int DK>
__global__ __launch_bounds__(512) void recurrent_bwd_kernel(Problem p, const In* __restrict__ d_o,
                                                            const float* __restrict__ dsf, GradPtrs g,
                                                            float* __restrict__ ws) {
  constexpr int NR = DK / 4;
  using RR = RowReduce16<NR>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;  // column slice
  const int j = lane & 15, gr = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, H = p.H, dv = p.dv;
  const int ns = int(dv / 16);
  const int col = wave * 16 + j;
  const int row0 = gr * NR;
  const BwdLayout L = bwd_layout(T, DK, dv);
  float* wsh = ws + bh * L.per_head;
  const int64_t nck = (T + kCB - 1) / kCB;

  const In* q = static_cast<const In*>(p.q);
  const In* k = static_cast<const In*>(p.k);
  const In* v = static_cast<const In*>(p.v);
  const In* al = static_cast<const In*>(p.alpha);
  const In* be = static_cast<const In*>(p.beta);
  const In* bev = static_cast<const In*>(p.beta_v);
  const In* jv = static_cast<const In*>(p.j);
  const In* et = static_cast<const In*>(p.eta);
  auto ld = [](const In* x) { return IO<In>::ld(x); };

  // (a, b, alpha) rows and w of this lane's column for token t
  auto token = [&](int64_t t, float (&a)[NR], float (&bb)[NR], float (&alpha)[NR], float& w)
      __attribute__((always_inline)) {
    const int64_t th = (b * T + t) * H + h;
    load_vec<NR>(k + th * DK + row0, a);
    const float vc = ld(v + th * dv + col);
    if (p.variant == GDN_VARIANT_ASYM) {
      const float e = ld(et + th);
      load_vec<NR>(jv + th * DK + row0, bb);
      load_vec<NR>(al + th * DK + row0, alpha);
#pragma unroll
      for (int r = 0; r < NR; ++r) bb[r] *= e;
      w = e * vc;
    } else if (p.variant == GDN_VARIANT_FG2) {
      float beta[NR];
      load_vec<NR>(be + th * DK + row0, beta);
      load_vec<NR>(al + th * DK + row0, alpha);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        a[r] *= sqrtf(beta[r]);
        bb[r] = a[r];
      }
      w = vc * sqrtf(bev ? ld(bev + th * dv + col) : ld(be + th * DK + col));
    } else {
      const float s = sqrtf(ld(be + th));
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        a[r] *= s;
        bb[r] = a[r];
      }
      if (p.variant == GDN_VARIANT_KDA) {
        load_vec<NR>(al + th * DK + row0, alpha);
      } else {
        const float gm = ld(al + th);
#pragma unroll
        for (int r = 0; r < NR; ++r) alpha[r] = gm;
      }
      w = s * vc;
    }
  };
  auto st_addr = [&](float* base, int r) { return base + int64_t(row0 + r) * dv + col; };
  auto fwd = [&](float (&S)[NR], int64_t t) __attribute__((always_inline)) {
    float a[NR], bb[NR], alpha[NR], w;
    token(t, a, bb, alpha, w);
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

  // ---- forward: checkpoints every kCB tokens ----
  float S[NR];
  const size_t sbase = size_t(bh) * DK * size_t(dv);
#pragma unroll
  for (int r = 0; r < NR; ++r) S[r] = p.s0 ? p.s0[sbase + size_t(row0 + r) * dv + col] : 0.0f;
  for (int64_t t = 0; t < T; ++t) {
    if (t % kCB == 0) {
      float* ck = wsh + L.ckpt + (t / kCB) * DK * dv;
#pragma unroll
      for (int r = 0; r < NR; ++r) *st_addr(ck, r) = S[r];
    }
    fwd(S, t);
  }

  // ---- backward, chunk by chunk in reverse ----
  float G[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) G[r] = dsf ? dsf[sbase + size_t(row0 + r) * dv + col] : 0.0f;
  float* cs = wsh + L.cs;
  float* part = wsh + L.part;
  float* dwb = wsh + L.dw;
  for (int64_t c = nck - 1; c >= 0; --c) {
    const int64_t t0 = c * kCB, t1 = min(T, t0 + kCB);
    {  // recompute the states before each token of the chunk
      float* ck = wsh + L.ckpt + c * DK * dv;
#pragma unroll
      for (int r = 0; r < NR; ++r) S[r] = *st_addr(ck, r);
      for (int64_t t = t0; t < t1; ++t) {
        float* dst = cs + (t - t0) * DK * dv;
#pragma unroll
        for (int r = 0; r < NR; ++r) *st_addr(dst, r) = S[r];
        fwd(S, t);
      }
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const int tl = int(t - t0);
      float a[NR], bb[NR], alpha[NR], w, qv[NR];
      token(t, a, bb, alpha, w);
      const int64_t th = (b * T + t) * H + h;
      load_vec<NR>(q + th * DK + row0, qv);
      const float doc = IO<In>::ld(d_o + th * dv + col);
      float Sp[NR], X[NR];
      const float* src = cs + int64_t(tl) * DK * dv;
      float bx = 0.0f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        Sp[r] = src[int64_t(row0 + r) * dv + col];
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
      if (gr == 0) dwb[int64_t(tl) * dv + col] = dw;
      float* pw = part + (int64_t(wave) * kCB + tl) * 4 * DK;
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
    }
    __syncthreads();
    // ---- the chunk's gradients: partials summed over the slices in order, then the
    // variant's chain rule; wave w takes tokens w, w + ns, ... ----
    for (int64_t t = t0 + wave; t < t1; t += ns) {
      const int tl = int(t - t0);
      const int64_t th = (b * T + t) * H + h;
      float sk = 0.0f, sv = 0.0f, sj = 0.0f, sal = 0.0f;  // per-token sums
      const float sbeta = (p.variant == GDN_VARIANT_KDA || p.variant == GDN_VARIANT_GDN) ? sqrtf(ld(be + th)) : 1.0f;
      const float e = p.variant == GDN_VARIANT_ASYM ? ld(et + th) : 0.0f;
      for (int r = lane; r < DK; r += 64) {
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int w2 = 0; w2 < ns; ++w2) {
          const float* pr = part + (int64_t(w2) * kCB + tl) * 4 * DK;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) s4[qd] += pr[qd * DK + r];
        }
        const float dq = s4[0], dab = s4[1] + s4[2], dal = s4[3];
        const int64_t ir = th * DK + r;
        g.dq[ir] = dq;
        const float kr = ld(k + ir);
        if (p.variant == GDN_VARIANT_FG2) {
          const float s = sqrtf(ld(be + ir));
          g.dk[ir] = s * dab;
          g.dalpha[ir] = dal;
          float db = kr * dab;
          if (!bev) db += ld(v + th * dv + r) * dwb[int64_t(tl) * dv + r];  // shared beta (dk == dv)
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
        const float dw = dwb[int64_t(tl) * dv + cc];
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
    __syncthreads();
  }
  if (g.ds0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) g.ds0[sbase + size_t(row0 + r) * dv + col] = G[r];
  }
}

template <typename In>
int launch_in(const Problem& p, const void* d_o, const float* dsf, const GradPtrs& g, float* ws,
              hipStream_t s) {
  const dim3 grid(unsigned(p.B * p.H));
  const dim3 block(unsigned(64 * (p.dv / 16)));
  const In* dO = static_cast<const In*>(d_o);
  switch (p.dk) {
    case 16: recurrent_bwd_kernel<In, 16><<<grid, block, 0, s>>>(p, dO, dsf, g, ws); break;
    case 32: recurrent_bwd_kernel<In, 32><<<grid, block, 0, s>>>(p, dO, dsf, g, ws); break;
    case 64: recurrent_bwd_kernel<In, 64><<<grid, block, 0, s>>>(p, dO, dsf, g, ws); break;
    case 128: recurrent_bwd_kernel<In, 128><<<grid, block, 0, s>>>(p, dO, dsf, g, ws); break;
    default: return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace

size_t bwd_workspace_bytes(const Problem& p) {
  return size_t(p.B * p.H) * size_t(bwd_layout(p.T, p.dk, p.dv).per_head) * sizeof(float);
}

int launch_recurrent_bwd(const Problem& p, const void* d_o, const float* dsf, const GradPtrs& g,
                         void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* w = static_cast<float*>(ws);
  return p.dtype == GDN_DTYPE_BF16 ? launch_in<uint16_t>(p, d_o, dsf, g, w, s)
                                   : launch_in<float>(p, d_o, dsf, g, w, s);
}

}  // namespace gdn
