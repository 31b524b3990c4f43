// Token-sequential recurrence (decode path and the library's second, independent
// GPU route):
//     S <- Diag(alpha_t) S;  u = w_t - S^T b_t;  S <- S + a_t u^T;  o_t = S^T q_t
// with (a, b, w, alpha) built per variant from the raw inputs as in gdn.h.
//
// One wave owns a 16-column slice of one (batch, head) state. Lane l = j + 16 g
// holds column j of the slice for the DK/4 contiguous key rows starting at
// g * DK/4, in fp32 registers for the whole sequence. Sums over key rows are a
// per-lane partial sum and two butterfly exchanges across the four lane groups.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename In, int DK>
__global__ __launch_bounds__(64) void recurrent_kernel(Problem p, float* __restrict__ state) {
  constexpr int NR = DK / 4;  // key rows per lane
  const int lane = threadIdx.x;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int slices = int(p.dv / 16);
  const int64_t bh = blockIdx.x / slices;
  const int slice = int(blockIdx.x % slices);
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t dk = DK, dv = p.dv, H = p.H, n_h = p.n_h;
  const int col = slice * 16 + j;
  const int row0 = g * NR;

  float S[NR];
  float* st = state + (bh * dk + row0) * dv + col;
#pragma unroll
  for (int r = 0; r < NR; ++r) S[r] = st[int64_t(r) * dv];

  const In* q = static_cast<const In*>(p.q);
  const In* k = static_cast<const In*>(p.k);
  const In* v = static_cast<const In*>(p.v);
  const In* al = static_cast<const In*>(p.alpha);
  const In* be = static_cast<const In*>(p.beta);
  const In* bev = static_cast<const In*>(p.beta_v);
  const In* jv = static_cast<const In*>(p.j);
  const In* et = static_cast<const In*>(p.eta);
  In* o = static_cast<In*>(p.o);

  for (int64_t t = 0; t < p.T; ++t) {
    const int64_t th = (b * p.T + t) * H + h;  // (b, t, h) flat index
    float qv[NR];
    load_vec<NR>(q + th * dk + row0, qv);

    if (p.variant == GDN_VARIANT_DELTAPRODUCT) {
      const float gate = IO<In>::ld(al + th);
#pragma unroll
      for (int r = 0; r < NR; ++r) S[r] *= gate;
      for (int i = 0; i < n_h; ++i) {
        const int64_t ti = th * n_h + i;
        float kv[NR];
        load_vec<NR>(k + ti * dk + row0, kv);
        const float bi = IO<In>::ld(be + ti);
        const float wv = bi * IO<In>::ld(v + ti * dv + col);
        float pr = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) pr += kv[r] * S[r];
        const float u = wv - bi * sum_over_groups(pr);  // w - (beta k)^T S
#pragma unroll
        for (int r = 0; r < NR; ++r) S[r] += kv[r] * u;
      }
    } else {
      float a[NR], bb[NR], alpha[NR];
      float wv;
      if (p.variant == GDN_VARIANT_ASYM) {
        load_vec<NR>(k + th * dk + row0, a);
        load_vec<NR>(jv + th * dk + row0, bb);
        load_vec<NR>(al + th * dk + row0, alpha);
        const float e = IO<In>::ld(et + th);
        if (p.stabilize) {
          const StabCoef sc = stab_coef<NR>(
              p.stabilize, e, [&](int i) { return KJD{a[i], bb[i], alpha[i]}; },
              [](float x) { return sum_over_groups(x); }, [](float x) { return max_over_groups(x); });
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            alpha[r] = stab_decay(sc, alpha[r]);
            bb[r] = stab_j(sc, a[r], bb[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) bb[r] *= e;
        wv = e * IO<In>::ld(v + th * dv + col);
      } else {
        load_vec<NR>(k + th * dk + row0, a);
        if (p.variant == GDN_VARIANT_FG2) {
          float beta[NR];
          load_vec<NR>(be + th * dk + row0, beta);
          load_vec<NR>(al + th * dk + row0, alpha);
#pragma unroll
          for (int r = 0; r < NR; ++r) a[r] *= sqrtf(beta[r]);
          const In* bw = bev ? bev : be;
          const int64_t bw_dim = bev ? dv : dk;
          wv = sqrtf(IO<In>::ld(bw + th * bw_dim + col)) * IO<In>::ld(v + th * dv + col);
        } else {
          const float sb = sqrtf(IO<In>::ld(be + th));
          if (p.variant == GDN_VARIANT_KDA) {
            load_vec<NR>(al + th * dk + row0, alpha);
          } else {
            const float gm = IO<In>::ld(al + th);
#pragma unroll
            for (int r = 0; r < NR; ++r) alpha[r] = gm;
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) a[r] *= sb;
          wv = sb * IO<In>::ld(v + th * dv + col);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) bb[r] = a[r];
      }
      float pr = 0.0f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        S[r] *= alpha[r];
        pr += bb[r] * S[r];
      }
      const float u = wv - sum_over_groups(pr);
#pragma unroll
      for (int r = 0; r < NR; ++r) S[r] += a[r] * u;
    }

    float ov = 0.0f;
#pragma unroll
    for (int r = 0; r < NR; ++r) ov += qv[r] * S[r];
    ov = sum_over_groups(ov);
    if (g == 0) IO<In>::st(o + th * dv + col, ov);
  }

#pragma unroll
  for (int r = 0; r < NR; ++r) st[int64_t(r) * dv] = S[r];
}

// Same recurrence, 32 value columns per wave for dk >= 32 and dv a multiple of 32:
// lane l = j + 8 g holds columns 4 j .. 4 j + 3 of the slice (one 16-byte vector)
// for the DK/8 contiguous key rows starting at g * DK/8, so that each state row of
// the slice is one 128-byte line read and written by eight lanes. Sums over key
// rows are a per-lane partial sum and three exchanges across the eight lane groups.
template <typename In, int DK>
__global__ __launch_bounds__(64) void recurrent_wide_kernel(Problem p, float* __restrict__ state) {
  constexpr int NR = DK / 8;  // key rows per lane
  const int lane = threadIdx.x;
  const int j = lane & 7;
  const int g = lane >> 3;
  const int slices = int(p.dv / 32);
  const int64_t bh = blockIdx.x / slices;
  const int slice = int(blockIdx.x % slices);
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t dk = DK, dv = p.dv, H = p.H, n_h = p.n_h;
  const int col = slice * 32 + 4 * j;
  const int row0 = g * NR;

  float S[NR][4];
  float* st = state + (bh * dk + row0) * dv + col;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float4 x = *reinterpret_cast<const float4*>(st + int64_t(r) * dv);
    S[r][0] = x.x, S[r][1] = x.y, S[r][2] = x.z, S[r][3] = x.w;
  }

  const In* q = static_cast<const In*>(p.q);
  const In* k = static_cast<const In*>(p.k);
  const In* v = static_cast<const In*>(p.v);
  const In* al = static_cast<const In*>(p.alpha);
  const In* be = static_cast<const In*>(p.beta);
  const In* bev = static_cast<const In*>(p.beta_v);
  const In* jv = static_cast<const In*>(p.j);
  const In* et = static_cast<const In*>(p.eta);
  In* o = static_cast<In*>(p.o);

  // S <- S + a u^T with u = w - (b^T S) reduced over the key rows
  auto delta = [&](const float (&a)[NR], const float (&bb)[NR], const float (&w)[4]) __attribute__((always_inline)) {
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float pr = 0.0f;
#pragma unroll
      for (int r = 0; r < NR; ++r) pr += bb[r] * S[r][c];
      u[c] = w[c] - sum_over_8_groups(pr);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) S[r][c] += a[r] * u[c];
  };

  for (int64_t t = 0; t < p.T; ++t) {
    const int64_t th = (b * p.T + t) * H + h;  // (b, t, h) flat index
    float qv[NR];
    load_vec<NR>(q + th * dk + row0, qv);

    if (p.variant == GDN_VARIANT_DELTAPRODUCT) {
      const float gate = IO<In>::ld(al + th);
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) S[r][c] *= gate;
      for (int i = 0; i < n_h; ++i) {
        const int64_t ti = th * n_h + i;
        float kv[NR], bk[NR], w[4];
        load_vec<NR>(k + ti * dk + row0, kv);
        load_vec<4>(v + ti * dv + col, w);
        const float bi = IO<In>::ld(be + ti);
#pragma unroll
        for (int r = 0; r < NR; ++r) bk[r] = bi * kv[r];
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] *= bi;
        delta(kv, bk, w);  // (I - beta k k^T) S + beta k v^T
      }
    } else {
      float a[NR], bb[NR], alpha[NR], w[4];
      load_vec<4>(v + th * dv + col, w);
      if (p.variant == GDN_VARIANT_ASYM) {
        load_vec<NR>(k + th * dk + row0, a);
        load_vec<NR>(jv + th * dk + row0, bb);
        load_vec<NR>(al + th * dk + row0, alpha);
        const float e = IO<In>::ld(et + th);
        if (p.stabilize) {
          const StabCoef sc = stab_coef<NR>(
              p.stabilize, e, [&](int i) { return KJD{a[i], bb[i], alpha[i]}; },
              [](float x) { return sum_over_8_groups(x); }, [](float x) { return max_over_8_groups(x); });
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            alpha[r] = stab_decay(sc, alpha[r]);
            bb[r] = stab_j(sc, a[r], bb[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) bb[r] *= e;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] *= e;
      } else {
        load_vec<NR>(k + th * dk + row0, a);
        if (p.variant == GDN_VARIANT_FG2) {
          float beta[NR], bw[4];
          load_vec<NR>(be + th * dk + row0, beta);
          load_vec<NR>(al + th * dk + row0, alpha);
#pragma unroll
          for (int r = 0; r < NR; ++r) a[r] *= sqrtf(beta[r]);
          if (bev)
            load_vec<4>(bev + th * dv + col, bw);
          else
            load_vec<4>(be + th * dk + col, bw);  // dk == dv
#pragma unroll
          for (int c = 0; c < 4; ++c) w[c] *= sqrtf(bw[c]);
        } else {
          const float sb = sqrtf(IO<In>::ld(be + th));
          if (p.variant == GDN_VARIANT_KDA) {
            load_vec<NR>(al + th * dk + row0, alpha);
          } else {
            const float gm = IO<In>::ld(al + th);
#pragma unroll
            for (int r = 0; r < NR; ++r) alpha[r] = gm;
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) a[r] *= sb;
#pragma unroll
          for (int c = 0; c < 4; ++c) w[c] *= sb;
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) bb[r] = a[r];
      }
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) S[r][c] *= alpha[r];
      delta(a, bb, w);
    }

    float ov[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x = 0.0f;
#pragma unroll
      for (int r = 0; r < NR; ++r) x += qv[r] * S[r][c];
      ov[c] = sum_over_8_groups(x);
    }
    if (g == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) IO<In>::st(o + th * dv + col + c, ov[c]);
    }
  }

#pragma unroll
  for (int r = 0; r < NR; ++r)
    *reinterpret_cast<float4*>(st + int64_t(r) * dv) = make_float4(S[r][0], S[r][1], S[r][2], S[r][3]);
}

template <typename In>
int launch_recurrent_t(const Problem& p, float* state, hipStream_t s) {
  if (p.dk >= 32 && p.dv % 32 == 0) {  // 128-byte state rows per wave
    const dim3 grid(unsigned(p.B * p.H * (p.dv / 32)));
    switch (p.dk) {
      case 32: recurrent_wide_kernel<In, 32><<<grid, 64, 0, s>>>(p, state); break;
      case 64: recurrent_wide_kernel<In, 64><<<grid, 64, 0, s>>>(p, state); break;
      case 128: recurrent_wide_kernel<In, 128><<<grid, 64, 0, s>>>(p, state); break;
      default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
  }
  const dim3 grid(unsigned(p.B * p.H * (p.dv / 16)));
  switch (p.dk) {
    case 16: recurrent_kernel<In, 16><<<grid, 64, 0, s>>>(p, state); break;
    case 32: recurrent_kernel<In, 32><<<grid, 64, 0, s>>>(p, state); break;
    case 64: recurrent_kernel<In, 64><<<grid, 64, 0, s>>>(p, state); break;
    case 128: recurrent_kernel<In, 128><<<grid, 64, 0, s>>>(p, state); break;
    default: return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

// s_final <- s0 (or zero) for T == 0.
__global__ void state_copy_kernel(const float* __restrict__ s0, float* __restrict__ s1, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) s1[i] = s0 ? s0[i] : 0.0f;
}

}  // namespace

int launch_recurrent(const Problem& p, float* state, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.dtype == GDN_DTYPE_BF16 ? launch_recurrent_t<uint16_t>(p, state, s)
                                   : launch_recurrent_t<float>(p, state, s);
}

int launch_state_copy(const Problem& p, void* stream) {
  const int64_t n = p.B * p.H * p.dk * p.dv;
  if (p.s0 == p.s_final) return 0;
  const unsigned blocks = unsigned((n + 255) / 256);
  state_copy_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(p.s0, p.s_final, n);
  return int(hipGetLastError());
}

}  // namespace gdn
