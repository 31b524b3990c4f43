// GDN2 stabilisers: token-wise transforms of the asymmetric variant's inputs that
// bound the spectral norm of its transition D (I - eta j k^T) (GDN2-stability page,
// "The Spectral Norm", "Simple Strategy", "Modifying Itself").
//
//   mode 1 (clip the decay)   D' = min(D, 1/rho),  rho = ||I - eta j k^T||_2
//   mode 2 (project j)        j' = s k + lam (j - s k),  s = j^T k / ||k||^2
//
// The formulas (norms folded into eta, the readings where the page gives no value)
// are in stab_coef; the same coefficients are applied inside the chunked and
// recurrent passes when gdn_args.stabilize asks for it.
//
// Both are HBM-bound streams (three dk-vectors and one scalar in, one dk-vector
// out per token and head). A row (one token and head) is spread over dk/4 adjacent
// lanes, four channels each, so a wave reads whole rows with 16-byte (fp32) or
// 8-byte (bf16) loads and reduces over the row with dk/4-lane butterflies.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off /= 2) x += __shfl_xor(x, off, 64);
  return x;
}

template <int LPR>
__device__ __forceinline__ float row_max(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off /= 2) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ void store4(float* p, const float x[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store4(uint16_t* p, const float x[4]) {
  uint2 u;
  u.x = uint32_t(f32_to_bf16(x[0])) | (uint32_t(f32_to_bf16(x[1])) << 16);
  u.y = uint32_t(f32_to_bf16(x[2])) | (uint32_t(f32_to_bf16(x[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

// One row per LPR = DK/4 lanes; grid-stride over rows. Every lane of a row takes the
// same trip count, so the butterflies only combine lanes that are active together.
template <typename In, int DK, int MODE>
__global__ __launch_bounds__(kThreads) void stabilize_kernel(const In* __restrict__ k,
                                                             const In* __restrict__ jv,
                                                             const In* __restrict__ D,
                                                             const In* __restrict__ eta,
                                                             In* out, int64_t rows) {
  constexpr int LPR = DK / 4;
  constexpr int RPB = kThreads / LPR;  // rows per block and pass
  const int c0 = (threadIdx.x % LPR) * 4;
  const int64_t stride = int64_t(gridDim.x) * RPB;
  for (int64_t r = int64_t(blockIdx.x) * RPB + threadIdx.x / LPR; r < rows; r += stride) {
    const int64_t base = r * DK + c0;
    float kk[4], jj[4], dd[4];
    load_vec<4>(k + base, kk);
    load_vec<4>(jv + base, jj);
    load_vec<4>(D + base, dd);
    const StabCoef sc = stab_coef<4>(
        MODE, IO<In>::ld(eta + r), [&](int i) { return KJD{kk[i], jj[i], dd[i]}; },
        [](float x) { return row_sum<LPR>(x); }, [](float x) { return row_max<LPR>(x); });
    float res[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) res[i] = MODE == 1 ? stab_decay(sc, dd[i]) : stab_j(sc, kk[i], jj[i]);
    store4(out + base, res);
  }
}

template <typename In, int MODE>
int launch_mode(const Problem& p, void* out, hipStream_t s) {
  const int64_t rows = p.B * p.T * p.H;
  const int lpr = int(p.dk / 4);
  const int64_t need = (rows + kThreads / lpr - 1) / (kThreads / lpr);
  const unsigned blocks = unsigned(need < (int64_t(1) << 20) ? need : (int64_t(1) << 20));
  const In* k = static_cast<const In*>(p.k);
  const In* j = static_cast<const In*>(p.j);
  const In* D = static_cast<const In*>(p.alpha);
  const In* e = static_cast<const In*>(p.eta);
  In* o = static_cast<In*>(out);
  switch (p.dk) {
    case 16: stabilize_kernel<In, 16, MODE><<<blocks, kThreads, 0, s>>>(k, j, D, e, o, rows); break;
    case 32: stabilize_kernel<In, 32, MODE><<<blocks, kThreads, 0, s>>>(k, j, D, e, o, rows); break;
    case 64: stabilize_kernel<In, 64, MODE><<<blocks, kThreads, 0, s>>>(k, j, D, e, o, rows); break;
    case 128: stabilize_kernel<In, 128, MODE><<<blocks, kThreads, 0, s>>>(k, j, D, e, o, rows); break;
    default: return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace

int launch_stabilize(const Problem& p, int mode, void* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == GDN_DTYPE_BF16)
    return mode == 1 ? launch_mode<uint16_t, 1>(p, out, s) : launch_mode<uint16_t, 2>(p, out, s);
  return mode == 1 ? launch_mode<float, 1>(p, out, s) : launch_mode<float, 2>(p, out, s);
}

}  // namespace gdn
