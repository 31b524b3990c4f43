// Device helpers shared by the gfx950 kernels: element conversion, vector loads,
// wave64 reductions and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bhalf8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

// ---- element conversion ------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(uint32_t(h) << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Input element types: float (fp32 I/O) or uint16_t holding bf16 bits.
template <typename In> struct IO;
template <> struct IO<float> {
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float x) { *p = x; }
};
template <> struct IO<uint16_t> {
  __device__ static __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void st(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

// Load N contiguous elements (N a multiple of 4) into fp32 registers. The address
// is aligned to 4 elements.
template <int N>
__device__ __forceinline__ void load_vec(const float* p, float* out) {
  static_assert(N % 4 == 0, "N multiple of 4");
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    float4 x = reinterpret_cast<const float4*>(p)[i];
    out[4 * i + 0] = x.x;
    out[4 * i + 1] = x.y;
    out[4 * i + 2] = x.z;
    out[4 * i + 3] = x.w;
  }
}
template <int N>
__device__ __forceinline__ void load_vec(const uint16_t* p, float* out) {
  static_assert(N % 4 == 0, "N multiple of 4");
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    uint2 x = reinterpret_cast<const uint2*>(p)[i];
    out[4 * i + 0] = __uint_as_float(x.x << 16);
    out[4 * i + 1] = __uint_as_float(x.x & 0xffff0000u);
    out[4 * i + 2] = __uint_as_float(x.y << 16);
    out[4 * i + 3] = __uint_as_float(x.y & 0xffff0000u);
  }
}

// Sum over the four lanes l, l^16, l^32, l^48 (every lane gets the total).
__device__ __forceinline__ float sum_over_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
// Max over the same four lanes with the gfx950 lane-swap instructions (no LDS):
// v_permlane32_swap pairs lane l with l^32 and v_permlane16_swap pairs l with l^16;
// the maximum of the two swapped registers is the pair's maximum in every lane.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
}

// Sum over all 64 lanes (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Sum and max over the eight lanes l ^ 8m (m = 0..7): DPP row_ror:8 pairs lane l with
// l ^ 8 inside each 16-lane row, then the four-group exchanges above.
__device__ __forceinline__ float sum_over_8_groups(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // lane ^ 8
  return sum_over_groups(x);                                                                       // ^ 16, ^ 32
}
__device__ __forceinline__ float max_over_8_groups(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  return max_over_groups(x);
}

// ---- GDN2 stabilisers --------------------------------------------------------------
// Per token and head of the asymmetric variant (GDN2-stability page, "The Spectral
// Norm", "Simple Strategy", "Modifying Itself"), with the norms of j and k folded
// into eta so that unit vectors are not required:
//   clip (mode 1)     D' = min(D, lim),  lim = 1 / rho,  rho = ||I - eta j k^T||_2
//                     = (e + sqrt(e^2 - 4 eta j^T k + 4)) / 2,  e = eta ||j|| ||k||
//   project (mode 2)  j' = s k + lam (j - s k),  s = j^T k / ||k||^2,
//                     c = eta j^T k,  g = max D,  tau = (c - 1) g + 1/g,
//                     lam = min(1, sqrt((tau^2 - c^2) / (eta^2 ||k||^2 ||j - s k||^2)))
// lam = 1 for a zero denominator (j parallel to k, or eta = 0); lam = 0 for
// tau^2 <= c^2 (the page's case without a solution, only reached with c < 0).
struct StabCoef {
  float lim, s, lam;  // D' = min(D, lim), j' = s k + lam (j - s k)
};
struct KJD {
  float k, j, d;
};

// Coefficients of one row whose channels are spread over several lanes: `at(i)`
// returns this lane's channel i (i < N) of k, j and D; `rsum` / `rmax` reduce over
// the lanes of the row. mode is uniform across the wave; 0 gives the identity.
template <int N, typename At, typename Sum, typename Max>
__device__ __forceinline__ StabCoef stab_coef(int mode, float eta, At at, Sum rsum, Max rmax) {
  StabCoef c{__builtin_inff(), 0.0f, 1.0f};
  if (mode == 0) return c;
  float jk = 0.0f, k2 = 0.0f, j2 = 0.0f, g = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const KJD x = at(i);
    jk += x.j * x.k;
    k2 += x.k * x.k;
    j2 += x.j * x.j;
    g = fmaxf(g, x.d);
  }
  jk = rsum(jk);
  k2 = rsum(k2);
  if (mode == 1) {
    j2 = rsum(j2);
    const float en = eta * sqrtf(j2) * sqrtf(k2);
    // en >= |eta j^T k| makes the radicand >= (en - 2)^2 >= 0; clamp rounding.
    const float rho = 0.5f * (en + sqrtf(fmaxf(en * en - 4.0f * eta * jk + 4.0f, 0.0f)));
    c.lim = 1.0f / rho;
    return c;
  }
  g = rmax(g);
  const float s = jk / k2;
  float p2 = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const KJD x = at(i);
    const float pe = x.j - s * x.k;
    p2 += pe * pe;
  }
  p2 = rsum(p2);
  const float cc = eta * jk;
  const float den = eta * eta * k2 * p2;  // ||eta ||k|| j||^2 - c^2 without cancellation
  // tau^2 - c^2 = (tau - c)(tau + c) = (1 - g)((1 + g)/g - c) (1 + g)(c + (1 - g)/g):
  // exactly 0 at g = 1 and no cancellation between tau^2 and c^2, where the square
  // root below is steepest.
  const float omg = 1.0f - g;
  const float num = omg * (1.0f + g) * ((1.0f + g) / g - cc) * (cc + omg / g);
  // fminf returns 1 for a NaN ratio, as for the zero denominator.
  c.s = s;
  c.lam = den <= 0.0f ? 1.0f : (num <= 0.0f ? 0.0f : fminf(1.0f, sqrtf(num / den)));
  return c;
}

__device__ __forceinline__ float stab_decay(const StabCoef& c, float d) { return fminf(d, c.lim); }
__device__ __forceinline__ float stab_j(const StabCoef& c, float k, float j) {
  return c.s * k + c.lam * (j - c.s * k);
}

// ---- MFMA wrappers -------------------------------------------------------------
// Every product below is a 16x16 output tile D += A B with A 16 x K and B K x 16,
// walked in 16-wide slices of K. Within a slice, lane l = i + 16 g (i = l % 16,
// g = l / 16) supplies the four A values A[i][4g .. 4g+3] and the four B values
// B[4g .. 4g+3][i]. The accumulator tile uses the same convention transposed:
// lane l holds D[4g + e][i], e = 0..3. So an accumulator tile of one product can be
// fed as the B slice of the next without moving data between lanes: the order of
// the summed index inside a slice is the same permutation on both operands.

// fp32: one slice = 4 MFMA 16x16x4 (K = 4 each, slot g holds k = 4g + e).
__device__ __forceinline__ float4v mma_slice_f32(const float a[4], const float b[4], float4v acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}

// fp16: two slices = one MFMA 16x16x32 (eight k values per lane: slice s0 in
// elements 0..3, slice s1 in elements 4..7).
__device__ __forceinline__ float4v mma_pair_f16(half8 a, half8 b, float4v acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ float4v mma_pair_bf16(bhalf8 a, bhalf8 b, float4v acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ half8 pack_f16(const float lo[4], const float hi[4]) {
  half8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (_Float16)lo[e];
    r[4 + e] = (_Float16)hi[e];
  }
  return r;
}

// Exact power of two that maps m into [2^target, 2^(target+1)) (1 for m == 0 or a
// non-finite m). Multiplying by it never rounds.
__device__ __forceinline__ float pow2_scale_for(float m, int target = 0) {
  if (!(m > 0.0f) || !(m < 3.0e38f)) return 1.0f;
  int e;
  frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
  const int x = min(max(target + 1 - e, -100), 100);
  return ldexpf(1.0f, x);
}

// Scale of one block of a column whose blocks are scaled separately and later
// brought to the column's common (smallest) scale: an all-zero block takes the
// largest scale so that it never sets the common one.
__device__ __forceinline__ float block_scale(float m, int target) {
  return m > 0.0f ? pow2_scale_for(m, target) : 0x1p100f;
}

}  // namespace gdn
