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
