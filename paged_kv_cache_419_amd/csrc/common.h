// Shared device helpers for the gfx950 kernels of the paged KV-cache data plane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// D = C + A * B on one 16x16x32 bf16 MFMA tile (fp32 accumulate).
// Lane l supplies A[l % 16][8 * (l / 16) + t] and B[8 * (l / 16) + t][l % 16]
// for t = 0..7, and receives C[4 * (l / 16) + i][l % 16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed pair of bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float wave_max_xor_16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Ordering of LDS accesses among the lanes of one wave (a wave-private region).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pkv
