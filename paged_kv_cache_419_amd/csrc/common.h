// Shared device helpers for the gfx950 kernels of the paged KV-cache data plane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: workgroups go round-robin to 8 accelerator dies
constexpr float kLog2e = 1.4426950408889634f;

// D = C + A * B on one 16x16x32 bf16 MFMA tile (fp32 accumulate).
// Lane l supplies A[l % 16][8 * (l / 16) + t] and B[8 * (l / 16) + t][l % 16]
// for t = 0..7, and receives C[4 * (l / 16) + i][l % 16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D = C + A * B on one 32x32x16 bf16 MFMA tile (fp32 accumulate).
// Lane l supplies A[l % 32][8 * (l / 32) + t] and B[8 * (l / 32) + t][l % 32]
// for t = 0..7, and receives C[8 * j + 4 * (l / 32) + i][l % 32] in element
// 4 * j + i (j, i = 0..3).
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// LDS pointers with the address space spelled out, so the compiler knows
// stores through them cannot touch global memory.
typedef __attribute__((address_space(3))) unsigned char* lds_bytes;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group,
// lane i addresses 4 consecutive 16-bit values that form row i / 4, columns
// 4 * (i % 4) .. +3 of a 4 x 16 block; lane j of the group receives column j
// (rows 0..3).
__device__ __forceinline__ uint2 lds_read_tr16(lds_bytes p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p));
}

// Direct-to-LDS load (gfx950 global_load_lds_dwordx4): every lane reads 16
// bytes at its own global address `src`; lane i's bytes land at LDS byte
// address `dst` + 16 * i (`dst` must be the same for the whole wave).  Issued
// from inline asm so that the compiler inserts no waits of its own for these
// loads; callers wait with barrier_after_loads.  M0 is saved and restored.
__device__ __forceinline__ void lds_dma16(const void* src, lds_bytes dst) {
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// The same barrier, written so the compiler sees the wait: it then knows that
// every vector-memory access it issued before, except the youngest N, has
// completed, and adds no waits of its own for them later.  The empty asm
// statements keep memory accesses from moving across.
template <int N>
__device__ __forceinline__ void barrier_after_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier once at most N vector-memory loads of this wave are still
// outstanding (direct-to-LDS loads included) and its LDS accesses are done:
// this wave's older loads have landed, younger ones stay in flight.  One asm statement with a memory
// clobber, so the compiler moves no memory access across it.
template <int N>
__device__ __forceinline__ void barrier_after_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Workgroup barrier once this wave's LDS accesses have completed.
__device__ __forceinline__ void barrier_after_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed pair of bf16 (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> bf16 bit pattern, round to nearest even.
__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Raw buffer descriptor over `num_bytes` bytes at `base`.  Loads at offsets
// past num_bytes return zeros without touching memory (hardware range check).
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data format, no swizzle

__device__ __forceinline__ buffer_rsrc make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(num_bytes),
                                           kRsrcWord3);
}

__device__ __forceinline__ u32x4 buffer_load16(buffer_rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0));
}

// The same descriptor as four scalar words, for inline asm.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(b), static_cast<uint32_t>(b >> 32) & 0xFFFFu, num_bytes,
               static_cast<uint32_t>(kRsrcWord3)};
}

// Direct-to-LDS 16-byte load through a raw buffer descriptor: lane i's 16
// bytes at byte voff + soff of the buffer go to LDS `dst` + 16 i (`dst` the
// same for the whole wave).  Dwords past the descriptor's num_records (soff
// included in the check) fetch nothing and write zeros.  Issued from inline
// asm, like lds_dma16, so the compiler adds no waits; M0 is saved and restored.
__device__ __forceinline__ void lds_dma16_buf(u32x4 desc, uint32_t voff, uint32_t soff, lds_bytes dst) {
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(desc), "s"(soff), "s"(lds_addr)
      : "memory");
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
