// store_kvcache: scatter each new token's K and V rows into the paged cache.
//
// "Nano-vLLM inference engine architecture" (blog.hotdry.top), PagedAttention
// section: the store kernel writes new keys and values at the offsets the slot
// mapping names inside the preallocated flat cache.  Here a token's row is
// Hkv * head_dim bf16 values (2 KiB at Hkv 8, d 128), moved as 16-byte pieces:
// one work item is one piece of K plus the same piece of V, and consecutive
// threads take consecutive pieces of a row, so every wave reads and writes whole
// contiguous rows.  A negative slot (padding entry) is skipped, and so is a
// slot at or past the end of the cache (the fused decode step does the same).
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kStoreThreads = 256;
// Pieces of K (and of V) per thread and loop pass.  One, with many small
// workgroups, was the fastest measured: 36k-token stores took 56 us against
// 59 (two per thread), 60 (four) and 65 (eight).
constexpr int kStoreUnroll = 1;

__global__ __launch_bounds__(kStoreThreads) void store_kvcache_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, u32x4* __restrict__ kc,
    u32x4* __restrict__ vc, const int32_t* __restrict__ slot_mapping, int64_t num_tokens,
    int64_t num_slots, int32_t pieces_per_row, int32_t tokens_per_block) {
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * tokens_per_block;
  const int64_t ntok = min(static_cast<int64_t>(tokens_per_block), num_tokens - tok0);
  const int32_t items = static_cast<int32_t>(ntok) * pieces_per_row;
  for (int32_t base = threadIdx.x; base < items; base += kStoreThreads * kStoreUnroll) {
    u32x4 kv[kStoreUnroll], vv[kStoreUnroll];
    int64_t dst[kStoreUnroll];
#pragma unroll
    for (int u = 0; u < kStoreUnroll; ++u) {
      const int32_t item = base + u * kStoreThreads;
      dst[u] = -1;
      if (item < items) {
        const int32_t t = item / pieces_per_row;
        const int32_t piece = item - t * pieces_per_row;
        const int64_t tok = tok0 + t;
        const int64_t slot = slot_mapping[tok];
        if (slot >= 0 && slot < num_slots) {
          const int64_t src = tok * pieces_per_row + piece;
          kv[u] = k[src];
          vv[u] = v[src];
          dst[u] = slot * pieces_per_row + piece;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kStoreUnroll; ++u) {
      if (dst[u] >= 0) {
        kc[dst[u]] = kv[u];
        vc[dst[u]] = vv[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_store_kvcache(const void* k, const void* v, void* k_cache, void* v_cache,
                                const int32_t* slot_mapping, int64_t num_tokens,
                                int64_t num_slots, int32_t row_elems, hipStream_t stream) {
  const int32_t pieces = row_elems / 8;  // 16-byte pieces of one token's row
  // kStoreUnroll pieces per thread once there are enough tokens; one token per
  // block at minimum so tiny batches still spread over the chip
  int64_t per_block = (static_cast<int64_t>(kStoreThreads) * kStoreUnroll) / pieces;
  if (per_block < 1) per_block = 1;
  if (num_tokens < 4096) per_block = (per_block + 3) / 4;
  if (per_block < 1) per_block = 1;
  const int64_t blocks = (num_tokens + per_block - 1) / per_block;
  hipLaunchKernelGGL(store_kvcache_kernel, dim3(static_cast<uint32_t>(blocks)),
                     dim3(kStoreThreads), 0, stream, static_cast<const u32x4*>(k),
                     static_cast<const u32x4*>(v), static_cast<u32x4*>(k_cache),
                     static_cast<u32x4*>(v_cache), slot_mapping, num_tokens, num_slots, pieces,
                     static_cast<int32_t>(per_block));
  return hipGetLastError();
}

}  // namespace pkv
