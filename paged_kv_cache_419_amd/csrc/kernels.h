// Launch entry points of the device kernels (host side, C++).  The C ABI in
// api.hip validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_store_kvcache(const void* k, const void* v, void* k_cache, void* v_cache,
                                const int32_t* slot_mapping, int64_t num_tokens,
                                int64_t num_slots, int32_t row_elems, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;   // [batch, Hq, n_split, D] when n_split > 1
  float* part_ml;  // [batch, Hq, n_split, 2]
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t group;        // query heads per kv head
  int32_t head_groups;  // ceil(group / 16): workgroups per kv head
  int32_t block_shift;  // log2(block_size)
  int32_t max_blocks_per_seq;
  int32_t split_tokens;
  int32_t n_split;
  int32_t max_context_len;
  int32_t work_order;   // 1: sequences longest first (batches up to 2048), 0: batch order
  int32_t order_shift;  // max_context_len >> order_shift < 256: length classes of the work order
  float scale_log2;     // scale * log2(e)
  // Fused store (all null / 0 otherwise): the new token of sequence b is row b
  // of k_new / v_new; it is attended from there and written to cache slot
  // slot_mapping[b] (skipped when outside [0, num_slots)).
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  int64_t num_slots;
  int32_t fused;
};

// Decode plan shared by the workspace query and the launch.
int32_t decode_auto_split(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_context_len);
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_tables;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int32_t group;
  int32_t block_shift;
  int32_t max_blocks_per_seq;
  int32_t max_seqlen_q;
  int32_t causal;
  float scale_log2;
  int64_t total_q;
};

// Workspace of the prefill launch: work queues and the list of (sequence,
// q tile) pairs, at most ceil(total_q / rows per workgroup) + num_seqs of them.
size_t prefill_workspace_bytes(int32_t num_seqs, int64_t total_q, int32_t group);
hipError_t launch_varlen_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream);

// Temperature / top-k sampling of one token per row of logits.
struct SampleArgs {
  const float* logits;  // [rows, vocab]
  const float* gumbel;  // [rows, vocab] standard Gumbel noise (read at the candidates)
  int32_t* tokens;      // [rows]
  int64_t rows, vocab;
  int32_t top_k;        // <= 0 or >= vocab: no restriction
  float inv_temperature;
  int32_t greedy;       // temperature <= 0: first maximum of the logits
};

hipError_t launch_topk_sample(const SampleArgs& a, hipStream_t stream);

}  // namespace pkv
