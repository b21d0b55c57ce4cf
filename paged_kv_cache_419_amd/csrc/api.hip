// C ABI of the paged KV-cache data plane: argument checks, launch planning and
// error reporting.  Nothing here allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"
#include "pagedkv.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int s = 0;
  while ((int64_t{1} << s) < x) ++s;
  return s;
}

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

pkv_status check_heads(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID_ARG, "head counts must be positive (q %d, kv %d)", num_q_heads,
                num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", head_dim);
  return PKV_OK;
}

pkv_status check_block_size(int32_t block_size) {
  if (!pow2(block_size) || block_size < 16)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d: must be a power of two >= 16", block_size);
  return PKV_OK;
}

int32_t resolve_split(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t max_ctx, int32_t split) {
  return split > 0 ? split : pkv::decode_auto_split(batch, hq, hkv, d, max_ctx);
}

int32_t num_splits(int32_t max_ctx, int32_t split) {
  const int32_t n = (max_ctx + split - 1) / split;
  return n < 1 ? 1 : n;
}

// Scratch of pkv_varlen_prefill_attention_noalloc: the prefill work list and
// queue counters that pkv_varlen_prefill_attention keeps in the caller's
// workspace, in a fixed array of device memory.  Each GPU the library runs on
// holds its own copy until the process ends; host code reaches it only through
// the device address looked up once per device (the array's name is not a
// device address in host code).
constexpr size_t kScratchBytes = PKV_PREFILL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there, with that device current).
pkv_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "device %d beyond the %d devices the static scratch serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "pagedkv 0.1.0 gfx950"; }

pkv_status pkv_store_kvcache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int64_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                             void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  if (num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_kv_heads %d and head_dim %d must be positive",
                num_kv_heads, head_dim);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", head_dim);
  if (num_slots <= 0) return fail(PKV_ERR_INVALID_ARG, "num_slots must be positive");
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "bf16 buffers must be 16-byte aligned");
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (num_tokens > (int64_t{1} << 31) - 1 || row > (int64_t{1} << 20))
    return fail(PKV_ERR_UNSUPPORTED, "num_tokens or row size too large");
  return hip_status(pkv::launch_store_kvcache(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                              num_slots, static_cast<int32_t>(row),
                                              static_cast<hipStream_t>(stream)),
                    "store_kvcache launch");
}

int32_t pkv_decode_split_tokens(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return 0;
  return pkv::decode_auto_split(batch, num_q_heads, num_kv_heads, head_dim, max_context_len);
}

size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_context_len,
                                  int32_t split_tokens) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || split_tokens < 0 || num_q_heads % num_kv_heads)
    return SIZE_MAX;
  if (batch == 0) return 0;
  const int32_t split = resolve_split(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, split_tokens);
  const int32_t n = num_splits(max_context_len, split);
  if (n == 1) return 0;
  return static_cast<size_t>(batch) * num_q_heads * n * (head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks and launch shared by the decode call and the fused store + decode
// call (k_new / v_new / slot_mapping are null for the former).
pkv_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t batch,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                       float scale, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                       const void* k_new, const void* v_new, const int32_t* slot_mapping,
                       int64_t num_slots, bool fused, void* stream, const char* what) {
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if ((st = check_block_size(block_size)) != PKV_OK) return st;
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (max_context_len < 0 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len %d outside [0, max_blocks_per_seq * block_size]",
                max_context_len);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (split_tokens < 0 || split_tokens % 32)
    return fail(PKV_ERR_INVALID_ARG, "split_tokens %d: 0 or a positive multiple of 32", split_tokens);
  if (fused && num_slots <= 0) return fail(PKV_ERR_INVALID_ARG, "num_slots must be positive");
  if (batch == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (fused && (!k_new || !v_new || !slot_mapping))
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (fused && (!aligned16(k_new) || !aligned16(v_new))))
    return fail(PKV_ERR_INVALID_ARG, "bf16 buffers must be 16-byte aligned");
  if (static_cast<int64_t>(num_kv_heads) * head_dim * 2 * 16 >= (int64_t{1} << 31))
    return fail(PKV_ERR_UNSUPPORTED, "num_kv_heads %d too large for 32-bit in-block offsets",
                num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t head_groups = (group + 15) / 16;
  const int32_t split = resolve_split(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, split_tokens);
  const int32_t n = num_splits(max_context_len, split);
  if (static_cast<int64_t>(batch) * num_kv_heads * head_groups * n > (int64_t{1} << 30))
    return fail(PKV_ERR_UNSUPPORTED, "more than 2^30 decode work items");
  if (static_cast<int64_t>(batch) * num_q_heads > (int64_t{1} << 30))
    return fail(PKV_ERR_UNSUPPORTED, "batch * num_q_heads beyond the launch grid");
  const size_t need = pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                 max_context_len, split_tokens);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? size_t{0} : workspace_bytes);
  if (need > 0 && !aligned16(workspace))
    return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = need > 0 ? static_cast<float*>(workspace) +
                             static_cast<size_t>(batch) * num_q_heads * n * head_dim
                       : nullptr;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.group = group;
  a.head_groups = head_groups;
  a.block_shift = log2i(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.split_tokens = split;
  a.n_split = n;
  a.max_context_len = max_context_len;
  // every workgroup reads all of context_lens to find its place: kept to
  // batches whose lengths fit a few per thread
  a.work_order = batch <= 2048 ? 1 : 0;
  a.order_shift = 0;
  while ((max_context_len >> a.order_shift) > 255) ++a.order_shift;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.num_slots = num_slots;
  a.fused = fused ? 1 : 0;
  return hip_status(pkv::launch_paged_decode(a, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

extern "C" {

pkv_status pkv_paged_decode_attention(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t batch,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t split_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                     scale, split_tokens, workspace, workspace_bytes, nullptr, nullptr, nullptr, 0,
                     false, stream, "paged_decode_attention launch");
}

pkv_status pkv_topk_sample(int32_t* tokens, const float* logits, const float* gumbel, int64_t rows,
                           int64_t vocab, int32_t top_k, float temperature, void* stream) {
  if (rows < 0 || vocab <= 0) return fail(PKV_ERR_INVALID_ARG, "rows < 0 or vocab <= 0");
  if (!std::isfinite(temperature)) return fail(PKV_ERR_INVALID_ARG, "temperature is not finite");
  const bool greedy = temperature <= 0.f;
  const float inv_t = greedy ? 0.f : 1.0f / temperature;
  if (!std::isfinite(inv_t)) return fail(PKV_ERR_INVALID_ARG, "temperature too small: 1/T overflows");
  if (vocab > (int64_t{1} << 31) - 1 || rows > (int64_t{1} << 31) - 1)
    return fail(PKV_ERR_UNSUPPORTED, "rows or vocab beyond 2^31 - 1");
  if (rows == 0) return ok();
  if (!tokens || !logits || (!greedy && !gumbel)) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv::SampleArgs a{};
  a.logits = logits;
  a.gumbel = gumbel;
  a.tokens = tokens;
  a.rows = rows;
  a.vocab = vocab;
  a.top_k = top_k;
  a.inv_temperature = inv_t;
  a.greedy = greedy ? 1 : 0;
  return hip_status(pkv::launch_topk_sample(a, static_cast<hipStream_t>(stream)), "topk_sample launch");
}

pkv_status pkv_store_and_decode(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t max_context_len, int64_t num_slots, float scale,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                     scale, split_tokens, workspace, workspace_bytes, k_new, v_new, slot_mapping,
                     num_slots, true, stream, "store_and_decode launch");
}

size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                   int32_t num_kv_heads) {
  if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads)
    return SIZE_MAX;
  if (num_seqs == 0 || total_q == 0) return 0;
  return pkv::prefill_workspace_bytes(num_seqs, total_q, num_q_heads / num_kv_heads);
}

pkv_status pkv_varlen_prefill_attention(void* out, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_k,
                                        const int32_t* block_tables, int32_t num_seqs,
                                        int64_t total_q, int32_t max_seqlen_q,
                                        int32_t max_seqlen_k, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_blocks_per_seq,
                                        float scale, int32_t causal, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size argument");
  pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if ((st = check_block_size(block_size)) != PKV_OK) return st;
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (static_cast<int64_t>(max_seqlen_k) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PKV_ERR_INVALID_ARG, "max_seqlen_k %d exceeds max_blocks_per_seq * block_size",
                max_seqlen_k);
  if (causal && max_seqlen_q > max_seqlen_k)
    return fail(PKV_ERR_INVALID_ARG, "causal prefill needs max_seqlen_q <= max_seqlen_k");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !cu_seqlens_q || !cu_seqlens_k || !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "bf16 buffers must be 16-byte aligned");
  if (total_q > (int64_t{1} << 31) - 1)
    return fail(PKV_ERR_UNSUPPORTED, "total_q beyond 2^31 - 1 rows");
  // output rows of one sequence and head are addressed with 32-bit offsets
  if (static_cast<int64_t>(max_seqlen_q) * num_q_heads * head_dim * 2 > (int64_t{1} << 31))
    return fail(PKV_ERR_UNSUPPORTED, "max_seqlen_q * num_q_heads * head_dim beyond 2^30");
  // work items (pairs x kv heads x head groups) are counted in 32 bits
  if ((total_q / 32 + num_seqs + 1) * static_cast<int64_t>(num_q_heads) > (int64_t{1} << 30))
    return fail(PKV_ERR_UNSUPPORTED, "too many prefill work items");
  const size_t need = pkv_prefill_workspace_bytes(num_seqs, total_q, num_q_heads, num_kv_heads);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? size_t{0} : workspace_bytes);
  if (!aligned16(workspace)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  pkv::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.block_tables = block_tables;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.group = num_q_heads / num_kv_heads;
  a.block_shift = log2i(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seqlen_q = max_seqlen_q;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.total_q = total_q;
  return hip_status(pkv::launch_varlen_prefill(a, workspace, static_cast<hipStream_t>(stream)),
                    "varlen_prefill_attention launch");
}

pkv_status pkv_varlen_prefill_attention_noalloc(void* out, const void* q, const void* k_cache,
                                                const void* v_cache, const int32_t* cu_seqlens_q,
                                                const int32_t* cu_seqlens_k,
                                                const int32_t* block_tables, int32_t num_seqs,
                                                int64_t total_q, int32_t max_seqlen_q,
                                                int32_t max_seqlen_k, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_blocks_per_seq,
                                                float scale, int32_t causal, void* stream) {
  const size_t need = pkv_prefill_workspace_bytes(num_seqs, total_q, num_q_heads, num_kv_heads);
  void* ws = nullptr;
  if (need != SIZE_MAX && need > 0 && max_seqlen_q > 0) {
    if (need > kScratchBytes)
      return fail(PKV_ERR_UNSUPPORTED,
                  "this batch needs %zu bytes of prefill scratch; the static scratch holds %zu "
                  "(pass a workspace to pkv_varlen_prefill_attention instead)",
                  need, kScratchBytes);
    const pkv_status st = scratch_ptr(&ws);
    if (st != PKV_OK) return st;
  }
  // the same checks and kernels as the workspace entry point, on the scratch
  return pkv_varlen_prefill_attention(out, q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k,
                                      block_tables, num_seqs, total_q, max_seqlen_q, max_seqlen_k,
                                      num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, scale, causal, ws,
                                      ws ? kScratchBytes : 0, stream);
}

}  // extern "C"
