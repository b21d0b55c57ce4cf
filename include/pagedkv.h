/*
 * pagedkv.h -- C ABI of the paged KV-cache data plane for MI355X (gfx950).
 *
 * Five operations of the data plane the Nano-vLLM write-ups describe, plus
 * the host-side block manager that feeds them (declared further down):
 *
 *   pkv_store_kvcache             write each new token's K and V rows into the
 *                                 block-paged cache at its slot-mapping entry
 *   pkv_paged_decode_attention    one query token per sequence attending to its
 *                                 whole cached history through its block table
 *   pkv_store_and_decode          both of the above for one decode step, in one
 *                                 kernel
 *   pkv_topk_sample               temperature / top-k sampling of the next token
 *   pkv_varlen_prefill_attention  causal attention over packed variable-length
 *                                 prompts (cu_seqlens), keys read through block
 *                                 tables, so blocks shared by prefix caching are
 *                                 read in place
 *
 * Sources: "Nano-vLLM part 1" (neutree.ai, translated on blog.itpub.net):
 * section 4.1 (fixed-size blocks, 256 tokens by default), 4.2 (prefix caching
 * by per-block hashes and reference counts), 4.3 (CPU control plane, GPU data
 * plane; freed blocks are not zeroed), 5.2 (prefill packs sequences with
 * cumulative lengths; decode passes positions and slot mappings), 5.3 (decode
 * steps replayed as captured graphs).  "Nano-vLLM inference engine
 * architecture" (blog.hotdry.top): the PagedAttention section (slot_mapping
 * into a flat slot-indexed cache, the store_kvcache kernel) and the low-level
 * optimisation section (a varlen prefill call and a KV-cache decode call).
 *
 * Conventions for every call
 * --------------------------
 *  - Pointers named as device buffers must be device memory (hipMalloc or
 *    equivalent); bf16 buffers must be 16-byte aligned.  All bf16 tensors are
 *    dense row-major with the shapes stated.
 *  - KV cache layout: k_cache and v_cache are separate bf16 tensors of shape
 *    [num_blocks * block_size, num_kv_heads, head_dim]; slot s of a cache is
 *    row s, the token at offset o of physical block b lives in slot
 *    b * block_size + o.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work and returns; ordering between calls is stream order.  No
 *    call allocates device memory, synchronises, or reads device memory from
 *    the host, so all of them may be captured into a HIP graph.
 *  - The caller owns every buffer.  The library keeps no state apart from a
 *    thread-local error message.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns PKV_ERR_INVALID_ARG or PKV_ERR_UNSUPPORTED and enqueues
 *    nothing.  PKV_ERR_HIP reports a launch failure.  pkv_last_error() then
 *    describes the failure.
 *  - Contents of device metadata (slots, block ids, lengths) are NOT checked:
 *    out-of-range slots or block ids, two new tokens with one slot, a context
 *    longer than its block table, or a store into a block another sequence
 *    reads (a shared prefix block) are undefined behaviour.
 *  - head_dim must be 64 or 128; block_size a power of two >= 16.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,  /* null pointer, misalignment, inconsistent sizes */
  PKV_ERR_UNSUPPORTED = 2,  /* a size this build has no kernel for */
  PKV_ERR_HIP = 3           /* the HIP runtime refused the launch */
} pkv_status;

/*
 * Store: for each i < num_tokens with slot_mapping[i] >= 0,
 *   k_cache[slot_mapping[i]] = k[i]  and  v_cache[slot_mapping[i]] = v[i]
 * (hotdry.top, PagedAttention section: new keys and values written at their
 * slot-mapping offsets; "Nano-vLLM part 1", section 5.2: decode passes the
 * slot mapping).  A negative slot is a padding entry and is skipped; a slot
 * >= num_slots is skipped too (as in pkv_store_and_decode).  Rows of the
 * cache not named by the mapping keep their contents bit for bit.
 *
 *   k, v          device bf16 [num_tokens, num_kv_heads, head_dim]
 *   k_cache,
 *   v_cache       device bf16 [num_slots, num_kv_heads, head_dim], updated in place
 *   slot_mapping  device int32 [num_tokens]
 * num_tokens == 0 is a no-op.
 */
pkv_status pkv_store_kvcache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int64_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                             void* stream);

/*
 * Workspace the decode call needs for its split-context partial results, in
 * bytes (0 when one pass per sequence suffices).  `split_tokens` as for
 * pkv_paged_decode_attention.  Returns SIZE_MAX for invalid sizes.
 */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_context_len,
                                  int32_t split_tokens);

/* The number of context tokens one workgroup covers for these sizes when
 * split_tokens == 0 (automatic choice): the whole context (max_context_len
 * rounded up to 32) when one kv head's K and V of it fit in 512 KiB
 * (max_context_len * head_dim <= 131072); otherwise a multiple of 256 in
 * [256, 32768] that gives about 2048 workgroups.  Pieces of 4096 tokens or
 * more over at least 2048 workgroups run one workgroup per CU. */
int32_t pkv_decode_split_tokens(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len);

/*
 * Decode attention: for each sequence b and query head h, with
 * n = context_lens[b], g = h / (num_q_heads / num_kv_heads) and
 * K_j, V_j the rows of kv head g at slot
 *   block_tables[b][j / block_size] * block_size + j % block_size,
 *   out[b][h] = sum_j softmax_j(scale * q[b][h] . K_j) * V_j,  j = 0 .. n-1
 * ("Nano-vLLM part 1", sections 2.4, 4.1 and 5.2; hotdry.top, the KV-cache
 * decode call).  context_lens counts the token stored for this step.  A
 * sequence with n == 0 gets a zero row.  fp32 accumulation, bf16 result
 * rounded to nearest even.
 *
 *   out           device bf16 [batch, num_q_heads, head_dim]
 *   q             device bf16 [batch, num_q_heads, head_dim]
 *   block_tables  device int32 [batch, max_blocks_per_seq]; entries past a
 *                 sequence's last block are ignored (-1 by convention)
 *   context_lens  device int32 [batch]; a value outside [0, max_context_len]
 *                 is taken as the nearest end of that range
 *   max_context_len  host-side bound: context_lens[b] <= max_context_len <=
 *                 max_blocks_per_seq * block_size (sizes the launch; no device
 *                 read).  Tokens beyond it are never visited.  Workgroups take
 *                 the sequences longest first in batches of up to 2048 (the
 *                 result does not depend on the order).
 *   split_tokens  context tokens per workgroup: 0 = automatic, else a positive
 *                 multiple of 32.  Sequences longer than one split are
 *                 processed in several workgroups whose partial softmax states
 *                 are merged by log-sum-exp in a second kernel.
 *   workspace     device buffer of at least pkv_decode_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0); scratch, contents
 *                 undefined afterwards.
 * batch == 0 is a no-op.  Any num_q_heads / num_kv_heads ratio is accepted.
 */
pkv_status pkv_paged_decode_attention(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t batch,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t split_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Fused decode step: for each sequence b, store its new token (row b of k_new
 * / v_new) into cache slot slot_mapping[b] and attend q[b] over positions
 * 0 .. context_lens[b]-1, the last of which is that new token -- the result
 * of pkv_store_kvcache followed by pkv_paged_decode_attention, in one launch
 * (the cache image is the same bit for bit; the output differs at most in
 * fp32 rounding order, as the new token is folded into the softmax state
 * last) ("Nano-vLLM
 * part 1", section 5.2: a decode step hands the slot mapping and the context
 * lengths to the GPU; hotdry.top, PagedAttention section: the store kernel,
 * and the low-level section: the KV-cache decode call).  The new token is
 * attended from k_new / v_new, not re-read from the cache, so
 * slot_mapping[b] is expected to be the slot of position context_lens[b]-1 in
 * block_tables[b] (the attention result does not depend on it).
 *
 *   k_new, v_new  device bf16 [batch, num_kv_heads, head_dim]
 *   slot_mapping  device int32 [batch]; negative entries (padding) and
 *                 entries >= num_slots store nothing
 *   num_slots     rows of each cache (num_blocks * block_size)
 *   other arguments as for pkv_paged_decode_attention (workspace sized by
 *   pkv_decode_workspace_bytes); k_cache / v_cache are written.
 * A row with context_lens[b] == 0 still stores its token and gets a zero
 * output row.
 */
pkv_status pkv_store_and_decode(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t max_context_len, int64_t num_slots, float scale,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Bytes of device workspace pkv_varlen_prefill_attention needs for these
 * sizes (its work list: one 64-byte record per (sequence, query tile) pair
 * and the work-queue counters).  0 when there is nothing to do; SIZE_MAX for
 * invalid sizes.
 */
size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                   int32_t num_kv_heads);

/*
 * Variable-length prefill attention over packed sequences.  Sequence i owns
 * query rows cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1 (Lq_i of them) and key
 * positions 0 .. Lk_i-1, Lk_i = cu_seqlens_k[i+1] - cu_seqlens_k[i], read from
 * the cache through block_tables[i] ("Nano-vLLM part 1", section 5.2:
 * cumulative sequence lengths; hotdry.top, the varlen prefill call).  Keys of
 * a cached prefix are simply positions whose blocks other tables list too
 * (section 4.2).  With causal != 0, query row r sits at absolute position
 * (Lk_i - Lq_i) + r and attends keys 0 .. that position (so Lk_i >= Lq_i is
 * required); otherwise it attends all Lk_i keys.  Each query row is
 *   out[row][h] = sum_j softmax_j(scale * q[row][h] . K_j) * V_j
 * with the kv head of h as for decode.  The K/V of every key position,
 * including this step's tokens, must already be in the cache
 * (pkv_store_kvcache first).  Rows that see no key get zeros.
 *
 *   out           device bf16 [total_q, num_q_heads, head_dim]
 *   q             device bf16 [total_q, num_q_heads, head_dim]
 *   cu_seqlens_q  device int32 [num_seqs + 1], cu[0] = 0, non-decreasing, cu[num_seqs] = total_q
 *   cu_seqlens_k  device int32 [num_seqs + 1], as above over key counts
 *   block_tables  device int32 [num_seqs, max_blocks_per_seq]
 *   max_seqlen_q, max_seqlen_k   host-side bounds on Lq_i and Lk_i (size the
 *                 launch; max_seqlen_k <= max_blocks_per_seq * block_size)
 *   workspace     device buffer of at least pkv_prefill_workspace_bytes(...)
 *                 bytes, 16-byte aligned; rewritten by every call (calls that
 *                 share one workspace must not overlap in time), contents
 *                 undefined afterwards.
 * num_seqs == 0 or total_q == 0 is a no-op.
 */
pkv_status pkv_varlen_prefill_attention(void* out, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_k,
                                        const int32_t* block_tables, int32_t num_seqs,
                                        int64_t total_q, int32_t max_seqlen_q,
                                        int32_t max_seqlen_k, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_blocks_per_seq,
                                        float scale, int32_t causal, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Bytes of the fixed per-GPU scratch of pkv_varlen_prefill_attention_noalloc. */
#define PKV_PREFILL_NOALLOC_SCRATCH_BYTES ((size_t)2 << 20)

/*
 * pkv_varlen_prefill_attention without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It computes exactly what
 * pkv_varlen_prefill_attention computes (same checks, same kernels, the same
 * output bit for bit) and allocates nothing: its work list lives in a fixed
 * device array of PKV_PREFILL_NOALLOC_SCRATCH_BYTES bytes (2 MiB),
 * which each GPU the library runs on holds from the first call there until
 * the process ends.  Batches whose pkv_prefill_workspace_bytes(...) exceeds
 * that size are refused with PKV_ERR_UNSUPPORTED before anything is enqueued
 * (about 32,000 (sequence, query tile) pairs: some 1 million query rows at
 * 4 query heads per kv head, whose tiles hold 32 rows).  Every call on one GPU uses that GPU's one array: calls that may
 * overlap in time on one GPU (different streams, different host threads) race
 * and must not be issued; each call rewrites the array from the start, so
 * stale contents from an earlier call do not matter.  Arguments as for
 * pkv_varlen_prefill_attention.
 */
pkv_status pkv_varlen_prefill_attention_noalloc(void* out, const void* q, const void* k_cache,
                                                const void* v_cache, const int32_t* cu_seqlens_q,
                                                const int32_t* cu_seqlens_k,
                                                const int32_t* block_tables, int32_t num_seqs,
                                                int64_t total_q, int32_t max_seqlen_q,
                                                int32_t max_seqlen_k, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_blocks_per_seq,
                                                float scale, int32_t causal, void* stream);

/*
 * Next-token sampling with temperature and top-k ("Nano-vLLM part 1",
 * section 5.4: the logits over the vocabulary become one token by sampling,
 * the temperature reshaping softmax(logits / T); hotdry.top, configuration
 * section: top_k bounds the candidates per step).  For each row r:
 *   candidates: entries whose logit is >= the top_k-th largest logit of the
 *     row (ties at that value all kept; every entry when top_k <= 0 or
 *     top_k >= vocab), the order being that of the fp32 values with
 *     -0 below +0;
 *   tokens[r] = the candidate i maximising fl(fl(logits[r][i] * fl(1/T)) +
 *     gumbel[r][i]) (each operation rounded in fp32, ties to the smallest i),
 *     which draws from softmax(logits / T) restricted to the candidates when
 *     gumbel holds independent standard Gumbel noise (the Gumbel-max identity);
 *   temperature <= 0: tokens[r] = the first index of the row's maximum logit.
 *
 *   tokens   device int32 [rows]
 *   logits   device fp32 [rows, vocab], finite or -inf (no NaN)
 *   gumbel   device fp32 [rows, vocab] (may be NULL when temperature <= 0);
 *            only the candidates' entries are read
 * rows == 0 is a no-op.  vocab and rows must be below 2^31.
 */
pkv_status pkv_topk_sample(int32_t* tokens, const float* logits, const float* gumbel, int64_t rows,
                           int64_t vocab, int32_t top_k, float temperature, void* stream);

/* ------------------------------------------------------------------------
 * Control plane: the block manager (host memory only, no GPU call).
 *
 * It decides which cache blocks each sequence uses and hands the data plane
 * its block tables and slot mappings ("Nano-vLLM part 1", section 4: fixed-size
 * blocks (4.1), prefix caching through a hash -> block id map with reference
 * counts (4.2), CPU-side metadata, freed blocks not cleared (4.3); section 3.2:
 * preemption when no block is left).  A full block's hash covers its tokens
 * and the hash of the block before it; a new sequence reuses the cached blocks
 * of its longest cached block-aligned prefix (always leaving at least one
 * block to compute); free blocks are handed out oldest-freed first, and a
 * freed block keeps its cached content until it is handed out again.  Not
 * thread-safe: one caller at a time per manager.
 * ------------------------------------------------------------------------ */
typedef struct pkv_block_manager pkv_block_manager;

#define PKV_BM_NO_SPACE (-1) /* not enough free blocks; nothing was changed */
#define PKV_BM_ERR_ARG (-2)  /* invalid argument or unknown / duplicate sequence id */

/* A manager of num_blocks blocks of block_size tokens (NULL on bad sizes). */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size);
void pkv_bm_destroy(pkv_block_manager* m);

/* Blocks that are free (cached content or not). */
int32_t pkv_bm_num_free(const pkv_block_manager* m);

/* Admit sequence seq_id with its n prompt tokens (host int32 ids): reuse the
 * cached blocks of its prefix, take free blocks for the rest.  Returns the
 * number of leading tokens whose K/V are already cached (a multiple of
 * block_size; the prefill computes and stores tokens from there on), or
 * PKV_BM_NO_SPACE / PKV_BM_ERR_ARG. */
int32_t pkv_bm_allocate(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t n);

/* Append one generated token to seq_id (a new block when the last one is
 * full).  0, or PKV_BM_NO_SPACE (the caller preempts a sequence and retries)
 * or PKV_BM_ERR_ARG. */
int32_t pkv_bm_append(pkv_block_manager* m, int64_t seq_id, int32_t token);

/* Release seq_id's blocks (finished or preempted).  0 or PKV_BM_ERR_ARG. */
int32_t pkv_bm_free(pkv_block_manager* m, int64_t seq_id);

/* Tokens of seq_id, or PKV_BM_ERR_ARG. */
int32_t pkv_bm_seq_len(const pkv_block_manager* m, int64_t seq_id);

/* Writes seq_id's block table into out[0 .. max_blocks-1] (-1 past its last
 * block; out may be NULL) and returns its number of blocks, or
 * PKV_BM_ERR_ARG. */
int32_t pkv_bm_block_table(const pkv_block_manager* m, int64_t seq_id, int32_t* out,
                           int32_t max_blocks);

/* Slots of positions from .. to-1 of seq_id
 * (block_table[p / block_size] * block_size + p % block_size) into out;
 * returns to - from, or PKV_BM_ERR_ARG. */
int32_t pkv_bm_slots(const pkv_block_manager* m, int64_t seq_id, int32_t from, int32_t to,
                     int32_t* out);

/* Reference count of a block (sequences using it), or PKV_BM_ERR_ARG. */
int32_t pkv_bm_ref_count(const pkv_block_manager* m, int32_t block_id);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
