// Paged decode attention for gfx950.
//
// One query token per sequence attends to every cached position of its
// sequence, read through the block table ("Nano-vLLM part 1", sections 2.4,
// 4.1 and 5.2; "Nano-vLLM inference engine architecture", the KV-cache decode
// call).  The result is softmax(scale * q K^T) V per query head; paging only
// changes where K_j and V_j are read.
//
// Work split.  A workgroup (4 waves) owns one (sequence, kv head, group of up
// to 16 query heads, context split).  All query heads that share the kv head
// are computed together, so every K/V byte is read from HBM once whatever the
// GQA ratio.  Waves take interleaved 32-token tiles of the split; each keeps
// an online-softmax state (running max m, running sum l, unnormalised output)
// and the four states are merged through LDS at the end.  When a sequence has
// more than one split, each split writes its merged (m, l, output) to the
// workspace and a second kernel combines the splits by log-sum-exp.
//
// Memory pipeline.  The kernel is bound by HBM, so each wave keeps the next
// tile's K and V loads in flight while it computes the current one (two
// register buffers).  A 16-token half of a tile always lies inside one cache
// block, so it is addressed by one buffer descriptor whose base is the block's
// slot row (64-bit, in scalar registers) and whose size is the number of live
// tokens in the half: lanes of tokens past the context read zeros from the
// hardware range check, never the stale (possibly NaN) contents of unused
// slots.  Per-lane offsets are constant for the whole loop.  Two workgroups
// are resident per CU, which short contexts need to hide each workgroup's
// start-up; long pieces of work run one per CU, where they stream faster
// (launch_paged_decode).
//
// Matrix cores.  Scores are computed transposed, S^T[token][head] = K Q^T, on
// 16x16x32 bf16 MFMA tiles: K rows go straight from HBM into the A operand,
// the zero-padded query heads form B.  The output lane layout of S^T is the
// B-operand layout P^T needs for O^T[d][head] = V^T P^T, so probabilities
// never leave their lanes and every lane owns one head's softmax state.  V^T
// as the A operand needs V transposed: each wave writes its V tile row-major
// into a private LDS region (rows padded to keep the transposed reads free of
// bank conflicts) and reads it back with the gfx950 transposing LDS load
// (ds_read_b64_tr_b16), four tokens of one column per lane and instruction.
// Exponentials use exp2 with scale * log2(e) folded in.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDecTile = 32;  // tokens per wave iteration: two 16-token MFMA tiles

template <int D>
struct DecodeShape {
  static constexpr int KK = D / 32;                       // MFMA k-steps over head_dim
  static constexpr int DB = D / 16;                       // 16-row d-blocks of O^T
  static constexpr int CH = D / 8;                        // 16-byte pieces per head row
  static constexpr int ROWS_PER_LOAD = kWave / CH;        // V rows one wave load covers
  static constexpr int VLOADS = kDecTile / ROWS_PER_LOAD; // V loads per lane per tile
  static constexpr int VROW = D * 2 + 32;                 // staged V row stride (bytes)
  static constexpr int LDS_STAGE = kDecWaves * kDecTile * VROW;
  static constexpr int LDS_MERGE = (2 * kDecWaves * 16 + kDecWaves * 16 * D) * 4;
  static constexpr int LDS = LDS_STAGE > LDS_MERGE ? LDS_STAGE : LDS_MERGE;
};

// K and V registers of one 32-token tile.
template <int D>
struct TileRegs {
  u32x4 k[2][DecodeShape<D>::KK];
  u32x4 v[DecodeShape<D>::VLOADS];
};

// Block-table entries are read with scalar loads: the index is the same for
// the whole wave and the table is never written by the kernel.
typedef const __attribute__((address_space(4))) int32_t* gtable;


// Buffer descriptor of the 16 token rows of one kv head starting at logical
// position j (a multiple of 16) of a sequence; `live` of them are readable
// (0 = none: the loads return zeros and touch no memory).
template <int D>
__device__ __forceinline__ buffer_rsrc half_rsrc(const uint16_t* cache, gtable bt, int j, int shift,
                                                 int64_t row_elems, int g, int live) {
  const int bmask = (1 << shift) - 1;
  const int64_t blk = bt[j >> shift];
  const uint16_t* p = cache + ((blk << shift) + (j & bmask)) * row_elems + static_cast<int64_t>(g) * D;
  return make_rsrc(p, static_cast<uint32_t>(live) * static_cast<uint32_t>(row_elems * 2));
}

// Issue the K and V loads of the tile starting at j0 (no branches: halves
// past the context get empty descriptors whose loads return zeros).  `jsafe`
// is a position known to lie inside the context; its block is looked up
// instead of a block past the end.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* kc, const uint16_t* vc,
                                          gtable bt, int j0, int t1, int jsafe, int shift,
                                          int64_t row_elems, int g, uint32_t koff,
                                          const uint32_t (&voff)[DecodeShape<D>::VLOADS]) {
  using S = DecodeShape<D>;
  // (readfirstlane keeps these provably wave-uniform, so the descriptors stay
  // in scalar registers)
  const int live0 = __builtin_amdgcn_readfirstlane(max(0, min(16, t1 - j0)));
  const int live1 = __builtin_amdgcn_readfirstlane(max(0, min(16, t1 - j0 - 16)));
  const int ja = live0 > 0 ? j0 : jsafe;
  const int jb = live1 > 0 ? j0 + 16 : ja;
  const buffer_rsrc k0 = half_rsrc<D>(kc, bt, ja, shift, row_elems, g, live0);
  const buffer_rsrc k1 = half_rsrc<D>(kc, bt, jb, shift, row_elems, g, live1);
  const buffer_rsrc v0 = half_rsrc<D>(vc, bt, ja, shift, row_elems, g, live0);
  const buffer_rsrc v1 = half_rsrc<D>(vc, bt, jb, shift, row_elems, g, live1);
#pragma unroll
  for (int kk = 0; kk < S::KK; ++kk) {
    r.k[0][kk] = buffer_load16(k0, koff + 64 * kk);
    r.k[1][kk] = buffer_load16(k1, koff + 64 * kk);
  }
#pragma unroll
  for (int e = 0; e < S::VLOADS; ++e) {
    const bool second = e * S::ROWS_PER_LOAD >= 16;
    r.v[e] = buffer_load16(second ? v1 : v0, voff[e]);
  }
}

// The fused call's new token as a tile of its own: row 0 of the tile is this
// kv head's row of k_new / v_new (whose rows have the cache's row stride, so
// the per-lane offsets are the same); the other rows fall outside the
// descriptors and read as zeros.
template <int D>
__device__ __forceinline__ void load_new_token(TileRegs<D>& r, const uint16_t* kn, const uint16_t* vn,
                                               uint32_t koff, const uint32_t (&voff)[DecodeShape<D>::VLOADS]) {
  using S = DecodeShape<D>;
  const buffer_rsrc k0 = make_rsrc(kn, D * 2);
  const buffer_rsrc v0 = make_rsrc(vn, D * 2);
  const buffer_rsrc none = make_rsrc(kn, 0);
#pragma unroll
  for (int kk = 0; kk < S::KK; ++kk) {
    r.k[0][kk] = buffer_load16(k0, koff + 64 * kk);
    r.k[1][kk] = buffer_load16(none, koff + 64 * kk);
  }
#pragma unroll
  for (int e = 0; e < S::VLOADS; ++e) {
    const bool second = e * S::ROWS_PER_LOAD >= 16;
    r.v[e] = buffer_load16(second ? none : v0, voff[e]);
  }
}

template <int D>
__device__ __forceinline__ void compute_tile(const TileRegs<D>& r, const u32x4 (&qb)[DecodeShape<D>::KK],
                                             f32x4 (&o)[DecodeShape<D>::DB], float& m, float& lsum,
                                             lds_bytes vst, int j0, int t1, int lane,
                                             float scale_log2) {
  using S = DecodeShape<D>;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;

  f32x4 s[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    s[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk) s[hf] = mfma16x16x32(r.k[hf][kk], qb[kk], s[hf]);
  }

  // Online softmax in the log2 domain; lane owns head n16 for tokens
  // 16*hf + 4*q4 + i of the tile.
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[hf][i] *= scale_log2;
  if (j0 + kDecTile > t1) {  // partial tile: mask the tokens past the context
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + hf * 16 + 4 * q4 + i >= t1) s[hf][i] = -INFINITY;
  }
  float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  mt = wave_max_xor_16_32(mt);
  const float m_new = fmaxf(m, mt);
  float p[2][4];
  float ps = 0.f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[hf][i] = fast_exp2(s[hf][i] - m_new);
      ps += p[hf][i];
    }
  if (__ballot(m_new > m) != 0) {  // rescale only when some running max grew
    const float alpha = fast_exp2(m - m_new);
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < S::DB; ++c) o[c] *= alpha;
    m = m_new;
  }
  lsum += ps;
  const u32x4 pb = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                    pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};

  // Stage V row-major, then read V^T operands with the transposing LDS load:
  // k-slot t of lane quarter q4 is token 16*(t/4) + 4*q4 + t%4, the token
  // order of the probabilities above.
  wave_lds_sync();
  {
    const int piece = lane % S::CH;
    const int row0 = lane / S::CH;
#pragma unroll
    for (int e = 0; e < S::VLOADS; ++e)
      *(lds_u32x4*)(vst + (e * S::ROWS_PER_LOAD + row0) * S::VROW + 16 * piece) = r.v[e];
  }
  wave_lds_sync();
  const lds_bytes rd = vst + (4 * q4 + (n16 >> 2)) * S::VROW + 8 * (n16 & 3);
#pragma unroll
  for (int c = 0; c < S::DB; ++c) {
    const uint2 lo = lds_read_tr16(rd + 32 * c);
    const uint2 hi = lds_read_tr16(rd + 16 * S::VROW + 32 * c);
    o[c] = mfma16x16x32(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, o[c]);
  }
}

// Inclusive sum over the workgroup's threads (one value each), in thread
// order; `part` holds kDecWaves ints of LDS.  Ends with a workgroup barrier.
__device__ __forceinline__ int workgroup_inclusive_sum(int v, int* part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  if (lane == kWave - 1) part[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += part[w];
  __syncthreads();
  return v;
}

// Sequence at place r of the batch in work order, and its context length:
// by context length, longest first, in length classes of 2^order_shift
// tokens (at most 256 classes), batch order inside a class.  Every workgroup
// derives the same order from context_lens: a histogram of the classes, a
// prefix sum that finds the class holding place r, and a prefix count that
// finds the sequence inside it.  Long sequences then start first and the
// short ones fill the end of the launch, so no CU is left with one long
// sequence after the others are done.  context_lens is read once (the
// workgroup needs its sequence's length anyway): up to kHeld lengths per
// thread stay in registers, larger batches read theirs again.  Lengths are
// clamped to [0, max_context_len].
struct SeqPick {
  int b;
  int ctx;
};

__device__ SeqPick sequence_in_work_order(const DecodeArgs& a, int r) {
  constexpr int kClasses = 256;
  constexpr int kPerThread = kClasses / kDecThreads;  // consecutive classes of one thread
  static_assert(kPerThread * kDecThreads == kClasses, "classes split evenly over the threads");
  constexpr int kHeld = 4;
  __shared__ int hist[kClasses];
  __shared__ int part[kDecWaves];
  __shared__ int pick[4];
  const int tid = threadIdx.x;
  const int per = (a.batch + kDecThreads - 1) / kDecThreads;  // sequences of this thread: a range
  const int j0 = tid * per;
  const int j1 = min(j0 + per, a.batch);
  auto len_at = [&](int j) { return min(max(a.context_lens[j], 0), a.max_context_len); };
  auto cls_of = [&](int len) { return 255 - (len >> a.order_shift); };  // 0 for the longest class
  int held[kHeld];
#pragma unroll
  for (int e = 0; e < kHeld; ++e) held[e] = j0 + e < j1 ? len_at(j0 + e) : 0;
  auto len_of = [&](int j) { return j - j0 < kHeld ? held[j - j0] : len_at(j); };
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) hist[tid * kPerThread + k] = 0;
  __syncthreads();
  for (int j = j0; j < j1; ++j) atomicAdd(&hist[cls_of(len_of(j))], 1);
  __syncthreads();
  int cnt[kPerThread], own = 0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) own += cnt[k] = hist[tid * kPerThread + k];
  int run = workgroup_inclusive_sum(own, part) - own;  // places before this thread's classes
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    if (r >= run && r < run + cnt[k]) {
      pick[0] = tid * kPerThread + k;
      pick[1] = r - run;
    }
    run += cnt[k];
  }
  __syncthreads();
  const int want = pick[0], rank = pick[1];
  int mine = 0;
  for (int j = j0; j < j1; ++j) mine += cls_of(len_of(j)) == want;
  const int upto = workgroup_inclusive_sum(mine, part);
  if (rank >= upto - mine && rank < upto) {
    int k = rank - (upto - mine);
    for (int j = j0; j < j1; ++j) {
      const int len = len_of(j);
      if (cls_of(len) == want) {
        if (k == 0) {
          pick[2] = j;
          pick[3] = len;
        }
        --k;
      }
    }
  }
  __syncthreads();
  return SeqPick{pick[2], pick[3]};
}

// (second bound: at least two waves per SIMD, i.e. up to 256 registers per lane)
template <int D>
__global__ __launch_bounds__(kDecThreads, 2) void paged_decode_kernel(DecodeArgs a) {
  using S = DecodeShape<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS];

  // Work item order: split index slowest, then kv head (and head group),
  // then sequence, so the first splits of all sequences start first and the
  // workgroups running at one time cover as many sequences (cache blocks) as
  // possible; this measured ~0.8 % faster on long contexts than sequence-major
  // order, where one sequence's kv heads run side by side.  Within a kv head
  // the sequences go longest first (sequence_in_work_order): 6 % faster at
  // 256 contexts of 100-1024 tokens and 4 % at 512 of 4k-32k tokens than
  // batch order.  Batches above 2048 sequences keep batch order (each
  // workgroup would read all of context_lens).
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_kv_heads * a.head_groups;
  const int64_t lin = blockIdx.x;
  const int split = static_cast<int>(lin / pairs);
  const int64_t pair = lin - split * pairs;
  const int gy = static_cast<int>(pair / a.batch);
  const int place = static_cast<int>(pair % a.batch);
  const SeqPick sp = a.work_order
                         ? sequence_in_work_order(a, place)
                         : SeqPick{place, min(max(a.context_lens[place], 0), a.max_context_len)};
  const int b = __builtin_amdgcn_readfirstlane(sp.b);
  const int g = gy / a.head_groups;
  const int hg = gy - g * a.head_groups;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n16 = lane & 15;
  const int q4 = lane >> 4;

  const int ctx = __builtin_amdgcn_readfirstlane(sp.ctx);
  const int t0 = split * a.split_tokens;
  const int heads_here = min(16, a.group - hg * 16);
  const int h0 = g * a.group + hg * 16;
  uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(b) * a.num_q_heads + h0) * D;

  // Fused call: the last position (the new token) is attended from k_new /
  // v_new, and the workgroup of head group 0 whose split holds it stores this
  // kv head's new K and V rows into cache slot slot_mapping[b].  No workgroup
  // of the call reads that slot.
  const bool last_split = split == max(0, ctx - 1) / a.split_tokens;
  const int64_t nrow = (static_cast<int64_t>(b) * a.num_kv_heads + g) * D;
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + nrow;
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new) + nrow;
  if (a.fused && last_split && hg == 0 && threadIdx.x < 2 * (D / 8)) {
    const int64_t slot = a.slot_mapping[b];
    if (slot >= 0 && slot < a.num_slots) {
      const int piece = threadIdx.x % (D / 8);
      const bool is_v = threadIdx.x >= D / 8;
      uint16_t* dst = static_cast<uint16_t*>(const_cast<void*>(is_v ? a.v_cache : a.k_cache)) +
                      (slot * a.num_kv_heads + g) * D + 8 * piece;
      *reinterpret_cast<u32x4*>(dst) = ldg16((is_v ? vn : kn) + 8 * piece);
    }
  }

  if (t0 >= ctx) {
    if (a.n_split == 1) {  // empty context: a zero row
      for (int i = threadIdx.x; i < heads_here * D; i += kDecThreads) out[i] = 0;
    }
    return;
  }
  // end of the positions read from the cache (the fused call's new token is not)
  const int t1 = a.fused ? min(ctx - 1, t0 + a.split_tokens) : min(ctx, t0 + a.split_tokens);

  // B operand of S^T = K Q^T: lane holds 8 values of query head n16.
  u32x4 qb[S::KK];
  {
    const bool hvalid = n16 < heads_here;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(b) * a.num_q_heads + h0 + n16) * D + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk) qb[kk] = hvalid ? ldg16(qp + 32 * kk) : u32x4{0, 0, 0, 0};
  }

  f32x4 o[S::DB];
#pragma unroll
  for (int c = 0; c < S::DB; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  gtable bt = (gtable)(a.block_tables) + static_cast<int64_t>(b) * a.max_blocks_per_seq;
  const int shift = a.block_shift;
  const int64_t row_elems = static_cast<int64_t>(a.num_kv_heads) * D;
  const uint32_t row_bytes = static_cast<uint32_t>(row_elems * 2);
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  lds_bytes vst = (lds_bytes)smem + wave * kDecTile * S::VROW;
  // Per-lane byte offsets inside a half: K lane (n16, q4) reads token n16,
  // head-dim values 8*q4 + 32*kk; V lane reads 16-byte piece lane % CH of row
  // lane / CH (+ ROWS_PER_LOAD per load).
  const uint32_t koff = n16 * row_bytes + 16 * q4;
  uint32_t voff[S::VLOADS];
#pragma unroll
  for (int e = 0; e < S::VLOADS; ++e)
    voff[e] = ((e * S::ROWS_PER_LOAD + lane / S::CH) & 15) * row_bytes + 16 * (lane % S::CH);

  // Software pipeline over this wave's tiles (wave, wave + 4, ...): the loads
  // of tile i + 1 are in flight while tile i is computed.
  constexpr int kStride = kDecWaves * kDecTile;
  const int j_first = t0 + wave * kDecTile;
  const int n_tiles = j_first < t1 ? (t1 - j_first + kStride - 1) / kStride : 0;
  if (n_tiles > 0) {
    TileRegs<D> ra, rb;
    load_tile<D>(ra, kc, vc, bt, j_first, t1, t0, shift, row_elems, g, koff, voff);
    // (the scheduling barriers keep the compiler from hoisting the current
    // tile's math, and with it a wait for the loads, above the next loads)
    for (int it = 0; it < n_tiles; it += 2) {
      const int j = j_first + it * kStride;
      load_tile<D>(rb, kc, vc, bt, j + kStride, t1, t0, shift, row_elems, g, koff, voff);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile<D>(ra, qb, o, m, lsum, vst, j, t1, lane, a.scale_log2);
      if (it + 1 >= n_tiles) break;
      load_tile<D>(ra, kc, vc, bt, j + 2 * kStride, t1, t0, shift, row_elems, g, koff, voff);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile<D>(rb, qb, o, m, lsum, vst, j + kStride, t1, lane, a.scale_log2);
    }
  }

  if (a.fused && last_split && wave == kDecWaves - 1) {  // the new token, by one wave
    TileRegs<D> rn;
    load_new_token<D>(rn, kn, vn, koff, voff);
    compute_tile<D>(rn, qb, o, m, lsum, vst, ctx - 1, ctx, lane, a.scale_log2);
  }

  // Merge the four waves' states.
  lsum = wave_sum_xor_16_32(lsum);
  __syncthreads();
  float* mw = reinterpret_cast<float*>(smem);
  float* lw = mw + kDecWaves * 16;
  float* ow = lw + kDecWaves * 16;
  if (q4 == 0) {
    mw[wave * 16 + n16] = m;
    lw[wave * 16 + n16] = lsum;
  }
  if (n16 < heads_here) {  // padding heads of the MFMA tile are never read back
#pragma unroll
    for (int c = 0; c < S::DB; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ow[(wave * 16 + n16) * D + 16 * c + 4 * q4 + i] = o[c][i];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < heads_here * D; idx += kDecThreads) {
    const int hl = idx / D;
    const int d = idx - hl * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, mw[w * 16 + hl]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mv = mw[w * 16 + hl];
      if (mv != -INFINITY) {
        const float e = fast_exp2(mv - M);
        L += e * lw[w * 16 + hl];
        O += e * ow[(w * 16 + hl) * D + d];
      }
    }
    if (a.n_split == 1) {
      out[idx] = bf16_bits(L > 0.f ? O / L : 0.f);
    } else {
      const int64_t pidx = (static_cast<int64_t>(b) * a.num_q_heads + h0 + hl) * a.n_split + split;
      a.part_o[pidx * D + d] = O;
      if (d == 0) {
        a.part_ml[2 * pidx] = M;
        a.part_ml[2 * pidx + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of the per-split states: out = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s, M = max_s m_s (scores are in the log2 domain).
template <int D>
__global__ __launch_bounds__(D) void paged_decode_combine_kernel(DecodeArgs a) {
  const int h = static_cast<int>(blockIdx.x % static_cast<uint32_t>(a.num_q_heads));
  const int b = static_cast<int>(blockIdx.x / static_cast<uint32_t>(a.num_q_heads));
  const int d = threadIdx.x;
  const int ctx = min(max(a.context_lens[b], 0), a.max_context_len);  // as the split kernel takes it
  const int n = min(a.n_split, (ctx + a.split_tokens - 1) / a.split_tokens);
  const int64_t base = (static_cast<int64_t>(b) * a.num_q_heads + h) * a.n_split;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, a.part_ml[2 * (base + s)]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < n; ++s) {
    const float e = fast_exp2(a.part_ml[2 * (base + s)] - M);
    L += e * a.part_ml[2 * (base + s) + 1];
    O += e * a.part_o[(base + s) * D + d];
  }
  uint16_t* out = static_cast<uint16_t*>(a.out);
  out[(static_cast<int64_t>(b) * a.num_q_heads + h) * D + d] =
      bf16_bits((n > 0 && L > 0.f) ? O / L : 0.f);
}

}  // namespace

int32_t decode_auto_split(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_context_len) {
  // A context whose K and V for one kv head fit in 512 KiB (1024 tokens at
  // head_dim 128, 2048 at 64) is never split: the split's second kernel costs
  // more than the extra workgroups save (3-6 us per call at batches of 1-64,
  // measured), while longer contexts at small batches gain from splitting.
  if (static_cast<int64_t>(max_context_len) * head_dim <= 131072)
    return max_context_len > 32 ? (max_context_len + 31) / 32 * 32 : 32;
  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t pairs = static_cast<int64_t>(batch) * num_kv_heads * ((group + 15) / 16);
  // Aim for at least ~2048 workgroups (eight per CU) so the tail is short;
  // never split below 256 tokens and never let one workgroup walk more than
  // kMaxSplit tokens (longer contexts then spread over several CUs).  Long
  // pieces run one workgroup per CU (launch_paged_decode), where fewer, longer
  // pieces stream best: at 512 contexts of 4k-32k tokens whole contexts take
  // 2.5 % less time than 8192-token pieces, and at 64-256 such contexts the
  // rule below is 2-4 % faster than pieces capped at 8192 with two workgroups
  // per CU (measured).
  constexpr int64_t kWantWGs = 2048;
  constexpr int64_t kMaxSplit = 32768;
  int64_t n = pairs > 0 ? (kWantWGs + pairs - 1) / pairs : 1;
  if (n < 1) n = 1;
  int64_t split = (static_cast<int64_t>(max_context_len) + n - 1) / n;
  split = (split + 255) / 256 * 256;
  if (split < 256) split = 256;
  if (split > kMaxSplit) split = kMaxSplit;
  return static_cast<int32_t>(split);
}

// LDS a decode workgroup asks for when it is to run alone on its CU: more
// than half of the CU's 160 KiB, so a second one cannot be resident.
constexpr uint32_t kOnePerCuLds = 96 * 1024;
static_assert(DecodeShape<128>::LDS < kOnePerCuLds && DecodeShape<64>::LDS < kOnePerCuLds, "LDS pad");

hipError_t launch_paged_decode(const DecodeArgs& args, hipStream_t stream) {
  const DecodeArgs& a = args;
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.n_split) * a.num_kv_heads *
                                        a.head_groups * a.batch));
  // Pieces of 4096 tokens and more, over a grid of at least 2048 workgroups
  // (eight rounds of the CUs), run one workgroup per CU: the long streams
  // then go 1.6-4 % faster than with two per CU (measured at 64-512 contexts
  // of 4k-32k tokens).  Short pieces keep two per CU, which they need to hide
  // their start-up latency (256 contexts of 100-1024 tokens take 15 % longer
  // at one).  The extra dynamic LDS is never touched; it only keeps a second
  // workgroup off the CU.
  const bool one_per_cu = a.split_tokens >= 4096 && grid.x >= 2048;
  if (a.head_dim == 128) {
    const uint32_t pad = one_per_cu ? kOnePerCuLds - DecodeShape<128>::LDS : 0;
    hipLaunchKernelGGL(paged_decode_kernel<128>, grid, dim3(kDecThreads), pad, stream, a);
  } else {
    const uint32_t pad = one_per_cu ? kOnePerCuLds - DecodeShape<64>::LDS : 0;
    hipLaunchKernelGGL(paged_decode_kernel<64>, grid, dim3(kDecThreads), pad, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.n_split == 1) return err;
  const dim3 cgrid(static_cast<uint32_t>(a.num_q_heads) * static_cast<uint32_t>(a.batch));
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(paged_decode_combine_kernel<128>, cgrid, dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(paged_decode_combine_kernel<64>, cgrid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pkv
