// Variable-length causal prefill attention over the paged cache, for gfx950.
//
// Sequences are packed by cumulative lengths ("Nano-vLLM part 1", section 5.2)
// and every key is read from the block-paged cache through the sequence's
// block table, so prefix blocks shared by prefix caching (section 4.2) are read
// in place ("Nano-vLLM inference engine architecture", the varlen prefill
// call).  Query row r of a sequence with Lq queries and Lk keys sits at
// absolute position (Lk - Lq) + r and, when causal, attends keys 0 .. that
// position.
//
// Work split.  A workgroup (4 waves) owns one (sequence, kv head, q tile).  Its
// waves cover up to four query heads of that kv head and 32 query rows each
// (4 heads x 32 rows at GQA ratio 4, 2 x 64 at ratio 2, 1 x 128 without GQA),
// so one K/V tile in LDS serves 128 (row, head) pairs.  Work items are ordered
// sequence, then q tile (latest first: those rows see the most keys), then kv
// head; workgroups go round-robin to the 8 XCDs, so with 8 | Hkv every XCD
// serves one kv head, and the q tiles of a sequence run close together in
// time on that XCD: the sequence's K/V for that head (and a shared prefix)
// stay in the XCD's L2 instead of being read from HBM once per q tile.
//
// Pipeline.  K and V tiles of 64 keys go straight from HBM into LDS with the
// gfx950 direct-to-LDS loads (global_load_lds_dwordx4), double-buffered: the
// next tile's loads are in flight while the current tile is computed.  Rows
// are stored with XOR-swizzled 16-byte chunks so that both the K operand reads
// and the transposing V reads are free of bank conflicts.  Key rows past Lk
// are redirected to key Lk - 1 (a live row), so stale or poisoned slots are
// never read; their scores are masked.
//
// Matrix cores.  Each wave computes S^T[key][row] = K Q^T on 32x32x16 bf16
// MFMAs with Q^T held in registers.  In that output layout a lane holds 32
// scores of one query row, so the online softmax needs a single cross-lane
// exchange per tile, and the probabilities already sit in the B-operand layout
// of O^T[d][row] += V^T P^T, whose V^T operand comes from ds_read_b64_tr_b16.
// fp32 accumulation; probabilities are rounded to bf16 for the second product.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfStages = 2;  // K/V tiles resident in LDS: the current one + 1 in flight
constexpr int kPfKeys = 64;  // keys per tile
constexpr int kPfKB = kPfKeys / 32;  // 32-key MFMA blocks per tile
constexpr int kPfU = kPfKeys / 16;   // 16-key k-blocks of the PV product per tile
constexpr int kPfRows = 32;  // query rows per wave (the N side of a 32x32 MFMA)
constexpr float kRescaleSlack = 8.f;  // log2 headroom of the lazy softmax rescale
constexpr unsigned short kSlackBf16Bits = 0x4380;  // bf16 bit pattern of 2^kRescaleSlack

template <int D>
struct PrefillShape {
  static constexpr int KS = D / 16;                 // k-steps of S^T = K Q^T
  static constexpr int DC = D / 32;                 // 32-row blocks of O^T
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int ROWB = D * 2;                // LDS bytes per key row
  static constexpr int TILE = kPfKeys * ROWB;       // one K (or V) tile
  static constexpr int RPL = kWave / CH;            // rows per wave-wide direct load
  static constexpr int LOADS = kPfKeys / kPfWaves / RPL;  // per wave, per tensor, per tile
};

// Chunk position of 16-byte chunk c of key row r in LDS (an involution in c).
// K: 16 consecutive rows read at one chunk hit 16 distinct bank groups.
// V: 4 consecutive rows x 4 consecutive chunks (one transposing read) hit 16.
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

struct SeqView {
  const uint16_t* kc;  // k_cache + g * D (elements)
  const uint16_t* vc;
  const __attribute__((address_space(4))) int32_t* bt;
  int lk;
  int shift;
  uint32_t row_bytes;
};

// Each wave loads rows 16 * wave .. 16 * wave + 15 of every K and V tile.
// Those 16 rows lie in one cache block (blocks hold >= 16 tokens and the rows
// start at a multiple of 16), so one block-table entry addresses them.
constexpr int kPfWaveRows = kPfKeys / kPfWaves;

// Block-table entry of this wave's rows of the tile starting at key k0 (a
// scalar load; issued one tile ahead of its use).
__device__ __forceinline__ int64_t tile_block(const SeqView& sv, int k0, int wave) {
  return sv.bt[min(k0 + wave * kPfWaveRows, sv.lk - 1) >> sv.shift];
}

// Per-lane byte offsets, inside a block, of this wave's direct-to-LDS loads of
// one tile, relative to the wave's first row: lane (row rr = lane / CH of
// load e, LDS position p = lane % CH) reads the chunk stored at p.  Only the
// offsets of load 0 are kept: load e reads rows e * RPL further on, and its
// K swizzle differs from load 0's by 4e in the chunk index (the row bits the
// swizzle takes from e sit above those it takes from the lane), i.e. by
// 64 e in the byte offset; the V swizzle does not depend on e.
template <int D>
struct TileLoadOffsets {
  uint32_t k;
  uint32_t v;
  __device__ __forceinline__ uint32_t koff(int e) const { return k ^ (64u * e); }
  __device__ __forceinline__ uint32_t voff(int) const { return v; }
};

template <int D>
__device__ __forceinline__ TileLoadOffsets<D> tile_load_offsets(int lane, int wave, uint32_t row_bytes) {
  using S = PrefillShape<D>;
  static_assert(S::LOADS * 4 <= S::CH, "swizzle step of load e stays inside the row");
  TileLoadOffsets<D> t;
  const int rel = lane / S::CH;             // row inside the wave's 16, load 0
  const int rr = wave * kPfWaveRows + rel;  // row inside the tile
  const int p = lane % S::CH;
  t.k = rel * row_bytes + 16 * (p ^ kswz<D>(rr));
  t.v = rel * row_bytes + 16 * (p ^ vswz<D>(rr));
  return t;
}

// This wave's share of one K/V tile: buffer descriptors that start at the
// wave's first row in the cache and end after its last live row (key < Lk),
// so the loads of rows past Lk fetch nothing and leave zeros in LDS (their
// scores are masked, and zero V rows add nothing); with no live row, or no
// tile to load, nothing is fetched at all.  kdst / vdst: the wave's first
// LDS row in the slot.
struct DmaJob {
  u32x4 kd;
  u32x4 vd;
  lds_bytes kdst;
  lds_bytes vdst;
  uint32_t row_bytes;
};

// blk is tile_block(sv, k0, wave); live = false for "nothing to load".
template <int D>
__device__ __forceinline__ DmaJob dma_job(const SeqView& sv, int64_t blk, int k0, int wave, bool live,
                                          lds_bytes kdst, lds_bytes vdst) {
  using S = PrefillShape<D>;
  const int r0 = k0 + wave * kPfWaveRows;
  const int nlive = live ? max(0, min(kPfWaveRows, sv.lk - r0)) : 0;
  const uint32_t nbytes = nlive > 0 ? (nlive - 1) * sv.row_bytes + S::ROWB : 0;
  const int64_t base =
      ((blk << sv.shift) + (r0 & ((1 << sv.shift) - 1))) * static_cast<int64_t>(sv.row_bytes);
  const char* kb = reinterpret_cast<const char*>(sv.kc) + (nlive > 0 ? base : 0);
  const char* vb = reinterpret_cast<const char*>(sv.vc) + (nlive > 0 ? base : 0);
  return DmaJob{rsrc_words(kb, nbytes), rsrc_words(vb, nbytes), kdst + wave * kPfWaveRows * S::ROWB,
                vdst + wave * kPfWaveRows * S::ROWB, sv.row_bytes};
}

// Load j of a DmaJob: the K loads first, then the V loads.
template <int D>
__device__ __forceinline__ void dma_one(const DmaJob& job, const TileLoadOffsets<D>& lo, int j) {
  using S = PrefillShape<D>;
  const int e = j % S::LOADS;
  const uint32_t step = static_cast<uint32_t>(e * S::RPL) * job.row_bytes;
  if (j < S::LOADS) {
    lds_dma16_buf(job.kd, lo.koff(e), step, job.kdst + e * S::RPL * S::ROWB);
  } else {
    lds_dma16_buf(job.vd, lo.voff(e), step, job.vdst + e * S::RPL * S::ROWB);
  }
}

template <int D>
__device__ __forceinline__ void dma_all(const DmaJob& job, const TileLoadOffsets<D>& lo) {
#pragma unroll
  for (int j = 0; j < 2 * PrefillShape<D>::LOADS; ++j) dma_one<D>(job, lo, j);
}

template <int D>
struct WaveState {
  u32x4 qb[PrefillShape<D>::KS];      // B operand Q^T per k-step
  f32x16 o[PrefillShape<D>::DC];      // O^T accumulators
  f32x16 lsum;                        // row sums of the bf16 weights (every element of a lane's column alike)
  float m;                            // running reference max (log2 domain) of this lane's row
};

// Scheduling shape for a block of M MFMAs fed by NR LDS reads: the first
// AHEAD reads go out before any MFMA, then each MFMA is followed by the next
// reads (evenly spread), so AHEAD reads stay in flight and the matrix core
// does not wait on LDS latency.
template <int M, int NR, int AHEAD>
__device__ __forceinline__ void sched_reads_ahead() {
  static_assert(AHEAD <= NR, "more reads ahead than reads");
  constexpr int kRest = NR - AHEAD;
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  constexpr int kPer = (kRest + M - 1) / M > 0 ? (kRest + M - 1) / M : 1;
  constexpr int kFull = kRest / kPer;  // MFMAs followed by kPer reads
  constexpr int kRem = kRest % kPer;   // reads after MFMA number kFull
#pragma unroll
  for (int i = 0; i < M; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < kFull) {
      __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);
    } else if (i == kFull && kRem > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, kRem, 0);
    }
  }
}

// Weights exp2(s c - m) of one 64-key tile, rounded to bf16 and packed in
// the B-operand order of the PV product: 16-key block u = 2 kb + hb, k-slots
// 0..3 are keys 16u + 4h + i, k-slots 4..7 are keys 16u + 8 + 4h + i.
__device__ __forceinline__ void tile_weights(const f32x16 (&s)[kPfKB], u32x4 (&pb)[kPfU], float m, float c) {
#pragma unroll
  for (int kb = 0; kb < kPfKB; ++kb) {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = fast_exp2(__builtin_fmaf(s[kb][v], c, -m));
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int j = 2 * hb;
      pb[2 * kb + hb] = u32x4{pack_bf16x2(p[4 * j], p[4 * j + 1]), pack_bf16x2(p[4 * j + 2], p[4 * j + 3]),
                              pack_bf16x2(p[4 * j + 4], p[4 * j + 5]),
                              pack_bf16x2(p[4 * j + 6], p[4 * j + 7])};
    }
  }
}

// True when some packed bf16 weight is >= 2^kRescaleSlack (or inf / NaN):
// weights are non-negative, so their bit patterns order like their values;
// a packed 16-bit max folds two weights per instruction.
__device__ __forceinline__ bool weights_overflow(const u32x4 (&pb)[kPfU]) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mx = __builtin_bit_cast(u16x2, pb[0][0]);
#pragma unroll
  for (int u = 0; u < kPfU; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (u != 0 || e != 0) {
        const u16x2 v = __builtin_bit_cast(u16x2, pb[u][e]);
        mx = __builtin_elementwise_max(mx, v);
      }
  const unsigned short lim = kSlackBf16Bits;
  return (mx[0] >= lim) || (mx[1] >= lim);
}

// One 64-key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// The next tile's loads (job) go out one after every kGap MFMAs of the S
// product, so the waves of a CU do not all queue their loads on the memory
// pipeline at once right after the barrier.
template <int D>
__device__ __forceinline__ void compute_tile(WaveState<D>& w, lds_bytes kt, lds_bytes vt,
                                             const uint32_t (&kaddr)[PrefillShape<D>::KS],
                                             const uint32_t (&vaddr)[PrefillShape<D>::DC],
                                             int k0, int lim, bool need_mask, int h,
                                             float c, const DmaJob& job,
                                             const TileLoadOffsets<D>& lo) {
  using S = PrefillShape<D>;
  constexpr int kGap = kPfKB * S::KS / (2 * S::LOADS);
  static_assert(kGap >= 1 && kGap * 2 * S::LOADS == kPfKB * S::KS, "loads per MFMA slot");
  f32x16 s[kPfKB];
#pragma unroll
  for (int kb = 0; kb < kPfKB; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const u32x4 a = *(const lds_u32x4*)(kt + kaddr[ks] + kb * 32 * S::ROWB);
      s[kb] = mfma32x32x16(a, w.qb[ks], s[kb]);
      const int i = kb * S::KS + ks;
      if (i % kGap == kGap - 1) dma_one<D>(job, lo, i / kGap);
    }
  }
  // Keep several K operand reads in flight ahead of the MFMAs (LDS latency is
  // a few MFMA issue slots).
  sched_reads_ahead<kPfKB * S::KS, kPfKB * S::KS, 4>();
  // element 4j + i of s[kb] is key k0 + 32 kb + 8 j + 4 h + i of this lane's row
  if (need_mask) {
#pragma unroll
    for (int kb = 0; kb < kPfKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (k0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3) > lim) s[kb][v] = -INFINITY;
  }
  // Weights p = exp2(s c - m) against the running reference m.  m only has
  // to bound the scores loosely: the weights are consistent with the sums and
  // O whatever m is.  It is first set from the first tile's max; afterwards
  // the max is not computed at all: the tile's weights are checked instead,
  // and only when some weight reaches 2^kRescaleSlack (its row's max rose by
  // that much, rare after the first tiles) is m raised and O rescaled.
  if (__ballot(w.m == -INFINITY) != 0) {  // first tile of this wave
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < kPfKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    w.m = mx * c;
  }
  u32x4 pb[kPfU];
  tile_weights(s, pb, w.m, c);
  if (__ballot(weights_overflow(pb)) != 0) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < kPfKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(w.m, mx * c);
    const float alpha = fast_exp2(w.m - m_new);
    w.lsum *= alpha;
#pragma unroll
    for (int cb = 0; cb < S::DC; ++cb) w.o[cb] *= alpha;
    w.m = m_new;
    tile_weights(s, pb, w.m, c);
  }
  // row sums on the matrix cores: (all-ones)^T P^T
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int u = 0; u < kPfU; ++u) w.lsum = mfma32x32x16(ones, pb[u], w.lsum);
#pragma unroll
  for (int u = 0; u < kPfU; ++u) {
#pragma unroll
    for (int cb = 0; cb < S::DC; ++cb) {
      const uint2 lo = lds_read_tr16(vt + vaddr[cb] + 16 * u * S::ROWB);
      const uint2 hi = lds_read_tr16(vt + vaddr[cb] + (16 * u + 8) * S::ROWB);
      w.o[cb] = mfma32x32x16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[u], w.o[cb]);
    }
  }
  sched_reads_ahead<kPfU * S::DC + kPfU, 2 * kPfU * S::DC, 8>();
}

// Start of tile step t: wait for this wave's loads of tile t (younger tiles
// stay in flight) and for its LDS reads of tile t - 1, sync the workgroup,
// then issue tile t + kPfStages - 1 into the slot tile t - 1 has just freed.
// blk_next carries the block-table entry of that tile, looked up a step ahead.
template <int D>
__device__ __forceinline__ lds_bytes kslot_of(lds_bytes lbase, int t) {
  return lbase + (t % kPfStages) * (2 * PrefillShape<D>::TILE);
}
template <int D>
__device__ __forceinline__ lds_bytes vslot_of(lds_bytes lbase, int t) {
  return kslot_of<D>(lbase, t) + PrefillShape<D>::TILE;
}

template <int D>
__device__ __forceinline__ void tile_sync(int t, int n_tiles) {
  using S = PrefillShape<D>;
  switch (min(n_tiles - 1 - t, kPfStages - 2)) {  // tiles younger than t in flight
    case 2: barrier_after_loads<2 * 2 * S::LOADS>(); break;
    case 1: barrier_after_loads<1 * 2 * S::LOADS>(); break;
    default: barrier_after_loads<0>(); break;
  }
}

template <int D>
__device__ __forceinline__ void tile_sync_and_issue(const SeqView& sv, int t, int n_tiles, int wave,
                                                    const TileLoadOffsets<D>& lo,
                                                    int64_t& blk_next, lds_bytes lbase) {
  tile_sync<D>(t, n_tiles);
  const int tn = t + kPfStages - 1;
  if (tn < n_tiles) {
    dma_all<D>(dma_job<D>(sv, blk_next, tn * kPfKeys, wave, true, kslot_of<D>(lbase, tn),
                          vslot_of<D>(lbase, tn)), lo);
    if (tn + 1 < n_tiles) blk_next = tile_block(sv, (tn + 1) * kPfKeys, wave);
  }
}

template <int D>
__global__ __launch_bounds__(kPfThreads, 2) void varlen_prefill_kernel(
    PrefillArgs a, int32_t heads_per_wg, int32_t head_groups, int32_t rows_per_wg,
    int32_t q_tiles) {
  using S = PrefillShape<D>;
  // kPfStages slots, each a K tile followed by a V tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kPfStages * 2 * S::TILE];

  // item = ((seq * q_tiles + q tile rank) * Hkv + g) * head_groups + hg
  int64_t rest = blockIdx.x;
  const int hg = static_cast<int>(rest % head_groups);
  rest /= head_groups;
  const int g = static_cast<int>(rest % a.num_kv_heads);
  rest /= a.num_kv_heads;
  const int qtile = q_tiles - 1 - static_cast<int>(rest % q_tiles);
  const int seq = static_cast<int>(rest / q_tiles);

  const int q_start = a.cu_q[seq];
  const int lq = a.cu_q[seq + 1] - q_start;
  const int lk = a.cu_k[seq + 1] - a.cu_k[seq];
  const int off = lk - lq;
  const int r0 = qtile * rows_per_wg;
  if (r0 >= lq) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int m32 = lane & 31;
  const int h = lane >> 5;
  const int hl = hg * heads_per_wg + wave % heads_per_wg;
  const bool hvalid = hl < a.group;
  const int head = g * a.group + (hvalid ? hl : 0);
  const int rbase = r0 + (wave / heads_per_wg) * kPfRows;
  const int row = rbase + m32;

  SeqView sv;
  sv.row_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;
  sv.kc = static_cast<const uint16_t*>(a.k_cache) + static_cast<int64_t>(g) * D;
  sv.vc = static_cast<const uint16_t*>(a.v_cache) + static_cast<int64_t>(g) * D;
  sv.bt = (const __attribute__((address_space(4))) int32_t*)(a.block_tables) +
          static_cast<int64_t>(seq) * a.max_blocks_per_seq;
  sv.lk = lk;
  sv.shift = a.block_shift;
  const lds_bytes lbase = (lds_bytes)smem;
  auto kslot = [&](int t) { return kslot_of<D>(lbase, t); };
  auto vslot = [&](int t) { return vslot_of<D>(lbase, t); };

  const int last_row = min(r0 + rows_per_wg, lq) - 1;
  const int kend = a.causal ? min(lk, off + last_row + 1) : lk;
  const int n_tiles = (kend + kPfKeys - 1) / kPfKeys;
  const TileLoadOffsets<D> lo = tile_load_offsets<D>(lane, wave, sv.row_bytes);
  for (int t = 0; t < min(n_tiles, kPfStages - 1); ++t)
    dma_all<D>(dma_job<D>(sv, tile_block(sv, t * kPfKeys, wave), t * kPfKeys, wave, true, kslot(t), vslot(t)),
               lo);
  // block of the next tile to issue, looked up one tile ahead
  int64_t blk_next = n_tiles >= kPfStages ? tile_block(sv, (kPfStages - 1) * kPfKeys, wave) : 0;

  WaveState<D> w;
  // With a negative scale, negate Q (exact in bf16) and use |scale|, so the
  // exponent scale c is positive and the row max of raw scores is the max.
  const float c = fabsf(a.scale_log2);
  {
    const bool live = hvalid && row < lq;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(q_start + (live ? row : 0)) * a.num_q_heads + head) * D +
                         8 * h;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) w.qb[ks] = live ? ldg16(qp + 16 * ks) : u32x4{0, 0, 0, 0};
    // Q (and tile 0) must have landed before the loop: a wait the compiler
    // sees, so it adds none inside the loop, where the only vector loads are
    // the direct-to-LDS ones it does not track.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (a.scale_log2 < 0.f) {
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) w.qb[ks] ^= 0x80008000u;
    }
  }
#pragma unroll
  for (int cb = 0; cb < S::DC; ++cb) w.o[cb] = f32x16{};
  w.m = -INFINITY;
  w.lsum = f32x16{};

  // last visible key of this lane's row (padding rows borrow the last row's)
  const int lim = a.causal ? min(off + min(row, lq - 1), lk - 1) : lk - 1;
  // smallest such limit over this wave's rows, and the wave's largest
  const int lim_lo = a.causal ? min(off + min(rbase, lq - 1), lk - 1) : lk - 1;
  const int lim_hi = a.causal ? min(off + min(rbase + kPfRows - 1, lq - 1), lk - 1) : lk - 1;

  // Per-lane LDS byte offsets of the MFMA operands inside a tile.
  uint32_t kaddr[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks)
    kaddr[ks] = m32 * S::ROWB + 16 * ((2 * ks + h) ^ kswz<D>(m32));
  uint32_t vaddr[S::DC];
  {
    const int gi = lane & 15;        // lane inside its 16-lane group
    const int dsub = (lane >> 4) & 1;
    const int vr = 4 * h + (gi >> 2);  // key row (mod 16) this lane addresses
#pragma unroll
    for (int cb = 0; cb < S::DC; ++cb) {
      const int chunk = 4 * cb + 2 * dsub + ((gi & 3) >> 1);
      vaddr[cb] = vr * S::ROWB + 16 * (chunk ^ vswz<D>(vr)) + 8 * (gi & 1);
    }
  }

  // Tile loop over a ring of kPfStages LDS slots, one barrier per tile: each
  // wave waits for its own loads of tile t (younger tiles stay in flight) and
  // for its LDS reads of tile t - 1, the workgroup syncs, and only then is
  // tile t + kPfStages - 1 issued into the slot tile t - 1 has just freed.
  // Tiles past lim_hi hold no key any row of this wave sees (they exist for
  // other row blocks of the workgroup); padding heads compute nothing.  The
  // computing tiles come first, in a loop of their own, so the accumulators
  // are updated unconditionally inside it.
  const int n_compute = hvalid ? min(n_tiles, lim_hi / kPfKeys + 1) : 0;
  int t = 0;
#pragma unroll 1
  for (; t < n_compute; ++t) {
    tile_sync<D>(t, n_tiles);
    const int k0 = t * kPfKeys;
    const bool need_mask = k0 + kPfKeys - 1 > lim_lo;
    const int tn = t + kPfStages - 1;
    // The next tile's loads ride along with this tile's MFMAs (with no next
    // tile they fetch nothing and zero the slot tile t - 1 has just freed).
    const DmaJob job = dma_job<D>(sv, blk_next, tn * kPfKeys, wave, tn < n_tiles, kslot(tn), vslot(tn));
    if (tn + 1 < n_tiles) blk_next = tile_block(sv, (tn + 1) * kPfKeys, wave);
    compute_tile<D>(w, kslot(t), vslot(t), kaddr, vaddr, k0, lim, need_mask, h, c, job, lo);
  }
#pragma unroll 1
  for (; t < n_tiles; ++t) tile_sync_and_issue<D>(sv, t, n_tiles, wave, lo, blk_next, lbase);
  // The last computing tile may have left zero-filling loads in flight: they
  // must land before the workgroup's LDS is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (!hvalid || row >= lq) return;
  const float lt = w.lsum[0];  // the sum over all keys of this lane's row
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* op = static_cast<uint16_t*>(a.out) +
                 (static_cast<int64_t>(q_start + row) * a.num_q_heads + head) * D + 4 * h;
#pragma unroll
  for (int cb = 0; cb < S::DC; ++cb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x16& ov = w.o[cb];
      const uint2 v = {pack_bf16x2(ov[4 * j] * inv, ov[4 * j + 1] * inv),
                       pack_bf16x2(ov[4 * j + 2] * inv, ov[4 * j + 3] * inv)};
      *reinterpret_cast<uint2*>(op + 32 * cb + 8 * j) = v;
    }
  }
}

}  // namespace

hipError_t launch_varlen_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int32_t heads_per_wg = (a.group % 4 == 0) ? 4 : ((a.group % 2 == 0) ? 2 : 1);
  const int32_t head_groups = a.group / heads_per_wg;
  const int32_t rows_per_wg = kPfRows * (kPfWaves / heads_per_wg);
  const int32_t q_tiles = (a.max_seqlen_q + rows_per_wg - 1) / rows_per_wg;
  const int64_t total =
      static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * head_groups * q_tiles;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(total));
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(varlen_prefill_kernel<128>, grid, dim3(kPfThreads), 0, stream, a,
                       heads_per_wg, head_groups, rows_per_wg, q_tiles);
  } else {
    hipLaunchKernelGGL(varlen_prefill_kernel<64>, grid, dim3(kPfThreads), 0, stream, a,
                       heads_per_wg, head_groups, rows_per_wg, q_tiles);
  }
  return hipGetLastError();
}

}  // namespace pkv
