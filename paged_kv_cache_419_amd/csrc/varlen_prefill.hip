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
// sequence (longest first), then q tile (latest first: those rows see the most
// keys), then kv head; workgroups go round-robin to the 8 XCDs, so with 8 | Hkv every XCD
// serves one kv head, and the q tiles of a sequence run close together in
// time on that XCD: the sequence's K/V for that head (and a shared prefix)
// stay in the XCD's L2 instead of being read from HBM once per q tile.
//
// Pipeline.  K and V tiles of 64 keys go straight from HBM into LDS with the
// gfx950 direct-to-LDS loads (global_load_lds_dwordx4), double-buffered: the
// next tile's loads are in flight while the current tile is computed.  Rows
// are stored with XOR-swizzled 16-byte chunks so that both the K operand reads
// and the transposing V reads are free of bank conflicts.  Key rows past Lk
// fall outside the wave's buffer descriptor, whose range ends after the last
// live row: they fetch nothing and arrive as zeros, so stale or poisoned slots
// are never read; their scores are masked.
//
// Matrix cores.  Each wave computes S^T[key][row] = K Q^T on 32x32x16 bf16
// MFMAs with Q^T held in registers.  In that output layout a lane holds 32
// scores of one query row, so the online softmax needs a single cross-lane
// exchange per tile, and the probabilities already sit in the B-operand layout
// of O^T[d][row] += V^T P^T, whose V^T operand comes from ds_read_b64_tr_b16.
// fp32 accumulation; probabilities are rounded to bf16 for the second product.
// A wave raises its priority while it issues MFMAs, so that of the two waves
// sharing a SIMD the one feeding the matrix core goes first (compute_tile).
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
constexpr float kSlackSum = 256.f;    // 2^kRescaleSlack
static_assert(kSlackSum == (1 << static_cast<int>(kRescaleSlack)), "2^slack");

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
// scalar load, issued at the end of a tile step and used in the next one: kept
// 32-bit until then, so nothing waits for it before the next step's barrier).
__device__ __forceinline__ int32_t tile_block(const SeqView& sv, int k0, int wave) {
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
  float lsum;                         // this lane's share of its row's weight sum (the other half: lane ^ 32)
  float m;                            // running reference max (log2 domain) of this lane's row
};

// Weights exp2(s c - m) of one 64-key tile, rounded to bf16 and packed in
// the B-operand order of the PV product: 16-key block u = 2 kb + hb, k-slots
// 0..3 are keys 16u + 4h + i, k-slots 4..7 are keys 16u + 8 + 4h + i.
// Returns the fp32 sum of this lane's 32 weights as rounded (the weights the
// PV product uses), taken two at a time by packed bf16 dot products with 1.
// (The dot product takes the bf16 pairs as built, not bit-cast back out of
// the packed words: hipcc 7.2 miscompiles the latter, reusing element 0.)
__device__ __forceinline__ float tile_weights(const f32x16 (&s)[kPfKB], u32x4 (&pb)[kPfU], float m, float c) {
  const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  float sum[2] = {0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kPfKB; ++kb) {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = fast_exp2(__builtin_fmaf(s[kb][v], c, -m));
    bf16x2 b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = bf16x2{static_cast<__bf16>(p[2 * e]), static_cast<__bf16>(p[2 * e + 1])};
      sum[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(b[e], one, sum[e & 1], false);
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      auto w = [&](int e) { return __builtin_bit_cast(uint32_t, b[4 * hb + e]); };
      pb[2 * kb + hb] = u32x4{w(0), w(1), w(2), w(3)};
    }
  }
  return sum[0] + sum[1];
}

// Largest s c over this lane's row (both lanes of the row: lane and lane ^ 32).
// c may be negative: the largest s c is then c times the smallest s.  Masked
// scores are -inf for c > 0 and +inf for c < 0, so they never win.
__device__ __forceinline__ float row_max_scaled(const f32x16 (&s)[kPfKB], float c) {
  float mx = s[0][0], mn = s[0][0];
#pragma unroll
  for (int kb = 0; kb < kPfKB; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      mx = fmaxf(mx, s[kb][v]);
      mn = fminf(mn, s[kb][v]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  mn = fminf(mn, __shfl_xor(mn, 32));
  return c > 0.f ? mx * c : mn * c;
}

// One 64-key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
//
// The instruction order is fixed by hand with scheduling fences (the
// compiler's own schedule waits for every LDS read right before the MFMA that
// uses it): the K operands are read kReadAhead MFMAs ahead, the two 32-key
// score blocks alternate so no MFMA waits on the one before it, and the next
// tile's loads (job) go out one after every kGap MFMAs of the S product, so
// the waves of a CU do not all queue their loads on the memory pipeline at
// once right after the barrier.  The first V^T operands are read before the
// softmax, so their latency hides behind it, and the rest stay kVAhead MFMAs
// ahead of the PV product.
//
// Wave priority: a wave issuing MFMAs is raised above one doing softmax
// arithmetic (2 during the S product, 3 during the PV product, 0 otherwise),
// so that when both waves of a SIMD have an instruction ready the matrix
// core is fed first and the other wave's VALU work fills its busy cycles.
// Measured 4-5 % faster on the prefix workload and 2.5-3 % on the varlen one
// than equal priorities (other levels, 1/3 or 3/3 or raising the softmax to
// 1, were within noise of this).
template <int D>
__device__ __forceinline__ void compute_tile(WaveState<D>& w, lds_bytes kt, lds_bytes vt,
                                             const uint32_t (&kaddr)[PrefillShape<D>::KS],
                                             const uint32_t (&vaddr)[PrefillShape<D>::DC],
                                             int k0, int lim, bool need_mask, int h,
                                             float c, float masked, const DmaJob& job,
                                             const TileLoadOffsets<D>& lo) {
  using S = PrefillShape<D>;
  static_assert(kPfKB == 2, "two interleaved score blocks");
  constexpr int kNS = kPfKB * S::KS;  // MFMAs of the S product
  constexpr int kNP = kPfU * S::DC;   // MFMAs of the PV product
  constexpr int kGap = kNS / (2 * S::LOADS);
  static_assert(kGap >= 1 && kGap * 2 * S::LOADS == kNS, "loads per MFMA slot");
  // (4 is ~1 % faster than 3 on the prefix workload with the wave priorities;
  // 2, 5 and V read-aheads of 2, 6 or 8 were no better)
  constexpr int kReadAhead = 4;
  constexpr int kVAhead = 4;
  static_assert(kReadAhead < kNS && kVAhead <= kNP, "read-ahead depth");

  u32x4 ka[kNS];
  auto kread = [&](int i) {  // operand of S MFMA i: key block i % 2, k-step i / 2
    ka[i] = *(const lds_u32x4*)(kt + kaddr[i >> 1] + (i & 1) * 32 * S::ROWB);
  };
  uint2 vlo[kNP], vhi[kNP];
  auto vread = [&](int j) {  // operand of PV MFMA j: 16-key block j / DC, d block j % DC
    const int u = j / S::DC, cb = j % S::DC;
    vlo[j] = lds_read_tr16(vt + vaddr[cb] + 16 * u * S::ROWB);
    vhi[j] = lds_read_tr16(vt + vaddr[cb] + (16 * u + 8) * S::ROWB);
  };

  f32x16 s[kPfKB];
#pragma unroll
  for (int i = 0; i < kReadAhead; ++i) kread(i);
  __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kNS; ++i) {
    if (i + kReadAhead < kNS) kread(i + kReadAhead);
    const int kb = i & 1, ks = i >> 1;
    s[kb] = mfma32x32x16(ka[i], w.qb[ks], ks == 0 ? f32x16{} : s[kb]);
    if (i % kGap == kGap - 1) dma_one<D>(job, lo, i / kGap);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < kVAhead; ++j) vread(j);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);

  // element 4j + i of s[kb] is key k0 + 32 kb + 8 j + 4 h + i of this lane's row
  if (need_mask) {
#pragma unroll
    for (int kb = 0; kb < kPfKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (k0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3) > lim) s[kb][v] = masked;
  }
  // Weights p = exp2(s c - m) against the running reference m.  m only has
  // to bound the scores loosely: the weights are consistent with the sums and
  // O whatever m is.  It is first set from the first tile's max; afterwards
  // the max is not computed at all: the tile's weight sums are checked
  // instead, and only when a lane's sum reaches 2^kRescaleSlack (so possibly
  // one of its weights did: its row's max rose by up to that much, rare after
  // the first tiles; inf and NaN also fail the check) is m raised to the
  // tile's max and O rescaled.
  if (__ballot(w.m == -INFINITY) != 0) w.m = row_max_scaled(s, c);  // first tile of this wave
  u32x4 pb[kPfU];
  float tsum = tile_weights(s, pb, w.m, c);
  if (__ballot(!(tsum < kSlackSum)) != 0) {
    const float m_new = fmaxf(w.m, row_max_scaled(s, c));
    const float alpha = fast_exp2(w.m - m_new);
    w.lsum *= alpha;
#pragma unroll
    for (int cb = 0; cb < S::DC; ++cb) w.o[cb] *= alpha;
    w.m = m_new;
    tsum = tile_weights(s, pb, w.m, c);
  }
  w.lsum += tsum;
  __builtin_amdgcn_s_setprio(3);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kNP; ++j) {
    if (j + kVAhead < kNP) vread(j + kVAhead);
    const int u = j / S::DC, cb = j % S::DC;
    w.o[cb] = mfma32x32x16(u32x4{vlo[j].x, vlo[j].y, vhi[j].x, vhi[j].y}, pb[u], w.o[cb]);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// LDS slot of ring position t: a K tile followed by a V tile.
template <int D>
__device__ __forceinline__ lds_bytes kslot_of(lds_bytes lbase, int t) {
  return lbase + (t % kPfStages) * (2 * PrefillShape<D>::TILE);
}
template <int D>
__device__ __forceinline__ lds_bytes vslot_of(lds_bytes lbase, int t) {
  return kslot_of<D>(lbase, t) + PrefillShape<D>::TILE;
}

// ---------------------------------------------------------------------------
// Work list and persistent workgroups.
//
// A work item is (sequence, q tile, kv head, head group).  A small plan
// kernel lists the (sequence, q tile) pairs that hold at least one query row,
// sequence by sequence (longest first) and latest q tile first, as records carrying what a
// workgroup needs to start on the pair; item i is pair i / ipp, kv head
// (i % ipp) % Hkv, head group (i % ipp) / Hkv (ipp = Hkv * head_groups).
// Items are dealt to eight queues, item i to queue i % 8, one queue per XCD:
// a workgroup takes items from the queue of the XCD it runs on (its hardware
// XCC id), so with 8 | Hkv each XCD serves one kv head, whatever the number
// of head groups, and the K/V it streams stay in its own L2.  A queue is a counter in the workspace
// bumped by one atomic per item; once its own queue is drained a workgroup
// takes items from the others.
//
// Exactly two workgroups per CU are launched, and each runs items back to
// back, so no workgroup waits on the hardware dispatcher, and the start of the
// next item overlaps the end of the current one: its record and its queue
// slot are fetched when the current item starts, its Q rows and its first K/V
// tile are loaded during the current item's last tile.  The LDS ring of K/V
// tiles simply runs on from one item into the next.

constexpr int kQueues = 8;        // one per XCD
constexpr int kQueueStride = 32;  // ints between queue counters (one 128-byte line each)
constexpr int kRecInts = 16;      // ints per pair record
constexpr int kWsCountersInts = kQueues * kQueueStride;
constexpr int kWsNPairsInt = kWsCountersInts;          // int index of the pair count
constexpr int kWsRecsInt = kWsCountersInts + 16;       // first record (64-byte aligned)
constexpr uint32_t kXccIdReg = (31u << 11) | 20u;      // s_getreg: HW_REG_XCC_ID, 32 bits

// Record of one (sequence, q tile) pair: sequence, q tile, first query row,
// Lq, Lk, and the block-table entries of tile 0's and tile 1's rows for waves
// 0..3 (so an item starts without reading the block table).
enum : int { kRecSeq = 0, kRecQtile, kRecQstart, kRecLq, kRecLk, kRecBlk0, kRecBlk1 = kRecBlk0 + 4 };
constexpr int kRecVecs = 4;  // 16-byte loads per record
static_assert(kRecBlk1 + 4 <= kRecVecs * 4 && kRecVecs * 4 <= kRecInts, "record layout");

struct PrefillSched {
  int* ws;               // workspace: queue counters, pair count, pair records
  int32_t heads_per_wg;  // query heads of one kv head per workgroup
  int32_t head_groups;   // group / heads_per_wg
  int32_t rows_per_wg;   // query rows per workgroup
};

// Entry of block table row `seq` holding key position k (clamped to the row,
// so the read stays inside the table whatever the sequence's length).
__device__ __forceinline__ int32_t block_entry(const PrefillArgs& a, int seq, int k) {
  return a.block_tables[static_cast<int64_t>(seq) * a.max_blocks_per_seq +
                        min(k >> a.block_shift, a.max_blocks_per_seq - 1)];
}

// Lists the pairs into the workspace (at most `cap` of them: the bound the
// workspace was sized for, which holds when cu_seqlens_q ends at total_q) and
// clears the queue counters.  Batches of up to 1024 sequences are listed
// longest first (by key count, ties in batch order), each sequence's q tiles
// together: the long items start first and short ones fill the end of the
// launch (~1 % faster at 64 sequences of 100-1024 tokens than batch
// order); their cu_seqlens and block-table entries are read once, all at
// the start, into LDS.  Larger batches keep batch order and read them where
// they are needed.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(PrefillArgs a, int32_t rows_per_wg,
                                                            int32_t cap, int* ws) {
  constexpr int kStaged = 1024;
  __shared__ int s_incl[1024];
  __shared__ int s_order[kStaged];  // place -> sequence, when staged
  __shared__ int4 s_seq[kStaged];   // q start, Lq, Lk of each sequence, when staged
  __shared__ int4 s_blk[kStaged];   // block-table entries of key rows 0, 16, 32, 48
  __shared__ int4 s_blk1[kStaged];  // and of rows 64, 80, 96, 112 (clamped to Lk - 1)
  __shared__ int s_total;
  const int tid = threadIdx.x;
  if (tid < kWsCountersInts) ws[tid] = 0;
  if (tid == 0) s_total = 0;
  const bool staged = a.num_seqs <= kStaged;
  auto seq_of = [&](int s) {
    const int q0 = a.cu_q[s];
    return int4{q0, a.cu_q[s + 1] - q0, a.cu_k[s + 1] - a.cu_k[s], 0};
  };
  auto blk_of = [&](int s) {
    return int4{block_entry(a, s, 0 * kPfWaveRows), block_entry(a, s, 1 * kPfWaveRows),
                block_entry(a, s, 2 * kPfWaveRows), block_entry(a, s, 3 * kPfWaveRows)};
  };
  // tile 1's rows, clamped to the last key as the attention kernel's block lookup does
  auto blk1_of = [&](int s, int lk) {
    auto e = [&](int w) { return block_entry(a, s, min(kPfKeys + w * kPfWaveRows, max(lk - 1, 0))); };
    return int4{e(0), e(1), e(2), e(3)};
  };
  if (staged) {
    if (tid < a.num_seqs) {
      const int4 sq = seq_of(tid);
      s_seq[tid] = sq;
      s_blk[tid] = blk_of(tid);
      s_blk1[tid] = blk1_of(tid, sq.z);
      s_incl[tid] = sq.z;
    }
    __syncthreads();
    if (tid < a.num_seqs) {
      const int lk = s_incl[tid];
      int place = 0;
      for (int j = 0; j < a.num_seqs; ++j) {
        const int o = s_incl[j];
        place += (o > lk) || (o == lk && j < tid);
      }
      s_order[place] = tid;
    }
  }
  __syncthreads();
  auto seq_at = [&](int i) { return staged ? s_order[i] : i; };
  auto info = [&](int s) { return staged ? s_seq[s] : seq_of(s); };
  for (int s0 = 0; s0 < a.num_seqs; s0 += 1024) {
    const int s = s0 + tid < a.num_seqs ? seq_at(s0 + tid) : a.num_seqs;
    const int lq = s < a.num_seqs ? info(s).y : 0;
    const int nqt = lq > 0 ? (lq + rows_per_wg - 1) / rows_per_wg : 0;
    s_incl[tid] = nqt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan of the pair counts
      const int v = tid >= d ? s_incl[tid - d] : 0;
      __syncthreads();
      s_incl[tid] += v;
      __syncthreads();
    }
    const int base = s_total;
    const int chunk = s_incl[1023];
    // one record per pair of this chunk of sequences, all threads together
    for (int r = tid; r < min(chunk, cap - base); r += 1024) {
      int lo = 0, hi = 1023;  // first thread whose inclusive count exceeds r
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_incl[mid] > r) hi = mid; else lo = mid + 1;
      }
      const int seq = seq_at(s0 + lo);
      const int first = s_incl[lo] - (lo > 0 ? s_incl[lo - 1] : 0);  // pairs of seq
      const int rank = r - (s_incl[lo] - first);
      const int4 sq = info(seq);
      const int4 bk = staged ? s_blk[seq] : blk_of(seq);
      const int4 bk1 = staged ? s_blk1[seq] : blk1_of(seq, sq.z);
      int4* rec = reinterpret_cast<int4*>(ws + kWsRecsInt + static_cast<int64_t>(base + r) * kRecInts);
      rec[0] = int4{seq, first - 1 - rank, sq.x, sq.y};
      rec[1] = int4{sq.z, bk.x, bk.y, bk.z};
      rec[2] = int4{bk.w, bk1.x, bk1.y, bk1.z};
      rec[3] = int4{bk1.w, 0, 0, 0};
    }
    __syncthreads();
    if (tid == 0) s_total = base + chunk;
    __syncthreads();
  }
  if (tid == 0) ws[kWsNPairsInt] = min(s_total, cap);
}

__device__ __forceinline__ int queue_size(int n_items, int q) {
  return n_items > q ? (n_items - q + kQueues - 1) / kQueues : 0;
}

// Item for slot `ticket` already taken in queue q0 (ticket < 0: none taken);
// when q0 is drained, takes an item from another queue.  -1 when all are.
__device__ int claim_item(int* counters, int n_items, int q0, int ticket) {
  if (ticket >= 0 && ticket < queue_size(n_items, q0)) return ticket * kQueues + q0;
  for (int k = 1; k < kQueues; ++k) {
    const int q = (q0 + k) & (kQueues - 1);
    const int size = queue_size(n_items, q);
    if (__atomic_load_n(&counters[q * kQueueStride], __ATOMIC_RELAXED) >= size) continue;
    const int j = atomicAdd(&counters[q * kQueueStride], 1);
    if (j < size) return j * kQueues + q;
  }
  return -1;
}

// One work item as seen by one wave (wave-uniform values).
struct Item {
  int seq, qtile, q_start, lq, lk, g, hg;
  int64_t blk0;  // block of this wave's rows of tile 0
  int32_t blk1;  // and of tile 1
};

// Every lane reads the same record (one request per wave), then the fields
// are made wave-uniform.
__device__ __forceinline__ void load_record(const int* ws, int pair, u32x4 (&r)[kRecVecs]) {
  const int* p = ws + kWsRecsInt + static_cast<int64_t>(pair) * kRecInts;
#pragma unroll
  for (int i = 0; i < kRecVecs; ++i) r[i] = ldg16(p + 4 * i);
}

__device__ __forceinline__ Item item_of(const PrefillSched& sc, int id, const u32x4 (&r)[kRecVecs], int wave,
                                        int ipp) {
  Item it;
  const int rem = id % ipp;
  const int hkv = ipp / sc.head_groups;
  it.g = rem % hkv;
  it.hg = rem / hkv;
  auto f = [&](int i) { return __builtin_amdgcn_readfirstlane(static_cast<int>(r[i >> 2][i & 3])); };
  it.seq = f(kRecSeq);
  it.qtile = f(kRecQtile);
  it.q_start = f(kRecQstart);
  it.lq = f(kRecLq);
  it.lk = f(kRecLk);
  const int b = wave == 0 ? f(kRecBlk0) : wave == 1 ? f(kRecBlk0 + 1) : wave == 2 ? f(kRecBlk0 + 2)
                                                                                   : f(kRecBlk0 + 3);
  it.blk0 = b;
  it.blk1 = wave == 0 ? f(kRecBlk1) : wave == 1 ? f(kRecBlk1 + 1) : wave == 2 ? f(kRecBlk1 + 2)
                                                                              : f(kRecBlk1 + 3);
  return it;
}

template <int D>
__device__ __forceinline__ SeqView seq_view(const PrefillArgs& a, const Item& it) {
  SeqView sv;
  sv.row_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;
  sv.kc = static_cast<const uint16_t*>(a.k_cache) + static_cast<int64_t>(it.g) * D;
  sv.vc = static_cast<const uint16_t*>(a.v_cache) + static_cast<int64_t>(it.g) * D;
  sv.bt = (const __attribute__((address_space(4))) int32_t*)(a.block_tables) +
          static_cast<int64_t>(it.seq) * a.max_blocks_per_seq;
  sv.lk = it.lk;
  sv.shift = a.block_shift;
  return sv;
}

// Number of K/V tiles the rows of an item's workgroup see.
__device__ __forceinline__ int item_tiles(const PrefillArgs& a, const PrefillSched& sc, const Item& it) {
  const int r0 = it.qtile * sc.rows_per_wg;
  const int last_row = min(r0 + sc.rows_per_wg, it.lq) - 1;
  const int kend = a.causal ? min(it.lk, it.lk - it.lq + last_row + 1) : it.lk;
  return (kend + kPfKeys - 1) / kPfKeys;
}

template <int D>
__global__ __launch_bounds__(kPfThreads, 2) void varlen_prefill_kernel(PrefillArgs a, PrefillSched sc) {
  using S = PrefillShape<D>;
  constexpr int kStores = S::DC * 4;  // output stores per wave and item
  // kPfStages slots, each a K tile followed by a V tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kPfStages * 2 * S::TILE];
  __shared__ int s_item[4];  // ids of coming items, published through the LDS
  const lds_bytes lbase = (lds_bytes)smem;
  auto kslot = [&](int t) { return kslot_of<D>(lbase, t); };
  auto vslot = [&](int t) { return vslot_of<D>(lbase, t); };

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int m32 = lane & 31;
  const int h = lane >> 5;
  const int xcc = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_s_getreg(kXccIdReg)) & (kQueues - 1);
  int* counters = sc.ws;
  const int ipp = a.num_kv_heads * sc.head_groups;
  const int n_items = sc.ws[kWsNPairsInt] * ipp;
  // Exponent scale of the raw scores (log2 domain).  A zero scale is taken as
  // a tiny one: every visible key then gets weight 1, and masked keys (score
  // -inf) still get 0.
  const float c = a.scale_log2 != 0.f ? a.scale_log2 : 1e-30f;
  const float masked = c > 0.f ? -INFINITY : INFINITY;  // score of a masked key: weight 0
  const uint32_t row_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;
  const TileLoadOffsets<D> lo = tile_load_offsets<D>(lane, wave, row_bytes);

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

  // This wave's query head and first row of an item, and its Q loads.
  auto wave_head = [&](const Item& it) {
    return it.g * a.group + it.hg * sc.heads_per_wg + wave % sc.heads_per_wg;
  };
  auto wave_rbase = [&](const Item& it) {
    return it.qtile * sc.rows_per_wg + (wave / sc.heads_per_wg) * kPfRows;
  };
  auto load_q = [&](const Item& it, u32x4 (&dst)[S::KS]) {
    const int row = wave_rbase(it) + m32;
    const bool live = row < it.lq;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(it.q_start + (live ? row : 0)) * a.num_q_heads +
                          wave_head(it)) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) dst[ks] = live ? ldg16(qp + 16 * ks) : u32x4{0, 0, 0, 0};
  };

  // Item ids go through a ring of four LDS slots: id(i) in slot i % 4.  The
  // id of item i + 2 is claimed by thread 0 when item i starts (with the
  // queue ticket it took during item i - 1) and read by every wave at item
  // i's last ring step, where the record of item i + 2 is loaded; item i + 1,
  // whose record is in registers by then, gets its Q rows and first K/V tile
  // loaded there.
  int ticket = -2;  // thread 0: queue slot taken for a later item (-2: the queues are drained)
  if (threadIdx.x == 0) {
    const int i0 = claim_item(counters, n_items, xcc, atomicAdd(&counters[xcc * kQueueStride], 1));
    const int i1 = i0 >= 0 ? claim_item(counters, n_items, xcc, atomicAdd(&counters[xcc * kQueueStride], 1)) : -1;
    s_item[0] = i0;
    s_item[1] = i1;
    ticket = i1 >= 0 ? atomicAdd(&counters[xcc * kQueueStride], 1) : -2;
  }
  __syncthreads();
  const int first_id = __builtin_amdgcn_readfirstlane(s_item[0]);
  if (first_id < 0) return;
  int nxt_id = __builtin_amdgcn_readfirstlane(s_item[1]);

  Item cur;
  WaveState<D> w;
  u32x4 rec[kRecVecs];
  {
    load_record(sc.ws, first_id / ipp, rec);
    cur = item_of(sc, first_id, rec, wave, ipp);
    dma_all<D>(dma_job<D>(seq_view<D>(a, cur), cur.blk0, 0, wave, item_tiles(a, sc, cur) > 0, kslot(0),
                          vslot(0)), lo);
    load_q(cur, w.qb);
    load_record(sc.ws, max(nxt_id, 0) / ipp, rec);
    // Once per workgroup: let everything land, so that the compiler knows no
    // load of this start is pending when the item loop begins.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  }

  int T = 0;  // ring position of the current tile (the tiles of all items, in order)
#pragma unroll 1
  for (int item_no = 0;; ++item_no) {
    if (threadIdx.x == 0)
      s_item[(item_no + 2) & 3] = ticket == -2 ? -1 : claim_item(counters, n_items, xcc, ticket);

    const SeqView sv = seq_view<D>(a, cur);
    const int head = wave_head(cur);
    const int rbase = wave_rbase(cur);
    const int row = rbase + m32;
    const int off = cur.lk - cur.lq;
    const int n_tiles = item_tiles(a, sc, cur);
    const int n_eff = max(n_tiles, 1);  // an item without keys still takes one (empty) ring step
    // last visible key of this lane's row (padding rows borrow the last row's)
    const int lim = a.causal ? min(off + min(row, cur.lq - 1), cur.lk - 1) : cur.lk - 1;
    // smallest such limit over this wave's rows, and the wave's largest
    const int lim_lo = a.causal ? min(off + min(rbase, cur.lq - 1), cur.lk - 1) : cur.lk - 1;
    const int lim_hi =
        a.causal ? min(off + min(rbase + kPfRows - 1, cur.lq - 1), cur.lk - 1) : cur.lk - 1;
    // Tiles past lim_hi hold no key any row of this wave sees (they exist for
    // other row blocks of the workgroup): the computing tiles come first, in
    // a loop of their own, so the accumulators are updated unconditionally.
    const int n_compute = min(n_tiles, lim_hi / kPfKeys + 1);

#pragma unroll
    for (int cb = 0; cb < S::DC; ++cb) w.o[cb] = f32x16{};
    w.m = -INFINITY;
    w.lsum = 0.f;

    // Start of ring step T (tile t of this item): wait for this wave's loads
    // of the tile (at an item's first tile, the previous item's output stores,
    // issued after them, may stay in flight) and for its LDS reads of the
    // previous tile, then sync the workgroup; the slot of the previous tile
    // is free from here on.
    auto sync_step = [&](int t) {
      if (t == 0 && item_no > 0) {
        barrier_after_vm<kStores>();
      } else {
        barrier_after_vm<0>();
      }
    };
    int32_t blk_next = n_eff > 1 ? cur.blk1 : 0;  // tile 1's block, from the record
    auto inner_step = [&](int t) -> DmaJob {  // loads of tile t + 1
      sync_step(t);
      return dma_job<D>(sv, blk_next, (t + 1) * kPfKeys, wave, t + 1 < n_tiles, kslot(T + 1), vslot(T + 1));
    };
    auto next_block = [&](int t) {  // block-table entry of tile t + 2, for the next step
      if (t + 2 < n_eff) blk_next = tile_block(sv, (t + 2) * kPfKeys, wave);
    };

    const int n_inner = n_eff - 1;
    int t = 0;
#pragma unroll 1
    for (; t < min(n_compute, n_inner); ++t, ++T) {
      const DmaJob job = inner_step(t);
      const int k0 = t * kPfKeys;
      compute_tile<D>(w, kslot(T), vslot(T), kaddr, vaddr, k0, lim, k0 + kPfKeys - 1 > lim_lo, h, c, masked, job, lo);
      next_block(t);
    }
#pragma unroll 1
    for (; t < n_inner; ++t, ++T) {
      dma_all<D>(inner_step(t), lo);
      next_block(t);
    }

    // Last ring step of the item: the loads that follow are the next item's
    // tile 0 (none after the last item, whose step then fetches nothing).
    sync_step(t);
    // Every word of the record stays allocated until here (no other value
    // may take a register a record load still writes).
    asm volatile("" ::"v"(rec[0]), "v"(rec[1]), "v"(rec[2]), "v"(rec[3]));
    const bool has_next = nxt_id >= 0;
    const Item nx = item_of(sc, max(nxt_id, 0), rec, wave, ipp);
    u32x4 qn[S::KS];
    {
      Item nq = nx;
      if (!has_next) nq.lq = 0;  // loads nothing
      load_q(nq, qn);
    }
    const DmaJob job = dma_job<D>(seq_view<D>(a, nx), nx.blk0, 0, wave, has_next && item_tiles(a, sc, nx) > 0,
                                  kslot(T + 1), vslot(T + 1));
    const int after = has_next ? __builtin_amdgcn_readfirstlane(s_item[(item_no + 2) & 3]) : -1;
    load_record(sc.ws, max(after, 0) / ipp, rec);
    if (threadIdx.x == 0) ticket = after >= 0 ? atomicAdd(&counters[xcc * kQueueStride], 1) : -2;
    if (t < n_compute) {
      const int k0 = t * kPfKeys;
      compute_tile<D>(w, kslot(T), vslot(T), kaddr, vaddr, k0, lim, k0 + kPfKeys - 1 > lim_lo, h, c, masked, job, lo);
    } else {
      dma_all<D>(job, lo);
    }
    ++T;

    // Output rows of this wave: buffer stores whose range ends after row Lq - 1
    // of this head, so the padding rows' stores are dropped by the hardware
    // (the count of store instructions stays kStores, whatever the rows).
    {
      const float lt = w.lsum + __shfl_xor(w.lsum, 32);  // the sum over all keys of this lane's row
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const uint32_t hrow = static_cast<uint32_t>(a.num_q_heads) * D * 2;  // bytes per token row
      const char* ob = static_cast<const char*>(a.out) +
                       (static_cast<int64_t>(cur.q_start) * a.num_q_heads + head) * D * 2;
      const buffer_rsrc orsrc = make_rsrc(ob, cur.lq > 0 ? (cur.lq - 1) * hrow + D * 2 : 0);
      const uint32_t obase = static_cast<uint32_t>(row) * hrow + 8 * h;
#pragma unroll
      for (int cb = 0; cb < S::DC; ++cb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& ov = w.o[cb];
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          const u32x2 v = {pack_bf16x2(ov[4 * j] * inv, ov[4 * j + 1] * inv),
                           pack_bf16x2(ov[4 * j + 2] * inv, ov[4 * j + 3] * inv)};
          __builtin_amdgcn_raw_buffer_store_b64(v, orsrc, static_cast<int>(obase + 2 * (32 * cb + 8 * j)), 0, 0);
        }
      }
    }
    if (!has_next) break;
    cur = nx;
    // The next item's Q rows take over here, after the output stores: the
    // empty asm keeps the compiler from moving the hand-over (and so its
    // wait for the Q loads, which would also wait for the next tile's loads
    // issued after them) to the start of the epilogue.
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      asm volatile("" : "+v"(qn[ks]));
      w.qb[ks] = qn[ks];
    }
    nxt_id = after;
  }
  // The last ring step's loads (zero fills) and the output stores must be
  // done before the workgroup's LDS is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

size_t prefill_workspace_bytes(int32_t num_seqs, int64_t total_q, int32_t group) {
  const int32_t heads_per_wg = (group % 4 == 0) ? 4 : ((group % 2 == 0) ? 2 : 1);
  const int64_t rows_per_wg = kPfRows * (kPfWaves / heads_per_wg);
  const int64_t cap = (total_q + rows_per_wg - 1) / rows_per_wg + num_seqs;
  return static_cast<size_t>(kWsRecsInt) * 4 + static_cast<size_t>(cap) * kRecInts * 4;
}

hipError_t launch_varlen_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream) {
  const int32_t heads_per_wg = (a.group % 4 == 0) ? 4 : ((a.group % 2 == 0) ? 2 : 1);
  PrefillSched sc;
  sc.ws = static_cast<int*>(workspace);
  sc.heads_per_wg = heads_per_wg;
  sc.head_groups = a.group / heads_per_wg;
  sc.rows_per_wg = kPfRows * (kPfWaves / heads_per_wg);
  const int64_t cap = static_cast<int64_t>((prefill_workspace_bytes(a.num_seqs, a.total_q, a.group) -
                                             static_cast<size_t>(kWsRecsInt) * 4) / (kRecInts * 4));
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, a, sc.rows_per_wg,
                     static_cast<int32_t>(cap), sc.ws);
  // two persistent workgroups per CU (more could not be resident)
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t max_items = cap * a.num_kv_heads * sc.head_groups;
  const int64_t grid = std::min<int64_t>(2 * static_cast<int64_t>(cus), max_items);
  if (grid <= 0) return hipGetLastError();
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(varlen_prefill_kernel<128>, dim3(static_cast<uint32_t>(grid)), dim3(kPfThreads), 0,
                       stream, a, sc);
  } else {
    hipLaunchKernelGGL(varlen_prefill_kernel<64>, dim3(static_cast<uint32_t>(grid)), dim3(kPfThreads), 0,
                       stream, a, sc);
  }
  return hipGetLastError();
}

}  // namespace pkv
