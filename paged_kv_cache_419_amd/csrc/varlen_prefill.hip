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
// so one K/V tile in LDS serves 128 (row, head) pairs.  Workgroup ids are
// remapped so that consecutive q tiles of one (sequence, kv head) run on the
// same XCD and share its L2.
//
// Per 64-key tile the workgroup copies K (row-major) and V (transposed, with
// the key order the MFMA k-slots use) into LDS; then each wave computes
// S^T[key][row] = K Q^T on 16x16x32 bf16 MFMAs (Q^T held in registers),
// applies the causal mask and an online softmax per query row (each lane owns
// one row of each 16-row block, so rescaling is lane-local and the
// probabilities already sit in the B-operand layout of the next product), and
// accumulates O^T[d][row] += V^T P^T on the same MFMA shape.  fp32 accumulation;
// probabilities are rounded to bf16 for the second product.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfKeys = 64;  // keys per LDS tile
constexpr int kPfRows = 32;  // query rows per wave: two 16-row MFMA blocks

template <int D>
struct PrefillShape {
  static constexpr int KK = D / 32;
  static constexpr int DB = D / 16;
  static constexpr int CH = D / 8;
  static constexpr int KROW = D * 2 + 16;          // LDS bytes per K row (padded)
  static constexpr int VTROW = kPfKeys * 2 + 16;   // LDS bytes per V^T row (one d)
  static constexpr int KLOADS = kPfKeys * CH / kPfThreads;
  static constexpr int LDS = kPfKeys * KROW + D * VTROW;
};

template <int D>
__global__ __launch_bounds__(kPfThreads, 2) void varlen_prefill_kernel(
    PrefillArgs a, int32_t heads_per_wg, int32_t head_groups, int32_t rows_per_wg,
    int32_t q_tiles, int64_t total_items, int64_t items_per_xcd) {
  using S = PrefillShape<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS];
  unsigned char* ks = smem;
  unsigned char* vts = smem + kPfKeys * S::KROW;

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of work items.
  const int64_t lin = blockIdx.x;
  const int64_t item = (lin % 8) * items_per_xcd + lin / 8;
  if (item >= total_items) return;
  int64_t rest = item;
  const int qt = static_cast<int>(rest % q_tiles);
  rest /= q_tiles;
  const int hg = static_cast<int>(rest % head_groups);
  rest /= head_groups;
  const int g = static_cast<int>(rest % a.num_kv_heads);
  const int seq = static_cast<int>(rest / a.num_kv_heads);

  const int q_start = a.cu_q[seq];
  const int lq = a.cu_q[seq + 1] - q_start;
  const int lk = a.cu_k[seq + 1] - a.cu_k[seq];
  const int off = lk - lq;
  const int qtile = q_tiles - 1 - qt;  // longer causal rows first within a sequence
  const int r0 = qtile * rows_per_wg;
  if (r0 >= lq) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int hl = hg * heads_per_wg + wave % heads_per_wg;
  const bool hvalid = hl < a.group;
  const int h = g * a.group + (hvalid ? hl : 0);
  const int rbase = r0 + (wave / heads_per_wg) * kPfRows;

  // B operands of S^T = K Q^T: lane holds 8 values of query row n16 per block.
  u32x4 qb[2][S::KK];
  int lim[2];  // last visible key position of this lane's row in each block
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = rbase + rb * 16 + n16;
    const bool live = hvalid && r < lq;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(q_start + r) * a.num_q_heads + h) * D + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk) qb[rb][kk] = live ? ldg16(qp + 32 * kk) : u32x4{0, 0, 0, 0};
    const int rc = min(r, lq - 1);  // padding rows borrow the last row's mask
    lim[rb] = a.causal ? min(off + rc, lk - 1) : lk - 1;
  }
  const int last_row = min(r0 + rows_per_wg, lq) - 1;
  const int kend = a.causal ? min(lk, off + last_row + 1) : lk;

  f32x4 o[2][S::DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < S::DB; ++c) o[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};

  const int32_t* bt = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks_per_seq;
  const int shift = a.block_shift;
  const int bmask = (1 << shift) - 1;
  const int64_t row_elems = static_cast<int64_t>(a.num_kv_heads) * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + static_cast<int64_t>(g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + static_cast<int64_t>(g) * D;

  for (int k0 = 0; k0 < kend; k0 += kPfKeys) {
    __syncthreads();  // the previous tile is consumed
    // K tile, row-major: one 16-byte piece per thread per load.
#pragma unroll
    for (int e = 0; e < S::KLOADS; ++e) {
      const int row = e * (kPfThreads / S::CH) + tid / S::CH;
      const int piece = tid % S::CH;
      const int key = k0 + row;
      u32x4 val = {0, 0, 0, 0};
      if (key < lk) {
        const int64_t slot = (static_cast<int64_t>(bt[key >> shift]) << shift) + (key & bmask);
        val = ldg16(kbase + slot * row_elems + 8 * piece);
      }
      *reinterpret_cast<u32x4*>(ks + row * S::KROW + 16 * piece) = val;
    }
    // V tile, transposed: a thread takes 4 consecutive keys x 8 values of d and
    // writes, for each d, the 4 keys as one 8-byte run of V^T row d.  Key k of
    // the tile goes to position 32*(k/32) + 8*((k%16)/4) + 4*((k%32)/16) + k%4,
    // the order in which the PV MFMA k-slots expect it.
    if (tid < 16 * S::CH) {
      const int quad = tid / S::CH;
      const int piece = tid % S::CH;
      u32x4 vk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + 4 * quad + e;
        vk[e] = u32x4{0, 0, 0, 0};
        if (key < lk) {
          const int64_t slot = (static_cast<int64_t>(bt[key >> shift]) << shift) + (key & bmask);
          vk[e] = ldg16(vbase + slot * row_elems + 8 * piece);
        }
      }
      const int pos = (quad / 8) * 32 + 8 * (quad % 4) + 4 * ((quad / 4) % 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int d = 8 * piece + 2 * w;
        const uint32_t lo0 = (vk[0][w] & 0xFFFFu) | (vk[1][w] << 16);
        const uint32_t lo1 = (vk[2][w] & 0xFFFFu) | (vk[3][w] << 16);
        const uint32_t hi0 = (vk[0][w] >> 16) | (vk[1][w] & 0xFFFF0000u);
        const uint32_t hi1 = (vk[2][w] >> 16) | (vk[3][w] & 0xFFFF0000u);
        *reinterpret_cast<uint2*>(vts + d * S::VTROW + 2 * pos) = uint2{lo0, lo1};
        *reinterpret_cast<uint2*>(vts + (d + 1) * S::VTROW + 2 * pos) = uint2{hi0, hi1};
      }
    }
    __syncthreads();
    if (!hvalid) continue;

    // S^T[key][row] for 4 key blocks x 2 row blocks.
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < S::KK; ++kk) {
        const u32x4 ka =
            *reinterpret_cast<const u32x4*>(ks + (kb * 16 + n16) * S::KROW + 2 * (32 * kk + 8 * q4));
        s[kb][0] = mfma16x16x32(ka, qb[0][kk], s[kb][0]);
        s[kb][1] = mfma16x16x32(ka, qb[1][kk], s[kb][1]);
      }
    }

    u32x4 pb[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + kb * 16 + 4 * q4 + i;
          const float x = key <= lim[rb] ? s[kb][rb][i] * a.scale_log2 : -INFINITY;
          s[kb][rb][i] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = wave_max_xor_16_32(mt);
      const float m_new = fmaxf(m[rb], mt);
      const float alpha = fast_exp2(m[rb] - m_new);
      float ps = 0.f;
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = fast_exp2(s[kb][rb][i] - m_new);
          ps += p[kb][i];
        }
      }
      l[rb] = l[rb] * alpha + ps;
      m[rb] = m_new;
#pragma unroll
      for (int c = 0; c < S::DB; ++c) o[rb][c] *= alpha;
#pragma unroll
      for (int g32 = 0; g32 < 2; ++g32) {
        pb[rb][g32] = u32x4{pack_bf16x2(p[2 * g32][0], p[2 * g32][1]),
                            pack_bf16x2(p[2 * g32][2], p[2 * g32][3]),
                            pack_bf16x2(p[2 * g32 + 1][0], p[2 * g32 + 1][1]),
                            pack_bf16x2(p[2 * g32 + 1][2], p[2 * g32 + 1][3])};
      }
    }

    // O^T[d][row] += V^T P^T.
#pragma unroll
    for (int c = 0; c < S::DB; ++c) {
#pragma unroll
      for (int g32 = 0; g32 < 2; ++g32) {
        const u32x4 va =
            *reinterpret_cast<const u32x4*>(vts + (16 * c + n16) * S::VTROW + 2 * (32 * g32 + 8 * q4));
        o[0][c] = mfma16x16x32(va, pb[0][g32], o[0][c]);
        o[1][c] = mfma16x16x32(va, pb[1][g32], o[1][c]);
      }
    }
  }

  if (!hvalid) return;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = wave_sum_xor_16_32(l[rb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int r = rbase + rb * 16 + n16;
    if (r >= lq) continue;
    uint16_t* op = static_cast<uint16_t*>(a.out) +
                   (static_cast<int64_t>(q_start + r) * a.num_q_heads + h) * D + 4 * q4;
#pragma unroll
    for (int c = 0; c < S::DB; ++c) {
      const uint2 w = {pack_bf16x2(o[rb][c][0] * inv, o[rb][c][1] * inv),
                       pack_bf16x2(o[rb][c][2] * inv, o[rb][c][3] * inv)};
      *reinterpret_cast<uint2*>(op + 16 * c) = w;
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
  const int64_t per_xcd = (total + 7) / 8;
  const dim3 grid(static_cast<uint32_t>(per_xcd * 8));
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(varlen_prefill_kernel<128>, grid, dim3(kPfThreads), 0, stream, a,
                       heads_per_wg, head_groups, rows_per_wg, q_tiles, total, per_xcd);
  } else {
    hipLaunchKernelGGL(varlen_prefill_kernel<64>, grid, dim3(kPfThreads), 0, stream, a,
                       heads_per_wg, head_groups, rows_per_wg, q_tiles, total, per_xcd);
  }
  return hipGetLastError();
}

}  // namespace pkv
