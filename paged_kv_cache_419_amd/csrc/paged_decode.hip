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
// Matrix cores.  Scores are computed transposed, S^T[token][head] = K Q^T, on
// 16x16x32 bf16 MFMA tiles: K rows go straight from HBM into the A operand
// (lane l holds 16 contiguous bytes of token row l % 16), the zero-padded query
// heads form B.  The output lane layout of S^T is exactly the B-operand layout
// P^T needs for O^T[d][head] = V^T P^T, so probabilities never leave their
// lanes, and every lane owns one head's softmax state (scale factors are
// lane-local).  V^T as the A operand needs V transposed: each wave stages its
// 32-token V tile in a private LDS region (row-major) and reads it back
// column-wise.  Exponentials use exp2 with scale * log2(e) folded in.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDecTile = 32;  // tokens per wave iteration: two 16-token MFMA tiles

template <int D>
struct DecodeShape {
  static constexpr int KK = D / 32;                      // MFMA k-steps over head_dim
  static constexpr int DB = D / 16;                      // 16-row d-blocks of O^T
  static constexpr int CH = D / 8;                       // 16-byte pieces per head row
  static constexpr int VROW = D * 2 + 16;                // staged V row stride (bytes)
  static constexpr int ROWS_PER_LOAD = kWave / CH;       // V rows one wave load covers
  static constexpr int VREGS = kDecTile / ROWS_PER_LOAD; // V loads per lane per tile
  static constexpr int LDS_STAGE = kDecWaves * kDecTile * VROW;
  static constexpr int LDS_MERGE = (2 * kDecWaves * 16 + kDecWaves * 16 * D) * 4;
  static constexpr int LDS = LDS_STAGE > LDS_MERGE ? LDS_STAGE : LDS_MERGE;
};

// k-slot t (0..7) of lane quarter q4 in a 32-token tile: tokens 4*q4+t of the
// first 16-token half for t < 4, 16+4*q4+(t-4) of the second for t >= 4.
__device__ __forceinline__ int tile_token(int q4, int t) {
  return (t < 4) ? (4 * q4 + t) : (12 + 4 * q4 + t);
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void paged_decode_kernel(DecodeArgs a) {
  using S = DecodeShape<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS];

  const int split = blockIdx.x;
  const int g = blockIdx.y / a.head_groups;
  const int hg = blockIdx.y - g * a.head_groups;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;

  const int ctx = a.context_lens[b];
  const int t0 = split * a.split_tokens;
  const int heads_here = min(16, a.group - hg * 16);
  const int h0 = g * a.group + hg * 16;
  uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(b) * a.num_q_heads + h0) * D;

  if (t0 >= ctx) {
    if (a.n_split == 1) {  // empty context: a zero row
      for (int i = threadIdx.x; i < heads_here * D; i += kDecThreads) out[i] = 0;
    }
    return;
  }
  const int t1 = min(ctx, t0 + a.split_tokens);

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

  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks_per_seq;
  const int shift = a.block_shift;
  const int bmask = (1 << shift) - 1;
  const int64_t row_elems = static_cast<int64_t>(a.num_kv_heads) * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + static_cast<int64_t>(g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + static_cast<int64_t>(g) * D;
  unsigned char* vst = smem + wave * kDecTile * S::VROW;
  const int vpiece = lane % S::CH;
  const int vrow0 = lane / S::CH;

  for (int j0 = t0 + wave * kDecTile; j0 < t1; j0 += kDecWaves * kDecTile) {
    // Slots of the two 16-token halves; a half never crosses a block boundary
    // because block_size >= 16 and j0 is a multiple of 16.
    const int64_t slot0 = (static_cast<int64_t>(bt[j0 >> shift]) << shift) + (j0 & bmask);
    const int j1 = j0 + 16;
    const int64_t slot1 =
        (j1 < t1) ? (static_cast<int64_t>(bt[j1 >> shift]) << shift) + (j1 & bmask) : slot0;

    u32x4 ka[2][S::KK];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool live = j0 + hf * 16 + n16 < t1;
      const uint16_t* kp = kbase + ((hf ? slot1 : slot0) + n16) * row_elems + 8 * q4;
#pragma unroll
      for (int kk = 0; kk < S::KK; ++kk) ka[hf][kk] = live ? ldg16(kp + 32 * kk) : u32x4{0, 0, 0, 0};
    }
    u32x4 vr[S::VREGS];
#pragma unroll
    for (int e = 0; e < S::VREGS; ++e) {
      const int row = e * S::ROWS_PER_LOAD + vrow0;
      const bool live = j0 + row < t1;
      const uint16_t* vp = vbase + ((row < 16 ? slot0 : slot1) + (row & 15)) * row_elems + 8 * vpiece;
      vr[e] = live ? ldg16(vp) : u32x4{0, 0, 0, 0};
    }

    f32x4 s[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      s[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < S::KK; ++kk) s[hf] = mfma16x16x32(ka[hf][kk], qb[kk], s[hf]);
    }

    // Online softmax in the log2 domain; lane owns head n16 for tokens 4*q4+i.
    float mt = -INFINITY;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = j0 + hf * 16 + 4 * q4 + i < t1;
        const float x = live ? s[hf][i] * a.scale_log2 : -INFINITY;
        s[hf][i] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = wave_max_xor_16_32(mt);
    const float m_new = fmaxf(m, mt);
    const float alpha = fast_exp2(m - m_new);
    float p[2][4];
    float ps = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[hf][i] = fast_exp2(s[hf][i] - m_new);
        ps += p[hf][i];
      }
    }
    lsum = lsum * alpha + ps;
    m = m_new;
#pragma unroll
    for (int c = 0; c < S::DB; ++c) o[c] *= alpha;
    const u32x4 pb = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                      pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};

    // Stage the V tile (row-major) and read V^T operands column-wise.
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < S::VREGS; ++e) {
      const int row = e * S::ROWS_PER_LOAD + vrow0;
      *reinterpret_cast<u32x4*>(vst + row * S::VROW + 16 * vpiece) = vr[e];
    }
    wave_lds_sync();
#pragma unroll
    for (int c = 0; c < S::DB; ++c) {
      const unsigned char* col = vst + (16 * c + n16) * 2;
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(col + tile_token(q4, t) * S::VROW);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(col + tile_token(q4, t + 1) * S::VROW);
        w[t / 2] = lo | (hi << 16);
      }
      o[c] = mfma16x16x32(u32x4{w[0], w[1], w[2], w[3]}, pb, o[c]);
    }
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
#pragma unroll
  for (int c = 0; c < S::DB; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ow[(wave * 16 + n16) * D + 16 * c + 4 * q4 + i] = o[c][i];
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
      out[idx] = static_cast<uint16_t>(bf16_rne(L > 0.f ? O / L : 0.f));
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
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int ctx = a.context_lens[b];
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
      static_cast<uint16_t>(bf16_rne((n > 0 && L > 0.f) ? O / L : 0.f));
}

}  // namespace

int32_t decode_auto_split(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t max_context_len) {
  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t pairs = static_cast<int64_t>(batch) * num_kv_heads * ((group + 15) / 16);
  // Aim for a few thousand workgroups so the 256 CUs stay busy to the end;
  // never split below 256 tokens and never let one workgroup walk more than 2048.
  const int64_t want = 4096;
  int64_t n = pairs > 0 ? (want + pairs - 1) / pairs : 1;
  if (n < 1) n = 1;
  int64_t split = (static_cast<int64_t>(max_context_len) + n - 1) / n;
  split = (split + 127) / 128 * 128;
  if (split < 256) split = 256;
  if (split > 2048) split = 2048;
  return static_cast<int32_t>(split);
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_split, a.num_kv_heads * a.head_groups, a.batch);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(paged_decode_kernel<128>, grid, dim3(kDecThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(paged_decode_kernel<64>, grid, dim3(kDecThreads), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.n_split == 1) return err;
  const dim3 cgrid(a.num_q_heads, a.batch);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(paged_decode_combine_kernel<128>, cgrid, dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(paged_decode_combine_kernel<64>, cgrid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pkv
