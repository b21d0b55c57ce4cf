// Temperature and top-k sampling of the next token from a row of logits.
//
// "Nano-vLLM part 1", section 5.4: the model's logits over the vocabulary are
// turned into a token by sampling; the temperature reshapes the distribution
// (softmax of logits / T: near 0 almost always the top token, large T
// flatter).  "Nano-vLLM inference engine architecture", the configuration
// section: top_k limits the candidates considered at each step.
//
// The draw uses the Gumbel-max identity: argmax_i (z_i / T + g_i), with g_i
// independent standard Gumbel noise, is distributed as softmax(z / T); with
// the argmax taken over the top-k candidates only, it samples the
// distribution restricted to them.  The noise is an input (one value per
// vocabulary entry, read only at the candidates), so the sampled token is a
// deterministic function of logits and noise: z_i * (1/T) and the sum are
// rounded separately in fp32 (no fused multiply-add), and ties go to the
// lowest index.  Candidates are the entries whose logit is >= the k-th
// largest (so ties at the threshold are all kept), ordered by the fp32 bit
// pattern mapped to an order-preserving unsigned key.  T <= 0 is greedy
// (the first maximum of the logits).
//
// One workgroup of 1024 threads per row.  Fast path (restricted top-k, large
// vocabulary): a threshold below the k-th largest logit is estimated from
// 1024 samples of the row, 64 evenly spaced runs of 16 entries (while the
// first part of the row is already streaming in), one pass over the row collects every entry at or
// above it into LDS (wave-ballot compaction), and the exact k-th
// largest and the draw are taken from those few entries (noise read at the
// candidates only), so the row is read once.  When the estimate fails (fewer
// than k or more than the LDS capacity collected: ties or odd distributions)
// the general path runs: four radix passes over the row (8-bit digits, a
// 256-bin LDS histogram each) find the k-th largest, and a last pass
// evaluates the candidates.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kSmThreads = 1024;
constexpr int kSmCap = 4096;       // entries the fast path can collect
constexpr int kSmMinVocab = 8192;  // smaller rows take the general path

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Better of two (value, index) pairs: larger value, then smaller index.
__device__ __forceinline__ void keep_best(float& v, int64_t& i, float v2, int64_t i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Workgroup-wide best (value, index); every thread gets the result.
__device__ void block_best(float& v, int64_t& i, float* sv, int64_t* si) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float v2 = __shfl_xor(v, off);
    const int64_t i2 = __shfl_xor(i, off);
    keep_best(v, i, v2, i2);
  }
  if (lane == 0) {
    sv[wave] = v;
    si[wave] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int w = 1; w < kSmThreads / kWave; ++w) keep_best(v, i, sv[w], si[w]);
  __syncthreads();
}

// Radix selection of the k-th largest key among n keys given by key_at(i)
// (0 <= i < n; every thread walks i = tid, tid + 1024, ...): four passes of
// 8-bit digits, each with its own 256-bin LDS histogram (hist: 4 x 256 ints,
// all cleared up front), scanned by one wave; two barriers per pass.  Keys
// often share their high digits (samples of a row do, and the candidates
// above a threshold all do), so each wave first adds up the lanes that share
// the digit of its first active lane and commits them with one atomic; the
// other lanes add one each.  Requires 0 < k <= n.
template <typename KeyAt>
__device__ uint32_t kth_largest_key(KeyAt key_at, int64_t n, int k, int* hist, uint32_t* s_digit,
                                    int* s_above) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  static_assert(kSmThreads == 4 * 256, "one histogram word per thread to clear");
  hist[tid] = 0;
  __syncthreads();
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    int* h = hist + 256 * pass;
    for (int64_t i = tid; i < n; i += kSmThreads) {
      const uint32_t key = key_at(i);
      const bool act = (key & mask) == prefix;
      const uint32_t d = (key >> shift) & 255;
      const uint64_t am = __ballot(act);
      if (am != 0) {
        const int leader = static_cast<int>(__builtin_ctzll(am));
        const uint32_t ld = static_cast<uint32_t>(__shfl(static_cast<int>(d), leader));
        const uint64_t same = __ballot(act && d == ld);
        if (lane == leader) {
          atomicAdd(&h[ld], static_cast<int>(__popcll(same)));
        } else if (act && d != ld) {
          atomicAdd(&h[d], 1);
        }
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l holds bins 4l .. 4l+3; suf = keys in the bins of lanes l .. 63
      const int4 hv = *reinterpret_cast<const int4*>(&h[4 * tid]);
      const int local = hv.x + hv.y + hv.z + hv.w;
      int suf = local;
      for (int off = 1; off < kWave; off <<= 1) {  // inclusive suffix scan over the lanes
        const int v = __shfl_down(suf, off);
        if (tid + off < kWave) suf += v;
      }
      const int above_lane = suf - local;  // keys whose digit is above this lane's bins
      // number of keys with digit >= 4l + j, and with digit > 4l + j
      const int ge[4] = {suf, above_lane + hv.y + hv.z + hv.w, above_lane + hv.z + hv.w, above_lane + hv.w};
      const int gt[4] = {ge[1], ge[2], ge[3], above_lane};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (ge[j] >= remaining && gt[j] < remaining) {  // exactly one bin of the row
          s_digit[pass] = static_cast<uint32_t>(4 * tid + j);
          s_above[pass] = gt[j];
        }
      }
    }
    __syncthreads();
    prefix |= s_digit[pass] << shift;
    mask |= 255u << shift;
    remaining -= s_above[pass];
  }
  // (the caller may reuse hist, s_digit and s_above only after a barrier)
  return prefix;
}

__global__ __launch_bounds__(kSmThreads) void topk_sample_kernel(SampleArgs a) {
  __shared__ __attribute__((aligned(16))) int hist[4 * 256];
  __shared__ float sv[kSmThreads / kWave];
  __shared__ int64_t si[kSmThreads / kWave];
  __shared__ uint32_t s_digit[4];
  __shared__ int s_above[4];

  const int64_t row = blockIdx.x;
  const int64_t V = a.vocab;
  const float* z = a.logits + row * V;
  const int tid = threadIdx.x;

  float best = -INFINITY;
  int64_t best_i = INT64_MAX;
  if (a.greedy) {
    for (int64_t i = tid; i < V; i += kSmThreads) keep_best(best, best_i, z[i], i);
    block_best(best, best_i, sv, si);
    if (tid == 0) a.tokens[row] = static_cast<int32_t>(best_i);
    return;
  }

  const float* g = a.gumbel + row * V;
  const bool restricted = a.top_k > 0 && a.top_k < V;

  if (restricted && V >= kSmMinVocab) {
    // Fast path.  Threshold: the s-th largest of 1024 samples of the row,
    // s chosen so that about 4 k entries of the row (at least 4 samples' worth)
    // lie above it: enough to hold the top k, few enough for the LDS.  (A row
    // where this fails is only slower: it takes the general path.)
    __shared__ uint32_t ckey[kSmCap];
    __shared__ int cidx[kSmCap];
    __shared__ uint32_t skey[kSmThreads];
    __shared__ int s_count;
    // The collect pass's first loads go out now, so that the row streams in
    // while the threshold is selected (kSmUnroll 16-byte loads per thread in
    // flight, 64 KiB per row; batches of 3-4 were the fastest measured, 8 was
    // ~3 % and 12-16 ~20 % slower: the first batch queues ahead of the sample
    // the threshold waits for).
    constexpr int kSmUnroll = 4;
    // 1024 samples in 64 evenly spaced runs of 16 consecutive entries: 64
    // cache lines per row (1024 lone entries would fetch 1024 lines)
    const int64_t sidx = static_cast<int64_t>(tid >> 4) * (V >> 6) + (tid & 15);
    // The sample is loaded first, straight into skey (a direct-to-LDS load:
    // it writes no register, so no register can be reused while it is in
    // flight), and waited for by count, so the batch's kSmUnroll loads stay
    // in flight: the compiler, waiting for a register load, would wait for
    // the batch as well.  A wrong count would only let the threshold read a
    // stale sample, which the exact selection below corrects.
    {
      const lds_bytes dst = (lds_bytes)skey + 4 * (tid & ~(kWave - 1));
      const uint32_t lds_addr =  // the same for the whole wave
          __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
      uint32_t saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %2\n\t"
          "global_load_lds_dword %1, off\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "v"(z + sidx), "s"(lds_addr)
          : "memory");
    }
    // Every wave's sample load goes out before any wave's batch loads (a
    // bare barrier: it orders the issue and waits for no memory), so the
    // samples do not queue behind 64 KiB of row data.
    __builtin_amdgcn_s_barrier();
    const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(z) & 15) == 0);
    const float4* z4 = reinterpret_cast<const float4*>(z);
    const int64_t n4 = V / 4;
    // (indices past the row are clamped to its last entry: the loads stay
    // unconditional, and the collect pass skips those entries)
    float4 first[kSmUnroll];
    static_assert(kSmUnroll == 4, "the wait below counts kSmUnroll loads");
    if (vec) {
#pragma unroll
      for (int u = 0; u < kSmUnroll; ++u) first[u] = z4[min(tid + static_cast<int64_t>(u) * kSmThreads, n4 - 1)];
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    skey[tid] = order_key(__uint_as_float(skey[tid]));
    if (tid == 0) s_count = 0;
    const int64_t want = (static_cast<int64_t>(kSmThreads) * 4 * a.top_k + V - 1) / V + 4;
    const int s_rank = static_cast<int>(min<int64_t>(want, kSmThreads));
    __syncthreads();
    // (every thread gets the same key back)
    const uint32_t tau0 = kth_largest_key([&](int64_t i) { return skey[i]; }, kSmThreads, s_rank, hist,
                                          s_digit, s_above);
    // Collect every entry with key >= tau0 (one wave-wide reservation per
    // step; entries past the capacity are counted, not stored).
    const int lane = tid & (kWave - 1);
    auto push = [&](bool take, uint32_t key, int64_t idx) {
      const uint64_t m = __ballot(take);
      if (m == 0) return;
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_count, __popcll(m));
      base = __shfl(base, 0);
      const int pos = base + __popcll(m & ((1ull << lane) - 1));
      if (take && pos < kSmCap) {
        ckey[pos] = key;
        cidx[pos] = static_cast<int>(idx);
      }
    };
    if (vec) {
      // The float tf whose key is tau0: !(f < tf) holds for every f with
      // key >= tau0 (also NaN, and -0 against +0, which the exact test then
      // drops), so one float compare per entry finds the few entries that
      // need the exact test.
      const float tf = __uint_as_float((tau0 & 0x80000000u) ? (tau0 & 0x7FFFFFFFu) : ~tau0);
      // kSmUnroll 16-byte loads per thread in flight, then their entries
      auto collect = [&](const float4 (&v)[kSmUnroll], int64_t i0) {
#pragma unroll
        for (int u = 0; u < kSmUnroll; ++u) {
          const int64_t i = i0 + u * kSmThreads;
          const bool live = i < n4;
          const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool maybe = live && !(e[c] < tf);
            if (__ballot(maybe) != 0) {
              const uint32_t key = order_key(e[c]);
              push(maybe && key >= tau0, key, 4 * i + c);
            }
          }
        }
      };
      collect(first, tid);
      for (int64_t i0 = tid + kSmUnroll * kSmThreads; i0 - tid < n4; i0 += kSmUnroll * kSmThreads) {
        float4 v[kSmUnroll];
#pragma unroll
        for (int u = 0; u < kSmUnroll; ++u) v[u] = z4[min(i0 + u * kSmThreads, n4 - 1)];
        // all kSmUnroll loads go out before the first entry is looked at
        __builtin_amdgcn_sched_barrier(0);
        collect(v, i0);
      }
    } else {
      for (int64_t i = tid; i - tid < V; i += kSmThreads) {
        const bool live = i < V;
        const uint32_t key = live ? order_key(z[i]) : 0u;
        push(live && key >= tau0, key, i);
      }
    }
    __syncthreads();
    const int count = s_count;
    if (count >= a.top_k && count <= kSmCap) {
      const uint32_t tau = kth_largest_key([&](int64_t i) { return ckey[i]; }, count, a.top_k, hist,
                                           s_digit, s_above);
      for (int j = tid; j < count; j += kSmThreads) {
        if (ckey[j] >= tau) {
          const int64_t i = cidx[j];
          keep_best(best, best_i, __fadd_rn(__fmul_rn(z[i], a.inv_temperature), g[i]), i);
        }
      }
      block_best(best, best_i, sv, si);
      if (tid == 0) a.tokens[row] = static_cast<int32_t>(best_i);
      return;
    }
    __syncthreads();  // the LDS scratch is reused below
  }

  // General path: the k-th largest key by radix passes over the row.
  const uint32_t tau = restricted
      ? kth_largest_key([&](int64_t i) { return order_key(z[i]); }, V, a.top_k, hist, s_digit, s_above)
      : 0u;  // every key
  for (int64_t i = tid; i < V; i += kSmThreads) {
    const float zi = z[i];
    if (order_key(zi) >= tau) keep_best(best, best_i, __fadd_rn(__fmul_rn(zi, a.inv_temperature), g[i]), i);
  }
  block_best(best, best_i, sv, si);
  if (tid == 0) a.tokens[row] = static_cast<int32_t>(best_i);
}

}  // namespace

hipError_t launch_topk_sample(const SampleArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_sample_kernel, dim3(static_cast<uint32_t>(a.rows)), dim3(kSmThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
