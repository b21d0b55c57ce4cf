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
// One workgroup of 1024 threads per row.  The k-th largest key is found by
// three radix passes over the row (11, 11 and 10 bits, a 2048-bin histogram
// in LDS each), a last pass evaluates the candidates; all passes read the
// logits with coalesced loads.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kSmThreads = 1024;
constexpr int kSmBins = 2048;

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

__global__ __launch_bounds__(kSmThreads) void topk_sample_kernel(SampleArgs a) {
  __shared__ int hist[kSmBins];
  __shared__ int suffix[kSmBins];
  __shared__ float sv[kSmThreads / kWave];
  __shared__ int64_t si[kSmThreads / kWave];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;

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

  // k-th largest key: digits from the top, each pass among the keys that
  // match the digits found so far.
  uint32_t prefix = 0, mask = 0;
  int remaining = a.top_k;
  if (a.top_k > 0 && a.top_k < V) {
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kBits[3] = {11, 11, 10};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int shift = kShift[p];
      const uint32_t nb = 1u << kBits[p];
      for (int b = tid; b < kSmBins; b += kSmThreads) hist[b] = 0;
      __syncthreads();
      for (int64_t i = tid; i < V; i += kSmThreads) {
        const uint32_t key = order_key(z[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
      }
      __syncthreads();
      // suffix sums: suffix[b] = number of matching keys with digit >= b
      for (int b = tid; b < kSmBins; b += kSmThreads) suffix[b] = b < static_cast<int>(nb) ? hist[b] : 0;
      __syncthreads();
      for (int d = 1; d < kSmBins; d <<= 1) {
        int add[2] = {0, 0};
        for (int j = 0; j < 2; ++j) {
          const int b = tid + j * kSmThreads;
          add[j] = b + d < kSmBins ? suffix[b + d] : 0;
        }
        __syncthreads();
        for (int j = 0; j < 2; ++j) suffix[tid + j * kSmThreads] += add[j];
        __syncthreads();
      }
      // the digit: the largest b with suffix[b] >= remaining (exactly one
      // b has suffix[b] >= remaining > suffix[b + 1])
      for (int j = 0; j < 2; ++j) {
        const int b = tid + j * kSmThreads;
        const int above = b + 1 < kSmBins ? suffix[b + 1] : 0;
        if (b < static_cast<int>(nb) && suffix[b] >= remaining && above < remaining) {
          s_digit = static_cast<uint32_t>(b);
          s_above = above;
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      mask |= (nb - 1) << shift;
      remaining -= s_above;
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;  // 0 (every key) when top_k does not restrict

  const float* g = a.gumbel + row * V;
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
