// Verification of a sampled draft by speculative sampling (Leviathan, Kalman,
// Matias, ICML 2023, Algorithm 1; Chen et al. 2023): the drafted token y_i of
// position i survives when U_i p_d(y_i) < p_t(y_i); the first rejected
// position n ends the block and the next token is drawn from the positive
// part of p_t - p_d there, or from p_t one past the block when every position
// survives.  p = softmax(L / T) for the target's and the draft's logits.
//
// Three launches on the caller's stream:
//   1. verify_stats_kernel, grid (B (K + 1), S1): the running (max, sum of
//      exp) of L / T over one vocabulary slice of one target row and, below
//      position K, of the draft row at the same position;
//   2. verify_draw_kernel, grid (B, S2): every workgroup of block b combines
//      the partials into log-normalisers, finds n (the accept tests are
//      cheap: two logits and one Philox word per position) and draws over its
//      vocabulary slice by Gumbel-max, merged with a 64-bit atomicMax key;
//   3. verify_finish_kernel: the key's index is the next token.
// The logit rows are read with coalesced 4-byte loads; the work is bound by
// HBM reads of B (2K + 1) V floats in pass 1 and at most 2 B V in pass 2.
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "lse.h"

namespace domino {

constexpr int kVThreads = kLseThreads;
constexpr int kVWaves = kLseWaves;

__global__ void __launch_bounds__(kVThreads) verify_stats_kernel(int K, int V, const float* __restrict__ target,
                                                                 const float* __restrict__ draft, float inv_t,
                                                                 float4* __restrict__ stats,
                                                                 unsigned long long* __restrict__ keys) {
  __shared__ LsePart red[kVWaves];
  const int row = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  const int b = row / (K + 1), i = row - b * (K + 1);
  long v0, v1;
  slice_bounds(V, s, S, v0, v1);
  if (s == 0 && i == 0 && threadIdx.x == 0) keys[b] = 0ull;
  const LsePart t = block_lse(target + (size_t)row * V, v0, v1, inv_t, red);
  LsePart d{-INFINITY, 0.f};
  if (i < K) d = block_lse(draft + ((size_t)b * K + i) * V, v0, v1, inv_t, red);
  if (threadIdx.x == 0) stats[(size_t)row * S + s] = float4{t.m, t.s, d.m, d.s};
}

__device__ __forceinline__ float uniform_from_word(uint32_t w) {
  return ((float)(w >> 9) + 0.5f) * 1.1920928955078125e-07f;
}

__global__ void __launch_bounds__(kVThreads) verify_draw_kernel(int K, int V, int S1, const float* __restrict__ target,
                                                                const float* __restrict__ draft,
                                                                const int32_t* __restrict__ tokens, float inv_t,
                                                                uint64_t seed, uint32_t offset,
                                                                const float4* __restrict__ stats,
                                                                unsigned long long* __restrict__ keys,
                                                                int32_t* __restrict__ accept) {
  __shared__ float lse_t[kMaxVerifyBlock + 1], lse_d[kMaxVerifyBlock];
  __shared__ int s_n;
  __shared__ unsigned long long s_key[kVWaves];
  const int b = blockIdx.x, s = blockIdx.y, S2 = gridDim.y;
  const int tid = threadIdx.x;
  if (tid == 0) s_n = K;
  for (int i = tid; i <= K; i += kVThreads) {
    LsePart t{-INFINITY, 0.f}, d{-INFINITY, 0.f};
    const float4* st = stats + ((size_t)b * (K + 1) + i) * S1;
    for (int q = 0; q < S1; ++q) {
      const float4 x = st[q];
      t = lse_merge(t, LsePart{x.x, x.y});
      d = lse_merge(d, LsePart{x.z, x.w});
    }
    lse_t[i] = t.m + logf(t.s);
    if (i < K) lse_d[i] = d.m + logf(d.s);
  }
  __syncthreads();
  // accept test of every drafted position; n = the first that fails
  for (int i = tid; i < K; i += kVThreads) {
    const int y = min(max(tokens[(size_t)b * K + i], 0), V - 1);
    const float pt = exp_hw(target[((size_t)b * (K + 1) + i) * V + y] * inv_t - lse_t[i]);
    const float pd = exp_hw(draft[((size_t)b * K + i) * V + y] * inv_t - lse_d[i]);
    const float u = uniform_from_word(philox_word(seed, offset, (uint32_t)b, (uint32_t)i, 0u));
    if (!(u * pd < pt)) atomicMin(&s_n, i);
  }
  __syncthreads();
  const int n = s_n;
  if (s == 0 && tid == 0) accept[b] = n;
  // Gumbel-max draw over this workgroup's vocabulary slice at position n
  const float* tr = target + ((size_t)b * (K + 1) + n) * V;
  const float* dr = draft + ((size_t)b * K + min(n, K - 1)) * V;
  const float lt = lse_t[n], ld = n < K ? lse_d[n] : 0.f;
  const long v0 = (long)V * s / S2, v1 = (long)V * (s + 1) / S2;
  unsigned long long best = 0ull;
  for (long v = v0 + tid; v < v1; v += kVThreads) {
    const float g = gumbel_from_word(philox_word(seed, offset + 1u, (uint32_t)b, (uint32_t)n, (uint32_t)v));
    float sc;
    if (n < K) {
      const float q = exp_hw(tr[v] * inv_t - lt) - exp_hw(dr[v] * inv_t - ld);
      sc = q > 0.f ? logf(q) + g : -INFINITY;
    } else {
      sc = tr[v] * inv_t + g;
    }
    const unsigned long long k = argmax_key(sc, (uint32_t)v);
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long x = __shfl_xor(best, o);
    best = x > best ? x : best;
  }
  if ((tid & 63) == 0) s_key[wave_id()] = best;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kVWaves; ++w) best = s_key[w] > best ? s_key[w] : best;
    if (best) atomicMax(keys + b, best);
  }
}

__global__ void verify_finish_kernel(int B, const unsigned long long* __restrict__ keys, int32_t* __restrict__ next) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) next[b] = key_token(keys[b]);
}

hipError_t launch_verify_sampled(int B, int K, int V, const float* target, const float* draft, const int32_t* tokens,
                                 float temperature, uint64_t seed, uint32_t offset, int32_t* accept, int32_t* next,
                                 const VerifyPlan& plan, void* workspace, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (K < 1 || K > kMaxVerifyBlock || V < 1) return hipErrorInvalidValue;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float4* stats = reinterpret_cast<float4*>(ws + plan.stats);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(ws + plan.keys);
  const float inv_t = 1.0f / temperature;
  hipLaunchKernelGGL(verify_stats_kernel, dim3((unsigned)(B * (K + 1)), (unsigned)plan.S1), dim3(kVThreads), 0, s, K,
                     V, target, draft, inv_t, stats, keys);
  hipLaunchKernelGGL(verify_draw_kernel, dim3((unsigned)B, (unsigned)plan.S2), dim3(kVThreads), 0, s, K, V, plan.S1,
                     target, draft, tokens, inv_t, seed, offset, stats, keys, accept);
  hipLaunchKernelGGL(verify_finish_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, B, keys, next);
  return hipGetLastError();
}

}  // namespace domino
