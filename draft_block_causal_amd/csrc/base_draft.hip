// Base-only drafting: every position's token from the frozen LM head's logits
// alone, with no causal correction.  This is the head-off configuration that
// the pages compare Domino with (the parallel backbone drafting on its own;
// [notes] §二.1(1) and the head ablation of §三; [explainer] §六): with the
// correction absent, L_i = L_i^base, so the K positions no longer depend on
// one another and are picked in one pass.
//
// Sampler as in the draft loop: greedy argmax, or Gumbel-max on L / T + G with
// the Philox4x32-10 word of counter (v >> 2, i, b, offset).
//
// grid (B K rows, S vocabulary slices of whole groups of 4 entries), 256
// threads: each thread takes groups of 4 consecutive entries (one Philox call
// per group), the workgroup's best (score, index) key goes to keys[i][b] by a
// 64-bit atomic max, and finalize_tokens turns the keys into tokens.  Bound by
// the HBM read of the B K V float32 logits.
#include "common.h"
#include "kernels.h"

namespace domino {

constexpr int kBdThreads = 256;

template <bool VEC>
__global__ void __launch_bounds__(kBdThreads)
    base_draft_kernel(int B, int K, int V, const float* __restrict__ base, float inv_t, int sampled, uint64_t seed,
                      uint32_t offset, unsigned long long* __restrict__ keys) {
  __shared__ unsigned long long red[kBdThreads / 64];
  const int row = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  const int b = row / K, i = row - b * K;
  const float* L = base + (size_t)row * V;
  const int ng = (V + 3) >> 2;
  const int g0 = (int)((long)ng * s / S), g1 = (int)((long)ng * (s + 1) / S);
  unsigned long long best = 0ull;
  for (int g = g0 + (int)threadIdx.x; g < g1; g += kBdThreads) {
    const int v0 = 4 * g;
    float x[4];
    if constexpr (VEC) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(L + v0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = q[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = v0 + e < V ? L[v0 + e] : 0.f;
    }
    u32x4 w = {0u, 0u, 0u, 0u};
    if (sampled) w = philox4(seed, offset, (uint32_t)b, (uint32_t)i, (uint32_t)g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sc = sampled ? x[e] * inv_t + gumbel_from_word(w[e]) : x[e];
      const unsigned long long k = v0 + e < V ? argmax_key(sc, (uint32_t)(v0 + e)) : 0ull;
      best = k > best ? k : best;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long x = __shfl_xor(best, o);
    best = x > best ? x : best;
  }
  if ((threadIdx.x & 63) == 0) red[wave_id()] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kBdThreads / 64; ++w) best = red[w] > best ? red[w] : best;
    if (best) atomicMax(keys + (size_t)i * B + b, best);
  }
}

hipError_t launch_base_draft(int B, int K, int V, const float* base, float temperature, uint64_t seed,
                             uint32_t offset, int32_t* tokens, void* workspace, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  unsigned long long* keys = static_cast<unsigned long long*>(workspace);
  hipError_t e = launch_fill_u64(keys, B * K, s);
  if (e != hipSuccess) return e;
  // about 2048 workgroups, each slice at least 1024 groups (4096 entries) long
  const long rows = (long)B * K, ng = (V + 3) / 4;
  long S = (2048 + rows - 1) / rows;
  S = S < 1 ? 1 : S;
  const long smax = ng / 1024 > 1 ? ng / 1024 : 1;
  S = S > smax ? smax : S;
  const bool vec = V % 4 == 0 && (reinterpret_cast<uintptr_t>(base) & 15u) == 0;
  const int sampled = temperature > 0.f ? 1 : 0;
  const float inv_t = sampled ? 1.0f / temperature : 0.f;
  auto kern = vec ? base_draft_kernel<true> : base_draft_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)rows, (unsigned)S), dim3(kBdThreads), 0, s, B, K, V, base, inv_t, sampled,
                     seed, offset, keys);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_finalize_tokens(B, K, keys, tokens, s);
}

}  // namespace domino
