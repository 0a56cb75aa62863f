// Streaming log-sum-exp over vocabulary slices (device helpers shared by the
// sampled-draft verification and the curriculum loss): a slice's running
// (max, sum of exp(x - max)) pair, merged across lanes, waves and slices so
// that an empty side (max = -inf, sum = 0) leaves the other unchanged.
#pragma once

#include <math.h>

#include "common.h"

namespace domino {

constexpr int kLseThreads = 256;
constexpr int kLseWaves = kLseThreads / 64;

struct LsePart {
  float m, s;
};

__device__ __forceinline__ LsePart lse_merge(LsePart a, LsePart b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return LsePart{m, 0.f};
  return LsePart{m, a.s * expf(a.m - m) + b.s * expf(b.m - m)};
}

__device__ __forceinline__ LsePart wave_lse(LsePart p) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    LsePart q{__shfl_xor(p.m, o), __shfl_xor(p.s, o)};
    p = lse_merge(p, q);
  }
  return p;
}

// Partial log-sum-exp of row[v0 .. v1) * inv_t over a workgroup of
// kLseThreads threads; thread 0 holds the result.  red: kLseWaves entries of
// LDS.  Every thread of the workgroup must call it.
__device__ inline LsePart block_lse(const float* __restrict__ row, long v0, long v1, float inv_t, LsePart* red) {
  LsePart p{-INFINITY, 0.f};
  for (long v = v0 + threadIdx.x; v < v1; v += kLseThreads) {
    const float x = row[v] * inv_t;
    if (x > p.m) {
      p.s = p.s * expf(p.m - x) + 1.f;
      p.m = x;
    } else {
      p.s += expf(x - p.m);
    }
  }
  p = wave_lse(p);
  const int wave = wave_id(), lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = p;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < kLseWaves; ++w) p = lse_merge(p, red[w]);
  __syncthreads();
  return p;
}

}  // namespace domino
