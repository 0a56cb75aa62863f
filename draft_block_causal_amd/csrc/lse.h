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

// e^x for the softmax terms (arguments x - max <= 0): 2^(x log2 e) on the
// hardware base-2 exponential, whose ~1 ulp plus the rounding of the product
// (|x| log2 e 2^-24 ln 2, 2e-6 relative at x = -30) is far inside the
// float32 log-sum-exp's own error over 10^5 entries; results below 2^-126
// flush to zero.  (The library expf adds a split product and range checks:
// 14 instructions against 2.)
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ LsePart lse_merge(LsePart a, LsePart b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return LsePart{m, 0.f};
  return LsePart{m, a.s * exp_hw(a.m - m) + b.s * exp_hw(b.m - m)};
}

__device__ __forceinline__ LsePart wave_lse(LsePart p) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    LsePart q{__shfl_xor(p.m, o), __shfl_xor(p.s, o)};
    p = lse_merge(p, q);
  }
  return p;
}

// Entries [v0, v1) of slice s of S over a row of V: boundaries fall on
// multiples of 4 (whole 16-byte groups), the last slice ends at V.
__device__ __forceinline__ void slice_bounds(long V, int s, int S, long& v0, long& v1) {
  v0 = s == 0 ? 0 : (V * s / S) & ~3L;
  v1 = s == S - 1 ? V : (V * (s + 1) / S) & ~3L;
}

// Folds four values into a running pair: one rescale when their maximum
// exceeds the running one, then four exponentials.
__device__ __forceinline__ LsePart lse_add4(LsePart p, float x0, float x1, float x2, float x3) {
  const float m4 = fmaxf(fmaxf(x0, x1), fmaxf(x2, x3));
  if (m4 > p.m) {
    p.s *= exp_hw(p.m - m4);  // (exp(-inf) = 0 for the empty pair)
    p.m = m4;
  }
  p.s += exp_hw(x0 - p.m) + exp_hw(x1 - p.m) + exp_hw(x2 - p.m) + exp_hw(x3 - p.m);
  return p;
}

// Partial log-sum-exp of row[v0 .. v1) * inv_t over a workgroup of
// kLseThreads threads; thread 0 holds the result.  red: kLseWaves entries of
// LDS.  Every thread of the workgroup must call it.  When the row and v0 are
// 16-byte aligned the body reads 16 B per lane, two loads in flight per
// thread, then the remaining whole 16-byte groups one load at a time; only
// the last (at most 3) entries are taken one by one.
__device__ inline LsePart block_lse(const float* __restrict__ row, long v0, long v1, float inv_t, LsePart* red) {
  LsePart p{-INFINITY, 0.f};
  long v = v0;
  if (((reinterpret_cast<uintptr_t>(row + v0)) & 15u) == 0) {
    constexpr long kStep = 8L * kLseThreads;  // entries per workgroup iteration
    const long nv = (v1 - v0) / kStep * kStep;
    const float4* r4 = reinterpret_cast<const float4*>(row + v0);
    for (long q = threadIdx.x; q < nv / 4; q += 2L * kLseThreads) {
      const float4 a = r4[q], b = r4[q + kLseThreads];
      p = lse_add4(p, a.x * inv_t, a.y * inv_t, a.z * inv_t, a.w * inv_t);
      p = lse_add4(p, b.x * inv_t, b.y * inv_t, b.z * inv_t, b.w * inv_t);
    }
    // the remaining whole 16-byte groups, one per thread at a time
    const long n4 = (v1 - v0) / 4;
    for (long q = nv / 4 + threadIdx.x; q < n4; q += kLseThreads) {
      const float4 a = r4[q];
      p = lse_add4(p, a.x * inv_t, a.y * inv_t, a.z * inv_t, a.w * inv_t);
    }
    v = v0 + 4 * n4;
  }
  for (v += threadIdx.x; v < v1; v += kLseThreads) {
    const float x = row[v] * inv_t;
    if (x > p.m) {
      p.s = p.s * exp_hw(p.m - x) + 1.f;
      p.m = x;
    } else {
      p.s += exp_hw(x - p.m);
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
