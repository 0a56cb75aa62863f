// Device helpers of the on-chip draft loops, whose workgroups exchange data
// through self-validating tagged 64-bit words: {tag (high 32 bits), payload}
// written and polled with relaxed agent-scope atomics, so no fence is needed
// (a reader accepts a word only once it carries the tag it expects).  Every
// wait is bounded and also ends once another workgroup has given up.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "common.h"

namespace domino {
namespace xchg {

__device__ __forceinline__ unsigned long long ld_word(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_word(unsigned long long* p, unsigned long long w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_f32(unsigned long long* p, float v, uint32_t tag) {
  put_word(p, ((unsigned long long)tag << 32) | __float_as_uint(v));
}
__device__ __forceinline__ float word_f32(unsigned long long w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ bool gave_up(const unsigned int* status) {
  return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Polls the words src[q] (skipping null entries) until each carries `tag` in
// its high word; x[q] holds the last value read (preloaded by the caller, so
// all first loads are in flight together).  Bounded: false once `limit`
// polls have failed or another workgroup gave up; limit 0 gives up at once.
template <int N>
__device__ __forceinline__ bool settle_all(const unsigned long long* const (&src)[N], uint32_t tag,
                                          const unsigned int* status, unsigned int limit,
                                          unsigned long long (&x)[N]) {
  // every exit follows a check of every load, so no load is left in flight
  // (a later wait would otherwise cover this wave's pending stores too)
  unsigned int spins = 0;
  while (true) {
    bool done = true;
#pragma unroll
    for (int q = 0; q < N; ++q) done &= !src[q] || (uint32_t)(x[q] >> 32) == tag;
    if (done && limit != 0u) return true;
    if (++spins > limit || ((spins & 63u) == 0u && gave_up(status))) return false;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (src[q] && (uint32_t)(x[q] >> 32) != tag) x[q] = ld_word(src[q]);
  }
}

// The same for N words base[q * stride], q < n (the others are not polled).
template <int N>
__device__ __forceinline__ bool settle_strided(const unsigned long long* base, size_t stride, int n, uint32_t tag,
                                              const unsigned int* status, unsigned int limit,
                                              unsigned long long (&x)[N]) {
  unsigned int spins = 0;
  while (true) {
    bool done = true;
#pragma unroll
    for (int q = 0; q < N; ++q) done &= q >= n || (uint32_t)(x[q] >> 32) == tag;
    if (done && limit != 0u) return true;
    if (++spins > limit || ((spins & 63u) == 0u && gave_up(status))) return false;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (q < n && (uint32_t)(x[q] >> 32) != tag) x[q] = ld_word(base + (size_t)q * stride);
  }
}

// Lanes 0..n-1 of one wave poll one word each, src0 + lane * stride, until it
// carries `tag`: a cheap "probably all there" signal before every thread
// loads (and tag-checks) its words of a published block, so that the whole
// grid does not re-poll thousands of words per round.
__device__ __forceinline__ bool wait_sentinels(const unsigned long long* src0, int n, size_t stride, uint32_t tag,
                                               const unsigned int* status, unsigned int limit) {
  const int lane = threadIdx.x & 63;
  const unsigned long long* src[1] = {lane < n ? src0 + (size_t)lane * stride : nullptr};
  unsigned long long x[1] = {src[0] ? ld_word(src[0]) : 0ull};
  return settle_all(src, tag, status, limit, x);
}

// Argmax key carrying the position tag: score (32) | tag (8) | 0xFFFFFF - v (24).
__device__ __forceinline__ unsigned long long tagged_key(float s, uint32_t v, uint32_t tag) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | ((unsigned long long)(tag & 0xFFu) << 24) |
         (unsigned long long)(0xFFFFFFu - v);
}
__device__ __forceinline__ bool key_tagged(unsigned long long k, uint32_t tag) {
  return k != 0ull && ((uint32_t)(k >> 24) & 0xFFu) == (tag & 0xFFu);
}
__device__ __forceinline__ int key_index(unsigned long long k) { return (int)(0xFFFFFFu - (uint32_t)(k & 0xFFFFFFull)); }

// 64-bit max across lanes with DPP moves (no LDS round trips): within each
// 16-lane row by rotations of 8 and 4 and two quad swaps, then across the
// four rows with lane reads (the result is wave-uniform).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_step(unsigned long long x) {
  const unsigned lo = __builtin_amdgcn_update_dpp(0u, (unsigned)x, CTRL, 0xF, 0xF, false);
  const unsigned hi = __builtin_amdgcn_update_dpp(0u, (unsigned)(x >> 32), CTRL, 0xF, 0xF, false);
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  return o > x ? o : x;
}
__device__ __forceinline__ unsigned long long row_max16(unsigned long long x) {
  x = dpp_max_step<0x128>(x);  // row_ror:8
  x = dpp_max_step<0x124>(x);  // row_ror:4
  x = dpp_max_step<0x4E>(x);   // quad_perm [2,3,0,1]
  return dpp_max_step<0xB1>(x);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ unsigned long long wave_max(unsigned long long x) {
  x = row_max16(x);
  unsigned long long m = 0ull;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const unsigned long long y = ((unsigned long long)__builtin_amdgcn_readlane((unsigned)(x >> 32), row * 16) << 32) |
                                 __builtin_amdgcn_readlane((unsigned)x, row * 16);
    m = y > m ? y : m;
  }
  return m;
}

// x = hi + lo as two bf16 values: hi = x truncated to bf16, lo = the remainder
// rounded to bf16 (about 16 significant bits together).
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  const uint32_t u = __float_as_uint(x) & 0xFFFF0000u;
  hi = (uint16_t)(u >> 16);
  lo = (uint16_t)f32_to_bf16_rne(x - __uint_as_float(u));
}

}  // namespace xchg

// The on-chip loops' workgroups wait on one another, so two such loops must
// never hold compute units at the same time: one loop could then wait for
// workgroups that cannot start until the other ends.  Within the process,
// every loop launch is ordered after the previous one on the same device,
// whatever stream either runs on: the launch first waits on an event that
// marks the end of the previous loop, then hands the event to its own loop
// kernel, whose dispatch records it as it completes (an extended launch with a
// stop event: no marker of its own on the stream, which costs ~2 us between
// back-to-back calls).  Under stream capture the ordering is the graph's (the
// event is neither waited on nor recorded: the launch gets a null event).
// Loops of other processes on the same device are not ordered by this; their
// bounded waits then give up instead of hanging.
class LoopOrder {
 public:
  static LoopOrder& get() {
    static LoopOrder o;
    return o;
  }
  // Enqueues `launch(stop)` on s after every earlier loop launch of this
  // device; `launch` passes `stop` as the stop event of its loop kernel's
  // extended launch (hipExtLaunchKernelGGL), or ignores a null one.
  template <class F>
  hipError_t run(hipStream_t s, F&& launch) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return launch(static_cast<hipEvent_t>(nullptr));
    std::lock_guard<std::mutex> lock(mu_);
    if (!ev_[dev]) {
      e = hipEventCreateWithFlags(&ev_[dev], hipEventDisableTiming);
      if (e != hipSuccess) {
        ev_[dev] = nullptr;
        return e;
      }
    } else if ((e = hipStreamWaitEvent(s, ev_[dev], 0)) != hipSuccess) {
      return e;
    }
    return launch(ev_[dev]);
  }

 private:
  static constexpr int kMaxDev = 64;
  std::mutex mu_;
  hipEvent_t ev_[kMaxDev] = {};
};

}  // namespace domino
