// Device-side building blocks shared by the Domino kernels (gfx950 / CDNA4).
//
// Matrix-core tiles: every product in the engine is "16 rows of activations
// times 16 rows of a [out, in] weight matrix", which is exactly one
// v_mfma_f32_16x16x32_bf16 per 32 input elements (bf16 weights) or four
// v_mfma_f32_16x16x4_f32 per 16 input elements (f32 weights).  A wave64 holds
// the operands as 16 bytes per lane:
//   lane = 16 * grp + col, grp in 0..3, col in 0..15
//   weight fragment     : W[n0 + col][k0 + grp * (16 B of elements) ...]
//   activation fragment : A[m0 + col][same k range]
//   accumulator         : lane holds D[4 * grp + j][col], j = 0..3
// Both operands use the same (grp, element) -> k assignment, so the
// contraction is over exactly the 64 bytes of K starting at k0 whatever order
// the instruction uses internally.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace domino {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

struct Bf16 {
  using elem = uint16_t;
  static constexpr int kPer16B = 8;
  __device__ __forceinline__ static float to_f32(elem e) { return bf16_to_f32(e); }
};
struct F32 {
  using elem = float;
  static constexpr int kPer16B = 4;
  __device__ __forceinline__ static float to_f32(elem e) { return e; }
};

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
// Branches on it then compile to scalar branches: a matrix-core instruction
// must not sit in a branch that the compiler lowers with a per-lane EXEC mask,
// which is what happens when the wave index is left in a vector register.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// acc += A_frag (16x(64 B of K)) * W_frag^T
template <class T>
__device__ __forceinline__ f32x4 mma16(f32x4 acc, u32x4 a, u32x4 w);

template <>
__device__ __forceinline__ f32x4 mma16<Bf16>(f32x4 acc, u32x4 a, u32x4 w) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, w),
                                                 acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mma16<F32>(f32x4 acc, u32x4 a, u32x4 w) {
  f32x4 af = __builtin_bit_cast(f32x4, a), wf = __builtin_bit_cast(f32x4, w);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], wf[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], wf[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], wf[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], wf[3], acc, 0, 0, 0);
  return acc;
}

// float32 activations as a matrix-core operand matching weight type T.
// For bf16 weights the value is split as x = hi + lo (hi = x truncated to
// bf16, lo = the remainder rounded to bf16), which keeps ~16 significant bits;
// both halves are multiplied and accumulated.  For f32 weights it is exact.
template <class T>
struct ActFrag;

template <>
struct ActFrag<Bf16> {
  u32x4 hi, lo;
  // 8 consecutive floats
  __device__ __forceinline__ void from_f32(const float* x) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t u = __float_as_uint(x[e]) & 0xFFFF0000u;
      h[e] = u >> 16;
      l[e] = f32_to_bf16_rne(x[e] - __uint_as_float(u));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hi[q] = h[2 * q] | (h[2 * q + 1] << 16);
      lo[q] = l[2 * q] | (l[2 * q + 1] << 16);
    }
  }
  __device__ __forceinline__ void zero() { hi = u32x4{0, 0, 0, 0}; lo = hi; }
  __device__ __forceinline__ f32x4 mma(f32x4 acc, u32x4 w) const {
    acc = mma16<Bf16>(acc, hi, w);
    return mma16<Bf16>(acc, lo, w);
  }
};

template <>
struct ActFrag<F32> {
  u32x4 v;
  __device__ __forceinline__ void from_f32(const float* x) {
    v = u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  }
  __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ f32x4 mma(f32x4 acc, u32x4 w) const { return mma16<F32>(acc, v, w); }
};

// Buffer descriptors for raw (untyped) loads: word 3 of the descriptor, and
// the cache-policy bit of a non-temporal load.  A raw buffer load whose offset
// (lane offset + immediate) is at or past the descriptor's byte count returns
// zero without touching memory.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadNonTemporal = 2;

// ---------------------------------------------------------------------------
// Philox4x32-10 counter-based generator (Salmon et al., SC'11): ten rounds of
// two 32x32->64 multiplies, with the key advanced by two Weyl constants
// between rounds.  Counter (v >> 2, pos, b, offset), key (seed lo, seed hi).
// ---------------------------------------------------------------------------
// All four output words of the counter (ctr, pos, b, offset): the words of
// vocabulary entries 4 ctr .. 4 ctr + 3.
__device__ __forceinline__ u32x4 philox4(uint64_t seed, uint32_t offset, uint32_t b, uint32_t pos, uint32_t ctr) {
  uint32_t x0 = ctr, x1 = pos, x2 = b, x3 = offset;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // each product as one 64-bit result (one v_mad_u64_u32 instead of a
    // low and a high multiply)
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0, p1 = (uint64_t)0xCD9E8D57u * x2;
    x0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
    x1 = (uint32_t)p1;
    x2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
    x3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{x0, x1, x2, x3};
}

__device__ __forceinline__ uint32_t philox_word(uint64_t seed, uint32_t offset, uint32_t b, uint32_t pos,
                                                uint32_t v) {
  const u32x4 x = philox4(seed, offset, b, pos, v >> 2);
  const uint32_t s = v & 3u;
  return s == 0 ? x[0] : s == 1 ? x[1] : s == 2 ? x[2] : x[3];
}

// Gumbel(0,1) sample from a Philox word: U = ((w >> 9) + 1/2) 2^-23 in (0,1),
// G = -ln(-ln U).  The logarithms use the hardware base-2 logarithm (about one
// ulp) times ln 2: U is exact, G is within a few ulps of a libm evaluation,
// and this transform runs once per vocabulary entry of every sampled position.
__device__ __forceinline__ float ln_hw(float x) { return __builtin_amdgcn_logf(x) * 0.69314718055994531f; }
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  const float u = ((float)(w >> 9) + 0.5f) * 1.1920928955078125e-07f;
  return -ln_hw(-ln_hw(u));
}

// 64-bit argmax key: larger score wins, then the lower index.  The score's
// bits are mapped to an unsigned order-preserving code (negative zero is
// folded onto positive zero so that equal scores tie).  Never 0, so 0 can
// mean "no candidate yet".
__device__ __forceinline__ unsigned long long argmax_key(float s, uint32_t v) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - v);
}

__device__ __forceinline__ int32_t key_token(unsigned long long k) {
  return (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

}  // namespace domino
