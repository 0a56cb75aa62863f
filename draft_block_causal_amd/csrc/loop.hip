// The Domino head's serial loop on gfx950 ([notes] §二.1(2) items 1-3;
// [explainer] §四): for each of the K positions, the GRU reads the embedding
// of the previous token, the low-rank correction is added to the base logits,
// and the next token is picked.
//
// Pages: [notes] "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn);
//        [explainer] the yhxrc.cn article on the Domino paper.
//
// Each position has three phases:
//   1. gru_partial_job  - GRU pre-activations W_ih e(prev) (split over K; not
//                         needed with the GRU input table) and W_hh g on the
//                         matrix cores, one 16-row tile per wave;
//   2. GRU gates -> new state g; u = SiLU(P + W1[:, d:] g)  (gates_kernel +
//                         u_kernel when kernel boundaries order the phases,
//                         gates_u_tile in the persistent kernel);
//   3. w2_sample_block  - L = L_base + W2 u + b2 (+ Gumbel noise), vocabulary
//                         argmax as a 64-bit key max.
// Two schedules run them:
//   * three kernels per position (Plain exchange: ordinary stores, kernel
//     boundaries order the phases);
//   * one persistent cooperative kernel (Tagged exchange): every value that
//     crosses workgroups is a 64-bit word {tag, payload} written and read with
//     relaxed agent-scope atomics; a consumer spins (bounded) until each word
//     carries the tag of the current position.  No grid barrier and no memory
//     fence is needed: each word validates itself.  Exchange buffers are
//     double-buffered by position parity and cleared before every call.
//     Reuse is safe because the phases form a chain: a buffer of parity q is
//     rewritten at position i + 2 only after every reader of position i has
//     produced an input that position i + 1 waits for.
#include <algorithm>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace domino {

struct Plain {
  static constexpr bool kTagged = false;
};
struct Tagged {
  static constexpr bool kTagged = true;
};

template <class T>
struct DevLoop {
  using E = typename T::elem;
  int B, K, d, V, H, r, KS;
  const E *embed, *w_ih, *w_hh, *b_ih, *b_hh, *w1, *w2, *b2;
  const float* base;
  const float* table;  // optional GRU input table [V][3H] = W_ih E^T + b_ih (three-kernel schedule)
  const int32_t *x_t, *teacher;
  float inv_temp;
  int sampled;
  uint64_t seed;
  uint32_t offset;
  float *logits, *states, *P, *part_ih, *part_hh, *u;
  const float* ppart;  // [S][B K][r] K-slice partials of P (S > 0), else P is whole
  int S;
  unsigned long long* keys;  // [K, B]  (three-kernel schedule)
  unsigned int* ctrl;        // [1]: non-zero once a persistent-kernel wait gave up
  int32_t* tokens;
  // persistent schedule: tagged exchange buffers, each [2 (parity)][...]
  unsigned long long* xpart;  // [2][KS + 1][B][3H]: W_ih slices, then W_hh
  unsigned long long* xg;     // [2][B][H]
  unsigned long long* xu;     // [2][B][r]
  unsigned long long* xkey;   // [2][G][B]
};

// ---------------------------------------------------------------------------
// tagged words
// ---------------------------------------------------------------------------
constexpr unsigned int kSpinLimit = 1u << 20;

__device__ __forceinline__ void put_word(unsigned long long* p, unsigned long long w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_f32(unsigned long long* p, float v, uint32_t tag) {
  put_word(p, ((unsigned long long)tag << 32) | __float_as_uint(v));
}

__device__ __forceinline__ bool gave_up(const unsigned int* status) {
  return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Bounded wait until *p carries `tag` in its high 32 bits.  Returns false when
// the wait gives up (too many polls, or another workgroup already gave up).
__device__ __forceinline__ bool wait_f32(const unsigned long long* p, uint32_t tag, const unsigned int* status,
                                         float& v) {
  unsigned int spins = 0;
  for (;;) {
    const unsigned long long w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) == tag) {
      v = __uint_as_float((uint32_t)w);
      return true;
    }
    if (++spins > kSpinLimit || ((spins & 63u) == 0u && gave_up(status))) {
      v = 0.f;
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Tagged argmax key: ordered score (32) | tag (8) | 0xFFFFFF - v (24).  Among
// keys of one position the order is (score, lower index); the reader checks
// the tag.  Requires V < 2^24.
__device__ __forceinline__ unsigned long long tagged_key(float s, uint32_t v, uint32_t tag) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | ((unsigned long long)(tag & 0xFFu) << 24) |
         (unsigned long long)(0xFFFFFFu - v);
}

__device__ __forceinline__ bool key_has_tag(unsigned long long k, uint32_t tag) {
  return k != 0ull && ((uint32_t)(k >> 24) & 0xFFu) == (tag & 0xFFu);
}

__device__ __forceinline__ int tagged_key_token(unsigned long long k) {
  return (int)(0xFFFFFFu - (uint32_t)(k & 0xFFFFFFull));
}

__device__ __forceinline__ int gru_jobs(int H, int KS, int step) {
  const int T3 = (3 * H) >> 4;
  return T3 * KS + (step > 0 ? T3 : 0);
}

// ---------------------------------------------------------------------------
// Phase 1, one wave job over 16-row tiles of the stacked gate rows (3H):
//   job < T3*KS : tile t, K-slice ks of W_ih e(tok)   -> slice ks
//   otherwise   : tile t of W_hh g_{step-1}           -> slice KS
// tok[b] (LDS) is the token each batch row feeds to the GRU at this step.
// Batch rows are the matrix-core M dimension (MT tiles of 16).
// ---------------------------------------------------------------------------
template <class T, int MT, class X>
__device__ bool gru_partial_job(const DevLoop<T>& p, int step, int job, const int* tok) {
  using E = typename T::elem;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int H = p.H, d = p.d, B = p.B;
  const int T3 = (3 * H) >> 4;
  const int n_ih = T3 * p.KS;
  const int G3 = 3 * H;
  const uint32_t tag = step + 1;
  const int par = step & 1;
  bool ok = true;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int slice, n;
  if (job < n_ih) {
    const int ks = job / T3, t = job - ks * T3;
    slice = ks;
    const int kc = d / p.KS;
    n = t * 16 + col;
    const unsigned char* wrow =
        reinterpret_cast<const unsigned char*>(p.w_ih + (size_t)n * d + (size_t)ks * kc) + grp * 16;
    const unsigned char* erow[MT];
    bool live[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int b = mt * 16 + col;
      live[mt] = b < B;
      const int tk = live[mt] ? tok[b] : 0;
      erow[mt] = reinterpret_cast<const unsigned char*>(p.embed + (size_t)tk * d + (size_t)ks * kc) + grp * 16;
    }
    const int bytes = kc * (int)sizeof(E);
#pragma unroll 4
    for (int kb = 0; kb < bytes; kb += 64) {
      const u32x4 w = ld16(wrow + kb);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a = live[mt] ? ld16(erow[mt] + kb) : u32x4{0, 0, 0, 0};
        acc[mt] = mma16<T>(acc[mt], a, w);
      }
    }
  } else {
    const int t = job - n_ih;
    slice = p.KS;
    n = t * 16 + col;
    const unsigned char* wrow = reinterpret_cast<const unsigned char*>(p.w_hh + (size_t)n * H) + grp * 16;
    constexpr int EPF = T::kPer16B;  // k elements per lane per fragment
#pragma unroll 2
    for (int k0 = 0; k0 < H; k0 += 4 * EPF) {
      const u32x4 w = ld16(wrow + (size_t)k0 * sizeof(E));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int b = mt * 16 + col;
        ActFrag<T> a;
        if (b < B) {
          float x[EPF];
          if constexpr (X::kTagged) {
            const unsigned long long* src = p.xg + ((size_t)(par ^ 1) * B + b) * H + k0 + grp * EPF;
#pragma unroll
            for (int e = 0; e < EPF; ++e) ok &= wait_f32(src + e, step, p.ctrl, x[e]);
          } else {
            const float* src = p.states + ((size_t)b * p.K + step - 1) * H + k0 + grp * EPF;
#pragma unroll
            for (int e = 0; e < EPF; e += 4) {
              const f32x4 v = *reinterpret_cast<const f32x4*>(src + e);
              x[e] = v[0];
              x[e + 1] = v[1];
              x[e + 2] = v[2];
              x[e + 3] = v[3];
            }
          }
          a.from_f32(x);
        } else {
          a.zero();
        }
        acc[mt] = a.mma(acc[mt], w);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = mt * 16 + grp * 4 + j;
      if (b < B) {
        if constexpr (X::kTagged) {
          put_f32(p.xpart + (((size_t)par * (p.KS + 1) + slice) * B + b) * G3 + n, acc[mt][j], tag);
        } else if (slice < p.KS) {
          p.part_ih[((size_t)slice * B + b) * G3 + n] = acc[mt][j];
        } else {
          p.part_hh[(size_t)b * G3 + n] = acc[mt][j];
        }
      }
    }
  return ok;
}

// ---------------------------------------------------------------------------
// Phase 2 for bottleneck rows 16t..16t+15 (one 256-thread workgroup).  For each
// slice of 16 batch rows it recomputes the new GRU state of those rows (every
// participating workgroup computes identical values; t == 0 stores them),
// then u = SiLU(P + W1[:, d:] g).  LDS: 16 x (H + 4) floats + 4 KB.
// ---------------------------------------------------------------------------
template <class T, class X>
__device__ bool gates_u_tile(const DevLoop<T>& p, int step, int t, unsigned char* smem) {
  using E = typename T::elem;
  const int H = p.H, B = p.B, G3 = 3 * H, KS = p.KS;
  float* gt = reinterpret_cast<float*>(smem);  // [16][H + 4]
  const int gstride = H + 4;
  float* red = gt + 16 * gstride;  // [4][16][16]
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int ldw1 = p.d + H;
  constexpr int EPF = T::kPer16B;
  const uint32_t tag = step + 1;
  const int par = step & 1;
  bool ok = true;

  for (int m0 = 0; m0 < B; m0 += 16) {
    for (int idx = threadIdx.x; idx < 16 * H; idx += blockDim.x) {
      const int rr = idx / H, j = idx - rr * H;
      const int b = m0 + rr;
      float g = 0.f;
      if (b < B) {
        float a3[3] = {0.f, 0.f, 0.f}, c3[3] = {0.f, 0.f, 0.f}, gp = 0.f;
        for (int q = 0; q < 3; ++q) {
          for (int ks = 0; ks < KS; ++ks) {
            float x;
            if constexpr (X::kTagged) {
              ok &= wait_f32(p.xpart + (((size_t)par * (KS + 1) + ks) * B + b) * G3 + q * H + j, tag, p.ctrl, x);
            } else {
              x = p.part_ih[((size_t)ks * B + b) * G3 + q * H + j];
            }
            a3[q] += x;
          }
          if (step > 0) {
            if constexpr (X::kTagged) {
              ok &= wait_f32(p.xpart + (((size_t)par * (KS + 1) + KS) * B + b) * G3 + q * H + j, tag, p.ctrl, c3[q]);
            } else {
              c3[q] = p.part_hh[(size_t)b * G3 + q * H + j];
            }
          }
          if (p.b_ih) a3[q] += T::to_f32(p.b_ih[q * H + j]);
          if (p.b_hh) c3[q] += T::to_f32(p.b_hh[q * H + j]);
        }
        if (step > 0) {
          if constexpr (X::kTagged) {
            ok &= wait_f32(p.xg + ((size_t)(par ^ 1) * B + b) * H + j, step, p.ctrl, gp);
          } else {
            gp = p.states[((size_t)b * p.K + step - 1) * H + j];
          }
        }
        const float rg = sigmoidf_(a3[0] + c3[0]);
        const float zg = sigmoidf_(a3[1] + c3[1]);
        const float ng = tanhf(a3[2] + rg * c3[2]);
        g = (1.f - zg) * ng + zg * gp;
        if (t == 0) {
          p.states[((size_t)b * p.K + step) * H + j] = g;
          if constexpr (X::kTagged) put_f32(p.xg + ((size_t)par * B + b) * H + j, g, tag);
        }
      }
      gt[rr * gstride + j] = g;
    }
    if constexpr (X::kTagged) {
      if (__syncthreads_or(!ok)) return false;
    } else {
      __syncthreads();
    }

    // u rows t*16 + col; the four waves take interleaved 64-byte K chunks
    const int row = t * 16 + col;
    const unsigned char* wrow =
        reinterpret_cast<const unsigned char*>(p.w1 + (size_t)row * ldw1 + p.d) + grp * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = wave * 4 * EPF; k0 < H; k0 += 16 * EPF) {
      const u32x4 w = ld16(wrow + (size_t)k0 * sizeof(E));
      ActFrag<T> a;
      a.from_f32(gt + col * gstride + k0 + grp * EPF);
      acc = a.mma(acc, w);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(wave * 16 + grp * 4 + j) * 16 + col] = acc[j];
    __syncthreads();
    {
      const int rr = threadIdx.x >> 4, c = threadIdx.x & 15;
      const int b = m0 + rr;
      if (b < B) {
        const float s = red[(0 * 16 + rr) * 16 + c] + red[(1 * 16 + rr) * 16 + c] +
                        red[(2 * 16 + rr) * 16 + c] + red[(3 * 16 + rr) * 16 + c];
        const int q = t * 16 + c;
        const float pre = p.P[((size_t)b * p.K + step) * p.r + q] + s;
        const float uv = pre * sigmoidf_(pre);
        if constexpr (X::kTagged)
          put_f32(p.xu + ((size_t)par * B + b) * p.r + q, uv, tag);
        else
          p.u[(size_t)b * p.r + q] = uv;
      }
    }
    __syncthreads();
  }
  return true;
}

template <class T>
__host__ __device__ constexpr int act_parts() {
  return (int)(sizeof(ActFrag<T>) / 16);  // bf16 weights: (hi, lo) pair; f32: one
}

template <class T>
__host__ __device__ inline size_t w2_lds_bytes(int r, int rows) {
  return (size_t)act_parts<T>() * rows * (r * sizeof(typename T::elem) + 16) + 4 * rows * sizeof(unsigned long long);
}

__host__ __device__ inline size_t gates_lds_bytes(int H) { return 16 * (size_t)(H + 4) * sizeof(float) + 4096; }

// ---------------------------------------------------------------------------
// Phase 3 for batch rows m0 .. m0 + 16*MT - 1 and vocabulary tiles
// bx, bx + nbx, ... (one 256-thread workgroup).  u is staged in LDS as
// matrix-core operands; each wave streams 16-row tiles of W2, adds b2 and the
// base logits, optionally stores the logits, draws Gumbel noise, and keeps a
// running argmax key per batch row; keys are reduced across lanes and waves.
// Plain: merged into keys[step][b] with a 64-bit atomic max.  Tagged: the
// workgroup's key is published in xkey[parity][bx][b].
// ---------------------------------------------------------------------------
template <class T, int MT, class X>
__device__ bool w2_sample_block(const DevLoop<T>& p, int step, int bx, int nbx, int m0, unsigned char* smem) {
  using E = typename T::elem;
  constexpr int EPF = T::kPer16B;
  constexpr int NPARTS = act_parts<T>();
  const int B = p.B, V = p.V, r = p.r;
  const int row_bytes = r * (int)sizeof(E);
  const int lds_stride = row_bytes + 16;
  constexpr int rows = 16 * MT;
  const uint32_t tag = step + 1;
  const int par = step & 1;
  unsigned long long* kred = reinterpret_cast<unsigned long long*>(smem + NPARTS * rows * lds_stride);
  bool ok = true;

  for (int idx = threadIdx.x; idx < rows * (r / EPF); idx += blockDim.x) {
    const int rr = idx / (r / EPF), c = idx - rr * (r / EPF);
    const int b = m0 + rr;
    ActFrag<T> a;
    if (b < B) {
      float x[EPF];
      if constexpr (X::kTagged) {
        const unsigned long long* src = p.xu + ((size_t)par * B + b) * r + c * EPF;
#pragma unroll
        for (int e = 0; e < EPF; ++e) ok &= wait_f32(src + e, tag, p.ctrl, x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < EPF; ++e) x[e] = p.u[(size_t)b * r + c * EPF + e];
      }
      a.from_f32(x);
    } else {
      a.zero();
    }
    const u32x4* parts = reinterpret_cast<const u32x4*>(&a);
#pragma unroll
    for (int q = 0; q < NPARTS; ++q) st16(smem + (q * rows + rr) * lds_stride + c * 16, parts[q]);
  }
  if constexpr (X::kTagged) {
    if (__syncthreads_or(!ok)) return false;
  } else {
    __syncthreads();
  }

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int ntiles = (V + 15) >> 4;
  unsigned long long best[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) best[mt][j] = 0ull;

  for (int t = bx * 4 + wave; t < ntiles; t += nbx * 4) {
    const int v = t * 16 + col;
    const unsigned char* wrow = reinterpret_cast<const unsigned char*>(p.w2 + (size_t)min(v, V - 1) * r) + grp * 16;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int kb = 0; kb < row_bytes; kb += 64) {
      const u32x4 w = ld16(wrow + kb);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NPARTS; ++q) {
          const u32x4 a = ld16(smem + (q * rows + mt * 16 + col) * lds_stride + grp * 16 + kb);
          acc[mt] = mma16<T>(acc[mt], a, w);
        }
    }
    if (v < V) {
      const float bv = p.b2 ? T::to_f32(p.b2[v]) : 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int b = m0 + mt * 16 + grp * 4 + j;
          if (b < B) {
            const size_t o = ((size_t)b * p.K + step) * V + v;
            const float L = p.base[o] + (acc[mt][j] + bv);
            if (p.logits) p.logits[o] = L;
            float s = L;
            if (p.sampled) s = L * p.inv_temp + gumbel_from_word(philox_word(p.seed, p.offset, b, step, v));
            const unsigned long long k = X::kTagged ? tagged_key(s, v, tag) : argmax_key(s, v);
            best[mt][j] = k > best[mt][j] ? k : best[mt][j];
          }
        }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      unsigned long long k = best[mt][j];
#pragma unroll
      for (int sh = 1; sh < 16; sh <<= 1) {
        const unsigned long long o = __shfl_xor(k, sh, 64);
        k = o > k ? o : k;
      }
      best[mt][j] = k;
    }
  if (col == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) kred[wave * rows + mt * 16 + grp * 4 + j] = best[mt][j];
  }
  __syncthreads();
  for (int rr = threadIdx.x; rr < rows; rr += blockDim.x) {
    unsigned long long k = kred[rr];
    for (int w = 1; w < 4; ++w) k = kred[w * rows + rr] > k ? kred[w * rows + rr] : k;
    const int b = m0 + rr;
    if (b < B) {
      if constexpr (X::kTagged) {
        // a workgroup without vocabulary tiles still publishes a tagged (lowest) key
        if (k == 0ull) k = (unsigned long long)(tag & 0xFFu) << 24;
        put_word(p.xkey + ((size_t)par * nbx + bx) * B + b, k);
      } else if (k != 0ull) {
        atomicMax(p.keys + (size_t)step * B + b, k);
      }
    }
  }
  __syncthreads();  // LDS is reused by the caller
  return true;
}

// ---------------------------------------------------------------------------
// Plain-schedule phase 3 for B > 1: batch rows m0 .. m0 + 16 MT - 1 (grid.y)
// against vocabulary tiles t = 4 blockIdx.x + wave, stepping by 4 gridDim.x.
// u is staged in LDS as matrix-core operands.  Each wave reads the NS 64-B
// K steps of its next tile of W2 (and that tile's base logits and b2) while
// it multiplies the current one: buffer descriptors sized to the valid rows
// make the loads past the last tile read zero, so every load is
// unconditional, and two register sets alternate.  Each 16 x 16 product tile
// is turned through a wave-private LDS patch so that a lane holds one batch
// row and four consecutive vocabulary entries: one Philox counter gives the
// four words it needs.  Argmax keys are reduced over lanes and waves and
// merged into keys[step][b] with a 64-bit atomic max.
// ---------------------------------------------------------------------------
template <class T>
__device__ void hh_unit(const DevLoop<T>& p, int step, int t, int m0);
template <class T, int NT, int MT>
__device__ void hh_block(const DevLoop<T>& p, int step, int n0, int m0, float* red);
// W_hh tiling of the W2 launch's units: 16 NT gate rows x 16 MT batch rows,
// and the LDS bytes of their reduction.  64 x 32 only where the W2 tile loop
// already runs two waves per SIMD (64-row slices); with 16- and 32-row
// slices 32 x 16 (more accumulators would take the launch from three waves
// per SIMD to two).
template <int MW>
struct HhTiling {
  static constexpr int NT = MW >= 4 ? 4 : 2, MT = MW >= 4 ? 2 : 1;
  static constexpr size_t kRedBytes = (size_t)4 * 16 * MT * (16 * NT + 1) * sizeof(float);
};

// VEC (V % 16 == 0: no partial tile, rows 16-B aligned): a lane's four base
// logits are one 16-B load and its four b2 entries one 8-B (bf16) load.
// LG: the logits are stored too (the caller asked for them).
// Workgroups x < gx_w2 of each batch slice stream W2.  hh_step > 0: the
// 3H/16 x ceil(B/16) 16 x 16 units of W_hh g for position hh_step (g of this
// position is final) are formed here too, which takes that product off the
// token-to-token path: by the workgroups x >= gx_w2, which do nothing else,
// when the grid has them, else by the W2 workgroups before their tiles
// (unit q in workgroup q mod the grid size).
template <class T, int MT, int NS, bool VEC, int D, bool LG>
__global__ void __launch_bounds__(256) w2_stream_kernel(DevLoop<T> p, int step, int hh_step, int gx_w2) {
  using E = typename T::elem;
  constexpr int EPF = T::kPer16B;
  constexpr int NPARTS = act_parts<T>();
  constexpr int rows = 16 * MT;
  constexpr int row_bytes = NS * 64;  // r * sizeof(E)
  constexpr int lds_stride = row_bytes + 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* tr = reinterpret_cast<float*>(smem + NPARTS * rows * lds_stride);          // [4][16][17]
  unsigned long long* kred = reinterpret_cast<unsigned long long*>(tr + 4 * 16 * 17);  // [4][rows]
  const int B = p.B, V = p.V, r = p.r, K = p.K;
  const int m0 = blockIdx.y * rows;
  // (trip counts are uniform over the workgroup: hh_unit synchronises it)
  const int hx = gridDim.x - gx_w2;  // W_hh-only workgroups per batch slice
  if (hh_step > 0) {
    // units of HhTiling<MT>::NT x ::MT 16-row tiles; the reduction uses the
    // LDS that u is staged into below
    using HT = HhTiling<MT>;
    const int tn = (3 * p.H + 16 * HT::NT - 1) / (16 * HT::NT);
    const int units = tn * ((B + 16 * HT::MT - 1) / (16 * HT::MT));
    float* hred = reinterpret_cast<float*>(smem);
    if (hx == 0) {
      for (int unit = blockIdx.y * gridDim.x + blockIdx.x; unit < units; unit += gridDim.x * gridDim.y)
        hh_block<T, HT::NT, HT::MT>(p, hh_step, (unit % tn) * 16 * HT::NT, (unit / tn) * 16 * HT::MT, hred);
    } else if ((int)blockIdx.x >= gx_w2) {
      for (int unit = blockIdx.y * hx + (blockIdx.x - gx_w2); unit < units; unit += hx * gridDim.y)
        hh_block<T, HT::NT, HT::MT>(p, hh_step, (unit % tn) * 16 * HT::NT, (unit / tn) * 16 * HT::MT, hred);
    }
  }
  if ((int)blockIdx.x >= gx_w2) return;

  // u rows -> LDS operands; each thread's fragments (rows * NS * 4 / 256 of
  // them, r = NS * 64 / sizeof(E) entries per row) are all loaded first
  {
    constexpr int kFrags = rows * NS * 4;  // EPF-entry fragments of the staged rows
    constexpr int kPer = (kFrags + 255) / 256;
    float x[kPer][EPF];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int idx = threadIdx.x + q * 256;
      const int rr = idx / (NS * 4), c = idx - rr * (NS * 4);
      const bool live = idx < kFrags && m0 + rr < B;
#pragma unroll
      for (int e = 0; e < EPF; e += 4) {
        const f32x4 v = live ? *reinterpret_cast<const f32x4*>(p.u + (size_t)(m0 + rr) * r + c * EPF + e)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
        x[q][e] = v[0];
        x[q][e + 1] = v[1];
        x[q][e + 2] = v[2];
        x[q][e + 3] = v[3];
      }
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int idx = threadIdx.x + q * 256;
      if (idx < kFrags) {
        const int rr = idx / (NS * 4), c = idx - rr * (NS * 4);
        ActFrag<T> a;
        a.from_f32(x[q]);
        const u32x4* parts = reinterpret_cast<const u32x4*>(&a);
#pragma unroll
        for (int pq = 0; pq < NPARTS; ++pq) st16(smem + (pq * rows + rr) * lds_stride + c * 16, parts[pq]);
      }
    }
  }
  __syncthreads();

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int eb = lane >> 2, eq = lane & 3;  // epilogue: batch row eb of a tile, entries 4 eq .. 4 eq + 3
  float* trw = tr + wave * 16 * 17;
  const int ntiles = (V + 15) >> 4;
  const int stride = __builtin_amdgcn_readfirstlane(gx_w2 * 4);  // (computed in a vector register otherwise)
  const int woff = col * row_bytes + grp * 16;
  // base logits of this position for the 16 batch rows of slice mt: one
  // descriptor per slice, based at its first row and ending after the last
  // batch row's V entries; lane offsets (eb K V + v) * 4 (checked on the host
  // to fit 31 bits)
  __amdgpu_buffer_rsrc_t brs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int live = min(max(B - (m0 + mt * 16), 0), 16);
    brs[mt] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.base + (live > 0 ? ((size_t)(m0 + mt * 16) * K + step) * V : 0)), (short)0,
        live > 0 ? ((live - 1) * K * V + V) * 4 : 0, kRsrcWord3);
  }
  const int boff = eb * K * V * 4;
  // the logits (when the caller asks for them) share that layout: rows past
  // the batch, and with a null pointer every row, lie past the descriptor's
  // end, where stores are dropped
  __amdgpu_buffer_rsrc_t lrs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int live = p.logits ? min(max(B - (m0 + mt * 16), 0), 16) : 0;
    lrs[mt] = __builtin_amdgcn_make_buffer_rsrc(p.logits + (live > 0 ? ((size_t)(m0 + mt * 16) * K + step) * V : 0),
                                                (short)0, live > 0 ? ((live - 1) * K * V + V) * 4 : 0, kRsrcWord3);
  }
  const __amdgpu_buffer_rsrc_t b2rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<E*>(p.b2 ? p.b2 : p.w2), (short)0, p.b2 ? V * (int)sizeof(E) : 0, kRsrcWord3);

  struct Stage {
    u32x4 w[NS];
    float base[MT][4];
    float b2[4];
  };
  auto load = [&](int t, Stage& st) {
    const int nrows = t < ntiles ? min(16, V - t * 16) : 0;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E*>(p.w2 + (t < ntiles ? (size_t)t * 16 * r : 0)), (short)0, nrows * row_bytes, kRsrcWord3);
#pragma unroll
    for (int kb = 0; kb < NS; ++kb) st.w[kb] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + kb * 64, 0, 0);
    const int v0 = t * 16 + 4 * eq;  // past V (or a dead tile): reads zero
    if constexpr (VEC) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(brs[mt], boff + v0 * 4, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.base[mt][i] = __uint_as_float(q[i]);
      }
      if constexpr (sizeof(E) == 2) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b64(b2rs, v0 * 2, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.b2[i] = __uint_as_float(((q[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16);
      } else {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(b2rs, v0 * 4, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.b2[i] = __uint_as_float(q[i]);
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st.base[mt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brs[mt], boff + (v0 + i) * 4, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned bits = sizeof(E) == 2 ? (unsigned)__builtin_amdgcn_raw_buffer_load_b16(b2rs, (v0 + i) * 2, 0, 0)
                                             : __builtin_amdgcn_raw_buffer_load_b32(b2rs, (v0 + i) * 4, 0, 0);
        st.b2[i] = sizeof(E) == 2 ? __uint_as_float(bits << 16) : __uint_as_float(bits);
      }
    }
  };
  unsigned long long best[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) best[mt] = 0ull;
  auto process = [&](int t, const Stage& st) {
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // u's operands come from LDS in the order (K step, slice, part); kAhead
    // reads stay in flight ahead of the product that takes them (read one at a
    // time, every product waited out a read's latency), the order pinned by
    // scheduling barriers
    constexpr int kF = NS * MT * NPARTS, kAhead = kF < 8 ? kF : 8;
    auto frag = [&](int i) {
      const int kb = i / (MT * NPARTS), mt = (i / NPARTS) % MT, q = i % NPARTS;
      return ld16(smem + (q * rows + mt * 16 + col) * lds_stride + grp * 16 + kb * 64);
    };
    u32x4 a[kF];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) a[i] = frag(i);
#pragma unroll
    for (int i = 0; i < kF; ++i) {
      if (i + kAhead < kF) a[i + kAhead] = frag(i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
      acc[(i / NPARTS) % MT] = mma16<T>(acc[(i / NPARTS) % MT], a[i], st.w[i / (MT * NPARTS)]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int v0 = t * 16 + 4 * eq;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) trw[(grp * 4 + j) * 17 + col] = acc[mt][j];
      const f32x4 d = f32x4{trw[eb * 17 + 4 * eq], trw[eb * 17 + 4 * eq + 1], trw[eb * 17 + 4 * eq + 2],
                            trw[eb * 17 + 4 * eq + 3]};
      // branch-free over the lanes (rows past the batch and entries past V
      // give no key): loads that only one side of a branch consumed would make
      // the compiler wait for them before the next prefetch reuses the registers
      const int b = m0 + mt * 16 + eb;
      float L[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) L[i] = st.base[mt][i] + (d[i] + st.b2[i]);
      // stores through the descriptor: no per-lane branch (entries past V get
      // an offset past its end)
      if constexpr (LG) {
        if constexpr (VEC) {
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{__float_as_uint(L[0]), __float_as_uint(L[1]), __float_as_uint(L[2]), __float_as_uint(L[3])},
              lrs[mt], boff + v0 * 4, 0, 0);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L[i]), lrs[mt],
                                                  v0 + i < V ? boff + (v0 + i) * 4 : (int)0x80000000u, 0, 0);
        }
      }
      // one uniform branch for the four entries' scores
      float sc[4];
      if (p.sampled) {
        const u32x4 words = philox4(p.seed, p.offset, (uint32_t)b, (uint32_t)step, (uint32_t)(v0 >> 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = L[i] * p.inv_temp + gumbel_from_word(words[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = L[i];
      }
      // lanes of rows past the batch keep keys that are never merged (the
      // reduction below skips those rows); entries past V (a partial last
      // tile) give no key
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        unsigned long long k = argmax_key(sc[i], (uint32_t)(v0 + i));
        if constexpr (!VEC) k = v0 + i < V ? k : 0ull;
        best[mt] = k > best[mt] ? k : best[mt];
      }
    }
  };

  // A ring of D register stages: the tiles D - 1 strides ahead are in flight
  // while a tile is multiplied (every load unconditional, so the compiler's
  // count of loads in flight stays exact).  (t is kept in a scalar register:
  // the descriptors built from it must be.)
  Stage st[D];
  int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load(t + i * stride, st[i]);
  while (t < ntiles) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      load(t + (D - 1) * stride, st[(i + D - 1) % D]);
      __builtin_amdgcn_sched_barrier(0);
      process(t, st[i]);
      t = __builtin_amdgcn_readfirstlane(t + stride);
      if (t >= ntiles) break;
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    unsigned long long k = best[mt];
#pragma unroll
    for (int sh = 1; sh < 4; sh <<= 1) {
      const unsigned long long o = __shfl_xor(k, sh, 64);
      k = o > k ? o : k;
    }
    if (eq == 0) kred[wave * rows + mt * 16 + eb] = k;
  }
  __syncthreads();
  for (int rr = threadIdx.x; rr < rows; rr += blockDim.x) {
    unsigned long long k = kred[rr];
    for (int w = 1; w < 4; ++w) k = kred[w * rows + rr] > k ? kred[w * rows + rr] : k;
    const int b = m0 + rr;
    if (b < B && k != 0ull) atomicMax(p.keys + (size_t)step * B + b, k);
  }
}

template <class T, int MT>
__host__ __device__ inline size_t w2_stream_lds_bytes(int r) {
  return (size_t)act_parts<T>() * 16 * MT * (r * sizeof(typename T::elem) + 16) + 4 * 16 * 17 * sizeof(float) +
         4 * 16 * MT * sizeof(unsigned long long);
}

// ---------------------------------------------------------------------------
// Plain-schedule phase 2, split in two launches:
//   gates_kernel - one thread per (batch row, GRU unit): the gates from the
//                  phase-1 partials (or the GRU input table row of the token)
//                  and the previous state -> states[b][step];
//   u_kernel     - u rows 16t..16t+15 for batch rows 16m..16m+15:
//                  SiLU(P + W1[:, d:] g) on the matrix cores.
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ int step_token(const DevLoop<T>& p, int step, int b) {
  int tk;
  if (step == 0)
    tk = p.x_t[b];
  else if (p.teacher)
    tk = p.teacher[(size_t)b * p.K + step - 1];
  else
    tk = key_token(p.keys[(size_t)(step - 1) * p.B + b]);
  return min(max(tk, 0), p.V - 1);
}

template <class T>
__global__ void __launch_bounds__(256) gates_kernel(DevLoop<T> p, int step) {
  const int H = p.H, G3 = 3 * H, KS = p.KS;
  const int b = blockIdx.y, j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= H) return;
  // the loads that do not depend on the token first, so that they are in
  // flight with the token's key load and the table row read after it
  float a3[3], c3[3] = {0.f, 0.f, 0.f};
  float gp = 0.f;
  if (step > 0) {
#pragma unroll
    for (int q = 0; q < 3; ++q) c3[q] = p.part_hh[(size_t)b * G3 + q * H + j];
    gp = p.states[((size_t)b * p.K + step - 1) * H + j];
  }
  // b_hh loaded unconditionally (from W_hh, 3H x H elements, when there is
  // no bias) and selected after: a load on one side of a branch made the
  // compiler wait for every load in flight after each
  const typename T::elem* bsrc = p.b_hh ? p.b_hh : p.w_hh;
  float bh[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const float v = T::to_f32(bsrc[q * H + j]);
    bh[q] = p.b_hh ? v : 0.f;
  }
  if (p.table) {
    const float* trow = p.table + (size_t)step_token(p, step, b) * G3;
#pragma unroll
    for (int q = 0; q < 3; ++q) a3[q] = trow[q * H + j];
  } else {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      float x = 0.f;
      for (int ks = 0; ks < KS; ++ks) x += p.part_ih[((size_t)ks * p.B + b) * G3 + q * H + j];
      a3[q] = x + (p.b_ih ? T::to_f32(p.b_ih[q * H + j]) : 0.f);
    }
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) c3[q] += bh[q];
  const float rg = sigmoidf_(a3[0] + c3[0]);
  const float zg = sigmoidf_(a3[1] + c3[1]);
  const float ng = tanhf(a3[2] + rg * c3[2]);
  p.states[((size_t)b * p.K + step) * H + j] = (1.f - zg) * ng + zg * gp;
}

// One wave's share of a 16 x 16 tile of W X^T: W rows wrow (lane column =
// output row, 16 B of K per lane), X rows xrow (fp32, lane column = batch
// row; null for a row past the batch), over matrix-core K steps s0 .. s0 + U - 1
// (steps past nsteps add zero).  Every load of the U steps is issued before
// the first product.
template <class T, int U>
__device__ __forceinline__ f32x4 wave_rows_dot(f32x4 acc, const unsigned char* wrow, const float* xrow, int s0,
                                               int nsteps) {
  using E = typename T::elem;
  constexpr int EPF = T::kPer16B;
  constexpr int KSTEP = 4 * EPF;
  u32x4 w[U];
  float x[U][EPF];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int s = s0 + u;
    const bool in = s < nsteps;
    w[u] = in ? ld16(wrow + (size_t)s * KSTEP * sizeof(E)) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < EPF; e += 4) {
      const f32x4 v = in && xrow ? *reinterpret_cast<const f32x4*>(xrow + s * KSTEP + e) : f32x4{0.f, 0.f, 0.f, 0.f};
      x[u][e] = v[0];
      x[u][e + 1] = v[1];
      x[u][e + 2] = v[2];
      x[u][e + 3] = v[3];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    ActFrag<T> a;
    a.from_f32(x[u]);
    acc = a.mma(acc, w[u]);
  }
  return acc;
}

// 16 output rows (W rows n0 .. n0 + 15) for batch rows m0 .. m0 + 15 of
// W[:, :ncols] X^T, with the 4 waves of a workgroup taking consecutive ranges
// of K steps; returns, for thread tid < 256, the sum for batch row m0 + tid / 16
// and output row n0 + tid % 16 (the four wave partials added in a fixed order).
template <class T>
__device__ __forceinline__ float block_rows_dot(const typename T::elem* W, int ldw, int n0, const float* X, int ldx,
                                                int m0, int B, int ncols) {
  using E = typename T::elem;
  constexpr int U = 8;
  constexpr int KSTEP = 4 * T::kPer16B;
  __shared__ float red[4][16][17];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int nsteps = ncols / KSTEP;
  const unsigned char* wrow = reinterpret_cast<const unsigned char*>(W + (size_t)(n0 + col) * ldw) + grp * 16;
  const float* xrow = m0 + col < B ? X + (size_t)(m0 + col) * ldx + grp * T::kPer16B : nullptr;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int per_wave = (nsteps + 3) / 4;
  for (int s0 = wave * per_wave; s0 < min(nsteps, (wave + 1) * per_wave); s0 += U)
    acc = wave_rows_dot<T, U>(acc, wrow, xrow, s0, min(nsteps, (wave + 1) * per_wave));
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wave][grp * 4 + j][col] = acc[j];
  __syncthreads();
  const int mm = (threadIdx.x >> 4) & 15, nn = threadIdx.x & 15;
  return red[0][mm][nn] + red[1][mm][nn] + red[2][mm][nn] + red[3][mm][nn];
}

// u rows 16t .. 16t+15 for batch rows 16m .. 16m+15: SiLU(P + W1[:, d:] g).
template <class T>
__global__ void __launch_bounds__(256) u_kernel(DevLoop<T> p, int step) {
  const int t = blockIdx.x, m0 = blockIdx.y * 16;
  const int b = m0 + (threadIdx.x >> 4), q = t * 16 + (threadIdx.x & 15);
  const size_t row = ((size_t)b * p.K + step) * p.r + q;
  // P (whole, or its S slices added in order) is read before the product, so
  // that its loads are in flight with the product's: the first kPReg slices
  // each into a register of its own (with a runtime trip count the compiler
  // waits for each load before issuing the next), added after the product
  constexpr int kPReg = 8;
  float pr[kPReg];
#pragma unroll
  for (int sl = 0; sl < kPReg; ++sl)
    pr[sl] = b < p.B && (sl < p.S || (sl == 0 && p.S == 0))
                 ? (p.S > 0 ? p.ppart[(size_t)sl * p.B * p.K * p.r + row] : p.P[row])
                 : 0.f;
  // batch row b's state at this position: states[b][step][:], row stride K * H
  const float sum = block_rows_dot<T>(p.w1 + p.d, p.d + p.H, t * 16, p.states + (size_t)step * p.H, p.K * p.H, m0,
                                      p.B, p.H);
  if (b < p.B) {
    float ph = 0.f;
#pragma unroll
    for (int sl = 0; sl < kPReg; ++sl) ph += pr[sl];  // slices past S are zero
    for (int sl = kPReg; sl < p.S; ++sl) ph += p.ppart[(size_t)sl * p.B * p.K * p.r + row];
    const float pre = ph + sum;
    p.u[(size_t)b * p.r + q] = pre * sigmoidf_(pre);
  }
}

// W_hh g_{step-1}: gate rows 16t .. 16t+15 for batch rows m0 .. m0+15 (one
// workgroup; every thread must call it).
template <class T>
__device__ void hh_unit(const DevLoop<T>& p, int step, int t, int m0) {
  const float sum = block_rows_dot<T>(p.w_hh, p.H, t * 16, p.states + (size_t)(step - 1) * p.H, p.K * p.H, m0, p.B,
                                      p.H);
  const int b = m0 + (threadIdx.x >> 4), n = t * 16 + (threadIdx.x & 15);
  if (b < p.B) p.part_hh[(size_t)b * 3 * p.H + n] = sum;
  __syncthreads();  // the reduction buffer is reused by the caller
}

template <class T>
__global__ void __launch_bounds__(256) hh_kernel(DevLoop<T> p, int step) {
  hh_unit(p, step, blockIdx.x, blockIdx.y * 16);
}

// W_hh g_{step-1} for gate rows n0 .. n0 + 16 NT - 1 and batch rows m0 ..
// m0 + 16 MT - 1 (one workgroup; every thread must call it; red: LDS for
// 4 x 16 MT x (16 NT + 1) floats).  A unit of 16 rows x 16 rows reads its
// 16 state rows (64 KB at H = 1024) for 16 gate rows of W_hh (32 KB); this
// one reads 16 MT state rows for 16 NT gate rows, so the states are read
// 3H / (16 NT) times per position instead of 3H / 16 (Qwen3 heads, 128
// blocks: 147 MB of cache traffic a position with 16 x 16 units, 49 MB with
// 64 x 32).  Same sums as hh_unit, in the same order: each wave one
// contiguous quarter of K in step order, the four partials added in wave
// order.  U steps of loads are in flight at once (addresses clamped, so
// every load is unconditional).
template <class T, int NT, int MT>
__device__ void hh_block(const DevLoop<T>& p, int step, int n0, int m0, float* red) {
  using E = typename T::elem;
  constexpr int EPF = T::kPer16B;
  constexpr int KSTEP = 4 * EPF;
  // steps of loads in flight: 128 VGPRs of operands, within the registers of
  // the W2 launch's tile loop (2 steps before: Qwen3-8B draft call at 128
  // blocks 1.033 -> 1.021 ms, unchanged at 32)
  constexpr int U = 128 / (4 * NT + MT * EPF) < 1 ? 1 : 128 / (4 * NT + MT * EPF);
  const int H = p.H, G3 = 3 * H;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int nsteps = H / KSTEP, per_wave = (nsteps + 3) / 4;
  const int s_begin = wave * per_wave, s_end = min(nsteps, s_begin + per_wave);
  const unsigned char* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    wrow[nt] = reinterpret_cast<const unsigned char*>(p.w_hh + (size_t)min(n0 + nt * 16 + col, G3 - 1) * H) + grp * 16;
  const float* X = p.states + (size_t)(step - 1) * H;
  const float* xrow[MT];
  bool xlive[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int b = m0 + mt * 16 + col;
    xlive[mt] = b < p.B;
    xrow[mt] = X + (size_t)min(b, p.B - 1) * p.K * H + grp * EPF;
  }
  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_begin; s0 < s_end; s0 += U) {
    u32x4 w[U][NT];
    float x[U][MT][EPF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u, s_end - 1);  // past s_end: a repeated step, multiplied by zero below
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w[u][nt] = ld16(wrow[nt] + (size_t)s * KSTEP * sizeof(E));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < EPF; e += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(xrow[mt] + s * KSTEP + e);
          x[u][mt][e] = v[0];
          x[u][mt][e + 1] = v[1];
          x[u][mt][e + 2] = v[2];
          x[u][mt][e + 3] = v[3];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = s0 + u < s_end;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float xs[EPF];
#pragma unroll
        for (int e = 0; e < EPF; ++e) xs[e] = in && xlive[mt] ? x[u][mt][e] : 0.f;
        ActFrag<T> a;
        a.from_f32(xs);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = a.mma(acc[nt][mt], w[u][nt]);
      }
    }
  }
  // partials [wave][batch row][gate row]
  constexpr int RS = 16 * NT + 1;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[(wave * 16 * MT + mt * 16 + grp * 4 + j) * RS + nt * 16 + col] = acc[nt][mt][j];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * MT * 16 * NT; i += blockDim.x) {
    const int mm = i / (16 * NT), nn = i - mm * (16 * NT);
    const int b = m0 + mm, n = n0 + nn;
    float sum = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) sum += red[(wv * 16 * MT + mm) * RS + nn];
    if (b < p.B && n < G3) p.part_hh[(size_t)b * G3 + n] = sum;
  }
  __syncthreads();  // red is reused by the caller
}


// ---------------------------------------------------------------------------
// three-kernels-per-position schedule
// ---------------------------------------------------------------------------
template <class T, int MT>
__global__ void __launch_bounds__(256) gru_partial_kernel(DevLoop<T> p, int step) {
  __shared__ int tok[16 * MT];
  for (int b = threadIdx.x; b < p.B && b < 16 * MT; b += blockDim.x) {
    int tk;
    if (step == 0)
      tk = p.x_t[b];
    else if (p.teacher)
      tk = p.teacher[(size_t)b * p.K + step - 1];
    else
      tk = key_token(p.keys[(size_t)(step - 1) * p.B + b]);
    tok[b] = min(max(tk, 0), p.V - 1);
  }
  __syncthreads();
  // the W_ih jobs only (without a GRU input table); hh_kernel forms W_hh g
  const int job = blockIdx.x * 4 + wave_id();
  if (job < ((3 * p.H) >> 4) * p.KS) gru_partial_job<T, MT, Plain>(p, step, job, tok);
}


template <class T, int MT>
__global__ void __launch_bounds__(256) w2_sample_kernel(DevLoop<T> p, int step, int /*hh_step: not fused here*/,
                                                        int /*gx_w2: the whole grid*/) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  w2_sample_block<T, MT, Plain>(p, step, blockIdx.x, gridDim.x, blockIdx.y * 16 * MT, smem);
}

// ---------------------------------------------------------------------------
// persistent schedule
// ---------------------------------------------------------------------------

// Reduce the tagged keys that all G workgroups published for position `step`
// (tag step + 1) into picked[b].  Runs on one wave.
template <class T>
__device__ bool reduce_keys(const DevLoop<T>& p, int step, int G, int* picked) {
  const int lane = threadIdx.x & 63;
  const uint32_t tag = step + 1;
  const int par = step & 1;
  bool ok = true;
  for (int b = 0; b < p.B; ++b) {
    unsigned long long best = 0ull;
    for (int w = lane; w < G; w += 64) {
      const unsigned long long* src = p.xkey + ((size_t)par * G + w) * p.B + b;
      unsigned long long k = 0ull;
      unsigned int spins = 0;
      for (;;) {
        k = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (key_has_tag(k, tag)) break;
        if (++spins > kSpinLimit || ((spins & 63u) == 0u && gave_up(p.ctrl))) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      best = k > best ? k : best;
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const unsigned long long o = __shfl_xor(best, sh, 64);
      best = o > best ? o : best;
    }
    if (lane == 0) picked[b] = tagged_key_token(best);
  }
  return ok;
}

template <class T>
__device__ void loop_failed(const DevLoop<T>& p) {
  if (threadIdx.x == 0) {
    atomicOr(p.ctrl, 1u);
    atomicOr(p.ctrl + 2, 1u);  // the call's status word (the next 64-bit control word)
  }
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < p.B * p.K; i += gridDim.x * blockDim.x) p.tokens[i] = -1;
}

template <class T, int MT>
__global__ void __launch_bounds__(256) draft_loop_persistent_kernel(DevLoop<T> p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int picked[16 * MT];
  __shared__ int tok[16 * MT];
  const int G = gridDim.x;
  const int wave = wave_id();
  const int n_u_tiles = p.r >> 4;
  for (int step = 0; step < p.K; ++step) {
    const int jobs = gru_jobs(p.H, p.KS, step);
    if (blockIdx.x * 4 < jobs) {
      // tokens picked at step - 1: every workgroup with GRU work reduces the keys itself
      bool ok = true;
      if (step > 0 && wave == 0) ok = reduce_keys(p, step - 1, G, picked);
      if (__syncthreads_or(!ok)) return loop_failed(p);
      for (int b = threadIdx.x; b < p.B; b += blockDim.x) {
        if (step > 0 && blockIdx.x == 0) p.tokens[(size_t)b * p.K + step - 1] = picked[b];
        const int tk = step == 0 ? p.x_t[b] : (p.teacher ? p.teacher[(size_t)b * p.K + step - 1] : picked[b]);
        tok[b] = min(max(tk, 0), p.V - 1);
      }
      __syncthreads();
      for (int job = blockIdx.x * 4 + wave; job < jobs; job += G * 4)
        ok &= gru_partial_job<T, MT, Tagged>(p, step, job, tok);
      if (__syncthreads_or(!ok)) return loop_failed(p);
    }
    for (int t = blockIdx.x; t < n_u_tiles; t += G)
      if (!gates_u_tile<T, Tagged>(p, step, t, smem)) return loop_failed(p);
    if (!w2_sample_block<T, MT, Tagged>(p, step, blockIdx.x, G, 0, smem)) return loop_failed(p);
  }
  if (blockIdx.x == 0) {
    bool ok = true;
    if (wave == 0) ok = reduce_keys(p, p.K - 1, G, picked);
    if (__syncthreads_or(!ok)) return loop_failed(p);
    for (int b = threadIdx.x; b < p.B; b += blockDim.x) p.tokens[(size_t)b * p.K + p.K - 1] = picked[b];
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <class K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <class T>
static DevLoop<T> make_dev(const LoopArgs& a) {
  using E = typename T::elem;
  DevLoop<T> p{};
  p.B = a.B;
  p.K = a.K;
  p.d = a.d;
  p.V = a.V;
  p.H = a.H;
  p.r = a.r;
  p.KS = a.ks;
  p.embed = static_cast<const E*>(a.embed);
  p.w_ih = static_cast<const E*>(a.w_ih);
  p.w_hh = static_cast<const E*>(a.w_hh);
  p.b_ih = static_cast<const E*>(a.b_ih);
  p.b_hh = static_cast<const E*>(a.b_hh);
  p.w1 = static_cast<const E*>(a.w1);
  p.w2 = static_cast<const E*>(a.w2);
  p.b2 = static_cast<const E*>(a.b2);
  p.base = a.base;
  p.table = a.table;
  p.x_t = a.x_t;
  p.teacher = a.teacher;
  p.inv_temp = a.inv_temp;
  p.sampled = a.sampled;
  p.seed = a.seed;
  p.offset = a.offset;
  p.logits = a.logits;
  p.states = a.states;
  p.P = a.P;
  p.ppart = a.ppart;
  p.S = 0;
  p.part_ih = a.part_ih;
  p.part_hh = a.part_hh;
  p.u = a.u;
  p.keys = a.keys;
  p.ctrl = reinterpret_cast<unsigned int*>(a.keys + (size_t)a.K * a.B);
  p.tokens = a.tokens;
  p.xpart = a.xpart;
  p.xg = a.xpart + 2 * (size_t)(a.ks + 1) * a.B * 3 * a.H;
  p.xu = p.xg + 2 * (size_t)a.B * a.H;
  p.xkey = p.xu + 2 * (size_t)a.B * a.r;
  return p;
}

// The W2 phase: the streaming kernel when a W2 row is 2 to 16 64-B steps,
// else the generic one.
template <class T, int MW>
struct W2Launch {
  void (*kern)(DevLoop<T>, int, int, int);
  size_t lds;
  dim3 grid;
  int gx_w2;      // workgroups per batch slice that stream W2 (the rest form W_hh g)
  bool fused_hh;  // the kernel forms W_hh g for the next position
};

// register stages of W2 tiles per wave in the streaming kernel (Qwen3-8B,
// draft call at 32 / 128 blocks: 0.622 / 1.40 ms with 2 stages, 0.690 / 1.79
// with 3, 0.711 / 2.07 with 4: more registers cost occupancy, and at 32 blocks
// the W_hh units then no longer fit in workgroups of their own)
constexpr int kW2Stages = 2;

template <class T, int MW, int NS>
static W2Launch<T, MW> w2_stream_plan(const DevLoop<T>& p, int num_cu) {
  const int ntiles = (p.V + 15) / 16;
  const size_t lds = std::max(w2_stream_lds_bytes<T, MW>(p.r), HhTiling<MW>::kRedBytes);
  // (a kernel of its own stores the logits: a store that might be in flight
  // costs the tile loop exact waits on its prefetches)
  auto kern = p.V % 16 == 0 ? (p.logits ? w2_stream_kernel<T, MW, NS, true, kW2Stages, true>
                                        : w2_stream_kernel<T, MW, NS, true, kW2Stages, false>)
                            : (p.logits ? w2_stream_kernel<T, MW, NS, false, kW2Stages, true>
                                        : w2_stream_kernel<T, MW, NS, false, kW2Stages, false>);
  // one workgroup per compute unit for each slice of 16 MW batch rows: each
  // wave then streams ~ntiles / (4 #CU) tiles, which amortises staging u and
  // the key reduction (measured at Qwen3 shapes, B = 8 / 32 / 128: 19 / 26 /
  // 51 us per position against 23 / 33 / 60 us with one wave per resident
  // slot and 3-4 tiles per wave)
  const int gx = std::max(1, std::min(num_cu, (ntiles + 3) / 4));
  const int gy = (p.B + 16 * MW - 1) / (16 * MW);
  // W_hh g in workgroups of its own when they fit beside the W2 ones (B = 8 /
  // 32 at Qwen3 shapes: the launch takes 17.0 / 28.2 us against 18.7 / 31.5
  // with the units inside the W2 workgroups), else inside the W2 workgroups
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), 256, lds) !=
      hipSuccess)
    per_cu = 1;
  using HT = HhTiling<MW>;
  const long units = (long)((3 * p.H + 16 * HT::NT - 1) / (16 * HT::NT)) * ((p.B + 16 * HT::MT - 1) / (16 * HT::MT));
  const long hx = (units + gy - 1) / gy;
  const bool own = (long)(gx + hx) * gy <= (long)per_cu * num_cu;
  return {kern, lds, dim3(gx + (own ? (int)hx : 0), gy), gx, true};
}

template <class T, int MW>
static W2Launch<T, MW> w2_plan(const DevLoop<T>& p, int num_cu) {
  const bool offsets_fit = (16LL * p.K * p.V + 16) * 4 < (1LL << 31);
  switch (offsets_fit ? p.r * (int)sizeof(typename T::elem) / 64 : 0) {
    case 2: return w2_stream_plan<T, MW, 2>(p, num_cu);
    case 4: return w2_stream_plan<T, MW, 4>(p, num_cu);
    case 8: return w2_stream_plan<T, MW, 8>(p, num_cu);
    case 16: return w2_stream_plan<T, MW, 16>(p, num_cu);
    default: break;
  }
  const int ntiles = (p.V + 15) / 16;
  const int gx = std::min((ntiles + 3) / 4, num_cu * 4);
  return {w2_sample_kernel<T, MW>, w2_lds_bytes<T>(p.r, 16 * MW), dim3(gx, (p.B + 16 * MW - 1) / (16 * MW)), gx,
          false};
}

template <class T, int MT>
static hipError_t multi_kernel_loop(const DevLoop<T>& p, int num_cu, hipStream_t s) {
  hipError_t e;
  constexpr int MW = MT > 4 ? 4 : MT;  // w2 rows per workgroup: 16 * MW (W2 read once per 64 rows)
  const W2Launch<T, MW> w2 = w2_plan<T, MW>(p, num_cu);
  if ((e = allow_lds(w2.kern, w2.lds)) != hipSuccess) return e;
  const dim3 ggrid((p.H + 255) / 256, p.B);
  const dim3 ugrid(p.r / 16, (p.B + 15) / 16);
  const int t3 = 3 * p.H / 16;
  const dim3 hgrid(t3, (p.B + 15) / 16);
  for (int step = 0; step < p.K; ++step) {
    if (!p.table) hipLaunchKernelGGL((gru_partial_kernel<T, MT>), dim3((t3 * p.KS + 3) / 4), dim3(256), 0, s, p, step);
    // W_hh g for this position: formed by the previous position's W2 launch
    // when it carries it, else a launch of its own
    if (step > 0 && !w2.fused_hh) hipLaunchKernelGGL(hh_kernel<T>, hgrid, dim3(256), 0, s, p, step);
    hipLaunchKernelGGL(gates_kernel<T>, ggrid, dim3(256), 0, s, p, step);
    hipLaunchKernelGGL(u_kernel<T>, ugrid, dim3(256), 0, s, p, step);
    const int hh_next = w2.fused_hh && step + 1 < p.K ? step + 1 : 0;
    hipLaunchKernelGGL(w2.kern, w2.grid, dim3(256), w2.lds, s, p, step, hh_next, w2.gx_w2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_finalize_tokens(p.B, p.K, p.keys, p.tokens, s);
}

// Returns an error when the grid cannot be co-resident (the caller falls back).
template <class T, int MT>
static hipError_t persistent_loop(const DevLoop<T>& p, int num_cu, int max_wg, hipStream_t s) {
  auto kern = draft_loop_persistent_kernel<T, MT>;
  const size_t lds = std::max(gates_lds_bytes(p.H), w2_lds_bytes<T>(p.r, 16 * MT));
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), 256, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
  const int G = std::min(num_cu * std::min(per_cu, 2), max_wg);
  DevLoop<T> pp = p;
  void* args[] = {&pp};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(G), dim3(256), args, (unsigned)lds, s);
}

// Blocks per call up to which the single-block loop runs once per block.
constexpr int kB1PerBlockMax = 2;
// Blocks per call up to which the several-block on-chip loop is the default.
constexpr int kBnDefaultMax = 16;

// Block b of a bf16 call as a call of its own (row pointers offset, the
// sampler keyed by b); hipErrorNotSupported before any launch if the
// single-block loop does not take these shapes.
static hipError_t b1_per_block(const LoopArgs& a, hipStream_t s) {
  LoopArgs a1 = a;
  a1.B = 1;
  if (a.dtype != 1 || !b1_supported(a1)) return hipErrorNotSupported;
  const size_t K = (size_t)a.K;
  for (int b = 0; b < a.B; ++b) {
    // block 0's pre-loop launch clears the whole key region, the call's status
    // word included; later blocks clear their own keys and control word only
    a1.clear_words = b == 0 ? a.K * a.B + 2 : a.K + 1;
    a1.hidden = static_cast<const uint16_t*>(a.hidden) + b * K * a.d;
    a1.base = a.base + b * K * a.V;
    a1.x_t = a.x_t + b;
    a1.teacher = a.teacher ? a.teacher + b * K : nullptr;
    a1.tokens = a.tokens + b * K;
    a1.logits = a.logits ? a.logits + b * K * a.V : nullptr;
    a1.states = a.states + b * K * a.H;
    a1.rng_block = a.rng_block + (uint32_t)b;
    const hipError_t e = launch_draft_b1(a1, s);
    if (e != hipSuccess) return e == hipErrorNotSupported && b > 0 ? hipErrorUnknown : e;
  }
  return hipSuccess;
}

template <class T, int MT>
static hipError_t run_loop(const LoopArgs& a, int mode, hipStream_t s) {
  const DevLoop<T> p = make_dev<T>(a);
  if constexpr (MT == 1) {
    if (mode != 2 && b1_supported(a)) {
      // on-chip-weight loop for a single block (needs the GRU input table); it
      // clears its own keys and exchange words and forms P in its pre-launch
      hipError_t e = launch_draft_b1(a, s);
      if (e != hipErrorNotSupported) return e;
      (void)hipGetLastError();  // the grid cannot be co-resident here: use another schedule
    } else if (mode != 2 && a.B <= kB1PerBlockMax) {
      // a few blocks: the single-block loop once per block, back to back on
      // the stream (at Qwen3-8B shapes ~157 us a block, against ~590 us for the
      // per-position kernels at B = 2 or 3); the workspace is reused in order
      hipError_t e = b1_per_block(a, s);
      if (e != hipErrorNotSupported) return e;
      (void)hipGetLastError();
    }
  }
  hipError_t e;
  PSplit ps;
  if (mode != 1 && a.dtype == 1 && p_split_shape(a.d, a.r, ps)) {
    // one launch: the keys [K, B] and control words cleared, and the
    // loop-invariant hidden half of the first correction projection (+ b1)
    // as K-slice partials that u_kernel adds up
    e = launch_p_partials(a.hidden, a.B * a.K, a.d, a.w1, a.d + a.H, a.r, a.b1, a.ppart, ps, a.keys,
                          a.K * a.B + 2, nullptr, 0, s);
    if (e != hipSuccess) return e;
    DevLoop<T> q = p;
    q.S = ps.S;
    return multi_kernel_loop<T, MT>(q, a.num_cu, s);
  }
  // keys [K, B] and the control words start at zero on every call
  e = launch_fill_u64(a.keys, a.K * a.B + 2, s);
  if (e != hipSuccess) return e;
  // loop-invariant hidden half of the first correction projection (+ b1)
  e = launch_panel_gemm(a.dtype, a.hidden, a.d, a.B * a.K, a.w1, a.d + a.H, a.r, a.d, a.b1, a.P, a.r, a.num_cu, s);
  if (e != hipSuccess) return e;
  if constexpr (MT <= 2) {
    if (mode == 1) {
      // the tagged exchange buffers start at zero (no valid tag) on every call
      e = launch_fill_u64(a.xpart, (int)a.xwords, s);
      if (e != hipSuccess) return e;
      return persistent_loop<T, MT>(p, a.num_cu, a.max_wg, s);
    }
  }
  return multi_kernel_loop<T, MT>(p, a.num_cu, s);
}

template <class T>
static hipError_t loop_t(const LoopArgs& a, int mode, hipStream_t s) {
  // several blocks of a bf16 head with its GRU input table: the on-chip loop
  // for several blocks per launch, from 2 to 16 blocks (one launch; measured
  // at Qwen3 shapes: 2 blocks 202 us against 307 us for the single-block loop
  // run twice, 8 blocks 253 us against 443 us for the per-position kernels,
  // 32 blocks in two launches 787 against 614 us), or for any count from 2
  // when forced
  if ((mode == 0 && a.B >= 2 && a.B <= kBnDefaultMax) || mode == 3) {
    if (bn_supported(a)) {
      const hipError_t e = launch_draft_bn(a, s);
      if (e != hipErrorNotSupported) return e;
      (void)hipGetLastError();  // the grid cannot be co-resident here: use another schedule
    }
  }
  if (a.B <= 16) return run_loop<T, 1>(a, mode, s);
  if (a.B <= 32) return run_loop<T, 2>(a, mode, s);
  if (a.B <= 64) return run_loop<T, 4>(a, mode, s);
  return run_loop<T, 8>(a, mode, s);
}

hipError_t launch_draft_loop(const LoopArgs& a, int mode, hipStream_t s) {
  if (!a.base) return a.B == 1 ? launch_draft_b1(a, s) : hipErrorNotSupported;  // only it forms the base logits
  if (a.dtype == 1) return loop_t<Bf16>(a, mode, s);
  return loop_t<F32>(a, mode, s);
}

}  // namespace domino
