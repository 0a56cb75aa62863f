// Domino draft-head kernels for gfx950.
//
// Pages (cited by title and section):
//   [notes]     "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn)
//   [explainer] the yhxrc.cn article on the Domino paper
//
// Kernels
//   panel_gemm      C = A W^T (+bias).  The frozen LM head over all block
//                   positions ([notes] §二.1(1)) and the loop-invariant hidden
//                   half of the first correction projection.
//   gru_partial     GRU gate pre-activations W_ih e(prev token) and W_hh g,
//                   split over K for parallelism ([notes] §二.1(2) item 1).
//   gru_gates_u     GRU gates -> new state; u = SiLU(P + W1_g g)
//                   ([notes] §二.1(2) item 2; [explainer] §四).
//   w2_sample       L = L_base + W2 u + b2, optional Gumbel noise, vocabulary
//                   argmax ([notes] §二.1(2) item 3).
//   finalize_tokens keys -> token ids.
//   accept_len      longest matching prefix ([notes] §一.1 item 1).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace domino {

constexpr int kPanelWaves = 8;

// ---------------------------------------------------------------------------
// panel_gemm: one workgroup stages a 16-row slice of A (all of K) in LDS; its
// waves then stream 16-row tiles of W from HBM, one matrix-core tile per 64 B
// of K, with no further synchronisation.  grid.y walks the 16-row slices of A.
// ---------------------------------------------------------------------------
template <class T>
__global__ void __launch_bounds__(kPanelWaves * 64)
    panel_gemm_kernel(const typename T::elem* __restrict__ A, int lda, int M,
                      const typename T::elem* __restrict__ W, int ldw, int N, int K,
                      const typename T::elem* __restrict__ bias, float* __restrict__ C, int ldc) {
  using E = typename T::elem;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int row_bytes = K * (int)sizeof(E);
  const int lds_stride = row_bytes + 16;
  const int m0 = blockIdx.y * 16;
  const int chunks = row_bytes >> 4;
  for (int idx = threadIdx.x; idx < 16 * chunks; idx += blockDim.x) {
    const int rr = idx / chunks, c = idx - rr * chunks;
    u32x4 v = {0, 0, 0, 0};
    if (m0 + rr < M) v = ld16(reinterpret_cast<const unsigned char*>(A + (size_t)(m0 + rr) * lda) + c * 16);
    st16(smem + rr * lds_stride + c * 16, v);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int ntiles = (N + 15) >> 4;
  const unsigned char* arow = smem + col * lds_stride + grp * 16;
  for (int t = blockIdx.x * kPanelWaves + wave; t < ntiles; t += gridDim.x * kPanelWaves) {
    const int n = t * 16 + col;
    const unsigned char* wrow =
        reinterpret_cast<const unsigned char*>(W + (size_t)min(n, N - 1) * ldw) + grp * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int kb = 0; kb < row_bytes; kb += 64) {
      const u32x4 w = ld16(wrow + kb);
      const u32x4 a = ld16(arow + kb);
      acc = mma16<T>(acc, a, w);
    }
    if (n < N) {
      const float bv = bias ? T::to_f32(bias[n]) : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + grp * 4 + j;
        if (m < M) C[(size_t)m * ldc + n] = acc[j] + bv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Token fed to the GRU at `step` for batch row b.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int loop_token(int step, int b, int K, int V, const int32_t* x_t,
                                          const int32_t* teacher, const unsigned long long* keys_prev) {
  int tok;
  if (step == 0)
    tok = x_t[b];
  else if (teacher)
    tok = teacher[(size_t)b * K + step - 1];
  else
    tok = key_token(keys_prev[b]);
  return min(max(tok, 0), V - 1);
}

// ---------------------------------------------------------------------------
// gru_partial: wave jobs over 16-row tiles of the stacked gate rows (3H).
//   job < n_ih : tile t, K-slice ks of W_ih e   -> part_ih[ks][b][3H]
//   otherwise  : tile t of W_hh g_prev          -> part_hh[b][3H]
// Batch rows live in the matrix-core M dimension, MT tiles of 16.
// ---------------------------------------------------------------------------
template <class T, int MT>
__global__ void __launch_bounds__(256)
    gru_partial_kernel(int B, int K, int V, int d, int H, int KS, int step, const int32_t* __restrict__ x_t,
                       const int32_t* __restrict__ teacher, const unsigned long long* __restrict__ keys_prev,
                       const typename T::elem* __restrict__ embed, const typename T::elem* __restrict__ w_ih,
                       const typename T::elem* __restrict__ w_hh, const float* __restrict__ g_prev,
                       int g_stride, float* __restrict__ part_ih, float* __restrict__ part_hh) {
  using E = typename T::elem;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int T3 = (3 * H) >> 4;
  const int n_ih = T3 * KS;
  const int n_hh = g_prev ? T3 : 0;
  const int job = blockIdx.x * 4 + wave;
  if (job >= n_ih + n_hh) return;
  const int G3 = 3 * H;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (job < n_ih) {
    const int ks = job / T3, t = job - ks * T3;
    const int kc = d / KS;
    const int n = t * 16 + col;
    const unsigned char* wrow =
        reinterpret_cast<const unsigned char*>(w_ih + (size_t)n * d + (size_t)ks * kc) + grp * 16;
    const unsigned char* erow[MT];
    bool live[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int b = mt * 16 + col;
      live[mt] = b < B;
      const int tok = live[mt] ? loop_token(step, b, K, V, x_t, teacher, keys_prev) : 0;
      erow[mt] = reinterpret_cast<const unsigned char*>(embed + (size_t)tok * d + (size_t)ks * kc) + grp * 16;
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
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = mt * 16 + grp * 4 + j;
        if (b < B) part_ih[((size_t)ks * B + b) * G3 + n] = acc[mt][j];
      }
  } else {
    const int t = job - n_ih;
    const int n = t * 16 + col;
    const unsigned char* wrow = reinterpret_cast<const unsigned char*>(w_hh + (size_t)n * H) + grp * 16;
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
          const float* src = g_prev + (size_t)b * g_stride + k0 + grp * EPF;
#pragma unroll
          for (int e = 0; e < EPF; e += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(src + e);
            x[e] = v[0]; x[e + 1] = v[1]; x[e + 2] = v[2]; x[e + 3] = v[3];
          }
          a.from_f32(x);
        } else {
          a.zero();
        }
        acc[mt] = a.mma(acc[mt], w);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = mt * 16 + grp * 4 + j;
        if (b < B) part_hh[(size_t)b * G3 + n] = acc[mt][j];
      }
  }
}

// ---------------------------------------------------------------------------
// gru_gates_u: workgroup t owns bottleneck rows 16t..16t+15.  For each slice
// of 16 batch rows it recomputes the new GRU state of those rows (identical in
// every workgroup; workgroup 0 stores it), then u = SiLU(P + W1[:, d:] g).
// ---------------------------------------------------------------------------
template <class T>
__global__ void __launch_bounds__(256)
    gru_gates_u_kernel(int B, int K, int d, int H, int r, int KS, int step, const float* __restrict__ part_ih,
                       const float* __restrict__ part_hh, const typename T::elem* __restrict__ b_ih,
                       const typename T::elem* __restrict__ b_hh, const float* __restrict__ g_prev, int g_stride,
                       float* __restrict__ g_out, int gout_stride, const typename T::elem* __restrict__ w1,
                       const float* __restrict__ P, float* __restrict__ u) {
  using E = typename T::elem;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* gt = reinterpret_cast<float*>(smem);           // [16][H + 4]
  const int gstride = H + 4;
  float* red = gt + 16 * gstride;                        // [4][16][16]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int G3 = 3 * H;
  const int t = blockIdx.x;
  const int ldw1 = d + H;
  constexpr int EPF = T::kPer16B;

  for (int m0 = 0; m0 < B; m0 += 16) {
    for (int idx = threadIdx.x; idx < 16 * H; idx += blockDim.x) {
      const int rr = idx / H, j = idx - rr * H;
      const int b = m0 + rr;
      float g = 0.f;
      if (b < B) {
        float ar = 0.f, az = 0.f, an = 0.f;
        for (int ks = 0; ks < KS; ++ks) {
          const float* p = part_ih + ((size_t)ks * B + b) * G3;
          ar += p[j];
          az += p[H + j];
          an += p[2 * H + j];
        }
        if (b_ih) {
          ar += T::to_f32(b_ih[j]);
          az += T::to_f32(b_ih[H + j]);
          an += T::to_f32(b_ih[2 * H + j]);
        }
        float cr = 0.f, cz = 0.f, cn = 0.f, gp = 0.f;
        if (g_prev) {
          const float* p = part_hh + (size_t)b * G3;
          cr = p[j];
          cz = p[H + j];
          cn = p[2 * H + j];
          gp = g_prev[(size_t)b * g_stride + j];
        }
        if (b_hh) {
          cr += T::to_f32(b_hh[j]);
          cz += T::to_f32(b_hh[H + j]);
          cn += T::to_f32(b_hh[2 * H + j]);
        }
        const float rg = sigmoidf_(ar + cr);
        const float zg = sigmoidf_(az + cz);
        const float ng = tanhf(an + rg * cn);
        g = (1.f - zg) * ng + zg * gp;
        if (t == 0) g_out[(size_t)b * gout_stride + j] = g;
      }
      gt[rr * gstride + j] = g;
    }
    __syncthreads();

    // u rows t*16 + col; the four waves take interleaved 64-byte K chunks
    const int row = t * 16 + col;
    const unsigned char* wrow =
        reinterpret_cast<const unsigned char*>(w1 + (size_t)row * ldw1 + d) + grp * 16;
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
        float s = red[(0 * 16 + rr) * 16 + c] + red[(1 * 16 + rr) * 16 + c] + red[(2 * 16 + rr) * 16 + c] +
                  red[(3 * 16 + rr) * 16 + c];
        const int q = t * 16 + c;
        const float pre = P[((size_t)b * K + step) * r + q] + s;
        u[(size_t)b * r + q] = pre * sigmoidf_(pre);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// w2_sample: u (all batch rows of this workgroup's slice) is staged in LDS as
// matrix-core operands; each wave streams 16-row tiles of W2, adds b2 and the
// base logits, optionally stores the logits, draws Gumbel noise, and keeps a
// running argmax key per batch row.  Keys are reduced across lanes, waves and
// finally workgroups (64-bit atomic max).
// ---------------------------------------------------------------------------
template <class T, int MT>
__global__ void __launch_bounds__(256)
    w2_sample_kernel(int B, int K, int V, int r, int step, const float* __restrict__ u,
                     const typename T::elem* __restrict__ w2, const typename T::elem* __restrict__ b2,
                     const float* __restrict__ base, float* __restrict__ logits, float inv_temp, int sampled,
                     uint64_t seed, uint32_t offset, unsigned long long* __restrict__ keys) {
  using E = typename T::elem;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int EPF = T::kPer16B;
  constexpr int NPARTS = sizeof(ActFrag<T>) / 16;  // 2 (hi, lo) for bf16, 1 for f32
  const int row_bytes = r * (int)sizeof(E);
  const int lds_stride = row_bytes + 16;
  const int rows = 16 * MT;
  const int m0 = blockIdx.y * rows;
  unsigned long long* kred = reinterpret_cast<unsigned long long*>(smem + NPARTS * rows * lds_stride);

  // stage u -> operand tiles; part p of row rr at smem + (p*rows + rr)*lds_stride
  for (int idx = threadIdx.x; idx < rows * (r / EPF); idx += blockDim.x) {
    const int rr = idx / (r / EPF), c = idx - rr * (r / EPF);
    const int b = m0 + rr;
    ActFrag<T> a;
    if (b < B)
      a.from_f32(u + (size_t)b * r + c * EPF);
    else
      a.zero();
    const u32x4* parts = reinterpret_cast<const u32x4*>(&a);
#pragma unroll
    for (int p = 0; p < NPARTS; ++p) st16(smem + (p * rows + rr) * lds_stride + c * 16, parts[p]);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int ntiles = (V + 15) >> 4;
  unsigned long long best[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) best[mt][j] = 0ull;

  for (int t = blockIdx.x * 4 + wave; t < ntiles; t += gridDim.x * 4) {
    const int v = t * 16 + col;
    const unsigned char* wrow =
        reinterpret_cast<const unsigned char*>(w2 + (size_t)min(v, V - 1) * r) + grp * 16;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int kb = 0; kb < row_bytes; kb += 64) {
      const u32x4 w = ld16(wrow + kb);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int p = 0; p < NPARTS; ++p) {
          const u32x4 a = ld16(smem + (p * rows + mt * 16 + col) * lds_stride + grp * 16 + kb);
          acc[mt] = mma16<T>(acc[mt], a, w);
        }
    }
    if (v < V) {
      const float bv = b2 ? T::to_f32(b2[v]) : 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int b = m0 + mt * 16 + grp * 4 + j;
          if (b < B) {
            const size_t o = ((size_t)b * K + step) * V + v;
            const float L = base[o] + (acc[mt][j] + bv);
            if (logits) logits[o] = L;
            float s = L;
            if (sampled) s = L * inv_temp + gumbel_from_word(philox_word(seed, offset, b, step, v));
            const unsigned long long k = argmax_key(s, v);
            best[mt][j] = k > best[mt][j] ? k : best[mt][j];
          }
        }
    }
  }
  // reduce over the 16 lanes of each group (same batch rows, different vocab)
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
    if (b < B && k != 0ull) atomicMax(keys + b, k);
  }
}

__global__ void fill_u64_kernel(unsigned long long* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

__global__ void finalize_tokens_kernel(int B, int K, const unsigned long long* __restrict__ keys,
                                       int32_t* __restrict__ tokens) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B * K) {
    const int b = i / K, step = i - b * K;
    tokens[i] = key_token(keys[(size_t)step * B + b]);
  }
}

__global__ void accept_len_kernel(int B, int K, const int32_t* __restrict__ draft,
                                  const int32_t* __restrict__ target, int32_t* __restrict__ accept) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* dr = draft + (size_t)b * K;
  const int32_t* tr = target + (size_t)b * K;
  int n = 0;
  while (n < K && dr[n] == tr[n]) ++n;
  accept[b] = n;
}

__global__ void debug_philox_kernel(uint64_t seed, uint32_t offset, int b, int pos, int v0, int n,
                                    uint32_t* __restrict__ out) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n) out[j] = philox_word(seed, offset, (uint32_t)b, (uint32_t)pos, (uint32_t)(v0 + j));
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <class K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <class T>
static hipError_t panel_gemm_t(const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                               const void* bias, float* C, int ldc, int num_cu, hipStream_t s) {
  using E = typename T::elem;
  const size_t lds = 16 * ((size_t)K * sizeof(E) + 16);
  auto kern = panel_gemm_kernel<T>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  const int ntiles = (N + 15) / 16;
  int gx = (ntiles + kPanelWaves - 1) / kPanelWaves;
  const int per_cu = lds > 80 * 1024 ? 1 : 2;
  gx = std::min(gx, std::max(1, num_cu * per_cu));
  dim3 grid(gx, (M + 15) / 16);
  hipLaunchKernelGGL(kern, grid, dim3(kPanelWaves * 64), lds, s, static_cast<const E*>(A), lda, M,
                     static_cast<const E*>(W), ldw, N, K, static_cast<const E*>(bias), C, ldc);
  return hipGetLastError();
}

hipError_t launch_panel_gemm(int dtype, const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                             const void* bias, float* C, int ldc, int num_cu, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == 1) return panel_gemm_t<Bf16>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
  return panel_gemm_t<F32>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
}

template <class T, int MT>
static hipError_t gru_partial_t(const LoopArgs& a, int step, hipStream_t s) {
  using E = typename T::elem;
  const int T3 = 3 * a.H / 16;
  const int jobs = T3 * a.ks + (step > 0 ? T3 : 0);
  const float* g_prev = step > 0 ? a.states + (size_t)(step - 1) * a.H : nullptr;
  hipLaunchKernelGGL((gru_partial_kernel<T, MT>), dim3((jobs + 3) / 4), dim3(256), 0, s, a.B, a.K, a.V, a.d,
                     a.H, a.ks, step, a.x_t, a.teacher, a.keys + (size_t)(step > 0 ? step - 1 : 0) * a.B,
                     static_cast<const E*>(a.embed), static_cast<const E*>(a.w_ih), static_cast<const E*>(a.w_hh),
                     g_prev, a.K * a.H, a.part_ih, a.part_hh);
  return hipGetLastError();
}

template <class T, int MT>
static hipError_t w2_sample_t(const LoopArgs& a, int step, hipStream_t s) {
  using E = typename T::elem;
  constexpr int NPARTS = sizeof(ActFrag<T>) / 16;
  const int rows = 16 * MT;
  const size_t lds = (size_t)NPARTS * rows * (a.r * sizeof(E) + 16) + 4 * rows * sizeof(unsigned long long);
  auto kern = w2_sample_kernel<T, MT>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  const int ntiles = (a.V + 15) / 16;
  int gx = std::min((ntiles + 3) / 4, a.num_cu * 4);
  dim3 grid(gx, (a.B + rows - 1) / rows);
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, a.B, a.K, a.V, a.r, step, a.u, static_cast<const E*>(a.w2),
                     static_cast<const E*>(a.b2), a.base, a.logits, a.inv_temp, a.sampled, a.seed, a.offset,
                     a.keys + (size_t)step * a.B);
  return hipGetLastError();
}

template <class T>
static hipError_t gates_u_t(const LoopArgs& a, int step, hipStream_t s) {
  using E = typename T::elem;
  const size_t lds = 16 * (size_t)(a.H + 4) * sizeof(float) + 4 * 16 * 16 * sizeof(float);
  auto kern = gru_gates_u_kernel<T>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  const float* g_prev = step > 0 ? a.states + (size_t)(step - 1) * a.H : nullptr;
  hipLaunchKernelGGL(kern, dim3(a.r / 16), dim3(256), lds, s, a.B, a.K, a.d, a.H, a.r, a.ks, step, a.part_ih,
                     a.part_hh, static_cast<const E*>(a.b_ih), static_cast<const E*>(a.b_hh), g_prev, a.K * a.H,
                     a.states + (size_t)step * a.H, a.K * a.H, static_cast<const E*>(a.w1), a.P, a.u);
  return hipGetLastError();
}

template <class T>
static hipError_t draft_loop_t(const LoopArgs& a, hipStream_t s) {
  hipError_t e;
  const int nk = a.K * a.B;
  hipLaunchKernelGGL(fill_u64_kernel, dim3((nk + 255) / 256), dim3(256), 0, s, a.keys, nk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // loop-invariant hidden half of the first correction projection (+ b1)
  e = launch_panel_gemm(a.dtype, a.hidden, a.d, a.B * a.K, a.w1, a.d + a.H, a.r, a.d, a.b1, a.P, a.r, a.num_cu, s);
  if (e != hipSuccess) return e;
  for (int step = 0; step < a.K; ++step) {
    if (a.B <= 16)
      e = gru_partial_t<T, 1>(a, step, s);
    else if (a.B <= 32)
      e = gru_partial_t<T, 2>(a, step, s);
    else if (a.B <= 64)
      e = gru_partial_t<T, 4>(a, step, s);
    else
      e = gru_partial_t<T, 8>(a, step, s);
    if (e != hipSuccess) return e;
    if ((e = gates_u_t<T>(a, step, s)) != hipSuccess) return e;
    e = a.B <= 16 ? w2_sample_t<T, 1>(a, step, s) : w2_sample_t<T, 2>(a, step, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(finalize_tokens_kernel, dim3((nk + 255) / 256), dim3(256), 0, s, a.B, a.K, a.keys, a.tokens);
  return hipGetLastError();
}

hipError_t launch_draft_loop(const LoopArgs& a, hipStream_t s) {
  if (a.dtype == 1) return draft_loop_t<Bf16>(a, s);
  return draft_loop_t<F32>(a, s);
}

hipError_t launch_accept_len(int B, int K, const int32_t* draft, const int32_t* target, int32_t* accept,
                             hipStream_t s) {
  hipLaunchKernelGGL(accept_len_kernel, dim3((B + 255) / 256), dim3(256), 0, s, B, K, draft, target, accept);
  return hipGetLastError();
}

hipError_t launch_debug_philox(uint64_t seed, uint32_t offset, int b, int pos, int v0, int n, uint32_t* out,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(debug_philox_kernel, dim3((n + 255) / 256), dim3(256), 0, s, seed, offset, b, pos, v0, n,
                     out);
  return hipGetLastError();
}

}  // namespace domino
