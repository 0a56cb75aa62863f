// Domino draft-head kernels for gfx950.
//
// Pages (cited by title and section):
//   [notes]     "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn)
//   [explainer] the yhxrc.cn article on the Domino paper
//
// Kernels
//   panel_gemm      C = A W^T (+bias).  The frozen LM head over all block
//                   positions ([notes] §二.1(1)) and the loop-invariant hidden
//                   half of the first correction projection (the row-streaming
//                   kernel for few rows is in rowstream.hip, the tiled GEMM for
//                   many rows in gemm.hip).
//   fill_u64        clears argmax keys and loop counters.
//   finalize_tokens keys -> token ids.
//   accept_len      longest matching prefix ([notes] §一.1 item 1).
//   debug_philox    the sampler's random words (test hook).
//   read_stream     a plain read of a buffer (calibration of the read bandwidth).
// The serial loop itself lives in loop.hip.
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

  const int wave = wave_id(), lane = threadIdx.x & 63;
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
// splitk_gemm: the same product for a 16-row slice of A, organised for
// streaming W at full bandwidth.  The 8 waves of a workgroup split K; each
// wave keeps its K range of the activation slice in registers for the whole
// kernel and streams its K range of one 16-row tile of W per iteration with
// every load of the next tile already in flight (double-buffered registers).
// The 8 partial 16x16 tiles are summed in LDS in a fixed order.
// KW = 64-byte K steps per wave (K * elem_size = 8 * 64 * KW).
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 8;

template <class T, int KW>
__global__ void __launch_bounds__(kSplitWaves * 64)
    splitk_gemm_kernel(const typename T::elem* __restrict__ A, int lda, int M,
                       const typename T::elem* __restrict__ W, int ldw, int N,
                       const typename T::elem* __restrict__ bias, float* __restrict__ C, int ldc) {
  __shared__ float red[kSplitWaves][16][17];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int m0 = blockIdx.y * 16;
  const size_t kbyte0 = (size_t)wave * KW * 64 + grp * 16;
  u32x4 af[KW];
  {
    const bool live = m0 + col < M;
    const unsigned char* arow = reinterpret_cast<const unsigned char*>(A + (size_t)(live ? m0 + col : 0) * lda) + kbyte0;
#pragma unroll
    for (int s = 0; s < KW; ++s) af[s] = live ? ld16(arow + s * 64) : u32x4{0, 0, 0, 0};
  }
  const int ntiles = (N + 15) >> 4;
  u32x4 wf[KW];
  int t = blockIdx.x;
  if (t < ntiles) {
    const unsigned char* wrow =
        reinterpret_cast<const unsigned char*>(W + (size_t)min(t * 16 + col, N - 1) * ldw) + kbyte0;
#pragma unroll
    for (int s = 0; s < KW; ++s) wf[s] = ld16(wrow + s * 64);
  }
  for (; t < ntiles; t += gridDim.x) {
    u32x4 wn[KW];
    const int tn = t + gridDim.x;
    if (tn < ntiles) {
      const unsigned char* wrow =
          reinterpret_cast<const unsigned char*>(W + (size_t)min(tn * 16 + col, N - 1) * ldw) + kbyte0;
#pragma unroll
      for (int s = 0; s < KW; ++s) wn[s] = ld16(wrow + s * 64);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KW; ++s) acc = mma16<T>(acc, af[s], wf[s]);
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][grp * 4 + j][col] = acc[j];
    __syncthreads();
    if (threadIdx.x < 256) {
      const int m = threadIdx.x >> 4, c = threadIdx.x & 15;
      const int n = t * 16 + c;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kSplitWaves; ++w) sum += red[w][m][c];
      if (m0 + m < M && n < N) C[(size_t)(m0 + m) * ldc + n] = sum + (bias ? T::to_f32(bias[n]) : 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KW; ++s) wf[s] = wn[s];
  }
}

// ---------------------------------------------------------------------------
// p_partials: the loop-invariant hidden half of the first correction
// projection, P = A W1[:, :d]^T + b1 for every block position
// ([notes] §二.1(2) item 2), as S partial sums over K slices, together with
// the clears the loop needs before it starts.  Each wave takes 512 B of K
// (8 matrix-core steps) of one 16-row tile of W1 for up to 64 rows of A
// (grid.y walks the 64-row groups); the waves of a workgroup add their
// products in LDS and the workgroup writes slice s: ppart[s][m][n], with b1
// in slice 0.  The consumer adds the S slices in a fixed order.  This spreads
// the W1 read over S x r / 16 workgroups instead of r / 16.
// ---------------------------------------------------------------------------
constexpr int kPreWaves = 4;  // waves per workgroup, at most
constexpr int kPreSteps = 8;  // 64-B K steps per wave
constexpr int kPreMt = 4;     // 16-row tiles of A per workgroup

__global__ void __launch_bounds__(kPreWaves * 64)
    p_partials_kernel(const uint16_t* __restrict__ A, int M, int lda, const uint16_t* __restrict__ w1, int ldw, int r,
                      const uint16_t* __restrict__ b1, float* __restrict__ ppart, int waves,
                      unsigned long long* __restrict__ z0, int n0, unsigned long long* __restrict__ z1, int n1) {
  __shared__ float red[kPreWaves][kPreMt][16][17];
  const int nthreads = gridDim.x * gridDim.y * blockDim.x;
  for (int i = (blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < n0 + n1; i += nthreads) {
    if (i < n0)
      z0[i] = 0ull;
    else
      z1[i - n0] = 0ull;
  }
  const int ntn = r >> 4;
  const int nt = blockIdx.x % ntn, ks = blockIdx.x / ntn;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int mt0 = blockIdx.y * kPreMt;
  const int mtiles = min(kPreMt, ((M + 15) >> 4) - mt0);
  if (wave < waves) {
    const size_t kb = (size_t)(ks * waves + wave) * (kPreSteps * 64) + grp * 16;
    const unsigned char* wrow = reinterpret_cast<const unsigned char*>(w1 + (size_t)(nt * 16 + col) * ldw) + kb;
    u32x4 wf[kPreSteps];
#pragma unroll
    for (int s = 0; s < kPreSteps; ++s) wf[s] = ld16(wrow + s * 64);
    for (int mt = 0; mt < mtiles; ++mt) {
      const int m = (mt0 + mt) * 16 + col;
      const unsigned char* arow = reinterpret_cast<const unsigned char*>(A + (size_t)min(m, M - 1) * lda) + kb;
      u32x4 a[kPreSteps];
#pragma unroll
      for (int s = 0; s < kPreSteps; ++s) a[s] = m < M ? ld16(arow + s * 64) : u32x4{0, 0, 0, 0};
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kPreSteps; ++s) acc = mma16<Bf16>(acc, a[s], wf[s]);
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][mt][grp * 4 + j][col] = acc[j];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < mtiles * 256; e += blockDim.x) {
    const int mt = e >> 8, mm = (e >> 4) & 15, c = e & 15;
    const int m = (mt0 + mt) * 16 + mm, n = nt * 16 + c;
    if (m < M) {
      float sum = 0.f;
      for (int w = 0; w < waves; ++w) sum += red[w][mt][mm][c];
      if (ks == 0 && b1) sum += bf16_to_f32(b1[n]);
      ppart[((size_t)ks * M + m) * r + n] = sum;
    }
  }
}

// z0[0..n0) and z1[0..n1) set to zero (grid-stride)
__global__ void __launch_bounds__(256) fill2_u64_kernel(unsigned long long* z0, int n0, unsigned long long* z1,
                                                        int n1) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n0 + n1; i += gridDim.x * blockDim.x) {
    if (i < n0)
      z0[i] = 0ull;
    else
      z1[i - n0] = 0ull;
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

// Calibration stream: each workgroup reads a contiguous range of the buffer
// with 16-B non-temporal loads, kReadInflight per thread in flight, and writes
// the XOR of its range's 32-bit words to sink[workgroup] (a plain store: one
// address updated by every workgroup would serialize them).
constexpr int kReadInflight = 8;
__global__ void __launch_bounds__(256) read_stream_kernel(const unsigned char* __restrict__ buf, size_t per_wg,
                                                          size_t total, uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[4];
  const size_t lo = (size_t)blockIdx.x * per_wg;
  const size_t hi = lo + per_wg < total ? lo + per_wg : total;
  constexpr size_t kStride = 256 * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t a0 = lo + threadIdx.x * 16; a0 < hi; a0 += kStride * kReadInflight) {
    u32x4 v[kReadInflight];
#pragma unroll
    for (int i = 0; i < kReadInflight; ++i) {
      const size_t a = a0 + (size_t)i * kStride;
      v[i] = a < hi ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(buf + a)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kReadInflight; ++i) acc ^= v[i];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
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

template <class T, int KW>
static hipError_t splitk_t(const void* A, int lda, int M, const void* W, int ldw, int N, const void* bias, float* C,
                           int ldc, int num_cu, hipStream_t s) {
  using E = typename T::elem;
  const int ntiles = (N + 15) / 16;
  dim3 grid(std::min(ntiles, num_cu), (M + 15) / 16);
  hipLaunchKernelGGL((splitk_gemm_kernel<T, KW>), grid, dim3(kSplitWaves * 64), 0, s, static_cast<const E*>(A), lda,
                     M, static_cast<const E*>(W), ldw, N, static_cast<const E*>(bias), C, ldc);
  return hipGetLastError();
}

// K split over 8 waves in 64-byte steps; returns hipErrorNotSupported for K
// that does not divide evenly into one of the compiled step counts.
template <class T>
static hipError_t splitk_dispatch(const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                                  const void* bias, float* C, int ldc, int num_cu, hipStream_t s) {
  const size_t row_bytes = (size_t)K * sizeof(typename T::elem);
  if (row_bytes % (64 * kSplitWaves)) return hipErrorNotSupported;
  switch (row_bytes / (64 * kSplitWaves)) {
    case 1: return splitk_t<T, 1>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 2: return splitk_t<T, 2>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 4: return splitk_t<T, 4>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 5: return splitk_t<T, 5>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 8: return splitk_t<T, 8>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 10: return splitk_t<T, 10>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 16: return splitk_t<T, 16>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_panel_gemm(int dtype, const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                             const void* bias, float* C, int ldc, int num_cu, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M <= 32 || (N <= 4096 && M <= 4096)) {  // few rows, or a small W: stream W at full bandwidth
    hipError_t e = launch_rowstream_gemm(dtype, A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (M <= 32) {
    const hipError_t e = dtype == 1 ? splitk_dispatch<Bf16>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s)
                                    : splitk_dispatch<F32>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (dtype == 1) {  // many rows: tiled matrix-core GEMM (W read once per XCD, re-used from L2)
    const hipError_t e = launch_gemm_bf16_tn(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (dtype == 1) return panel_gemm_t<Bf16>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
  return panel_gemm_t<F32>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
}

hipError_t launch_p_partials(const void* A, int M, int lda, const void* w1, int ldw, int r, const void* b1,
                             float* ppart, const PSplit& ps, unsigned long long* z0, int n0, unsigned long long* z1,
                             int n1, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int gy = (M + 16 * kPreMt - 1) / (16 * kPreMt);
  if (gy > 65535) return hipErrorNotSupported;
  hipLaunchKernelGGL(p_partials_kernel, dim3(ps.S * (r / 16), gy), dim3(kPreWaves * 64), 0, s,
                     static_cast<const uint16_t*>(A), M, lda, static_cast<const uint16_t*>(w1), ldw, r,
                     static_cast<const uint16_t*>(b1), ppart, ps.waves, z0, n0, z1, n1);
  return hipGetLastError();
}

hipError_t launch_fill2_u64(unsigned long long* z0, int n0, unsigned long long* z1, int n1, hipStream_t s) {
  const int n = n0 + n1;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill2_u64_kernel, dim3(std::min((n + 255) / 256, 1024)), dim3(256), 0, s, z0, n0, z1, n1);
  return hipGetLastError();
}

hipError_t launch_fill_u64(unsigned long long* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u64_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_finalize_tokens(int B, int K, const unsigned long long* keys, int32_t* tokens, hipStream_t s) {
  const int n = B * K;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_tokens_kernel, dim3((n + 255) / 256), dim3(256), 0, s, B, K, keys, tokens);
  return hipGetLastError();
}

hipError_t launch_accept_len(int B, int K, const int32_t* draft, const int32_t* target, int32_t* accept,
                             hipStream_t s) {
  hipLaunchKernelGGL(accept_len_kernel, dim3((B + 255) / 256), dim3(256), 0, s, B, K, draft, target, accept);
  return hipGetLastError();
}

hipError_t launch_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  // bytes per workgroup, rounded up to 4 KiB (a multiple of 16: every load stays in range)
  const size_t per = ((bytes + kReadGrid - 1) / kReadGrid + 4095) / 4096 * 4096;
  hipLaunchKernelGGL(read_stream_kernel, dim3(kReadGrid), dim3(256), 0, s, static_cast<const unsigned char*>(buf),
                     per, bytes, sink);
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
