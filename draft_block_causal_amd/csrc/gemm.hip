// Tiled bf16 GEMM on the gfx950 matrix cores:
//     C[M][N] (float32) = A[M][K] (bf16) * W[N][K]^T (bf16) (+ bias[N])
// Both operands are K-contiguous ([rows, K] row-major), as the LM head
// (hidden x W_lm^T, [notes] §二.1(1)) and the GRU input projection of the
// embedding table are.
//
// Block tile 128 x 128, K tile 64, 256 threads = 4 waves in a 2 x 2 grid of
// 64 x 64 wave tiles (4 x 4 v_mfma_f32_16x16x32_bf16 accumulators each).  The
// K loop is double-buffered: the next K tile is fetched from HBM into
// registers while the current one is consumed from LDS.  LDS rows are padded
// by 16 bytes so that the 16 rows of a fragment read fall into distinct banks.
//
// Block order: workgroups are dispatched round-robin over the 8 XCDs, so block
// b runs on XCD b % 8.  Blocks are numbered so that one XCD processes every
// M tile of a given N tile back to back: the W tile is then fetched from HBM
// once and re-read from that XCD's L2.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace domino {

constexpr int kGBM = 128, kGBN = 128, kGBK = 64;
constexpr int kGThreads = 256;
constexpr int kGRow = kGBK * 2;     // bytes of K per tile row
constexpr int kGLds = kGRow + 16;   // padded LDS row stride
constexpr int kXcds = 8;

__global__ void __launch_bounds__(kGThreads, 2)
    gemm_bf16_tn_kernel(const uint16_t* __restrict__ A, int lda, int M, const uint16_t* __restrict__ W, int ldw,
                        int N, int K, const uint16_t* __restrict__ bias, float* __restrict__ C, int ldc, int num_m,
                        int num_n) {
  __shared__ __attribute__((aligned(16))) unsigned char sA[2][kGBM * kGLds];
  __shared__ __attribute__((aligned(16))) unsigned char sW[2][kGBN * kGLds];
  // ---- tile of this block (XCD-grouped) ----
  const int b = blockIdx.x;
  const int xcd = b % kXcds, local = b / kXcds;
  const int n_per_xcd = (num_n + kXcds - 1) / kXcds;
  const int nl = local / num_m, mt = local - nl * num_m;
  const int nt = nl * kXcds + xcd;
  if (nl >= n_per_xcd || nt >= num_n) return;
  const int m0 = mt * kGBM, n0 = nt * kGBN;

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: 128 rows x 8 chunks of 16 B per operand, 4 chunks per thread
  const unsigned char* ag[4];
  const unsigned char* wg[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * kGThreads;
    const int row = c >> 3, seg = c & 7;
    const int ar = min(m0 + row, M - 1), wr = min(n0 + row, N - 1);
    ag[i] = reinterpret_cast<const unsigned char*>(A + (size_t)ar * lda) + seg * 16;
    wg[i] = reinterpret_cast<const unsigned char*>(W + (size_t)wr * ldw) + seg * 16;
    lds_off[i] = row * kGLds + seg * 16;
  }
  u32x4 ra[4], rw[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(ag[i] + (size_t)k0 * 2);
      rw[i] = ld16(wg[i] + (size_t)k0 * 2);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(sA[buf] + lds_off[i], ra[i]);
      st16(sW[buf] + lds_off[i], rw[i]);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kGBK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * kGBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 af[4], wf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = ld16(sA[buf] + (wm * 64 + i * 16 + col) * kGLds + kk * 64 + grp * 16);
        wf[i] = ld16(sW[buf] + (wn * 64 + i * 16 + col) * kGLds + kk * 64 + grp * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma16<Bf16>(acc[i][j], af[i], wf[j]);
    }
    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*grp + q of each 16 x 16 tile, column col ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + col;
    if (n >= N) continue;
    const float bv = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * 64 + i * 16 + grp * 4 + q;
        if (m < M) C[(size_t)m * ldc + n] = acc[i][j][q] + bv;
      }
  }
}

// ---------------------------------------------------------------------------
// Large-M variant: block tile 256 x 256, 256 threads = 4 waves in a 2 x 2 grid
// of 128 x 128 wave tiles (8 x 8 accumulators each, 256 registers per lane,
// held in AGPRs: one wave per SIMD may use 512).  Per 32-wide K step a wave
// reads 8 + 8 fragments from LDS for 64 matrix-core products, twice the
// operand reuse of the 64 x 64 wave tile above.
// Operands go from HBM straight into LDS (global_load_lds, 16 B per lane, no
// staging registers) through a ring of kHStages K tiles of 32, so the loads of
// a tile are issued kHStages - 1 tiles (~1.5 us of products) before use.  An
// LDS row is 64 bytes (4 chunks of 16 B); chunk c of row r sits in slot
// c ^ ((r >> 2) & 3), which makes the 16-row fragment reads conflict-free.
// Same XCD-grouped block order as above.
// ---------------------------------------------------------------------------
constexpr int kHBM = 256, kHBN = 256, kHBK = 32;
constexpr int kHStages = 4;
constexpr int kHRow = kHBK * 2;                     // 64 bytes of K per LDS row
constexpr int kHStage = (kHBM + kHBN) * kHRow;      // 32 KB per stage
constexpr int kHLoads = kHBM * kHRow / 1024 / 4;    // 1 KB loads per wave per operand per stage (4)

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// s_waitcnt with only the vector-memory count limited (expcnt, lgkmcnt at max)
#define DOMINO_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

__global__ void __launch_bounds__(kGThreads, 1)
    gemm_bf16_tn_256_kernel(const uint16_t* __restrict__ A, int lda, int M, const uint16_t* __restrict__ W, int ldw,
                            int N, int K, const uint16_t* __restrict__ bias, float* __restrict__ C, int ldc, int num_m,
                            int num_n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.x;
  const int xcd = b % kXcds, local = b / kXcds;
  const int n_per_xcd = (num_n + kXcds - 1) / kXcds;
  const int nl = local / num_m, mt = local - nl * num_m;
  const int nt = nl * kXcds + xcd;
  if (nl >= n_per_xcd || nt >= num_n) return;
  const int m0 = mt * kHBM, n0 = nt * kHBN;

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;

  // DMA: load i of this wave covers tile rows 16 * (wave * kHLoads + i) + lane / 4,
  // LDS slot lane & 3 of that row, i.e. global chunk (lane & 3) ^ ((lane >> 4) & 3)
  const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const unsigned char* ag[kHLoads];
  const unsigned char* wg[kHLoads];
#pragma unroll
  for (int i = 0; i < kHLoads; ++i) {
    const int row = 16 * (wave * kHLoads + i) + (lane >> 2);
    const int ar = min(m0 + row, M - 1), wr = min(n0 + row, N - 1);
    ag[i] = reinterpret_cast<const unsigned char*>(A + (size_t)ar * lda) + dchunk * 16;
    wg[i] = reinterpret_cast<const unsigned char*>(W + (size_t)wr * ldw) + dchunk * 16;
  }
  auto issue = [&](int kt) {
    unsigned char* sA = smem + (kt % kHStages) * kHStage;
    unsigned char* sW = sA + kHBM * kHRow;
#pragma unroll
    for (int i = 0; i < kHLoads; ++i) {
      const int blk = (wave * kHLoads + i) * 1024;
      __builtin_amdgcn_global_load_lds((gptr_t)(ag[i] + (size_t)kt * kHRow),
                                       (lptr_t)(sA + blk), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(wg[i] + (size_t)kt * kHRow),
                                       (lptr_t)(sW + blk), 16, 0, 0);
    }
  };
  // fragment reads: row r = base + col, chunk grp -> slot grp ^ ((r >> 2) & 3) (base % 16 == 0)
  const int fslot = (grp ^ ((col >> 2) & 3)) * 16;

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kHBK;
  constexpr int kPerStage = 2 * kHLoads;  // DMA instructions of one stage per wave
#pragma unroll
  for (int s = 0; s < kHStages - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of tile kt are done once at most the younger stages are in flight
    const int ahead = min(kHStages - 2, nk - 1 - kt);
    static_assert(kHStages - 2 <= 3, "wait counts below cover at most three younger stages");
    if (ahead >= 3)
      DOMINO_WAIT_VM(3 * kPerStage);
    else if (ahead == 2)
      DOMINO_WAIT_VM(2 * kPerStage);
    else if (ahead == 1)
      DOMINO_WAIT_VM(kPerStage);
    else
      DOMINO_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();  // every wave's loads of tile kt are in LDS; tile kt - 1 is consumed
    if (kt + kHStages - 1 < nk) issue(kt + kHStages - 1);
    const unsigned char* sA = smem + (kt % kHStages) * kHStage;
    const unsigned char* sW = sA + kHBM * kHRow;
    u32x4 af[8], wf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      af[i] = ld16(sA + (wm * 128 + i * 16 + col) * kHRow + fslot);
      wf[i] = ld16(sW + (wn * 128 + i * 16 + col) * kHRow + fslot);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mma16<Bf16>(acc[i][j], af[i], wf[j]);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // all 16 fragment reads first,
    __builtin_amdgcn_sched_group_barrier(0x008, 64, 0);  // then the 64 products
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = n0 + wn * 128 + j * 16 + col;
    if (n >= N) continue;
    const float bv = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * 128 + i * 16 + grp * 4 + q;
        if (m < M) C[(size_t)m * ldc + n] = acc[i][j][q] + bv;
      }
  }
}

hipError_t launch_gemm_bf16_tn(const void* A, int lda, int M, const void* W, int ldw, int N, int K, const void* bias,
                               float* C, int ldc, hipStream_t s) {
  if (M >= kHBM && K % kHBK == 0) {
    const int num_m = (M + kHBM - 1) / kHBM, num_n = (N + kHBN - 1) / kHBN;
    const int n_per_xcd = (num_n + kXcds - 1) / kXcds;
    const long blocks = (long)n_per_xcd * num_m * kXcds;
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    const size_t lds = (size_t)kHStages * kHStage;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_tn_256_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_bf16_tn_256_kernel, dim3((unsigned)blocks), dim3(kGThreads), lds, s,
                       static_cast<const uint16_t*>(A), lda, M, static_cast<const uint16_t*>(W), ldw, N, K,
                       static_cast<const uint16_t*>(bias), C, ldc, num_m, num_n);
    return hipGetLastError();
  }
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % kGBK) return hipErrorNotSupported;
  const int num_m = (M + kGBM - 1) / kGBM, num_n = (N + kGBN - 1) / kGBN;
  const int n_per_xcd = (num_n + kXcds - 1) / kXcds;
  const long blocks = (long)n_per_xcd * num_m * kXcds;
  if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
  hipLaunchKernelGGL(gemm_bf16_tn_kernel, dim3((unsigned)blocks), dim3(kGThreads), 0, s,
                     static_cast<const uint16_t*>(A), lda, M, static_cast<const uint16_t*>(W), ldw, N, K,
                     static_cast<const uint16_t*>(bias), C, ldc, num_m, num_n);
  return hipGetLastError();
}

}  // namespace domino
