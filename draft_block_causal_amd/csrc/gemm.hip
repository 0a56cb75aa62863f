// Tiled bf16 GEMM on the gfx950 matrix cores:
//     C[M][N] (float32) = A[M][K] (bf16) * W[N][K]^T (bf16) (+ bias[N])
// Both operands are K-contiguous ([rows, K] row-major), as the LM head
// (hidden x W_lm^T, [notes] §二.1(1)) and the GRU input projection of the
// embedding table are.
//
// Block order: workgroups are dispatched round-robin over the 8 XCDs, so block
// b runs on XCD b % 8.  Blocks are numbered so that one XCD processes every
// M tile of a given N tile back to back: the W tile is then fetched from HBM
// once and re-read from that XCD's L2.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace domino {

constexpr int kGThreads = 256;
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// Big-tile kernel: block tile BM x 256 (BM = 256, or 128 for 33 .. 255 rows),
// NW = 4 or 8 waves.  BM = 256: a 2 x 2 grid of 128 x 128 wave tiles (4 waves)
// or a 2 x 4 grid of 128 x 64 (8 waves, two per SIMD); BM = 128: four
// 128 x 64 wave tiles side by side (4 waves) or a 2 x 4 grid of 64 x 64
// (8 waves).  Accumulators live in
// AGPRs (one wave per SIMD may use 512 registers, two 256).  Per 32-wide K step a wave
// reads 8 A and 8 (or 4) W fragments from LDS for 64 (or 32) products.
// Operands go from HBM straight into LDS (global_load_lds, 16 B per lane, no
// staging registers) through a ring of kStages K tiles of 32 (4 x 32 KB for
// BM = 256, 6 x 24 KB for BM = 128), so the loads of a tile are issued
// kStages - 1 tiles before use.  An LDS row is 64 bytes (4 chunks of 16 B);
// chunk c of row r sits in slot c ^ ((r >> 1) & 3): a 16-B read is served 8
// lanes (128 B, all 32 banks) at a time, and the 8 lanes of a fragment read
// (rows r .. r + 7, one chunk) then touch 8 different 16-B bank groups (two
// rows share a 128-B line; the XOR separates rows r and r + 2).  Same
// XCD-grouped block order as above.  With 8 waves the K loop runs as a
// ping-pong of the two wave groups (memory phase against product phase, see
// the loop).  The operand fill into LDS is what bounds it: BM x 256 outputs
// per (BM + 256) x 64 B filled per K step; streaming the same operand bytes
// into registers alone, with no LDS and no products, takes 0.365 ms for the
// Qwen3-8B LM head at 512 rows, and through the LDS DMA path 0.49 ms.
// ---------------------------------------------------------------------------
template <int BM, int NW = 4, int BN = 256>
struct BigTile {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBN = BN, kBK = 32;
  static constexpr int kRow = kBK * 2;                    // 64 bytes of K per LDS row
  static constexpr int kStage = (BM + kBN) * kRow;        // bytes per ring stage
  static constexpr int kStages = BM == 256 ? 4 : 6;       // 128 KB or 144 KB of LDS
  static constexpr int kALoads = BM * kRow / 1024 / NW;   // 1 KB A loads per wave per stage
  static constexpr int kWLoads = kBN * kRow / 1024 / NW;  // 1 KB W loads per wave per stage
  static constexpr int kPerStage = kALoads + kWLoads;     // DMA instructions of one stage per wave
  static constexpr int kWavesN = BM == 256 && NW == 4 ? 2 : 4;  // wave grid (NW / kWavesN) x kWavesN
  static constexpr int kFW = kBN / kWavesN / 16;          // W fragments per wave (8 or 4)
  static constexpr int kFA = BM / (NW / kWavesN) / 16;    // A fragments per wave (8, or 4 for 128 x 256 / 8)
  static_assert(BM == 256 || BM == 128, "block height");
  static_assert(BN == 256 || BN == 128, "block width");
  static_assert(NW == 4 || NW == 8, "waves");
  static_assert((kStages - 2) * kPerStage < 64, "vector-memory count field");
};

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// s_waitcnt with only the vector-memory count limited (expcnt, lgkmcnt at max)
#define DOMINO_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// Wait until at most `ahead` younger stages of this wave's loads are in flight.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (MAXA >= 4) {
    if (ahead >= 4) {
      DOMINO_WAIT_VM(4 * PER);
      return;
    }
  }
  if constexpr (MAXA >= 3) {
    if (ahead >= 3) {
      DOMINO_WAIT_VM(3 * PER);
      return;
    }
  }
  if (ahead >= 2) {
    DOMINO_WAIT_VM(2 * PER);
  } else if (ahead == 1) {
    DOMINO_WAIT_VM(PER);
  } else {
    DOMINO_WAIT_VM(0);
  }
}

// The same with lgkmcnt(0) as well: this wave's LDS reads have returned.
#define DOMINO_WAIT_VM_LGK0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0070)
template <int PER, int MAXA>
__device__ __forceinline__ void wait_stages_lgk0(int ahead) {
  if constexpr (MAXA >= 4) {
    if (ahead >= 4) {
      DOMINO_WAIT_VM_LGK0(4 * PER);
      return;
    }
  }
  if constexpr (MAXA >= 3) {
    if (ahead >= 3) {
      DOMINO_WAIT_VM_LGK0(3 * PER);
      return;
    }
  }
  if (ahead >= 2) {
    DOMINO_WAIT_VM_LGK0(2 * PER);
  } else if (ahead == 1) {
    DOMINO_WAIT_VM_LGK0(PER);
  } else {
    DOMINO_WAIT_VM_LGK0(0);
  }
}

// MODE selects what a launch computes:
//   kPlain   C = A W^T (+ bias), the XCD-grouped block order above;
//   kSplitK  blockIdx.y = slice s of K: A columns s K .. s K + K - 1 against W
//            columns (s K) mod w_wrap .., written to C + s c_slice (partial
//            products; K must divide w_wrap); blocks in plain (m, n) order,
//            since few N tiles would leave XCDs idle in the grouped order;
//   kWrapT   W column k is read as k mod w_wrap (one wrap at most), and C is
//            stored transposed, C[n][m] at C + n ldc + m (c_slice != 0: C is
//            16-byte aligned and ldc, M multiples of 4, for 16-byte stores).
enum GemmMode { kPlain = 0, kSplitK = 1, kWrapT = 2 };

template <int BM, int MODE, int NW, int BN>
__global__ void __launch_bounds__(NW * 64, 1)
    gemm_bf16_tn_big_kernel(const uint16_t* __restrict__ A, int lda, int M, const uint16_t* __restrict__ W, int ldw,
                            int N, int K, const uint16_t* __restrict__ bias, float* __restrict__ C, int ldc, int num_m,
                            int num_n, int w_wrap, size_t c_slice) {
  using BT = BigTile<BM, NW, BN>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.x;
  int mt, nt;
  if constexpr (MODE == kSplitK) {
    mt = b % num_m;
    nt = b / num_m;
    const int k0 = (int)blockIdx.y * K;
    A += k0;
    W += k0 >= w_wrap ? k0 - w_wrap : k0;
    C += (size_t)blockIdx.y * c_slice;
  } else {
    const int xcd = b % kXcds, local = b / kXcds;
    const int n_per_xcd = (num_n + kXcds - 1) / kXcds;
    const int nl = local / num_m;
    mt = local - nl * num_m;
    nt = nl * kXcds + xcd;
    if (nl >= n_per_xcd || nt >= num_n) return;
  }
  const int m0 = mt * BM, n0 = nt * BT::kBN;

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int wm = wave / BT::kWavesN, wn = wave % BT::kWavesN;

  // DMA: load i of this wave covers tile rows 16 * (wave * loads + i) + lane / 4,
  // LDS slot lane & 3 of that row, i.e. global chunk (lane & 3) ^ ((lane >> 3) & 3)
  const int dchunk = (lane & 3) ^ ((lane >> 3) & 3);
  const unsigned char* ag[BT::kALoads];
  const unsigned char* wg[BT::kWLoads];
#pragma unroll
  for (int i = 0; i < BT::kALoads; ++i) {
    const int row = 16 * (wave * BT::kALoads + i) + (lane >> 2);
    ag[i] = reinterpret_cast<const unsigned char*>(A + (size_t)min(m0 + row, M - 1) * lda) + dchunk * 16;
  }
#pragma unroll
  for (int i = 0; i < BT::kWLoads; ++i) {
    const int row = 16 * (wave * BT::kWLoads + i) + (lane >> 2);
    wg[i] = reinterpret_cast<const unsigned char*>(W + (size_t)min(n0 + row, N - 1) * ldw) + dchunk * 16;
  }
  auto issue = [&](int kt) {
    unsigned char* sA = smem + (kt % BT::kStages) * BT::kStage;
    unsigned char* sW = sA + BM * BT::kRow;
#pragma unroll
    for (int i = 0; i < BT::kALoads; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(ag[i] + (size_t)kt * BT::kRow),
                                       (lptr_t)(sA + (wave * BT::kALoads + i) * 1024), 16, 0, 0);
    size_t wk = (size_t)kt * BT::kRow;
    if constexpr (MODE == kWrapT) {
      if (kt * BT::kBK >= w_wrap) wk -= (size_t)w_wrap * 2;
    }
#pragma unroll
    for (int i = 0; i < BT::kWLoads; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(wg[i] + wk), (lptr_t)(sW + (wave * BT::kWLoads + i) * 1024), 16, 0,
                                       0);
  };
  // fragment reads: row r = base + col, chunk grp -> slot grp ^ ((r >> 1) & 3) (base % 16 == 0)
  const int fslot = (grp ^ ((col >> 1) & 3)) * 16;

  f32x4 acc[BT::kFA][BT::kFW];
#pragma unroll
  for (int i = 0; i < BT::kFA; ++i)
#pragma unroll
    for (int j = 0; j < BT::kFW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BT::kBK;
#pragma unroll
  for (int s = 0; s < BT::kStages - 1; ++s)
    if (s < nk) issue(s);
  if constexpr (NW == 8) {
    // Ping-pong: waves 0-3 (wm = 0, one per SIMD) and 4-7 (wm = 1) alternate
    // between a memory phase (fragment reads of step kt, DMA issue of step
    // kt + kStages - 1, wait for this wave's part of step kt + 1) and a product
    // phase, one phase apart, with a barrier between phases.  Each SIMD then
    // runs one wave's products while its other wave reads, instead of both
    // reading and then both multiplying (Qwen3-8B LM head, 512 rows of
    // Gaussian data, one launch per step: 0.629 -> 0.586 ms; 20 launches back
    // to back: 0.766 -> 0.706 ms).  Ordering: stage kt + 1 is complete for every wave before the
    // barrier that precedes its first read; the slot refilled in the memory
    // phase of step kt held step kt - 1, whose reads (both groups, lgkmcnt(0)
    // before their barriers) ended at least one barrier earlier.
    wait_stages_lgk0<BT::kPerStage, BT::kStages - 2>(min(BT::kStages - 2, nk - 1));
    __builtin_amdgcn_s_barrier();
    if (wm == 1) __builtin_amdgcn_s_barrier();  // the second group starts one phase later
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      const unsigned char* sA = smem + (kt % BT::kStages) * BT::kStage;
      const unsigned char* sW = sA + BM * BT::kRow;
      u32x4 af[BT::kFA], wf[BT::kFW];
#pragma unroll
      for (int i = 0; i < BT::kFA; ++i) af[i] = ld16(sA + (wm * BT::kFA * 16 + i * 16 + col) * BT::kRow + fslot);
#pragma unroll
      for (int j = 0; j < BT::kFW; ++j) wf[j] = ld16(sW + (wn * BT::kFW * 16 + j * 16 + col) * BT::kRow + fslot);
      if (kt + BT::kStages - 1 < nk) issue(kt + BT::kStages - 1);
      // fragments in registers (their slot may be refilled after the barrier),
      // and this wave's part of step kt + 1 in LDS
      wait_stages_lgk0<BT::kPerStage, BT::kStages - 2>(max(0, min(BT::kStages - 2, nk - 2 - kt)));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < BT::kFA; ++i)
#pragma unroll
        for (int j = 0; j < BT::kFW; ++j) acc[i][j] = mma16<Bf16>(acc[i][j], af[i], wf[j]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
    }
    if (wm == 0) __builtin_amdgcn_s_barrier();  // equal barrier counts in both groups
  } else
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of tile kt are done once at most the younger stages are in flight
    wait_stages<BT::kPerStage, BT::kStages - 2>(min(BT::kStages - 2, nk - 1 - kt));
    __builtin_amdgcn_s_barrier();  // every wave's loads of tile kt are in LDS; tile kt - 1 is consumed
    if (kt + BT::kStages - 1 < nk) issue(kt + BT::kStages - 1);
    const unsigned char* sA = smem + (kt % BT::kStages) * BT::kStage;
    const unsigned char* sW = sA + BM * BT::kRow;
    u32x4 af[BT::kFA], wf[BT::kFW];
#pragma unroll
    for (int i = 0; i < BT::kFA; ++i) af[i] = ld16(sA + (wm * BT::kFA * 16 + i * 16 + col) * BT::kRow + fslot);
#pragma unroll
    for (int j = 0; j < BT::kFW; ++j) wf[j] = ld16(sW + (wn * BT::kFW * 16 + j * 16 + col) * BT::kRow + fslot);
#pragma unroll
    for (int i = 0; i < BT::kFA; ++i)
#pragma unroll
      for (int j = 0; j < BT::kFW; ++j) acc[i][j] = mma16<Bf16>(acc[i][j], af[i], wf[j]);
    __builtin_amdgcn_sched_group_barrier(0x100, BT::kFA + BT::kFW, 0);  // all fragment reads first,
    __builtin_amdgcn_sched_group_barrier(0x008, BT::kFA * BT::kFW, 0);  // then the products
  }

#pragma unroll
  for (int j = 0; j < BT::kFW; ++j) {
    const int n = n0 + wn * BT::kFW * 16 + j * 16 + col;
    if (n >= N) continue;
    if constexpr (MODE == kWrapT) {
      // a lane's 4 values are consecutive in C[n][:]: one 16-byte store when
      // C and ldc allow it (c_slice != 0; then M % 4 == 0 as well)
#pragma unroll
      for (int i = 0; i < BT::kFA; ++i) {
        const int m = m0 + wm * BT::kFA * 16 + i * 16 + grp * 4;
        if (c_slice) {
          if (m < M) *reinterpret_cast<f32x4*>(C + (size_t)n * ldc + m) = acc[i][j];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (m + q < M) C[(size_t)n * ldc + m + q] = acc[i][j][q];
        }
      }
    } else {
      const float bv = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
      for (int i = 0; i < BT::kFA; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + wm * BT::kFA * 16 + i * 16 + grp * 4 + q;
          if (m < M) C[(size_t)m * ldc + n] = acc[i][j][q] + bv;
        }
    }
  }
}

template <int BM, int MODE, int NW = 4, int BN = 256>
static hipError_t launch_big(const void* A, int lda, int M, const void* W, int ldw, int N, int K, const void* bias,
                             float* C, int ldc, int slices, int w_wrap, size_t c_slice, hipStream_t s) {
  using BT = BigTile<BM, NW, BN>;
  const int num_m = (M + BM - 1) / BM, num_n = (N + BT::kBN - 1) / BT::kBN;
  const int n_per_xcd = (num_n + kXcds - 1) / kXcds;
  const long blocks = MODE == kSplitK ? (long)num_m * num_n : (long)n_per_xcd * num_m * kXcds;
  if (blocks > 0x7FFFFFFF || slices > 65535) return hipErrorNotSupported;
  const size_t lds = (size_t)BT::kStages * BT::kStage;
  const void* fn = reinterpret_cast<const void*>(gemm_bf16_tn_big_kernel<BM, MODE, NW, BN>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_bf16_tn_big_kernel<BM, MODE, NW, BN>), dim3((unsigned)blocks, (unsigned)slices), dim3(BT::kThreads),
                     lds, s, static_cast<const uint16_t*>(A), lda, M, static_cast<const uint16_t*>(W), ldw, N, K,
                     static_cast<const uint16_t*>(bias), C, ldc, num_m, num_n, w_wrap, c_slice);
  return hipGetLastError();
}

// One M tile (M <= BM): num_n BM x 256 tiles on num_cu CUs (one workgroup
// each) take ceil(num_n / num_cu) rounds.  When the last round would hold at
// most half the CUs, its tiles run as twice as many BM x 128 tiles in a second
// launch: each moves (BM + 128) / (BM + 256) of a wide tile's operand bytes
// per K step, so the last round takes 2/3 (BM = 128) or 3/4 (BM = 256) of the
// time, with no partial sums (Qwen3-4B LM head, 128 rows: 0.217 -> 0.203 ms;
// Qwen3-8B, 48 / 64 / 128 rows: 0.332 / 0.337 / 0.354 -> 0.315 / 0.320 /
// 0.331 ms).
template <int BM, int NW>
static hipError_t launch_one_m_tile(const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                                    const void* bias, float* C, int ldc, int num_cu, hipStream_t s) {
  const int num_n = (N + 255) / 256;
  const int tail = num_cu > 0 ? num_n % num_cu : 0;
  if (M > BM || num_n < num_cu || tail == 0 || 2 * tail > num_cu)
    return launch_big<BM, kPlain, NW>(A, lda, M, W, ldw, N, K, bias, C, ldc, 1, 0, 0, s);
  const int n_full = (num_n - tail) * 256;  // columns in the full rounds
  hipError_t e = launch_big<BM, kPlain, NW>(A, lda, M, W, ldw, n_full, K, bias, C, ldc, 1, 0, 0, s);
  if (e != hipSuccess) return e;
  return launch_big<BM, kPlain, NW, 128>(A, lda, M, static_cast<const uint16_t*>(W) + (size_t)n_full * ldw, ldw,
                                         N - n_full, K, bias ? static_cast<const uint16_t*>(bias) + n_full : nullptr,
                                         C + n_full, ldc, 1, 0, 0, s);
}

hipError_t launch_gemm_bf16_tn(const void* A, int lda, int M, const void* W, int ldw, int N, int K, const void* bias,
                               float* C, int ldc, int num_cu, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % BigTile<256>::kBK) return hipErrorNotSupported;
  // 256 x 256 tiles with two waves per SIMD: one wave's fragment reads run
  // beside the other's products (Qwen3-8B LM head, 512 rows: 0.831 -> 0.802 ms
  // against one wave per SIMD)
  if (M >= 256) return launch_one_m_tile<256, 8>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
  // 33 .. 255 rows: 128-row tiles, with 8 waves and the ping-pong loop for
  // long rows (Qwen3-8B LM head, K = 4096, at 48 / 64 / 128 rows: 0.359 /
  // 0.367 / 0.389 -> 0.330 / 0.334 / 0.352 ms), else 4 waves (Qwen3-4B, K =
  // 2560, 128 rows: 0.217 ms against 0.220 with 8)
  return K >= 4096 ? launch_one_m_tile<128, 8>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s)
                   : launch_one_m_tile<128, 4>(A, lda, M, W, ldw, N, K, bias, C, ldc, num_cu, s);
}

hipError_t launch_gemm_bf16_tn_splitk(const void* A, int lda, int M, const void* W, int ldw, int N, int kc,
                                      int slices, int w_wrap, float* C, int ldc, size_t c_slice, hipStream_t s) {
  if (M <= 0 || N <= 0 || slices <= 0) return hipSuccess;
  if (kc <= 0 || kc % BigTile<256>::kBK || w_wrap <= 0 || w_wrap % kc) return hipErrorNotSupported;
  return M >= 256 ? launch_big<256, kSplitK, 8>(A, lda, M, W, ldw, N, kc, nullptr, C, ldc, slices, w_wrap, c_slice, s)
                  : launch_big<128, kSplitK>(A, lda, M, W, ldw, N, kc, nullptr, C, ldc, slices, w_wrap, c_slice, s);
}

hipError_t launch_gemm_bf16_tn_wrapt(const void* A, int lda, int M, const void* W, int ldw, int N, int K, int w_wrap,
                                     float* C, int ldc, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % BigTile<256>::kBK || w_wrap % BigTile<256>::kBK || w_wrap <= 0 || K > 2 * w_wrap)
    return hipErrorNotSupported;
  const size_t vec = (reinterpret_cast<uintptr_t>(C) & 15u) == 0 && ldc % 4 == 0 && M % 4 == 0;
  return M >= 256 ? launch_big<256, kWrapT, 8>(A, lda, M, W, ldw, N, K, nullptr, C, ldc, 1, w_wrap, vec, s)
                  : launch_big<128, kWrapT>(A, lda, M, W, ldw, N, K, nullptr, C, ldc, 1, w_wrap, vec, s);
}
}  // namespace domino
