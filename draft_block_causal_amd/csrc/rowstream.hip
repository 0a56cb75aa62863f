// Row-streaming LM-head kernel: C = A W^T (+bias) for at most 32 rows of A,
// bound by the single read of W from HBM.  Used for the frozen LM head over
// the K positions of a block ([notes] §二.1(1); [explainer] §三) and for the
// hidden half of the first correction projection.
//
// Pages (cited by title and section):
//   [notes]     "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn)
//   [explainer] the yhxrc.cn article on the Domino paper
#include "common.h"
#include "kernels.h"

namespace domino {

constexpr int kRowStreamWaves = 8;

// ---------------------------------------------------------------------------
// rowstream_gemm: the split-K product above with W read the way HBM streams
// best.  A load instruction of the split-K kernel covers 64 B of each of 16
// rows; here each covers whole 16-B chunks of contiguous runs of one or a
// few rows (two runs of 512 B when d = 4096 bf16), read non-temporally since
// W is used once.  Each wave writes its row slices into a private LDS tile and
// reads them back in the matrix-core operand layout (row = lane column), in
// passes of at most 512 B per row so that the tile stays 8 KB.  The 16-B
// chunks of row r are stored XOR-swizzled by r & 15, so both the row-wise
// writes and the column-wise reads touch 16 distinct bank groups per 16 lanes.
// W and the bias are read through buffer descriptors sized to the valid rows
// of the tile: rows past N, and the prefetch past the last tile, read as zero
// without touching memory, so every load is unconditional and the next tile
// is always in flight while the current one is multiplied (two register
// buffers used in turn, so no copies).  The partial tiles of the 8 waves are
// summed in LDS in a fixed order; the two halves of the loop use separate
// reduction buffers, so one barrier per tile suffices.  Finished output tiles
// stay in LDS and are written after the workgroup's last tile: C stores mixed
// into the W stream cost ~8 % of HBM read throughput, as scattered writes.
// KW in {4, 8, 16}.
// ---------------------------------------------------------------------------
template <int KW>
struct RowStream {
  static constexpr int kSlice = KW * 64;                         // bytes of a row per wave
  static constexpr int kPass = kSlice < 512 ? kSlice : 512;      // bytes of a row per LDS pass
  static constexpr int kPasses = kSlice / kPass;
  static constexpr int kChunks = kPass / 16;                     // 16-B chunks per row and pass
  static constexpr int kRowsPerLoad = 64 / kChunks;              // rows one load instruction covers
  static constexpr int kLoadsPerPass = 16 / kRowsPerLoad;
  static constexpr int kStepsPerPass = kPass / 64;               // matrix-core K steps per pass
  static constexpr size_t kTileLds = 16 * kPass;                 // one wave's transposition tile
  static constexpr int kRed = kRowStreamWaves * 16 * 17;             // floats per reduction buffer
  static constexpr size_t kFixedLds = kRowStreamWaves * kTileLds + 2 * kRed * sizeof(float);
  static constexpr int kOutTileFloats = 256;                     // one 16 x 16 output tile
  static_assert(kChunks >= 16 && kRowsPerLoad >= 1 && kPasses * kLoadsPerPass == KW, "row-stream shape");
};
constexpr size_t kMaxLds = 160 * 1024;


template <class T>
__device__ __forceinline__ unsigned load_elem_bits(__amdgpu_buffer_rsrc_t r, int off);
template <>
__device__ __forceinline__ unsigned load_elem_bits<Bf16>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <>
__device__ __forceinline__ unsigned load_elem_bits<F32>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <class T>
__device__ __forceinline__ float elem_bits_to_f32(unsigned u);
template <>
__device__ __forceinline__ float elem_bits_to_f32<Bf16>(unsigned u) { return __uint_as_float(u << 16); }
template <>
__device__ __forceinline__ float elem_bits_to_f32<F32>(unsigned u) { return __uint_as_float(u); }

template <class T, int KW, bool BIAS>
__global__ void __launch_bounds__(kRowStreamWaves * 64)
    rowstream_gemm_kernel(const typename T::elem* __restrict__ A, int lda, int M,
                          const typename T::elem* __restrict__ W, int ldw, int N,
                          const typename T::elem* __restrict__ bias, float* __restrict__ C, int ldc,
                          int out_tiles, int G, int groups) {
  using RS = RowStream<KW>;
  using E = typename T::elem;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  // x: the workgroup's W range (tiles x, x + G, ...); y: its 16-row slice of A.
  // groups > 1 (a 1-D grid of G * groups): the `groups` slices of one W range
  // get consecutive numbers on one XCD (workgroups go round-robin over the 8
  // XCDs), so they stream the same W tiles at about the same time and all but
  // the first read hit that XCD's L2.
  int x, y;
  if (groups > 1) {
    const int b = blockIdx.x, local = b >> 3;
    y = local % groups;
    x = (b & 7) + 8 * (local / groups);
  } else {
    x = blockIdx.x;
    y = blockIdx.y;
  }
  const int m0 = y * 16;
  unsigned char* tile = smem + (size_t)wave * RS::kTileLds;
  float* red = reinterpret_cast<float*>(smem + kRowStreamWaves * RS::kTileLds);
  float* obuf = reinterpret_cast<float*>(smem + RS::kFixedLds);  // out_tiles finished 16 x 16 tiles

  u32x4 af[KW];
  {
    const bool live = m0 + col < M;
    const unsigned char* arow = reinterpret_cast<const unsigned char*>(A + (size_t)(live ? m0 + col : 0) * lda) +
                                (size_t)wave * RS::kSlice + grp * 16;
#pragma unroll
    for (int s = 0; s < KW; ++s) af[s] = live ? ld16(arow + s * 64) : u32x4{0, 0, 0, 0};
  }
  const int ntiles = (N + 15) >> 4;
  const int row_bytes = ldw * (int)sizeof(E);
  // load jj of pass p: row jj * kRowsPerLoad + lrow, chunk lchunk of the pass
  const int lrow = lane / RS::kChunks, lchunk = lane % RS::kChunks;
  const int voff = lrow * row_bytes + wave * RS::kSlice + lchunk * 16;
  const __amdgpu_buffer_rsrc_t brs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(BIAS ? bias : W), (short)0, BIAS ? N * (int)sizeof(E) : 0,
                                        kRsrcWord3);
  const int rcol = threadIdx.x & 15;  // output column of a reducing thread

  // Load jj of a pass reads rows jj * kRowsPerLoad ... of the tile through a
  // descriptor based at its first row and sized to those of its rows below N
  // (none past the last tile), so one lane offset serves every load and the
  // range check covers every row.
  auto stage = [&](int t, u32x4 (&dst)[KW], unsigned& bv) {
    const int rows = t < ntiles ? min(16, N - t * 16) : 0;
    const E* base = W + (t < ntiles ? (size_t)t * 16 * ldw : 0);
#pragma unroll
    for (int jj = 0; jj < RS::kLoadsPerPass; ++jj) {
      // (rows >= 0; a clamp on both sides for jj = 0 becomes a vector med3 and
      // the descriptor a per-lane value)
      const int rj = jj == 0 ? min(rows, RS::kRowsPerLoad) : min(max(rows - jj * RS::kRowsPerLoad, 0), RS::kRowsPerLoad);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<E*>(base + (rj > 0 ? (size_t)jj * RS::kRowsPerLoad * ldw : 0)), (short)0, rj * row_bytes,
          kRsrcWord3);
#pragma unroll
      for (int p = 0; p < RS::kPasses; ++p)
        dst[p * RS::kLoadsPerPass + jj] =
            __builtin_amdgcn_raw_buffer_load_b128(r, voff + p * RS::kPass, 0, kLoadNonTemporal);
    }
    bv = BIAS ? load_elem_bits<T>(brs, (t * 16 + rcol) * (int)sizeof(E)) : 0u;
  };
  auto process = [&](int i, int t, const u32x4 (&w)[KW], unsigned bv, float* rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < RS::kPasses; ++p) {
#pragma unroll
      for (int jj = 0; jj < RS::kLoadsPerPass; ++jj) {
        const int r = jj * RS::kRowsPerLoad + lrow;
        st16(tile + r * RS::kPass + ((lchunk ^ (r & 15)) << 4), w[p * RS::kLoadsPerPass + jj]);
      }
#pragma unroll
      for (int ss = 0; ss < RS::kStepsPerPass; ++ss) {
        const u32x4 b = ld16(tile + col * RS::kPass + (((ss * 4 + grp) ^ col) << 4));
        acc = mma16<T>(acc, af[p * RS::kStepsPerPass + ss], b);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[(wave * 16 + grp * 4 + j) * 17 + col] = acc[j];
    // converted by every wave, outside the branch below: a load that only one
    // side of a branch consumes makes the compiler drain the prefetch later
    float bias_n = elem_bits_to_f32<T>(bv);
    if (BIAS) asm volatile("" : "+v"(bias_n));  // keeps the compiler from sinking it into the branch
    __syncthreads();
    if (threadIdx.x < 256) {
      const int m = threadIdx.x >> 4;
      float sum = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < kRowStreamWaves; ++w8) sum += rb[(w8 * 16 + m) * 17 + rcol];
      sum += bias_n;
      if (i < out_tiles) {
        obuf[i * RS::kOutTileFloats + threadIdx.x] = sum;
      } else {  // more tiles than the LDS holds: store directly
        const int n = t * 16 + rcol;
        if (m0 + m < M && n < N) C[(size_t)(m0 + m) * ldc + n] = sum;
      }
    }
  };

  u32x4 w0[KW], w1[KW];
  unsigned b0, b1;
  int t = x, i = 0;
  stage(t, w0, b0);
  // The scheduling barriers keep each prefetch ahead of the LDS traffic of
  // the tile in hand; left alone, the compiler sinks the loads below it and
  // the wait for the current tile then drains the prefetch as well.
  while (t < ntiles) {
    stage(t + G, w1, b1);
    __builtin_amdgcn_sched_barrier(0);
    process(i, t, w0, b0, red);
    t += G;
    ++i;
    if (t >= ntiles) break;
    stage(t + G, w0, b0);
    __builtin_amdgcn_sched_barrier(0);
    process(i, t, w1, b1, red + RS::kRed);
    t += G;
    ++i;
  }
  // the held output tiles, local tile k = global tile x + k * G
  __syncthreads();
  const int held = min(i, out_tiles);
  for (int e = threadIdx.x; e < held * RS::kOutTileFloats; e += kRowStreamWaves * 64) {
    const int k = e >> 8, m = (e >> 4) & 15;
    const int n = (x + k * G) * 16 + (e & 15);
    if (m0 + m < M && n < N) C[(size_t)(m0 + m) * ldc + n] = obuf[e];
  }
}

template <class T, int KW>
static hipError_t rowstream_t(const void* A, int lda, int M, const void* W, int ldw, int N, const void* bias,
                              float* C, int ldc, int num_cu, hipStream_t s) {
  using E = typename T::elem;
  using RS = RowStream<KW>;
  auto kern = bias ? rowstream_gemm_kernel<T, KW, true> : rowstream_gemm_kernel<T, KW, false>;
  const int ntiles = (N + 15) / 16;
  // 17 .. 32 rows with a large W: the two 16-row slices share W ranges
  // through L2 (Qwen3-8B LM head, 32 rows: 226 us against 383 us with one W
  // read from HBM per slice; four slices sharing a range took 396 us at 64
  // rows, slower than the tiled kernel); else one W range per compute unit
  // and slice
  const int slices = (M + 15) / 16;
  const bool grouped = slices == 2 && num_cu % (8 * slices) == 0 && ntiles >= num_cu;
  const int gx = grouped ? num_cu / slices : std::min(ntiles, num_cu);
  // hold every output tile of a workgroup in LDS when it fits
  const int per_wg = (ntiles + gx - 1) / gx;
  const int fit = (int)((kMaxLds - RS::kFixedLds) / (RS::kOutTileFloats * sizeof(float)));
  const int out_tiles = std::min(per_wg, fit);
  const size_t lds = RS::kFixedLds + (size_t)out_tiles * RS::kOutTileFloats * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid = grouped ? dim3(gx * slices) : dim3(gx, slices);
  hipLaunchKernelGGL(kern, grid, dim3(kRowStreamWaves * 64), lds, s, static_cast<const E*>(A), lda, M,
                     static_cast<const E*>(W), ldw, N, static_cast<const E*>(bias), C, ldc, out_tiles, gx,
                     grouped ? slices : 1);
  return hipGetLastError();
}


// Returns hipErrorNotSupported unless K * elem_size is 8 * 64 * KW bytes with
// KW in {4, 8, 16} and every W row starts 16-byte aligned.  Each 16-row slice
// of A streams all of W (two slices share it through L2, above), so more than
// 32 rows are taken only for a small W and a moderate M (N, M <= 4096: the
// hidden half of the first correction projection at B > 2), whose re-reads
// come from the caches.
hipError_t launch_rowstream_gemm(int dtype, const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                                 const void* bias, float* C, int ldc, int num_cu, hipStream_t s) {
  const size_t elem = dtype == 1 ? 2 : 4;
  const size_t row_bytes = (size_t)K * elem;
  if ((M > 32 && (N > 4096 || M > 4096)) || row_bytes % (64 * kRowStreamWaves) || ((size_t)ldw * elem) % 16)
    return hipErrorNotSupported;
  switch (row_bytes / (64 * kRowStreamWaves)) {
    case 4: return dtype == 1 ? rowstream_t<Bf16, 4>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s)
                              : rowstream_t<F32, 4>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 8: return dtype == 1 ? rowstream_t<Bf16, 8>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s)
                              : rowstream_t<F32, 8>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    case 16: return dtype == 1 ? rowstream_t<Bf16, 16>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s)
                               : rowstream_t<F32, 16>(A, lda, M, W, ldw, N, bias, C, ldc, num_cu, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace domino
