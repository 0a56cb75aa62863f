// Backward through time of the teacher-forced GRU causal encoder ([notes]
// §二.1(2) item 1 and §二.2(1)): from dg[b][i], the gradient of a loss with
// respect to each state g_i from outside the recurrence, to the gradients of
// W_ih, W_hh, b_ih and b_hh.  The forward is g_i = GRU(E[tok_i], g_{i-1}),
// g_{-1} = 0, tok_0 = x_t, tok_i = teacher[i - 1]; PyTorch GRUCell gates
// r | z | n with the reset applied to W_hn g + b_hn.
//
// Launches on the caller's stream, all float32 with sums in a fixed order:
//   1. gb_gather_kernel: per row (b, i) the token's embedding row and the
//      previous state (zero at i = 0);
//   2. the pre-activations of every row, independent of the backward:
//      a = W_ih e + b_ih (the tiled matrix-core GEMM on the gathered rows) and
//      c = W_hh g_prev + b_hh (float32 states: gb_matvec_kernel; bf16 heads:
//      the states split hi / lo by gb_hilo_kernel, split-K partials of the
//      tiled GEMM, added in slice order with the bias by gb_csum_kernel);
//   3. per position i = K-1 … 0: gb_elem_kernel (the gate derivatives of
//      every row of position i: da, dc and the direct part z dg of the carry)
//      and gb_carry_kernel (W_hhᵀ dc, the rest of the gradient reaching
//      g_{i-1}, its 3H terms split over P workgroups and their waves, the P
//      partial sums added by the next gb_elem_kernel; bf16 heads:
//      gb_carrym_kernel on the matrix cores against W_hh transposed once by
//      gb_whht_kernel);
//   4. gb_outer_kernel twice: dW_ih = Σ da eᵀ, db_ih = Σ da and
//      dW_hh = Σ dc g_prevᵀ, db_hh = Σ dc over every row; bf16 heads from
//      kGbMfmaRows rows on: the operands re-laid by gb_tsplit_kernel and the
//      tiled matrix-core GEMM twice, the bias sums from per-tile partials
//      (gb_bsum_kernel).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace domino {

constexpr int kGbThreads = 256;
constexpr int kGbWaves = kGbThreads / 64;
constexpr int kGbQ = 16;  // output rows per thread in the outer-product sums
constexpr int kGbCarryNB = kGruCarryBlocks;  // blocks per carry workgroup from 8 blocks up

// x_e[row][:] = E[tok(row)][:] (head dtype) and x_g[row][:] = states[b][i - 1][:] (zero at i = 0).
template <class T>
__global__ void gb_gather_kernel(int B, int K, int d, int H, int V, const int32_t* __restrict__ x_t,
                                 const int32_t* __restrict__ teacher, const typename T::elem* __restrict__ embed,
                                 const float* __restrict__ states, typename T::elem* __restrict__ x_e,
                                 float* __restrict__ x_g, int32_t* __restrict__ tok) {
  const int row = blockIdx.x, b = row / K, i = row - b * K;
  int t = i == 0 ? x_t[b] : teacher[(size_t)b * K + i - 1];
  t = min(max(t, 0), V - 1);
  if (threadIdx.x == 0) tok[row] = t;
  for (int k = threadIdx.x; k < d; k += blockDim.x) x_e[(size_t)row * d + k] = embed[(size_t)t * d + k];
  for (int k = threadIdx.x; k < H; k += blockDim.x)
    x_g[(size_t)row * H + k] = i == 0 ? 0.f : states[((size_t)b * K + i - 1) * H + k];
}

// out[row][q] = W[q][:] . x[row][:] + bias[q] for q in the workgroup's 64 rows
// of W (blockIdx.y); x (float32) staged in LDS; rows of W split over the
// lanes of a wave, four at a time.
template <class T>
__global__ void __launch_bounds__(kGbThreads) gb_matvec_kernel(int N, int n, const typename T::elem* __restrict__ W,
                                                               const typename T::elem* __restrict__ bias,
                                                               const float* __restrict__ x, float* __restrict__ out) {
  using E = typename T::elem;
  constexpr int EPF = T::kPer16B;
  extern __shared__ __attribute__((aligned(16))) float xs[];
  const int row = blockIdx.x, n0 = blockIdx.y * 64;
  for (int k = threadIdx.x; k < n; k += kGbThreads) xs[k] = x[(size_t)row * n + k];
  __syncthreads();
  const int wave = wave_id(), lane = threadIdx.x & 63;
  for (int q0 = n0 + wave * 4; q0 < min(N, n0 + 64); q0 += kGbWaves * 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = lane * EPF; k < n; k += 64 * EPF) {
      u32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = q0 + j < N ? ld16(W + (size_t)(q0 + j) * n + k) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const E* e = reinterpret_cast<const E*>(&w[j]);
#pragma unroll
        for (int c = 0; c < EPF; ++c) acc[j] += T::to_f32(e[c]) * xs[k + c];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = acc[j];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0 && q0 + j < N) out[(size_t)row * N + q0 + j] = s + (bias ? T::to_f32(bias[q0 + j]) : 0.f);
    }
  }
}

// xs[row][:] = hi | lo of x_g[row][:] (hi truncated to bf16, lo the rest
// rounded to bf16), the matrix-core operand for c = W_hh g_prev.
__global__ void gb_hilo_kernel(int R, int H, const float* __restrict__ x_g, uint16_t* __restrict__ xs) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x, row = blockIdx.y;
  if (k >= H) return;
  const float x = x_g[(size_t)row * H + k];
  const uint32_t t = __float_as_uint(x) & 0xFFFF0000u;
  xs[(size_t)row * 2 * H + k] = (uint16_t)(t >> 16);
  xs[(size_t)row * 2 * H + H + k] = (uint16_t)f32_to_bf16_rne(x - __uint_as_float(t));
}

// c[row][q] = Σ_s cpart[s][row][q] (slice order) + b_hh[q].
__global__ void gb_csum_kernel(long n, int G3, int S, const float* __restrict__ cpart,
                               const uint16_t* __restrict__ bias, float* __restrict__ c) {
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += cpart[(size_t)s * n + e];
  c[e] = v + (bias ? bf16_to_f32(bias[e % G3]) : 0.f);
}

// Gate derivatives of the rows of position i, one thread per (b, unit j).
// The carry reaching this position is carry[0] (the direct part) plus the P
// partial sums carry[1 .. P] of the previous gb_carry_kernel, in that order.
__global__ void gb_elem_kernel(int B, int K, int H, int i, int P, const float* __restrict__ a,
                               const float* __restrict__ c, const float* __restrict__ x_g,
                               const float* __restrict__ dg, float* __restrict__ carry, float* __restrict__ da,
                               float* __restrict__ dc) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x, b = blockIdx.y;
  if (j >= H) return;
  const size_t row = (size_t)b * K + i, G3 = 3 * (size_t)H;
  const float* ar = a + row * G3;
  const float* cr = c + row * G3;
  const float r = sigmoidf_(ar[j] + cr[j]);
  const float z = sigmoidf_(ar[H + j] + cr[H + j]);
  const float n = tanhf(ar[2 * H + j] + r * cr[2 * H + j]);
  const float gp = x_g[row * H + j];
  const size_t BH = (size_t)B * H;
  float cin = carry[(size_t)b * H + j];
  for (int p = 1; p <= P; ++p) cin += carry[p * BH + (size_t)b * H + j];
  const float d_g = dg[row * H + j] + cin;
  const float d_n = d_g * (1.f - z);
  const float d_z = d_g * (gp - n);
  const float d_pn = d_n * (1.f - n * n);
  const float d_pr = d_pn * cr[2 * H + j] * r * (1.f - r);
  const float d_pz = d_z * z * (1.f - z);
  da[row * G3 + j] = d_pr;
  da[row * G3 + H + j] = d_pz;
  da[row * G3 + 2 * H + j] = d_pn;
  dc[row * G3 + j] = d_pr;
  dc[row * G3 + H + j] = d_pz;
  dc[row * G3 + 2 * H + j] = d_pn * r;
  carry[(size_t)b * H + j] = d_g * z;  // the direct part; gb_carry_kernel adds W_hhᵀ dc
}

// carry[1 + p][b][j] = Σ_q W_hh[q][j] dc[row(b, i)][q] over group p
// (blockIdx.z) of the 3H terms: a workgroup takes 64 units j (one per lane)
// of NB blocks b (each W_hh value loaded once for the NB blocks); its 4 waves
// take a quarter of the group each, eight loads in flight per lane, and the
// quarter sums are added in wave order.
template <class T, int NB>
__global__ void __launch_bounds__(kGbThreads) gb_carry_kernel(int B, int K, int H, int i,
                                                              const typename T::elem* __restrict__ w_hh,
                                                              const float* __restrict__ dc, float* __restrict__ carry) {
  __shared__ float part[kGbWaves][NB][64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int j = blockIdx.x * 64 + lane, b0 = blockIdx.y * NB, G3 = 3 * H;
  const int nb = min(NB, B - b0);
  const int parts = (int)gridDim.z * kGbWaves, idx = (int)blockIdx.z * kGbWaves + wave;
  const int qa = (int)((long)G3 * idx / parts), qb = (int)((long)G3 * (idx + 1) / parts);
  const float* d[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) d[t] = dc + ((size_t)(b0 + min(t, nb - 1)) * K + i) * G3;
  float acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = 0.f;
  if (j < H) {
    int q = qa;
    for (; q + 8 <= qb; q += 8) {
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = T::to_f32(w_hh[(size_t)(q + u) * H + j]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int t = 0; t < NB; ++t) acc[t] += w[u] * d[t][q + u];
    }
    for (; q < qb; ++q) {
      const float w = T::to_f32(w_hh[(size_t)q * H + j]);
#pragma unroll
      for (int t = 0; t < NB; ++t) acc[t] += w * d[t][q];
    }
  }
#pragma unroll
  for (int t = 0; t < NB; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave == 0 && j < H)
    for (int t = 0; t < nb; ++t) {
      float sum = part[0][t][lane];
      for (int w = 1; w < kGbWaves; ++w) sum += part[w][t][lane];
      carry[(1 + blockIdx.z) * (size_t)B * H + (size_t)(b0 + t) * H + j] = sum;
    }
}

// bf16 heads: whhT[j][q] = W_hh[q][j] (once per call), 64 x 64 tiles through LDS.
__global__ void __launch_bounds__(kGbThreads) gb_whht_kernel(int H, const uint16_t* __restrict__ w_hh,
                                                             uint16_t* __restrict__ whhT) {
  __shared__ uint16_t t[64][66];
  const int G3 = 3 * H, j0 = blockIdx.x * 64, q0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int qq = (tid >> 6) + 4 * i, jj = tid & 63;
    t[qq][jj] = q0 + qq < G3 && j0 + jj < H ? w_hh[(size_t)(q0 + qq) * H + j0 + jj] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int jj = (tid >> 6) + 4 * i, qq = tid & 63;
    if (j0 + jj < H && q0 + qq < G3) whhT[(size_t)(j0 + jj) * G3 + q0 + qq] = t[qq][jj];
  }
}

// bf16 heads: carry[1 + p][b][j] = Σ_q W_hh[q][j] dc[row(b, i)][q] over group
// p (blockIdx.z) of the 3H terms on the matrix cores: 16 blocks (blockIdx.y)
// x 64 units (16 per wave), dc split hi + lo, the group's K steps in order
// with eight steps of loads in flight.  3H a multiple of 32 gridDim.z.
__global__ void __launch_bounds__(kGbThreads) gb_carrym_kernel(int B, int K, int H, int i,
                                                               const uint16_t* __restrict__ whhT,
                                                               const float* __restrict__ dc,
                                                               float* __restrict__ carry) {
  const int wave = wave_id(), lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int G3 = 3 * H, b0 = blockIdx.y * 16, j0 = blockIdx.x * 64 + wave * 16;
  if (j0 >= H) return;  // (uniform over the wave; no barrier below)
  const int steps = G3 / 32 / (int)gridDim.z, s_begin = (int)blockIdx.z * steps;
  const int b = min(b0 + col, B - 1), jr = min(j0 + col, H - 1);
  const float* arow = dc + ((size_t)b * K + i) * G3 + grp * 8;
  const unsigned char* wrow = reinterpret_cast<const unsigned char*>(whhT + (size_t)jr * G3) + grp * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kU = 8;
  for (int s0 = 0; s0 < steps; s0 += kU) {
    u32x4 w[kU];
    float x[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int st = s_begin + min(s0 + u, steps - 1);  // past the group: a repeated step, zeroed below
      w[u] = ld16(wrow + (size_t)st * 64);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(arow + (size_t)st * 32);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(arow + (size_t)st * 32 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[u][e] = v0[e];
        x[u][e + 4] = v1[e];
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float xs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[e] = s0 + u < steps ? x[u][e] : 0.f;
      ActFrag<Bf16> a;
      a.from_f32(xs);
      acc = a.mma(acc, w[u]);
    }
  }
  const int j = j0 + col;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int bb = b0 + grp * 4 + q;
    if (bb < B && j < H) carry[(1 + blockIdx.z) * (size_t)B * H + (size_t)bb * H + j] = acc[q];
  }
}

// out[q][k] = Σ_rows A[row][q] X[row][k] for q0 .. q0 + 15 (X of type XE);
// bias[q] = Σ_rows A[row][q] from the workgroups with blockIdx.x == 0.  The
// A values of 64 rows at a time are staged in LDS (read as broadcasts).
constexpr int kGbRowsLds = 64;
template <class XE>
__global__ void __launch_bounds__(kGbThreads) gb_outer_kernel(int R, int Q, int N, const float* __restrict__ A,
                                                              const XE* __restrict__ X, float* __restrict__ out,
                                                              float* __restrict__ bias) {
  __shared__ float as[kGbRowsLds][kGbQ];
  const int k = blockIdx.x * kGbThreads + threadIdx.x, q0 = blockIdx.y * kGbQ;
  const int nq = min(kGbQ, Q - q0);
  float acc[kGbQ];
#pragma unroll
  for (int q = 0; q < kGbQ; ++q) acc[q] = 0.f;
  float bsum = 0.f;
  for (int r0 = 0; r0 < R; r0 += kGbRowsLds) {
    const int nr = min(kGbRowsLds, R - r0);
    __syncthreads();
    for (int e = threadIdx.x; e < kGbRowsLds * kGbQ; e += kGbThreads) {
      const int rr = e / kGbQ, q = e % kGbQ;
      as[rr][q] = rr < nr && q < nq ? A[(size_t)(r0 + rr) * Q + q0 + q] : 0.f;
    }
    __syncthreads();
    if (blockIdx.x == 0 && (int)threadIdx.x < nq)
      for (int rr = 0; rr < nr; ++rr) bsum += as[rr][threadIdx.x];
    if (k < N)
      for (int rr = 0; rr < nr; ++rr) {
        float x;
        if constexpr (sizeof(XE) == 2)
          x = bf16_to_f32(X[(size_t)(r0 + rr) * N + k]);
        else
          x = X[(size_t)(r0 + rr) * N + k];
#pragma unroll
        for (int q = 0; q < kGbQ; ++q) acc[q] += as[rr][q] * x;
      }
  }
  if (k < N)
    for (int q = 0; q < nq; ++q) out[(size_t)(q0 + q) * N + k] = acc[q];
  if (blockIdx.x == 0 && bias && (int)threadIdx.x < nq) bias[q0 + threadIdx.x] = bsum;
}

// bf16 heads: the two weight gradients as matrix-core GEMMs over the rows,
// dW_ih = [da_hi | da_lo] [e | e]^T and dW_hh = [dc_hi | dc_hi | dc_lo]
// [g_hi | g_lo | g_hi]^T (x = hi + lo as in the correction-head backward, the
// lo lo term dropped), each operand re-laid with the rows along K.  Job j
// (blockIdx.z) of one launch: Y[n][p Rp + r] = part p of X[r][n] as bf16 for
// r < R (zero up to Rp); bit p of `lo_parts` set: the remainder x - hi
// rounded to bf16, else hi = x truncated to bf16 (for bf16 X, x itself).  One
// 64 x 64 tile of X per workgroup through LDS; with `bpart`, the tile's
// column sums (its rows in order) go to bpart[blockIdx.y][n].
// (KJob, KJobs: kernels.h)
__global__ void __launch_bounds__(256) gb_tsplit_kernel(int R, int Rp, KJobs jobs) {
  __shared__ float t[64][65];
  const KJob& jb = jobs.j[blockIdx.z];
  const int N = jb.N, n0 = blockIdx.x * 64, r0 = blockIdx.y * 64, tid = threadIdx.x;
  if (n0 >= N) return;  // (uniform over the workgroup)
  {
    const int c = tid & 63, n = n0 + c;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int rr = (tid >> 6) + 4 * j, r = r0 + rr;
      float x = 0.f;
      if (r < R && n < N)
        x = jb.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(jb.X)[(size_t)r * N + n])
                    : static_cast<const float*>(jb.X)[(size_t)r * N + n];
      t[rr][c] = x;
    }
  }
  __syncthreads();
  if (jb.bpart && tid < 64 && n0 + tid < N) {
    float sum = 0.f;
    for (int rr = 0; rr < 64; ++rr) sum += t[rr][tid];
    jb.bpart[(size_t)blockIdx.y * N + n0 + tid] = sum;
  }
  const int c = tid >> 2, rq = (tid & 3) * 16, n = n0 + c;
  if (n >= N || r0 + rq >= Rp) return;  // (Rp is a multiple of 32: 16-row runs never straddle it)
  uint32_t hi[16], lo[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float x = t[rq + e][c];
    const uint32_t u = __float_as_uint(x) & 0xFFFF0000u;
    hi[e] = u >> 16;
    lo[e] = f32_to_bf16_rne(x - __uint_as_float(u));
  }
  uint16_t* dst = jb.Y + (size_t)n * jb.nparts * Rp + r0 + rq;
  for (int p = 0; p < jb.nparts; ++p) {
    const uint32_t* v = (jb.lo_parts >> p) & 1u ? lo : hi;
    st16(dst + (size_t)p * Rp, u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)});
    st16(dst + (size_t)p * Rp + 8,
         u32x4{v[8] | (v[9] << 16), v[10] | (v[11] << 16), v[12] | (v[13] << 16), v[14] | (v[15] << 16)});
  }
}

// bias y[n] = the tiles' column sums added in tile order (blockIdx.y: which
// of the two).
__global__ void gb_bsum_kernel(int tiles, int N, const float* __restrict__ bpart0, float* __restrict__ bias0,
                               const float* __restrict__ bpart1, float* __restrict__ bias1) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const float* bpart = blockIdx.y ? bpart1 : bpart0;
  float* bias = blockIdx.y ? bias1 : bias0;
  if (n >= N || !bias) return;
  float sum = 0.f;
  for (int i = 0; i < tiles; ++i) sum += bpart[(size_t)i * N + n];
  bias[n] = sum;
}

hipError_t launch_rows_to_k(int R, int Rp, const KJobs& jobs, int njobs, int nmax, hipStream_t s) {
  if (R <= 0 || njobs <= 0) return hipSuccess;
  if (njobs > 4 || Rp % 32 || Rp < R) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gb_tsplit_kernel, dim3((nmax + 63) / 64, (Rp + 63) / 64, njobs), dim3(256), 0, s, R, Rp, jobs);
  return hipGetLastError();
}

hipError_t launch_tile_colsums(int tiles, int N, const float* bpart0, float* sum0, const float* bpart1, float* sum1,
                               hipStream_t s) {
  if (N <= 0 || (!sum0 && !sum1)) return hipSuccess;
  hipLaunchKernelGGL(gb_bsum_kernel, dim3((N + 255) / 256, 2), dim3(256), 0, s, tiles, N, bpart0, sum0, bpart1, sum1);
  return hipGetLastError();
}

// Rows (blocks x positions) from which bf16 heads take the weight gradients
// to the matrix cores (Qwen3-8B: at 512 rows 112 against 342 us with the
// float32 outer products; at 16 rows ~50 against 24 us, the launches' fixed
// cost)
constexpr int kGbMfmaRows = 128;

template <class T>
static hipError_t gru_backward_t(const GruBackwardArgs& g, int num_cu, hipStream_t s) {
  using E = typename T::elem;
  const int B = g.B, K = g.K, d = g.d, H = g.H, V = g.V, R = B * K, G3 = 3 * H;
  const GruBackwardPlan& pl = g.plan;
  unsigned char* ws = static_cast<unsigned char*>(g.workspace);
  E* x_e = reinterpret_cast<E*>(ws + pl.x_e);
  float* x_g = reinterpret_cast<float*>(ws + pl.x_g);
  float* a = reinterpret_cast<float*>(ws + pl.a);
  float* c = reinterpret_cast<float*>(ws + pl.c);
  float* da = reinterpret_cast<float*>(ws + pl.da);
  float* dc = reinterpret_cast<float*>(ws + pl.dc);
  float* carry = reinterpret_cast<float*>(ws + pl.carry);
  int32_t* tok = reinterpret_cast<int32_t*>(ws + pl.tok);
  hipLaunchKernelGGL(gb_gather_kernel<T>, dim3(R), dim3(256), 0, s, B, K, d, H, V, g.x_t, g.teacher,
                     static_cast<const E*>(g.embed), g.states, x_e, x_g, tok);
  hipError_t e = launch_panel_gemm(g.dtype, x_e, d, R, g.w_ih, d, G3, d, g.b_ih, a, G3, num_cu, s);
  if (e != hipSuccess) return e;
  if (pl.S > 0) {
    // bf16: c = [g_hi | g_lo] [W_hh ; W_hh]^T + b_hh as split-K partials on the matrix cores
    uint16_t* xs = reinterpret_cast<uint16_t*>(ws + pl.xs);
    float* cpart = reinterpret_cast<float*>(ws + pl.cpart);
    hipLaunchKernelGGL(gb_hilo_kernel, dim3((H + 255) / 256, R), dim3(256), 0, s, R, H, x_g, xs);
    e = launch_gemm_bf16_tn_splitk(xs, 2 * H, R, g.w_hh, H, G3, 2 * H / pl.S, pl.S, H, cpart, G3,
                                   (size_t)R * G3, s);
    if (e != hipSuccess) return e;
    const long n = (long)R * G3;
    hipLaunchKernelGGL(gb_csum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, G3, pl.S, cpart,
                       static_cast<const uint16_t*>(g.b_hh), c);
  } else {
    const size_t lds = (size_t)H * sizeof(float);
    if (lds > 65536) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(gb_matvec_kernel<T>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gb_matvec_kernel<T>, dim3(R, (G3 + 63) / 64), dim3(kGbThreads), lds, s, G3, H,
                       static_cast<const E*>(g.w_hh), static_cast<const E*>(g.b_hh), x_g, c);
  }
  const int P = pl.carry_parts;
  // bf16 heads: the carried gradient on the matrix cores against W_hh
  // transposed once per call (Qwen3-8B, 32 blocks: 16.4 us a position with
  // the float32 kernel)
  uint16_t* whhT = pl.S > 0 && pl.whhT ? reinterpret_cast<uint16_t*>(ws + pl.whhT) : nullptr;
  if (whhT)
    hipLaunchKernelGGL(gb_whht_kernel, dim3((H + 63) / 64, (G3 + 63) / 64), dim3(kGbThreads), 0, s, H,
                       static_cast<const uint16_t*>(g.w_hh), whhT);
  e = launch_fill_u64(reinterpret_cast<unsigned long long*>(carry), (int)(((size_t)(1 + P) * B * H + 1) / 2), s);
  if (e != hipSuccess) return e;
  const dim3 eg((H + 255) / 256, B);
  for (int i = K - 1; i >= 0; --i) {
    hipLaunchKernelGGL(gb_elem_kernel, eg, dim3(256), 0, s, B, K, H, i, i == K - 1 ? 0 : P, a, c, x_g, g.dg,
                       carry, da, dc);
    if (i > 0 && whhT)
      hipLaunchKernelGGL(gb_carrym_kernel, dim3((H + 63) / 64, (B + 15) / 16, P), dim3(kGbThreads), 0, s, B, K, H, i,
                         whhT, dc, carry);
    else if (i > 0)
      hipLaunchKernelGGL((B >= kGbCarryNB ? gb_carry_kernel<T, kGbCarryNB> : gb_carry_kernel<T, 1>),
                         dim3((H + 63) / 64, B >= kGbCarryNB ? (B + kGbCarryNB - 1) / kGbCarryNB : B, P),
                         dim3(kGbThreads), 0, s, B, K, H, i, static_cast<const E*>(g.w_hh), dc, carry);
  }
  if (pl.S > 0 && R >= kGbMfmaRows) {
    const int Rp = pl.Rp, tiles = (Rp + 63) / 64;
    uint16_t* daT = reinterpret_cast<uint16_t*>(ws + pl.daT);
    uint16_t* eT = reinterpret_cast<uint16_t*>(ws + pl.eT);
    uint16_t* dcT = reinterpret_cast<uint16_t*>(ws + pl.dcT);
    uint16_t* gT = reinterpret_cast<uint16_t*>(ws + pl.gT);
    float* bpart = reinterpret_cast<float*>(ws + pl.bpart);
    float* bpart_hh = bpart + (size_t)tiles * G3;
    KJobs jobs{};
    jobs.j[0] = {da, daT, g.d_b_ih ? bpart : nullptr, G3, 2, 0, 0b10u};
    jobs.j[1] = {x_e, eT, nullptr, d, 2, 1, 0b00u};
    jobs.j[2] = {dc, dcT, g.d_b_hh ? bpart_hh : nullptr, G3, 3, 0, 0b100u};
    jobs.j[3] = {x_g, gT, nullptr, H, 3, 0, 0b010u};
    e = launch_rows_to_k(R, Rp, jobs, 4, std::max(std::max(G3, d), H), s);
    if (e != hipSuccess) return e;
    e = launch_tile_colsums(tiles, G3, bpart, g.d_b_ih, bpart_hh, g.d_b_hh, s);
    if (e != hipSuccess) return e;
    e = launch_gemm_bf16_tn(daT, 2 * Rp, G3, eT, 2 * Rp, d, 2 * Rp, nullptr, g.d_w_ih, d, num_cu, s);
    if (e != hipSuccess) return e;
    e = launch_gemm_bf16_tn(dcT, 3 * Rp, G3, gT, 3 * Rp, H, 3 * Rp, nullptr, g.d_w_hh, H, num_cu, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gb_outer_kernel<E>, dim3((d + kGbThreads - 1) / kGbThreads, (G3 + kGbQ - 1) / kGbQ),
                     dim3(kGbThreads), 0, s, R, G3, d, da, x_e, g.d_w_ih, g.d_b_ih);
  hipLaunchKernelGGL(gb_outer_kernel<float>, dim3((H + kGbThreads - 1) / kGbThreads, (G3 + kGbQ - 1) / kGbQ),
                     dim3(kGbThreads), 0, s, R, G3, H, dc, x_g, g.d_w_hh, g.d_b_hh);
  return hipGetLastError();
}

hipError_t launch_gru_backward(const GruBackwardArgs& g, int num_cu, hipStream_t s) {
  if (g.B <= 0) return hipSuccess;
  return g.dtype == 1 ? gru_backward_t<Bf16>(g, num_cu, s) : gru_backward_t<F32>(g, num_cu, s);
}

}  // namespace domino
