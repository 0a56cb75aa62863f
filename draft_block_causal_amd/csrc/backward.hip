// Backward through the low-rank correction head ([notes] §二.1(2) items 2-3):
// from G = d loss / d L_final (every block and position, [R = B K][V]) to the
// gradients of W2, b2, W1, b1 and of the GRU states.  With x_i = [h_i ; g_i],
// z_i = W1 x_i + b1, u_i = SiLU(z_i):
//   dW2 = Σ_i G_i u_iᵀ, db2 = Σ_i G_i, du_i = W2ᵀ G_i,
//   dz_i = du_i ⊙ SiLU'(z_i), dW1 = Σ_i dz_i x_iᵀ, db1 = Σ_i dz_i,
//   dg_i = W1[:, d:]ᵀ dz_i.
// Launches on the caller's stream, every sum in a fixed order (no atomics, so
// two calls give the same bits).  float32 heads, all on the vector ALUs:
//   1. bw_z_kernel     (R x r / 64): z and u of each row, 64 outputs per
//                      workgroup, rows of W1 split over the lanes of a wave;
//   2. bw_dw2_kernel   (V / 256 x r / 32): dW2 and db2, one vocabulary entry
//                      per thread, u staged in LDS 64 rows at a time;
//   3. bw_du_kernel    (S vocabulary slices x R / 64 x r / 256): partial W2ᵀ G
//                      over a slice for 64 rows (G and W2 staged in LDS,
//                      16 x 4 register tiles), W2 read once per 64 rows;
//   4. bw_dz_kernel    (R r / 64): the S partials added, a quarter of the
//                      slices per wave, times SiLU'(z);
//   5. bw_dw1_kernel   ((d + H) / 256 x r / 16): dW1 and db1;
//   6. bw_dg_kernel    (H / 64 x R / 16): the state gradient, the r terms split
//                      over the waves of a workgroup.
// bf16 heads replace 2 and 3 by bw_split_kernel (G re-laid along both axes,
// db2), bw_w2t_kernel, bw_us_kernel and two launches of the tiled bf16 GEMM
// on the matrix cores (dW2, and the du partials over vocabulary slices).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace domino {

constexpr int kBwThreads = 256;
constexpr int kBwWaves = kBwThreads / 64;
constexpr int kBwRowsDu = 64;   // rows per du workgroup
constexpr int kBwQDw2 = 32;     // outputs of a W2 row per dW2 thread
constexpr int kBwRowsLds = 64;  // u rows staged per round in the dW2 kernel
constexpr int kBwQDw1 = 16;     // W1 rows per dW1 thread
constexpr int kBwRowsDg = 16;   // rows per dg thread

__device__ __forceinline__ float bw_wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// bf16 heads: z and u of 16 rows (blockIdx.y) x 16 bottleneck rows
// (blockIdx.x) on the matrix cores, [h ; g] against W1's rows: the hidden
// part with exact bf16 operands, the state part split hi + lo (as in the
// loop's u).  The K steps of each part are split over the four waves in
// order, kZuU steps of loads in flight per wave, and the wave partials added
// in wave order.  d and H multiples of 32.
constexpr int kZuU = 8;
__global__ void __launch_bounds__(kBwThreads) bw_zu_kernel(int R, int d, int H, int r,
                                                           const uint16_t* __restrict__ hidden,
                                                           const float* __restrict__ states,
                                                           const uint16_t* __restrict__ w1,
                                                           const uint16_t* __restrict__ b1, float* __restrict__ z,
                                                           float* __restrict__ u) {
  __shared__ float red[kBwWaves][16][17];
  const int q0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int wave = wave_id(), lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int n = d + H;
  // (rows past R and W1 rows past r read clamped rows; their outputs are not stored)
  const int row = min(m0 + col, R - 1), qrow = min(q0 + col, r - 1);
  const unsigned char* wrow = reinterpret_cast<const unsigned char*>(w1 + (size_t)qrow * n) + grp * 16;
  const unsigned char* hrow = reinterpret_cast<const unsigned char*>(hidden + (size_t)row * d) + grp * 16;
  const float* grow = states + (size_t)row * H + grp * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  {
    const int ns = d / 32, per = (ns + kBwWaves - 1) / kBwWaves, sb = wave * per, se = min(ns, sb + per);
    for (int s0 = sb; s0 < se; s0 += kZuU) {
      u32x4 w[kZuU], a[kZuU];
#pragma unroll
      for (int i = 0; i < kZuU; ++i) {
        const int st = min(s0 + i, se - 1);  // past se: a repeated step, its A operand zeroed below
        w[i] = ld16(wrow + (size_t)st * 64);
        a[i] = ld16(hrow + (size_t)st * 64);
      }
#pragma unroll
      for (int i = 0; i < kZuU; ++i) {
        const u32x4 ai = s0 + i < se ? a[i] : u32x4{0, 0, 0, 0};
        acc = mma16<Bf16>(acc, ai, w[i]);
      }
    }
  }
  {
    const int ns = H / 32, per = (ns + kBwWaves - 1) / kBwWaves, sb = wave * per, se = min(ns, sb + per);
    const unsigned char* wg = wrow + (size_t)d * 2;
    for (int s0 = sb; s0 < se; s0 += kZuU) {
      u32x4 w[kZuU];
      float x[kZuU][8];
#pragma unroll
      for (int i = 0; i < kZuU; ++i) {
        const int st = min(s0 + i, se - 1);
        w[i] = ld16(wg + (size_t)st * 64);
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(grow + (size_t)st * 32);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(grow + (size_t)st * 32 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[i][e] = v0[e];
          x[i][e + 4] = v1[e];
        }
      }
#pragma unroll
      for (int i = 0; i < kZuU; ++i) {
        float xs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xs[e] = s0 + i < se ? x[i][e] : 0.f;
        ActFrag<Bf16> a;
        a.from_f32(xs);
        acc = a.mma(acc, w[i]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wave][grp * 4 + j][col] = acc[j];
  __syncthreads();
  const int mm = threadIdx.x >> 4, nn = threadIdx.x & 15;  // 256 threads: 16 x 16 outputs
  const int m = m0 + mm, q = q0 + nn;
  if (m < R && q < r) {
    float sum = 0.f;
#pragma unroll
    for (int wv = 0; wv < kBwWaves; ++wv) sum += red[wv][mm][nn];
    const float zz = sum + (b1 ? bf16_to_f32(b1[q]) : 0.f);
    z[(size_t)m * r + q] = zz;
    u[(size_t)m * r + q] = zz * sigmoidf_(zz);
  }
}

// bf16 heads, for dg on the matrix cores: w1gT[j][q] = W1[q][d + j] (the
// state columns of W1, transposed so that the product's K, the bottleneck
// rows, is contiguous), one 64 x 64 tile per workgroup through LDS.
__global__ void __launch_bounds__(kBwThreads) bw_w1gt_kernel(int d, int H, int r, const uint16_t* __restrict__ w1,
                                                             uint16_t* __restrict__ w1gT) {
  __shared__ uint16_t t[64][66];
  const int j0 = blockIdx.x * 64, q0 = blockIdx.y * 64, tid = threadIdx.x;
  const int n = d + H;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int qq = (tid >> 6) + 4 * i, jj = tid & 63;
    t[qq][jj] = q0 + qq < r && j0 + jj < H ? w1[(size_t)(q0 + qq) * n + d + j0 + jj] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int jj = (tid >> 6) + 4 * i, qq = tid & 63;
    if (j0 + jj < H && q0 + qq < r) w1gT[(size_t)(j0 + jj) * r + q0 + qq] = t[qq][jj];
  }
}

// bf16 heads: dg = dz W1[:, d:] for 16 rows (blockIdx.y) x 64 state columns
// (blockIdx.x, 16 per wave) on the matrix cores, dz split hi + lo, every K
// step's loads issued first.  r a multiple of 32.
__global__ void __launch_bounds__(kBwThreads) bw_dgm_kernel(int R, int H, int r, const float* __restrict__ dz,
                                                            const uint16_t* __restrict__ w1gT,
                                                            float* __restrict__ dg) {
  const int wave = wave_id(), lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int m0 = blockIdx.y * 16, j0 = blockIdx.x * 64 + wave * 16;
  if (j0 >= H) return;  // (uniform over the wave; no barrier below)
  const int row = min(m0 + col, R - 1), jrow = min(j0 + col, H - 1);
  const float* arow = dz + (size_t)row * r + grp * 8;
  const unsigned char* wrow = reinterpret_cast<const unsigned char*>(w1gT + (size_t)jrow * r) + grp * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kU = 8;
  const int ns = r / 32;
  for (int s0 = 0; s0 < ns; s0 += kU) {
    u32x4 w[kU];
    float x[kU][8];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int st = min(s0 + i, ns - 1);  // past ns: a repeated step, its A operand zeroed below
      w[i] = ld16(wrow + (size_t)st * 64);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(arow + (size_t)st * 32);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(arow + (size_t)st * 32 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[i][e] = v0[e];
        x[i][e + 4] = v1[e];
      }
    }
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      float xs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[e] = s0 + i < ns ? x[i][e] : 0.f;
      ActFrag<Bf16> a;
      a.from_f32(xs);
      acc = a.mma(acc, w[i]);
    }
  }
  const int j = j0 + col;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int m = m0 + grp * 4 + jj;
    if (m < R && j < H) dg[(size_t)m * H + j] = acc[jj];
  }
}

// z = W1 [h ; g] + b1 and u = SiLU(z) for row `row`; x staged in LDS.
template <class T>
__global__ void __launch_bounds__(kBwThreads) bw_z_kernel(int d, int H, int r, const typename T::elem* __restrict__ hidden,
                                                          const float* __restrict__ states,
                                                          const typename T::elem* __restrict__ w1,
                                                          const typename T::elem* __restrict__ b1,
                                                          float* __restrict__ z, float* __restrict__ u) {
  using E = typename T::elem;
  constexpr int EPF = T::kPer16B;
  extern __shared__ __attribute__((aligned(16))) float xs[];  // [d + H]
  const int row = blockIdx.x, n = d + H, n0 = blockIdx.y * 64;  // outputs n0 .. n0 + 63 of the row
  for (int k = threadIdx.x; k < d; k += kBwThreads) xs[k] = T::to_f32(hidden[(size_t)row * d + k]);
  for (int k = threadIdx.x; k < H; k += kBwThreads) xs[d + k] = states[(size_t)row * H + k];
  __syncthreads();
  const int wave = wave_id(), lane = threadIdx.x & 63;
  for (int q0 = n0 + wave * 4; q0 < min(r, n0 + 64); q0 += kBwWaves * 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = lane * EPF; k < n; k += 64 * EPF) {
      u32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = q0 + j < r ? ld16(w1 + (size_t)(q0 + j) * n + k) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const E* e = reinterpret_cast<const E*>(&w[j]);
#pragma unroll
        for (int c = 0; c < EPF; ++c) acc[j] += T::to_f32(e[c]) * xs[k + c];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float s = bw_wave_sum(acc[j]);
      if (lane == 0 && q0 + j < r) {
        const float zz = s + (b1 ? T::to_f32(b1[q0 + j]) : 0.f);
        z[(size_t)row * r + q0 + j] = zz;
        u[(size_t)row * r + q0 + j] = zz * sigmoidf_(zz);
      }
    }
  }
}

// dW2[v][q0 .. q0 + 31] = Σ_rows G[row][v] u[row][q]; db2[v] = Σ_rows G[row][v] (blockIdx.y == 0).
// ROWS_OUT: the finished 256 x 32 tile goes through LDS so that the stores
// write whole 128-byte rows (each thread's own 32 values lie 4r bytes from its
// neighbour's); used for up to 64 rows, where the stores dominate (at
// Qwen3-8B shapes: one block 72 against 203 us, but 32 blocks 1.88 against
// 1.14 ms, the tile's LDS lowering the occupancy of the longer accumulation).
template <bool ROWS_OUT>
__global__ void __launch_bounds__(kBwThreads) bw_dw2_kernel(int R, int V, int r, const float* __restrict__ G,
                                                            const float* __restrict__ u, float* __restrict__ dw2,
                                                            float* __restrict__ db2) {
  __shared__ float us[kBwRowsLds][kBwQDw2];
  __shared__ float tile[ROWS_OUT ? kBwThreads : 1][kBwQDw2 + 1];
  const int vb = blockIdx.x * kBwThreads, v = vb + threadIdx.x, q0 = blockIdx.y * kBwQDw2;
  const int nq = min(kBwQDw2, r - q0);
  float acc[kBwQDw2];
#pragma unroll
  for (int q = 0; q < kBwQDw2; ++q) acc[q] = 0.f;
  float gsum = 0.f;
  for (int r0 = 0; r0 < R; r0 += kBwRowsLds) {
    const int nr = min(kBwRowsLds, R - r0);
    __syncthreads();
    for (int e = threadIdx.x; e < kBwRowsLds * kBwQDw2; e += kBwThreads) {
      const int rr = e / kBwQDw2, q = e % kBwQDw2;
      us[rr][q] = rr < nr && q < nq ? u[(size_t)(r0 + rr) * r + q0 + q] : 0.f;
    }
    __syncthreads();
    if (v < V)
      for (int rr = 0; rr < nr; ++rr) {
        const float g = G[(size_t)(r0 + rr) * V + v];
        gsum += g;
#pragma unroll
        for (int q = 0; q < kBwQDw2; ++q) acc[q] += g * us[rr][q];
      }
  }
  if (blockIdx.y == 0 && db2 && v < V) db2[v] = gsum;
  if constexpr (ROWS_OUT) {
#pragma unroll
    for (int q = 0; q < kBwQDw2; ++q) tile[threadIdx.x][q] = acc[q];
    __syncthreads();
    for (int e = threadIdx.x; e < kBwThreads * kBwQDw2; e += kBwThreads) {
      const int vl = e / kBwQDw2, q = e % kBwQDw2;
      if (vb + vl < V && q < nq) dw2[(size_t)(vb + vl) * r + q0 + q] = tile[vl][q];
    }
  } else {
    if (v >= V) return;
    for (int q = 0; q < nq; ++q) dw2[(size_t)v * r + q0 + q] = acc[q];
  }
}

// part[s][row][q] = Σ_{v in slice s} G[row][v] W2[v][q] for rows m0 .. m0 + 63
// and columns q0 .. q0 + 255 (q0 = 256 blockIdx.z).  G and W2 are staged in
// LDS 64 vocabulary entries at a time with coalesced loads.  Thread (wave w,
// lane l) holds a 16-row x 4-column tile: rows m0 + 16 w .., columns
// q0 + 4 l ..; the lanes of a wave share their rows, so each LDS read of G is
// a broadcast that feeds four multiply-adds.
constexpr int kBwVChunk = 64;
template <class T>
__global__ void __launch_bounds__(kBwThreads) bw_du_kernel(int R, int V, int r, const float* __restrict__ G,
                                                           const typename T::elem* __restrict__ w2,
                                                           float* __restrict__ part) {
  __shared__ float gs[kBwRowsDu][kBwVChunk];
  __shared__ __attribute__((aligned(16))) float ws[kBwVChunk][256];
  const int s = blockIdx.x, S = gridDim.x, m0 = blockIdx.y * kBwRowsDu, q0 = blockIdx.z * 256;
  const int nr = min(kBwRowsDu, R - m0), nq = min(256, r - q0);
  const long v0 = (long)V * s / S, v1 = (long)V * (s + 1) / S;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int ql = lane * 4;       // first of this thread's 4 columns within the block
  const bool live = ql < nq;     // r is a multiple of 32, so all 4 or none
  float acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = 0.f;
  for (long vc = v0; vc < v1; vc += kBwVChunk) {
    const int nv = (int)min((long)kBwVChunk, v1 - vc);
    __syncthreads();
    for (int e = threadIdx.x; e < kBwRowsDu * kBwVChunk; e += kBwThreads) {
      const int i = e / kBwVChunk, vv = e % kBwVChunk;
      gs[i][vv] = i < nr && vv < nv ? G[(size_t)(m0 + i) * V + vc + vv] : 0.f;
    }
    for (int e = threadIdx.x; e < kBwVChunk * 256; e += kBwThreads) {
      const int vv = e >> 8, c = e & 255;
      ws[vv][c] = vv < nv && c < nq ? T::to_f32(w2[(size_t)(vc + vv) * r + q0 + c]) : 0.f;
    }
    __syncthreads();
    if (live)
      for (int vv = 0; vv < nv; ++vv) {
        const float4 w = *reinterpret_cast<const float4*>(&ws[vv][ql]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float g = gs[wave * 16 + i][vv];
          acc[i][0] += g * w.x;
          acc[i][1] += g * w.y;
          acc[i][2] += g * w.z;
          acc[i][3] += g * w.w;
        }
      }
  }
  if (!live) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = wave * 16 + i;
    if (row < nr)
#pragma unroll
      for (int c = 0; c < 4; ++c) part[((size_t)s * R + m0 + row) * r + q0 + ql + c] = acc[i][c];
  }
}

// dz = (Σ_s part[s]) ⊙ SiLU'(z): 64 entries per workgroup, each wave adds a
// quarter of the slices in order (eight loads in flight), and the quarter
// sums are added in wave order.
__global__ void __launch_bounds__(kBwThreads) bw_dz_kernel(int R, int r, int S, const float* __restrict__ part,
                                                           const float* __restrict__ z, float* __restrict__ dz) {
  __shared__ float ps[kBwWaves][64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const long n = (long)R * r, e = (long)blockIdx.x * 64 + lane;
  const int sa = S * wave / kBwWaves, sb = S * (wave + 1) / kBwWaves;
  float du = 0.f;
  if (e < n) {
    int s = sa;
    for (; s + 8 <= sb; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(s + u) * n + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) du += v[u];
    }
    for (; s < sb; ++s) du += part[(size_t)s * n + e];
  }
  ps[wave][lane] = du;
  __syncthreads();
  if (wave == 0 && e < n) {
    const float t = (ps[0][lane] + ps[1][lane]) + (ps[2][lane] + ps[3][lane]);
    const float zz = z[e], sg = sigmoidf_(zz);
    dz[e] = t * sg * (1.f + zz * (1.f - sg));
  }
}

// dW1[q][k] = Σ_rows dz[row][q] x[row][k] for q0 .. q0 + 15; db1 from the
// workgroups with blockIdx.x == 0.  The dz values of 64 rows at a time are
// staged in LDS (read as broadcasts).
template <class T>
__global__ void __launch_bounds__(kBwThreads) bw_dw1_kernel(int R, int d, int H, int r,
                                                            const typename T::elem* __restrict__ hidden,
                                                            const float* __restrict__ states,
                                                            const float* __restrict__ dz, float* __restrict__ dw1,
                                                            float* __restrict__ db1) {
  __shared__ float zs[kBwRowsLds][kBwQDw1];
  const int k = blockIdx.x * kBwThreads + threadIdx.x, q0 = blockIdx.y * kBwQDw1, n = d + H;
  const int nq = min(kBwQDw1, r - q0);
  // rows of group blockIdx.z; with several groups the sums are partials
  const int ga = (int)((long)R * blockIdx.z / gridDim.z), gb = (int)((long)R * (blockIdx.z + 1) / gridDim.z);
  if (gridDim.z > 1) {
    dw1 += (size_t)blockIdx.z * r * n;
    if (db1) db1 += (size_t)blockIdx.z * r;
  }
  float acc[kBwQDw1];
#pragma unroll
  for (int q = 0; q < kBwQDw1; ++q) acc[q] = 0.f;
  float bsum = 0.f;
  for (int r0 = ga; r0 < gb; r0 += kBwRowsLds) {
    const int nr = min(kBwRowsLds, gb - r0);
    __syncthreads();
    for (int e = threadIdx.x; e < kBwRowsLds * kBwQDw1; e += kBwThreads) {
      const int rr = e / kBwQDw1, q = e % kBwQDw1;
      zs[rr][q] = rr < nr && q < nq ? dz[(size_t)(r0 + rr) * r + q0 + q] : 0.f;
    }
    __syncthreads();
    if (blockIdx.x == 0 && (int)threadIdx.x < nq)
      for (int rr = 0; rr < nr; ++rr) bsum += zs[rr][threadIdx.x];
    if (k < n)
      for (int rr = 0; rr < nr; ++rr) {
        const int row = r0 + rr;
        const float x = k < d ? T::to_f32(hidden[(size_t)row * d + k]) : states[(size_t)row * H + k - d];
#pragma unroll
        for (int q = 0; q < kBwQDw1; ++q) acc[q] += zs[rr][q] * x;
      }
  }
  if (k < n)
    for (int q = 0; q < nq; ++q) dw1[(size_t)(q0 + q) * n + k] = acc[q];
  if (blockIdx.x == 0 && db1 && (int)threadIdx.x < nq) db1[q0 + threadIdx.x] = bsum;
}

// out[e] = Σ_g part[g][e] in group order (dW1 and db1 from row groups).
__global__ void bw_gsum_kernel(long n, int G, const float* __restrict__ part, float* __restrict__ out) {
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float v = 0.f;
  for (int g = 0; g < G; ++g) v += part[(size_t)g * n + e];
  out[e] = v;
}

// dg[row][j] = Σ_q dz[row][q] W1[q][d + j] for rows m0 .. m0 + 15: a
// workgroup takes 64 units j (one per lane); its 4 waves take a quarter of
// the r terms each, with the 16 rows' dz in LDS, and the quarter sums are
// added in wave order.
template <class T>
__global__ void __launch_bounds__(kBwThreads) bw_dg_kernel(int R, int d, int H, int r,
                                                           const typename T::elem* __restrict__ w1,
                                                           const float* __restrict__ dz, float* __restrict__ dg) {
  extern __shared__ __attribute__((aligned(16))) float zs[];  // [kBwRowsDg][r], then [kBwWaves][kBwRowsDg][64]
  float* part = zs + kBwRowsDg * r;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int j = blockIdx.x * 64 + lane, m0 = blockIdx.y * kBwRowsDg;
  const int nr = min(kBwRowsDg, R - m0);
  for (int e = threadIdx.x; e < kBwRowsDg * r; e += kBwThreads) {
    const int i = e / r, q = e % r;
    zs[e] = i < nr ? dz[(size_t)(m0 + i) * r + q] : 0.f;
  }
  __syncthreads();
  const int qa = r * wave / kBwWaves, qb = r * (wave + 1) / kBwWaves;
  float acc[kBwRowsDg];
#pragma unroll
  for (int i = 0; i < kBwRowsDg; ++i) acc[i] = 0.f;
  if (j < H)
    for (int q = qa; q < qb; ++q) {
      const float w = T::to_f32(w1[(size_t)q * (d + H) + d + j]);
#pragma unroll
      for (int i = 0; i < kBwRowsDg; ++i) acc[i] += zs[i * r + q] * w;
    }
#pragma unroll
  for (int i = 0; i < kBwRowsDg; ++i) part[(wave * kBwRowsDg + i) * 64 + lane] = acc[i];
  __syncthreads();
  if (wave == 0 && j < H)
    for (int i = 0; i < nr; ++i) {
      float sum = part[i * 64 + lane];
      for (int w = 1; w < kBwWaves; ++w) sum += part[(w * kBwRowsDg + i) * 64 + lane];
      dg[(size_t)(m0 + i) * H + j] = sum;
    }
}

// ---------------------------------------------------------------------------
// bf16 heads: the two large contractions on the matrix cores.  The float32
// operands are split as x = hi + lo (hi = x truncated to bf16, lo = the
// remainder rounded to bf16, about 16 significant bits together) and the
// products expanded, in the tiled bf16 GEMM:
//   du  = G W2 = [G_hi | G_lo] [W2 ; W2]     split-K partials over vocabulary slices,
//   dW2 = G^T u = G_hi^T u_hi + G_lo^T u_hi + G_hi^T u_lo, stored as [V][r].
// Both GEMM operands are K-contiguous, so G, W2 and u are re-laid first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bw_split(float x, uint32_t& h, uint32_t& l) {
  const uint32_t t = __float_as_uint(x) & 0xFFFF0000u;
  h = t >> 16;
  l = f32_to_bf16_rne(x - __uint_as_float(t));
}

// One pass over G [R][V] (256 columns per workgroup, 32 rows per round):
// gs [R][2 Vp] = hi | lo along the vocabulary (zero past V), gt [V][2 Rp] =
// hi | lo along the rows (zero past R), and db2[v] = the column sums of G in
// row order.  VEC: V % 4 == 0 and G 16-byte aligned, rows read as float4.
template <bool VEC>
__global__ void __launch_bounds__(kBwThreads) bw_split_kernel(int R, int V, int Vp, int Rp, const float* __restrict__ G,
                                                              uint16_t* __restrict__ gs, uint16_t* __restrict__ gt,
                                                              float* __restrict__ db2) {
  __shared__ __attribute__((aligned(16))) float t[32][260];
  const int v0 = blockIdx.x * 256, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int v = v0 + lane * 4;  // this lane's 4 columns in the row-wise phase
  const int vt = v0 + tid;      // this thread's column in the transposed phase
  float colsum = 0.f;
  for (int rc = 0; rc < Rp; rc += 32) {
    float4 g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = rc + wave * 8 + j;
      const float* src = G + (size_t)row * V + v;
      if constexpr (VEC) {
        g[j] = row < R && v < V ? *reinterpret_cast<const float4*>(src) : float4{0.f, 0.f, 0.f, 0.f};
      } else {
        g[j].x = row < R && v < V ? src[0] : 0.f;
        g[j].y = row < R && v + 1 < V ? src[1] : 0.f;
        g[j].z = row < R && v + 2 < V ? src[2] : 0.f;
        g[j].w = row < R && v + 3 < V ? src[3] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = rc + wave * 8 + j;
      *reinterpret_cast<float4*>(&t[wave * 8 + j][lane * 4]) = g[j];
      if (row < R && v < Vp) {
        uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
        bw_split(g[j].x, h0, l0);
        bw_split(g[j].y, h1, l1);
        bw_split(g[j].z, h2, l2);
        bw_split(g[j].w, h3, l3);
        uint16_t* dst = gs + (size_t)row * 2 * Vp + v;
        *reinterpret_cast<uint2*>(dst) = uint2{h0 | (h1 << 16), h2 | (h3 << 16)};
        *reinterpret_cast<uint2*>(dst + Vp) = uint2{l0 | (l1 << 16), l2 | (l3 << 16)};
      }
    }
    __syncthreads();
    if (vt < V) {
      uint16_t* dst = gt + (size_t)vt * 2 * Rp + rc;
#pragma unroll
      for (int k8 = 0; k8 < 32; k8 += 8) {
        uint32_t h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = t[k8 + e][tid];
          colsum += x;
          bw_split(x, h[e], l[e]);
        }
        u32x4 hv, lv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = h[2 * q] | (h[2 * q + 1] << 16);
          lv[q] = l[2 * q] | (l[2 * q + 1] << 16);
        }
        st16(dst + k8, hv);
        st16(dst + Rp + k8, lv);
      }
    }
    __syncthreads();
  }
  if (db2 && vt < V) db2[vt] = colsum;
}

// w2t [r][Vp] = W2^T (zero past V); 64 vocabulary rows x 32 columns per workgroup.
__global__ void __launch_bounds__(kBwThreads) bw_w2t_kernel(int V, int r, int Vp, const uint16_t* __restrict__ w2,
                                                            uint16_t* __restrict__ w2t) {
  __shared__ uint16_t tw[64][34];
  const int v0 = blockIdx.x * 64, q0 = blockIdx.y * 32, tid = threadIdx.x;
  {
    const int vv = tid >> 2, q8 = (tid & 3) * 8;
    const u32x4 x = v0 + vv < V ? ld16(w2 + (size_t)(v0 + vv) * r + q0 + q8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tw[vv][q8 + 2 * q] = (uint16_t)(x[q] & 0xFFFFu);
      tw[vv][q8 + 2 * q + 1] = (uint16_t)(x[q] >> 16);
    }
  }
  __syncthreads();
  const int q = tid >> 3, v8 = (tid & 7) * 8;
  u32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (uint32_t)tw[v8 + 2 * e][q] | ((uint32_t)tw[v8 + 2 * e + 1][q] << 16);
  st16(w2t + (size_t)(q0 + q) * Vp + v0 + v8, y);
}

// us [r][3 Rp] = u_hi^T | u_hi^T | u_lo^T (zero past R).
__global__ void bw_us_kernel(int R, int r, int Rp, const float* __restrict__ u, uint16_t* __restrict__ us) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x, q = blockIdx.y;
  if (k >= Rp) return;
  uint32_t h, l;
  bw_split(k < R ? u[(size_t)k * r + q] : 0.f, h, l);
  uint16_t* dst = us + (size_t)q * 3 * Rp + k;
  dst[0] = (uint16_t)h;
  dst[Rp] = (uint16_t)h;
  dst[2 * Rp] = (uint16_t)l;
}

template <class T>
static hipError_t backward_t(const BackwardArgs& a, hipStream_t s) {
  using E = typename T::elem;
  const int R = a.R, V = a.V, r = a.r, d = a.d, H = a.H;
  const BackwardPlan& pl = a.plan;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  float* z = reinterpret_cast<float*>(ws + pl.z);
  float* u = reinterpret_cast<float*>(ws + pl.u);
  float* dz = reinterpret_cast<float*>(ws + pl.dz);
  float* part = reinterpret_cast<float*>(ws + pl.part);
  const E* hidden = static_cast<const E*>(a.hidden);
  const E* w1 = static_cast<const E*>(a.w1);
  const size_t lds = (size_t)(d + H) * sizeof(float);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(bw_z_kernel<T>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (std::is_same<T, Bf16>::value && d % 32 == 0 && H % 32 == 0) {
    // on the matrix cores (Qwen3-8B, 32 blocks: 80 us as float32 vector dot products)
    hipLaunchKernelGGL(bw_zu_kernel, dim3((r + 15) / 16, (R + 15) / 16), dim3(kBwThreads), 0, s, R, d, H, r,
                       reinterpret_cast<const uint16_t*>(hidden), a.states, reinterpret_cast<const uint16_t*>(w1),
                       static_cast<const uint16_t*>(a.b1), z, u);
  } else {
    hipLaunchKernelGGL(bw_z_kernel<T>, dim3(R, (r + 63) / 64), dim3(kBwThreads), lds, s, d, H, r, hidden, a.states,
                       w1, static_cast<const E*>(a.b1), z, u);
  }
  if (pl.mfma) {
    if constexpr (std::is_same<T, Bf16>::value) {
      uint16_t* gs = reinterpret_cast<uint16_t*>(ws + pl.gs);
      uint16_t* gt = reinterpret_cast<uint16_t*>(ws + pl.gt);
      uint16_t* w2t = reinterpret_cast<uint16_t*>(ws + pl.w2t);
      uint16_t* us = reinterpret_cast<uint16_t*>(ws + pl.us);
      const int Vp = pl.Vp, Rp = pl.Rp;
      const bool vec = V % 4 == 0 && (reinterpret_cast<uintptr_t>(a.grad) & 15u) == 0;
      hipLaunchKernelGGL(vec ? bw_split_kernel<true> : bw_split_kernel<false>, dim3((Vp + 255) / 256),
                         dim3(kBwThreads), 0, s, R, V, Vp, Rp, a.grad, gs, gt, a.d_b2);
      hipLaunchKernelGGL(bw_w2t_kernel, dim3(Vp / 64, r / 32), dim3(kBwThreads), 0, s, V, r, Vp,
                         static_cast<const uint16_t*>(a.w2), w2t);
      hipLaunchKernelGGL(bw_us_kernel, dim3((Rp + 255) / 256, r), dim3(256), 0, s, R, r, Rp, u, us);
      hipError_t e = launch_gemm_bf16_tn_wrapt(us, 3 * Rp, r, gt, 2 * Rp, V, 3 * Rp, 2 * Rp, a.d_w2, r, s);
      if (e != hipSuccess) return e;
      e = launch_gemm_bf16_tn_splitk(gs, 2 * Vp, R, w2t, Vp, r, pl.kc, pl.S, Vp, part, r, (size_t)R * r, s);
      if (e != hipSuccess) return e;
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    auto dw2_kern = R <= kBwRowsLds ? bw_dw2_kernel<true> : bw_dw2_kernel<false>;
    hipLaunchKernelGGL(dw2_kern, dim3((V + kBwThreads - 1) / kBwThreads, (r + kBwQDw2 - 1) / kBwQDw2),
                       dim3(kBwThreads), 0, s, R, V, r, a.grad, u, a.d_w2, a.d_b2);
    hipLaunchKernelGGL(bw_du_kernel<T>, dim3(pl.S, (R + kBwRowsDu - 1) / kBwRowsDu, (r + 255) / 256),
                       dim3(kBwThreads), 0, s, R, V, r, a.grad, static_cast<const E*>(a.w2), part);
  }
  hipLaunchKernelGGL(bw_dz_kernel, dim3((unsigned)(((long)R * r + 63) / 64)), dim3(kBwThreads), 0, s, R, r, pl.S,
                     part, z, dz);
  if (pl.w1m) {
    // dW1 on the matrix cores: [dz_hi | dz_lo] [h | h]^T for the hidden
    // columns, [dz_hi | dz_lo | dz_hi] [g_hi | g_hi | g_lo]^T for the state
    // columns, as S1 split-K slices added in slice order (Qwen3-8B, 32
    // blocks: 73 + 12 us with the float32 row groups)
    const int Rp = pl.Rp, S1 = pl.S1, tiles = (Rp + 63) / 64, n1 = d + H;
    uint16_t* dzT = reinterpret_cast<uint16_t*>(ws + pl.dzT);
    uint16_t* hT = reinterpret_cast<uint16_t*>(ws + pl.hT);
    uint16_t* gT = reinterpret_cast<uint16_t*>(ws + pl.gT);
    float* bp1 = reinterpret_cast<float*>(ws + pl.bp1);
    KJobs jobs{};
    jobs.j[0] = {dz, dzT, a.d_b1 ? bp1 : nullptr, r, 3, 0, 0b010u};
    jobs.j[1] = {hidden, hT, nullptr, d, 2, 1, 0b00u};
    jobs.j[2] = {a.states, gT, nullptr, H, 3, 0, 0b100u};
    hipError_t e = launch_rows_to_k(R, Rp, jobs, 3, std::max(std::max(r, d), H), s);
    if (e != hipSuccess) return e;
    e = launch_tile_colsums(tiles, r, bp1, a.d_b1, nullptr, nullptr, s);
    if (e != hipSuccess) return e;
    float* w1out = S1 > 1 ? reinterpret_cast<float*>(ws + pl.dw1p) : a.d_w1;
    e = S1 > 1 ? launch_gemm_bf16_tn_splitk(dzT, 3 * Rp, r, hT, 2 * Rp, d, 2 * Rp / S1, S1, 2 * Rp, w1out, n1,
                                            (size_t)r * n1, s)
               : launch_gemm_bf16_tn(dzT, 3 * Rp, r, hT, 2 * Rp, d, 2 * Rp, nullptr, w1out, n1, 0, s);
    if (e != hipSuccess) return e;
    e = S1 > 1 ? launch_gemm_bf16_tn_splitk(dzT, 3 * Rp, r, gT, 3 * Rp, H, 3 * Rp / S1, S1, 3 * Rp, w1out + d, n1,
                                            (size_t)r * n1, s)
               : launch_gemm_bf16_tn(dzT, 3 * Rp, r, gT, 3 * Rp, H, 3 * Rp, nullptr, w1out + d, n1, 0, s);
    if (e != hipSuccess) return e;
    if (S1 > 1) {
      const long nw = (long)r * n1;
      hipLaunchKernelGGL(bw_gsum_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, nw, S1, w1out, a.d_w1);
    }
  } else {
    const int G1 = pl.G1;
    float* w1out = G1 > 1 ? reinterpret_cast<float*>(ws + pl.dw1p) : a.d_w1;
    float* b1out = G1 > 1 ? (a.d_b1 ? reinterpret_cast<float*>(ws + pl.db1p) : nullptr) : a.d_b1;
    hipLaunchKernelGGL(bw_dw1_kernel<T>,
                       dim3((d + H + kBwThreads - 1) / kBwThreads, (r + kBwQDw1 - 1) / kBwQDw1, G1),
                       dim3(kBwThreads), 0, s, R, d, H, r, hidden, a.states, dz, w1out, b1out);
    if (G1 > 1) {
      const long n1 = (long)r * (d + H);
      hipLaunchKernelGGL(bw_gsum_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, n1, G1, w1out,
                         a.d_w1);
      if (a.d_b1)
        hipLaunchKernelGGL(bw_gsum_kernel, dim3((unsigned)((r + 255) / 256)), dim3(256), 0, s, (long)r, G1, b1out,
                           a.d_b1);
    }
  }
  if (a.d_states && pl.w1gT) {
    // on the matrix cores (Qwen3-8B, 32 blocks: 35 us for the float32 vector kernel)
    uint16_t* w1gT = reinterpret_cast<uint16_t*>(ws + pl.w1gT);
    hipLaunchKernelGGL(bw_w1gt_kernel, dim3((H + 63) / 64, (r + 63) / 64), dim3(kBwThreads), 0, s, d, H, r,
                       static_cast<const uint16_t*>(a.w1), w1gT);
    hipLaunchKernelGGL(bw_dgm_kernel, dim3((H + 63) / 64, (R + 15) / 16), dim3(kBwThreads), 0, s, R, H, r, dz, w1gT,
                       a.d_states);
  } else if (a.d_states) {
    const size_t dg_lds = ((size_t)kBwRowsDg * r + (size_t)kBwWaves * kBwRowsDg * 64) * sizeof(float);
    if (dg_lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(bw_dg_kernel<T>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)dg_lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bw_dg_kernel<T>, dim3((H + 63) / 64, (R + kBwRowsDg - 1) / kBwRowsDg), dim3(kBwThreads),
                       dg_lds, s, R, d, H, r, w1, dz, a.d_states);
  }
  return hipGetLastError();
}

hipError_t launch_correction_backward(const BackwardArgs& a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  return a.dtype == 1 ? backward_t<Bf16>(a, s) : backward_t<F32>(a, s);
}

}  // namespace domino
