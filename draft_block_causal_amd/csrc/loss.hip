// Base-anchored curriculum loss of the Domino head's training ([notes]
// §二.2(2)): loss = (1 - λ) L_final + λ L_base, where L_x is the cross-entropy
// of the logits x (base, or teacher-forced final, [notes] §二.2(1)) against
// the reference token of each position, weighted by w_i = γ^i along the block
// (Σ_i w_i CE_i / Σ_i w_i) and averaged over blocks; optionally its gradients
// with respect to both logit tensors, (coef) (softmax(x) - onehot(y)).
//
// Launches on the caller's stream:
//   1. loss_stats_kernel, grid (B K rows, S slices): the (max, sum of exp) of
//      one vocabulary slice of the base and of the final row;
//   2. loss_rows_kernel: per row, the two log-normalisers, the two
//      cross-entropies and the row's weighted term;
//   3. loss_sum_kernel, one workgroup: the loss, summed in a fixed order (so
//      two runs give the same bits);
//   4. loss_grad_kernel, grid (B K rows, S slices), when gradients are asked
//      for: each entry read once and its gradient written (in place allowed).
// Bound by HBM: 2 B K V floats read in pass 1, and 2 B K V read + written in
// pass 4.
#include <math.h>

#include <cmath>

#include "common.h"
#include "kernels.h"
#include "lse.h"

namespace domino {

__global__ void __launch_bounds__(kLseThreads) loss_stats_kernel(int V, const float* __restrict__ base,
                                                                 const float* __restrict__ final_,
                                                                 float4* __restrict__ stats) {
  __shared__ LsePart red[kLseWaves];
  const int row = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  long v0, v1;
  slice_bounds(V, s, S, v0, v1);
  const LsePart b = block_lse(base + (size_t)row * V, v0, v1, 1.f, red);
  const LsePart f = block_lse(final_ + (size_t)row * V, v0, v1, 1.f, red);
  if (threadIdx.x == 0) stats[(size_t)row * S + s] = float4{b.m, b.s, f.m, f.s};
}

__device__ __forceinline__ int clamp_token(int y, int V) { return min(max(y, 0), V - 1); }

// One thread per row: log-normalisers, cross-entropies and the weighted term
// w_i ((1 - λ) CE_final + λ CE_base).
__global__ void loss_rows_kernel(int rows, int K, int V, int S, const float* __restrict__ base,
                                 const float* __restrict__ final_, const int32_t* __restrict__ targets, float lam,
                                 float gamma, const float4* __restrict__ stats, float2* __restrict__ lse,
                                 float* __restrict__ contrib, float* __restrict__ ce_base,
                                 float* __restrict__ ce_final) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  LsePart b{-INFINITY, 0.f}, f{-INFINITY, 0.f};
  for (int q = 0; q < S; ++q) {
    const float4 x = stats[(size_t)row * S + q];
    b = lse_merge(b, LsePart{x.x, x.y});
    f = lse_merge(f, LsePart{x.z, x.w});
  }
  const float lb = b.m + logf(b.s), lf = f.m + logf(f.s);
  const int y = clamp_token(targets[row], V);
  const float cb = lb - base[(size_t)row * V + y];
  const float cf = lf - final_[(size_t)row * V + y];
  lse[row] = float2{lb, lf};
  const int i = row % K;
  contrib[row] = powf(gamma, (float)i) * ((1.f - lam) * cf + lam * cb);
  if (ce_base) ce_base[row] = cb;
  if (ce_final) ce_final[row] = cf;
}

// loss = Σ_rows contrib / (Σ_i w_i · B): each thread adds rows t, t + 256, ...
// in order, then a fixed pairwise tree over the 256 partial sums.
__global__ void __launch_bounds__(256) loss_sum_kernel(int rows, const float* __restrict__ contrib, float scale,
                                                       float* __restrict__ loss) {
  __shared__ float part[256];
  float acc = 0.f;
  for (int r = threadIdx.x; r < rows; r += 256) acc += contrib[r];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = part[0] * scale;
}

// d loss / d x = coef_x (softmax(x) - onehot(y)), coef_final = (1 - λ) w_i / (Σw B),
// coef_base = λ w_i / (Σw B).  Each entry is read and then written by the same
// thread, so the gradient may overwrite its logits.
__global__ void __launch_bounds__(kLseThreads) loss_grad_kernel(int K, int V, const float* base, const float* final_,
                                                                const int32_t* __restrict__ targets, float lam,
                                                                float gamma, float scale,
                                                                const float2* __restrict__ lse, float* grad_base,
                                                                float* grad_final) {
  const int row = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  long v0, v1;
  slice_bounds(V, s, S, v0, v1);
  const int y = clamp_token(targets[row], V);
  const float w = powf(gamma, (float)(row % K)) * scale;
  const float cb = lam * w, cf = (1.f - lam) * w;
  const float2 l = lse[row];
  const size_t o = (size_t)row * V;
  long vs = v0;
  // 16 B per lane where every tensor's row slice is 16-byte aligned
  const uintptr_t al = reinterpret_cast<uintptr_t>(base + o + v0) | reinterpret_cast<uintptr_t>(final_ + o + v0) |
                       reinterpret_cast<uintptr_t>(grad_base ? grad_base + o + v0 : base + o + v0) |
                       reinterpret_cast<uintptr_t>(grad_final ? grad_final + o + v0 : final_ + o + v0);
  if ((al & 15u) == 0) {
    const long n4 = (v1 - v0) / 4;
    for (long q = threadIdx.x; q < n4; q += kLseThreads) {
      const long v = v0 + 4 * q;
      const float h0 = v == y, h1 = v + 1 == y, h2 = v + 2 == y, h3 = v + 3 == y;
      if (grad_base) {
        const float4 x = *reinterpret_cast<const float4*>(base + o + v);
        *reinterpret_cast<float4*>(grad_base + o + v) =
            float4{cb * (exp_hw(x.x - l.x) - h0), cb * (exp_hw(x.y - l.x) - h1), cb * (exp_hw(x.z - l.x) - h2),
                   cb * (exp_hw(x.w - l.x) - h3)};
      }
      if (grad_final) {
        const float4 x = *reinterpret_cast<const float4*>(final_ + o + v);
        *reinterpret_cast<float4*>(grad_final + o + v) =
            float4{cf * (exp_hw(x.x - l.y) - h0), cf * (exp_hw(x.y - l.y) - h1), cf * (exp_hw(x.z - l.y) - h2),
                   cf * (exp_hw(x.w - l.y) - h3)};
      }
    }
    vs = v0 + 4 * n4;
  }
  for (long v = vs + threadIdx.x; v < v1; v += kLseThreads) {
    const float hot = v == y ? 1.f : 0.f;
    if (grad_base) {
      const float x = base[o + v];
      grad_base[o + v] = cb * (exp_hw(x - l.x) - hot);
    }
    if (grad_final) {
      const float x = final_[o + v];
      grad_final[o + v] = cf * (exp_hw(x - l.y) - hot);
    }
  }
}

hipError_t launch_curriculum_loss(int B, int K, int V, const float* base, const float* final_,
                                  const int32_t* targets, float lam, float gamma, float* loss, float* ce_base,
                                  float* ce_final, float* grad_base, float* grad_final, const LossPlan& plan,
                                  void* workspace, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float4* stats = reinterpret_cast<float4*>(ws + plan.stats);
  float2* lse = reinterpret_cast<float2*>(ws + plan.lse);
  float* contrib = reinterpret_cast<float*>(ws + plan.contrib);
  const int rows = B * K;
  double wsum = 0.0;
  for (int i = 0; i < K; ++i) wsum += std::pow((double)gamma, (double)i);
  const float scale = (float)(1.0 / (wsum * B));
  hipLaunchKernelGGL(loss_stats_kernel, dim3((unsigned)rows, (unsigned)plan.S), dim3(kLseThreads), 0, s, V, base,
                     final_, stats);
  hipLaunchKernelGGL(loss_rows_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, rows, K, V, plan.S,
                     base, final_, targets, lam, gamma, stats, lse, contrib, ce_base, ce_final);
  hipLaunchKernelGGL(loss_sum_kernel, dim3(1), dim3(256), 0, s, rows, contrib, scale, loss);
  if (grad_base || grad_final)
    hipLaunchKernelGGL(loss_grad_kernel, dim3((unsigned)rows, (unsigned)plan.S), dim3(kLseThreads), 0, s, K, V,
                       base, final_, targets, lam, gamma, scale, lse, grad_base, grad_final);
  return hipGetLastError();
}

}  // namespace domino
