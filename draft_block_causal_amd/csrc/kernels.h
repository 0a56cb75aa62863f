// Host-side launchers of the Domino kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "loss_plan.h"
#include "psplit.h"
#include "verify_plan.h"

namespace domino {

// C[m, n] = sum_k A[m, k] W[n, k] (+ bias[n]) for m < M, n < N, in float32.
// dtype 0 = f32, 1 = bf16 for A, W and bias.  K * elem_size must be a multiple
// of 64 and at most 8192 bytes.  Pointers 16-byte aligned, lda/ldw rows too.
hipError_t launch_panel_gemm(int dtype, const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                             const void* bias, float* C, int ldc, int num_cu, hipStream_t s);

// The same product by the row-streaming kernel (rowstream.hip) for M <= 32,
// or M, N <= 4096; hipErrorNotSupported otherwise, or unless
// K * elem_size is 2, 4 or 8 KB and W rows are 16-byte aligned.
hipError_t launch_rowstream_gemm(int dtype, const void* A, int lda, int M, const void* W, int ldw, int N, int K,
                                 const void* bias, float* C, int ldc, int num_cu, hipStream_t s);

// P = A W1[:, :d]^T + b1 (bf16 A rows of lda elements, W1 rows of ldw) as S
// partial sums over K slices, ppart[S][M][r] float32 (b1 in slice 0), plus
// zeroing z0[0..n0) and z1[0..n1) (z1 may be null).  p_split_shape gives the
// slicing for hidden size d (psplit.h).
hipError_t launch_p_partials(const void* A, int M, int lda, const void* w1, int ldw, int r, const void* b1,
                             float* ppart, const PSplit& ps, unsigned long long* z0, int n0, unsigned long long* z1,
                             int n1, hipStream_t s);

// Tiled bf16 matrix-core GEMM, C = A W^T (+bias), K % 32 == 0 (else hipErrorNotSupported);
// num_cu: compute units of the device (sizes the last round of tiles).
hipError_t launch_gemm_bf16_tn(const void* A, int lda, int M, const void* W, int ldw, int N, int K, const void* bias,
                               float* C, int ldc, int num_cu, hipStream_t s);
// Split-K partial products: slice s of `slices` multiplies A columns s kc ..
// s kc + kc - 1 by W columns (s kc) mod w_wrap .. and writes C + s c_slice.
hipError_t launch_gemm_bf16_tn_splitk(const void* A, int lda, int M, const void* W, int ldw, int N, int kc,
                                      int slices, int w_wrap, float* C, int ldc, size_t c_slice, hipStream_t s);
// C[n][m] = sum_k A[m][k] W[n][k mod w_wrap] (K <= 2 w_wrap), stored transposed.
hipError_t launch_gemm_bf16_tn_wrapt(const void* A, int lda, int M, const void* W, int ldw, int N, int K, int w_wrap,
                                     float* C, int ldc, hipStream_t s);

struct LoopArgs {
  int dtype;
  int B, K, d, V, H, r;
  const void *embed, *w_ih, *w_hh, *b_ih, *b_hh, *w1, *b1, *w2, *b2;
  const void* hidden;
  const float* base;     // [B, K, V], or null: the single-block loop forms the base logits from lm_head
  const void* lm_head;   // [V, d] (read only where base is null)
  const int32_t* x_t;
  const int32_t* teacher;
  float inv_temp;
  int sampled;
  uint64_t seed;
  uint32_t offset;
  int32_t* tokens;
  float* logits;
  float* states;  // [B, K, H]
  uint32_t rng_block;  // block index of row 0 in the sampler's counter (rows are rng_block + b)
  // workspace pieces
  unsigned long long* keys;  // [K, B], followed by 2 u64 of loop control (barrier counter, status)
  float* P;                  // [B, K, r]
  float* ppart;              // B = 1: [S <= 16][K][r] K-slice partials of P
  float* part_ih;            // [KS, B, 3H]
  float* part_hh;            // [B, 3H]
  float* u;                  // [B, r]
  const float* table;  // [V, 3H] = W_ih E^T + b_ih, or nullptr
  // persistent schedules: tagged exchange words
  unsigned long long* xpart;
  size_t xwords;
  int max_wg;
  int ks;
  int num_cu;
  // the call's status word (keys + K B + 1 of the whole call): 0 while every
  // block's loop completes, 1 once one gave up; cleared by the call's first launch
  unsigned int* call_status;
  // polls a wait of the on-chip loops makes before giving up; 0 makes every
  // wait give up at its first check (a host-forced give-up for tests)
  unsigned int spin_limit;
  // key words the single-block loop's pre-loop launch clears (keys + control words)
  int clear_words;
};

// Runs the K-position loop.  mode: 0 = default (three kernels per position),
// 1 = one persistent cooperative kernel (B <= 32), 2 = three kernels per position.
hipError_t launch_draft_loop(const LoopArgs& a, int mode, hipStream_t s);

// The single-block (B = 1) loop with on-chip weights: b1_supported() tells
// whether it takes these arguments (host-side checks only); launch_draft_b1
// returns hipErrorNotSupported when the device does not fit it (the caller
// then uses another schedule).  It enqueues its own pre-loop kernel, which
// clears a.keys and the exchange words and writes the hidden half of the
// first correction projection to a.ppart.
bool b1_supported(const LoopArgs& a);
hipError_t launch_draft_b1(const LoopArgs& a, hipStream_t s);
size_t b1_exchange_words(int H, int r, int max_wg);

// The several-block loop with on-chip weights (loop_bn.hip), up to 32 blocks
// per launch (a call of more blocks runs launches of about equal size, each
// with its own pre-loop kernel): bn_supported() tells whether it takes these
// arguments (host-side checks only); bn_exchange_words() is the exchange
// region it needs for `batch` blocks.
bool bn_supported(const LoopArgs& a);
hipError_t launch_draft_bn(const LoopArgs& a, hipStream_t s);
size_t bn_exchange_words(int batch, int max_wg, int H, int r);

hipError_t launch_fill_u64(unsigned long long* p, int n, hipStream_t s);
hipError_t launch_fill2_u64(unsigned long long* z0, int n0, unsigned long long* z1, int n1, hipStream_t s);
constexpr unsigned int kDefaultSpinLimit = 1u << 20;  // about a second of polling
hipError_t launch_finalize_tokens(int B, int K, const unsigned long long* keys, int32_t* tokens, hipStream_t s);

// Sampled-draft verification (verify.hip): accept[b] and next[b] from the
// target's [B][K + 1][V] and the draft's [B][K][V] float32 logits; the
// workspace follows verify_plan(B, K, V).
hipError_t launch_verify_sampled(int B, int K, int V, const float* target, const float* draft, const int32_t* tokens,
                                 float temperature, uint64_t seed, uint32_t offset, int32_t* accept, int32_t* next,
                                 const VerifyPlan& plan, void* workspace, hipStream_t s);

// Backward through the correction head (backward.hip).
struct BackwardPlan {
  int S;     // slices of the du partials (vocabulary slices; bf16: hi and lo halves)
  int mfma;  // bf16 head: W2^T G and G^T u on the matrix cores
  int kc, Vp, Rp;  // (mfma) vocabulary entries per slice, padded vocabulary, padded rows
  // byte offsets of z, u, dz [R][r] and part [S][R][r] (float32), and with
  // mfma of gs [R][2 Vp], gt [V][2 Rp], w2t [r][Vp], us [r][3 Rp] (bf16); workspace bytes
  size_t z, u, dz, part, gs, gt, w2t, us, total;
  // dW1, db1: the rows split over G1 groups (G1 > 1: partial sums dw1p
  // [G1][r][n1] and db1p [G1][r] float32, added in group order)
  int G1;
  size_t dw1p, db1p;
  // bf16 heads with r % 32 == 0: W1's state columns transposed, w1gT [H][r]
  // bf16, for dg on the matrix cores (0: the float32 kernel)
  size_t w1gT;
  // bf16 heads from kBwW1MfmaRows rows (d, H, r multiples of 32): dW1 on the
  // matrix cores, S1 split-K slices (partials in dw1p when S1 > 1), operands
  // dzT [r][3 Rp] (dz hi | lo | hi), hT [d][2 Rp], gT [H][3 Rp] (g hi | hi |
  // lo), db1 tile sums bp1 [Rp / 64][r]
  int w1m, S1;
  size_t dzT, hT, gT, bp1;
};
constexpr int kBwW1MfmaRows = 128;
constexpr int kBwDw1Rows = 128;  // rows per dW1 group
inline BackwardPlan backward_plan(int R, int r, int V, int dtype, int n1, int H) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BackwardPlan p{};
  if (dtype == 1) {
    const long bm = R >= 256 ? 256 : 128;
    const long tiles = ((R + bm - 1) / bm) * ((r + 255) / 256);
    long half = 128 / tiles;
    const long hmax = (V + 511) / 512;  // slices of at least 512 entries
    if (half > hmax) half = hmax;
    if (half < 1) half = 1;
    p.mfma = 1;
    p.kc = (int)(64 * ((V + 64 * half - 1) / (64 * half)));
    p.Vp = (int)(half * p.kc);
    p.Rp = (R + 31) / 32 * 32;
    p.S = (int)(2 * half);
  } else {
    const long groups = (R + 63) / 64;
    long S = (512 + groups - 1) / groups;
    const long smax = V / 512 > 1 ? V / 512 : 1;  // slices of at least 512 entries
    p.S = (int)(S < 1 ? 1 : S > smax ? smax : S);
  }
  const size_t m = up((size_t)R * r * sizeof(float));
  size_t off = 0;
  p.z = off;
  off += m;
  p.u = off;
  off += m;
  p.dz = off;
  off += m;
  p.part = off;
  off += up((size_t)p.S * R * r * sizeof(float));
  if (p.mfma) {
    p.gs = off;
    off += up((size_t)R * 2 * p.Vp * 2);
    p.gt = off;
    off += up((size_t)V * 2 * p.Rp * 2);
    p.w2t = off;
    off += up((size_t)r * p.Vp * 2);
    p.us = off;
    off += up((size_t)r * 3 * p.Rp * 2);
  }
  {
    const int g = (R + kBwDw1Rows - 1) / kBwDw1Rows;
    p.G1 = g < 1 ? 1 : g > 8 ? 8 : g;
  }
  if (p.G1 > 1) {
    p.dw1p = off;
    off += up((size_t)p.G1 * r * n1 * 4);
    p.db1p = off;
    off += up((size_t)p.G1 * r * 4);
  }
  p.w1gT = 0;
  if (dtype == 1 && r % 32 == 0) {
    p.w1gT = off;
    off += up((size_t)H * r * 2);
  }
  const int d = n1 - H;
  p.w1m = dtype == 1 && R >= kBwW1MfmaRows && r % 32 == 0 && d % 32 == 0 && H % 32 == 0;
  if (p.w1m) {
    const size_t Rp = (size_t)p.Rp;
    // the largest slice count within the dW1 partial buffer dividing Rp / 32
    p.S1 = 1;
    for (int sl = p.G1; sl > 1; --sl)
      if ((p.Rp / 32) % sl == 0) {
        p.S1 = sl;
        break;
      }
    p.dzT = off;
    off += up((size_t)r * 3 * Rp * 2);
    p.hT = off;
    off += up((size_t)d * 2 * Rp * 2);
    p.gT = off;
    off += up((size_t)H * 3 * Rp * 2);
    p.bp1 = off;
    off += up((Rp + 63) / 64 * (size_t)r * 4);
  }
  p.total = off;
  return p;
}
struct BackwardArgs {
  int dtype, R, d, H, r, V;
  const void *hidden, *w1, *b1, *w2;
  const float *states, *grad;
  float *d_w2, *d_b2, *d_w1, *d_b1, *d_states;
  void* workspace;
  BackwardPlan plan;
};
hipError_t launch_correction_backward(const BackwardArgs& a, hipStream_t s);

// Backward through time of the teacher-forced GRU (gru_backward.hip).
constexpr int kGruCarryBlocks = 8;  // blocks sharing each W_hh load in the carry, from 8 blocks up
// Rows-to-K re-layout for the matrix-core weight gradients (gru_backward.hip):
// job j of a launch, Y[n][p Rp + r] = part p of X[r][n] as bf16 for r < R
// (zero up to Rp, a multiple of 32); bit p of lo_parts set: the remainder
// x - hi rounded to bf16, else hi = x truncated to bf16 (bf16 X: x itself);
// with bpart, each 64-row tile's column sums in row order, bpart[tile][n].
struct KJob {
  const void* X;  // [R][N] row-major: float32, or bf16 when bf16 = 1
  uint16_t* Y;    // [N][nparts Rp]
  float* bpart;
  int N, nparts, bf16;
  unsigned lo_parts;
};
struct KJobs {
  KJob j[4];
};
// njobs <= 4; nmax: the largest N of the jobs.
hipError_t launch_rows_to_k(int R, int Rp, const KJobs& jobs, int njobs, int nmax, hipStream_t s);
// sum_i[n] = bpart_i[0][n] + ... + bpart_i[tiles - 1][n] in tile order (sum_i nullptr: skipped).
hipError_t launch_tile_colsums(int tiles, int N, const float* bpart0, float* sum0, const float* bpart1, float* sum1,
                               hipStream_t s);

struct GruBackwardPlan {
  size_t x_e, x_g, a, c, da, dc, carry, tok, total;  // byte offsets; workspace bytes
  int carry_parts;  // P
  // bf16 heads: c = W_hh g_prev on the matrix cores, g_prev split hi | lo
  // (xs [R][2H] bf16) and S split-K partials (cpart [S][R][3H] float32)
  int S;
  size_t xs, cpart;
  // bf16 heads: the weight gradients on the matrix cores, operands re-laid
  // with the rows (padded to Rp, a multiple of 32) along K: daT [3H][2 Rp]
  // (da hi | lo), eT [d][2 Rp] (the embedding rows twice), dcT [3H][3 Rp]
  // (dc hi | hi | lo), gT [H][3 Rp] (g_prev hi | lo | hi), and the bias
  // sums' per-64-row partials bpart [2][Rp / 64][3H]
  int Rp;
  size_t daT, eT, dcT, gT, bpart;
  // bf16 heads with 3H a multiple of 32 carry_parts: W_hh transposed, whhT
  // [H][3H] bf16, for the carried gradient W_hh^T dc on the matrix cores
  // (0: the float32 kernel)
  size_t whhT;
};
inline GruBackwardPlan gru_backward_plan(int B, int K, int d, int H, int elem) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t R = (size_t)B * K, G3 = 3 * (size_t)H;
  GruBackwardPlan p{};
  size_t off = 0;
  p.x_e = off;
  off += up(R * d * elem);
  p.x_g = off;
  off += up(R * H * 4);
  p.a = off;
  off += up(R * G3 * 4);
  p.c = off;
  off += up(R * G3 * 4);
  p.da = off;
  off += up(R * G3 * 4);
  p.dc = off;
  off += up(R * G3 * 4);
  {
    // groups of the 3H terms of W_hh^T dc (the carry is [1 + P][B][H]: the
    // direct part, then one partial sum per group), about 256 workgroups
    const long wgs = ((long)H + 63) / 64 * (B >= kGruCarryBlocks ? (B + kGruCarryBlocks - 1) / kGruCarryBlocks : B);
    long P = 256 / wgs;
    P = P < 1 ? 1 : P > 8 ? 8 : P;
    // bf16 heads: a power of two, so that the matrix-core carry kernel's K
    // groups are whole 32-wide steps (3H a multiple of 32 P)
    if (elem == 2)
      while (P & (P - 1)) --P;
    p.carry_parts = (int)P;
  }
  p.carry = off;
  off += up(((size_t)(1 + p.carry_parts) * B * H + 1) / 2 * 8);
  p.tok = off;
  off += up(R * 4);
  if (elem == 2) {
    // slices of K = 2H: kc = H / half, a multiple of 32 that divides H, with
    // about 512 workgroups over the R x 3H output tiles
    const long bm = R >= 256 ? 256 : 128;
    const long tiles = (((long)R + bm - 1) / bm) * (((long)G3 + 255) / 256);
    long half = 1;
    while (4 * half * tiles <= 512 && H % (2 * half) == 0 && (H / (2 * half)) % 32 == 0) half *= 2;
    p.S = (int)(2 * half);
    p.xs = off;
    off += up(R * 2 * H * 2);
    p.cpart = off;
    off += up((size_t)p.S * R * G3 * 4);
    p.Rp = (int)((R + 31) / 32 * 32);
    const size_t Rp = (size_t)p.Rp;
    p.daT = off;
    off += up(G3 * 2 * Rp * 2);
    p.eT = off;
    off += up((size_t)d * 2 * Rp * 2);
    p.dcT = off;
    off += up(G3 * 3 * Rp * 2);
    p.gT = off;
    off += up((size_t)H * 3 * Rp * 2);
    p.bpart = off;
    off += up(2 * ((Rp + 63) / 64) * G3 * 4);
    p.whhT = 0;
    if (G3 % (32 * (size_t)p.carry_parts) == 0) {
      p.whhT = off;
      off += up((size_t)H * G3 * 2);
    }
  }
  p.total = off;
  return p;
}
struct GruBackwardArgs {
  int dtype, B, K, d, H, V;
  const void *embed, *w_ih, *w_hh, *b_ih, *b_hh;
  const int32_t *x_t, *teacher;
  const float *states, *dg;
  float *d_w_ih, *d_w_hh, *d_b_ih, *d_b_hh;
  void* workspace;
  GruBackwardPlan plan;
};
hipError_t launch_gru_backward(const GruBackwardArgs& g, int num_cu, hipStream_t s);

// Base-only drafting (base_draft.hip): tokens[b][i] picked from base[b][i][:]
// alone (greedy, or Gumbel-max when temperature > 0); workspace holds B K
// 64-bit keys.
hipError_t launch_base_draft(int B, int K, int V, const float* base, float temperature, uint64_t seed,
                             uint32_t offset, int32_t* tokens, void* workspace, hipStream_t s);

// Base-anchored curriculum loss (loss.hip) over [B][K][V] float32 base and
// final logits with targets [B][K]; ce_*, grad_* may be null; the workspace
// follows loss_plan(B, K, V).
hipError_t launch_curriculum_loss(int B, int K, int V, const float* base, const float* final_,
                                  const int32_t* targets, float lam, float gamma, float* loss, float* ce_base,
                                  float* ce_final, float* grad_base, float* grad_final, const LossPlan& plan,
                                  void* workspace, hipStream_t s);

hipError_t launch_accept_len(int B, int K, const int32_t* draft, const int32_t* target, int32_t* accept,
                             hipStream_t s);

constexpr int kReadGrid = 2048;  // workgroups of the calibration read (entries of its sink)
hipError_t launch_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_debug_philox(uint64_t seed, uint32_t offset, int b, int pos, int v0, int n, uint32_t* out,
                               hipStream_t s);

}  // namespace domino
