// Single-block (B = 1) draft loop with the head's per-position weights held
// on chip ([notes] §二.1(2) items 1-3; [explainer] §四).
//
// Pages: [notes] "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn);
//        [explainer] the yhxrc.cn article on the Domino paper.
//
// One launch of G = #CU workgroups (256 threads, 4 waves each, one workgroup
// per compute unit) runs the whole K-position loop.  Re-reading W2 and W_hh
// from HBM at every position would cost ~85 MB per position; each workgroup
// instead loads its share once and keeps it resident:
//   * W2:   a contiguous range of 16-row vocabulary tiles, up to NR per wave,
//           in registers;
//   * W_hh: a contiguous range of U_hh "k-steps" (16 gate rows x 32 inputs)
//           of the stacked [3H, H] matrix, in registers (all workgroups but
//           the unit ones);
//   * W1[:, d:] (the GRU half of the first correction projection): the
//           kUnitWGs "unit" workgroups hold the columns of their H / kUnitWGs
//           GRU units in LDS, in place of some of their W2 tiles.
// The GRU input term W_ih e(y) + b_ih is read from the per-head table
// T[y] = W_ih E[y] + b_ih (domino_prepare_gru_table): one row gather per
// position instead of a 25 MB matrix-vector product.
//
// Per position i (every exchanged word is {tag = i + 1, payload}, written and
// polled with relaxed agent-scope atomics, double-buffered by the parity of i):
//   B(i)   the kUnitWGs unit workgroups: y_{i-1} from the G argmax keys,
//          T[y_{i-1}] for their units, W_hh g_{i-1} from the partials, gates,
//          new state g_i (-> states, x_g), their share of W1[:, d:] g_i on
//          the matrix cores, unit workgroup s < S adding slice s of
//          P_i = W1[:, :d] h_i + b1                                -> x_pu
//   C(i)   every workgroup: u = SiLU(sum of the shares), its W2 tiles
//          on the matrix cores, + b2 + base logits (+ Gumbel), argmax -> x_key
//   A(i+1) the other workgroups (the W_hh owners), after publishing their
//          key: W_hh g_i partials of their k-range, from g_i staged in C(i)
//                                                                  -> x_hh
// The only exchanges on the token-to-token path are the key gather and the
// u shares; A(i+1) overlaps the key gather and the T row read of B(i+1).
// A wave's loads wait for the completion of its earlier stores (one counter
// covers both), so each role polls before it publishes wherever it can.
// Every wait is bounded: a workgroup that gives up records it in `status`
// and all others leave at their next poll; the tokens are then -1.
//
// The workgroups wait on one another, so all G must be resident at once.  The
// kernel is an ordinary launch (a cooperative launch costs ~20 us more per
// call in the runtime): the host checks that one workgroup fits per compute
// unit, and as G is the compute-unit count every workgroup starts as soon as
// earlier work on the device has left the compute units.  Work on other
// streams that keeps compute units busy only delays the loop; a wait gives up
// after about a second, so even a loop that cannot complete ends.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"
#include <hip/hip_ext.h>

#include "xchg.h"

namespace domino {
namespace b1 {
using namespace xchg;

// One wave per SIMD: each wave may use 512 registers (256 VGPRs + 256 AGPRs),
// which is where the workgroup's whole share of W2 lives.
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kNR = 10;  // W2 tiles per wave, held in registers
constexpr int kUnitWGs = 8;
constexpr int kUnitMax = 128;  // GRU units per unit workgroup (H <= 1024)
constexpr int kMaxWgTiles = kNR * kWaves;  // W2 tiles per workgroup
constexpr int kStreamPositions = 16;       // positions of a block whose base logits the kernel can form itself
// LM-head widths the kernel streams (64-B steps per wave-quarter of a row):
// d = 2560 and d = 4096 (the Qwen3-4B and Qwen3-8B hidden sizes)
constexpr int kStreamKw4B = 2560 * 2 / kWaves / 64;
constexpr int kStreamKw8B = 4096 * 2 / kWaves / 64;
constexpr int kUHW = 8;  // W_hh k-steps per wave: the only shape a grid of 200..256 workgroups takes
constexpr int kPRows = 256 / kUnitWGs;  // rows of P = W1[:, :d] h + b1 a unit workgroup forms (fused; r = 256)
typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
constexpr int kWaitVmem0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters left alone


struct Params {
  int d, V, H, r, K;
  int KH;      // 32-element k-steps per W_hh row: H / 32
  int U_hh;    // W_hh k-steps per W_hh owner (multiple of 2 * kWaves)
  int ntiles;  // ceil(V / 16)
  int ut;      // W2 tiles of a unit workgroup (the others share the remainder evenly)
  const uint16_t *w_hh, *b_hh, *w1, *w2, *b2, *b1;
  const float* table;     // [V][3H]: W_ih E[v] + b_ih
  const float* base;   // [K][V], or null: the kernel forms its range's base logits itself
  const uint16_t *lm_head, *hidden;  // [V][d], [K][d] (base == null)
  const float* ppart;  // [S][K][r]: P = W1[:, :d] h + b1 = sum over s of ppart[s] (b1 in s = 0)
  int S;
  const int32_t *x_t, *teacher;
  float inv_temp;
  int sampled;
  uint64_t seed;
  uint32_t offset;
  uint32_t rng_b;  // the block's index in the sampler's counter
  float *logits, *states;
  int32_t* tokens;
  unsigned int* status;       // this launch's give-up flag: the other workgroups leave at their next poll
  unsigned int* call_status;  // the call's status word (see domino_draft_status)
  unsigned int spin_limit;    // polls before a wait gives up; 0: every wait gives up at once
  unsigned long long* x_hh;   // [2][G][2 segments][16]
  unsigned long long* x_g;    // [2][H]
  unsigned long long* x_pu;   // [2][kUnitWGs][r]
  unsigned long long* x_key;  // [2][G]
};

// Max over the G keys published for one position, on one wave; every load of a
// lane is in flight before the first is checked.
__device__ __forceinline__ bool gather_keys(const unsigned long long* keys, int G, uint32_t tag,
                                            const unsigned int* status, unsigned int limit,
                                            unsigned long long& best) {
  constexpr int kMaxPer = 4;  // G <= 256
  const int lane = threadIdx.x & 63;
  unsigned long long k[kMaxPer];
  const unsigned long long* src[kMaxPer];
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    src[q] = lane + q * 64 < G ? keys + lane + q * 64 : nullptr;
    k[q] = src[q] ? ld_word(src[q]) : 0ull;
  }
  bool ok = true;
  unsigned int spins = 0;
  while (true) {
    bool done = true;
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) done &= !src[q] || key_tagged(k[q], tag);
    if (done && limit != 0u) break;
    if (++spins > limit || ((spins & 63u) == 0u && gave_up(status))) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q)
      if (src[q] && !key_tagged(k[q], tag)) k[q] = ld_word(src[q]);
  }
  best = 0ull;
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) best = k[q] > best ? k[q] : best;
  best = wave_max(best);
  return ok;
}

// Word offset, within the parity-0 half of x_hh, of the o-th W_hh partial of
// gate row `row` (the W_hh owners, i.e. the workgroups after the unit ones,
// numbered from 0, whose k-step range covers the row's tile, each holding it
// in segment 0 (its first tile) or 1), or -1 when the tile has fewer owners.
__device__ __forceinline__ int hh_partial_offset(const Params& p, int row, int o, int G) {
  const int t = row >> 4, c = row & 15;
  const int lo = (t * p.KH) / p.U_hh, hi = (t * p.KH + p.KH - 1) / p.U_hh;
  const int ow = lo + o;
  if (ow > hi) return -1;
  const int seg = ((ow * p.U_hh) / p.KH == t) ? 0 : 1;
  return (ow * 2 + seg) * 16 + c;
}

// The argmax key of one entry: L_i[v] = (W2 u)[v] + (base + b2)[v], scored
// as L_i[v] (greedy) or L_i[v] / T + Gumbel noise.  Entries past the
// workgroup's range or the vocabulary carry a bias of -inf and never win.
template <bool SAMPLED>
__device__ __forceinline__ unsigned long long entry_key(float L, float inv_temp, float noise, uint32_t v, uint32_t tag) {
  return tagged_key(SAMPLED ? L * inv_temp + noise : L, v, tag);
}

struct Lds {
  int pool, ghl, utile, lbs, b2s, gum, uhl, gs_prev, zero, red, lb, px, total;
};

// The pool holds a unit workgroup's W1 columns, or a W_hh owner's k-steps,
// both as matrix-core fragments [.. 16-row tiles][.. k-steps][64 lanes][16 B].
__host__ __device__ inline Lds lds_layout(int U_hh, int H, int r, bool fused) {
  Lds L{};
  int off = 0;
  L.pool = off;
  const int unit_pool = r * (H / kUnitWGs) * 2, owner_pool = U_hh * 1024;
  off += unit_pool > owner_pool ? unit_pool : owner_pool;
  L.ghl = off;
  off += 2 * H * 2;  // g split into bf16 hi and lo rows (W_hh owners)
  L.utile = off;
  off += 2 * r * 2;  // u split into bf16 hi and lo rows
  L.lbs = off;
  off += kMaxWgTiles * 16 * 4;  // base logits + b2 of this workgroup's vocabulary range
  L.b2s = off;
  off += kMaxWgTiles * 16 * 4;  // b2 of the same range
  L.gum = off;
  off += kMaxWgTiles * 16 * 4;  // Gumbel noise of the same range at this position (sampling)
  L.uhl = off;
  off += 2 * kUnitMax * 2;  // a unit workgroup's g split into bf16 hi and lo rows
  L.gs_prev = off;
  off += kUnitMax * 4;
  L.zero = off;
  off += 16;  // 16 zero bytes: the A operand of the lanes of rows 2-15
  L.red = off;
  off += kWaves * 2 * 16 * 4;
  L.lb = off;
  off += fused ? kStreamPositions * kMaxWgTiles * 16 * 4 : 0;  // base logits + b2 of every position (fused)
  L.px = off;
  off += fused ? kStreamPositions * kPRows * 4 : 0;  // a unit workgroup's rows of P for every position (fused)
  L.total = off;
  return L;
}

// Vectors enter the matrix cores as the A operand of a 16x16x32 product with
// only two live rows: x is split into bf16 halves x = hi + lo, stored as two
// LDS rows (hl[j] = hi, hl[n + j] = lo); row 0 of the operand (col == 0
// lanes) carries hi and row 1 (col == 1 lanes) carries lo, so one instruction
// forms both products and the result is D[0][c] + D[1][c] = acc[0] + acc[1]
// on the grp == 0 lanes.  The lanes of rows 2-15 read 16 zero bytes.
__device__ __forceinline__ void split_store(uint16_t* hl, int n, int j, float x) {
  const uint32_t u = __float_as_uint(x) & 0xFFFF0000u;
  hl[j] = (uint16_t)(u >> 16);
  hl[n + j] = (uint16_t)f32_to_bf16_rne(x - __uint_as_float(u));
}
__device__ __forceinline__ u32x4 row_frag(const uint16_t* hl, int n, int k0, int col, int grp, const void* zero) {
  return ld16(col < 2 ? static_cast<const void*>(hl + col * n + k0 + grp * 8) : zero);
}

// Bytes of LDS the fused base-logit stream borrows from the pool: each
// wave's transposition tile and two reduction buffers.
__host__ __device__ constexpr int stream_scratch_bytes() { return kWaves * 16 * 512 + 2 * kWaves * 16 * 17 * 4; }

// Base logits of this workgroup's vocabulary range for every position
// ([notes] §二.1(1): the frozen LM head over the block's hidden states, in one
// pass): lb[i][e] = sum_k hidden[i][k] W_lm[16 t_lo + e][k] + b2[16 t_lo + e]
// (-inf past the vocabulary); then, for a unit workgroup u (nx = 2), rows
// 32 u .. 32 u + 31 of the hidden half of the first correction projection,
// px[i][c] = sum_k hidden[i][k] W1[32 u + c][k] + b1[32 u + c]
// ([notes] §二.1(2) item 2: the hidden state's share of the bottleneck
// input), streamed the same way as two more tiles.  W_lm's rows are read once, from HBM, the way
// it streams best: each wave takes a quarter of K (KW 64-B steps of each
// row), and a load instruction covers 512 contiguous bytes of each of two rows,
// read non-temporally through buffer descriptors sized to the valid rows (rows
// past V read zero); a quarter of K that 512 B does not divide goes in 256-B
// passes of four rows.  The wave writes its slices into a private LDS tile
// (16-B chunks XOR-swizzled by row) and reads them back as matrix-core
// operands against the 16 positions' hidden states held in registers; the
// four waves' partial sums are added in LDS in a fixed order.  The next tile's
// loads are in flight while a tile is multiplied.
template <int KW>
__device__ void stream_base(const Params& p, int t_lo, int nt, int nx, int x_row0, unsigned char* scratch, float* lb,
                            float* px) {
  constexpr int kSlice = KW * 64;
  constexpr int kPass = kSlice % 512 == 0 ? 512 : 256;
  constexpr int kPasses = kSlice / kPass;
  constexpr int kChunks = kPass / 16;
  constexpr int kRowsPerLoad = 64 / kChunks;
  constexpr int kLoadsPerPass = 16 / kRowsPerLoad;
  constexpr int kStepsPerPass = kPass / 64;
  static_assert(kSlice % kPass == 0 && kPasses * kLoadsPerPass == KW, "stream shape");
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int V = p.V, d = p.d;
  unsigned char* tile = scratch + wave * 16 * kPass;
  float* red = reinterpret_cast<float*>(scratch + kWaves * 16 * 512);
  u32x4 af[KW];
  {
    const bool live = col < p.K;
    const unsigned char* arow =
        reinterpret_cast<const unsigned char*>(p.hidden + (size_t)(live ? col : 0) * d) + wave * kSlice + grp * 16;
#pragma unroll
    for (int s = 0; s < KW; ++s) af[s] = live ? ld16(arow + s * 64) : u32x4{0, 0, 0, 0};
  }
  const int lrow = lane / kChunks, lchunk = lane % kChunks;
  const int ldw1 = d + p.H;  // W1 row length (hidden half first)
  auto stage = [&](int j, u32x4 (&dst)[KW]) {
    // tile j < nt: LM head rows 16 (t_lo + j) ..; nt <= j < nt + nx: W1 rows
    // x_row0 + 16 (j - nt) ..; later: nothing (every load reads zero)
    const bool lm = j < nt, w1t = !lm && j < nt + nx;
    const int rows = lm ? min(16, V - (t_lo + j) * 16) : w1t ? 16 : 0;
    const int ld = lm ? d : ldw1;
    const uint16_t* base = lm ? p.lm_head + (size_t)(t_lo + j) * 16 * d
                              : w1t ? p.w1 + (size_t)(x_row0 + 16 * (j - nt)) * ldw1 : p.lm_head;
    const int row_bytes = ld * 2;
    const int voff = lrow * row_bytes + wave * kSlice + lchunk * 16;
#pragma unroll
    for (int jj = 0; jj < kLoadsPerPass; ++jj) {
      const int rj =
          jj == 0 ? min(rows, kRowsPerLoad) : min(max(rows - jj * kRowsPerLoad, 0), kRowsPerLoad);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base + (rj > 0 ? (size_t)jj * kRowsPerLoad * ld : 0)), (short)0, rj * row_bytes,
          kRsrcWord3);
#pragma unroll
      for (int q = 0; q < kPasses; ++q)
        dst[q * kLoadsPerPass + jj] = __builtin_amdgcn_raw_buffer_load_b128(r, voff + q * kPass, 0, kLoadNonTemporal);
    }
  };
  auto process = [&](int j, const u32x4 (&w)[KW], float* rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
#pragma unroll
      for (int jj = 0; jj < kLoadsPerPass; ++jj) {
        const int r = jj * kRowsPerLoad + lrow;
        st16(tile + r * kPass + ((lchunk ^ (r & 15)) << 4), w[q * kLoadsPerPass + jj]);
      }
#pragma unroll
      for (int ss = 0; ss < kStepsPerPass; ++ss) {
        const u32x4 b = ld16(tile + col * kPass + (((ss * 4 + grp) ^ col) << 4));
        acc = mma16<Bf16>(acc, af[q * kStepsPerPass + ss], b);
      }
    }
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) rb[(wave * 16 + grp * 4 + jq) * 17 + col] = acc[jq];
    __syncthreads();
    // thread: position tid / 16, entry tid % 16 of the tile
    const int m = tid >> 4, c = tid & 15;
    float sum = 0.f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) sum += rb[(wv * 16 + m) * 17 + c];
    if (j < nt) {
      const int v = (t_lo + j) * 16 + c;
      lb[m * kMaxWgTiles * 16 + j * 16 + c] = v < V ? sum + (p.b2 ? bf16_to_f32(p.b2[v]) : 0.f) : -INFINITY;
    } else {
      const int row = x_row0 + 16 * (j - nt) + c;
      px[m * kPRows + 16 * (j - nt) + c] = sum + (p.b1 ? bf16_to_f32(p.b1[row]) : 0.f);
    }
  };
  u32x4 w0[KW], w1[KW];
  const int ntot = nt + nx;
  int j = 0;
  stage(0, w0);
  // the scheduling barriers keep each prefetch ahead of the tile in hand
  while (j < ntot) {
    stage(j + 1, w1);
    __builtin_amdgcn_sched_barrier(0);
    process(j, w0, red);
    if (++j >= ntot) break;
    stage(j + 1, w0);
    __builtin_amdgcn_sched_barrier(0);
    process(j, w1, red + kWaves * 16 * 17);
    ++j;
  }
  // slots without a tile never win
  for (int i = tid; i < kStreamPositions * kMaxWgTiles * 16; i += kThreads)
    if (i % (kMaxWgTiles * 16) >= nt * 16) lb[i] = -INFINITY;
}

template <int UHW, int NR, int RK, bool SAMPLED, bool LOGITS, int SKW>
__global__ void __launch_bounds__(kThreads, 1) draft_b1_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ unsigned long long s_key[kWaves];
  __shared__ int s_tok;
  const int w = blockIdx.x, G = gridDim.x;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int H = p.H, V = p.V, r = p.r;
  const int T3 = (3 * H) >> 4;
  const Lds L = lds_layout(p.U_hh, H, r, SKW > 0);
  unsigned char* pool = smem + L.pool;
  uint16_t* ghl = reinterpret_cast<uint16_t*>(smem + L.ghl);
  uint16_t* utile = reinterpret_cast<uint16_t*>(smem + L.utile);
  uint16_t* uhl = reinterpret_cast<uint16_t*>(smem + L.uhl);
  float* gs_prev = reinterpret_cast<float*>(smem + L.gs_prev);
  const void* zero = smem + L.zero;
  float* red = reinterpret_cast<float*>(smem + L.red);
  float* lbs = reinterpret_cast<float*>(smem + L.lbs);
  float* b2s = reinterpret_cast<float*>(smem + L.b2s);
  float* gum = reinterpret_cast<float*>(smem + L.gum);
  float* lbt = reinterpret_cast<float*>(smem + L.lb);
  float* pxt = reinterpret_cast<float*>(smem + L.px);
  const int units = H / kUnitWGs;
  const int ksu = units / 32;  // k-steps of a unit workgroup's W1 columns
  const bool unit_wg = w < kUnitWGs;

  // ---------------- resident weights ----------------
  int t_lo, t_hi;
  {
    const int rest = p.ntiles - kUnitWGs * p.ut, others = G - kUnitWGs;
    if (unit_wg) {
      t_lo = w * p.ut;
      t_hi = t_lo + p.ut;
    } else {
      const int o = w - kUnitWGs;
      t_lo = kUnitWGs * p.ut + (int)((long)o * rest / others);
      t_hi = kUnitWGs * p.ut + (int)((long)(o + 1) * rest / others);
    }
  }
  const int nt = t_hi - t_lo;
  // fused: the base logits of the range for every position first, while the
  // registers and the pool are still free
  if constexpr (SKW > 0) {
    stream_base<SKW>(p, t_lo, nt, unit_wg ? kPRows / 16 : 0, w * kPRows, pool, lbt, pxt);
    __syncthreads();
  }
  // W2: tile s * kWaves + wave of this workgroup's range, 8 k-step fragments each
  u32x4 w2r[NR][RK];
#pragma unroll
  for (int s = 0; s < NR; ++s) {
    const int j = s * kWaves + wave;
    const int v = min((t_lo + j) * 16 + col, V - 1);
#pragma unroll
    for (int k = 0; k < RK; ++k)
      w2r[s][k] = j < nt ? ld16(p.w2 + (size_t)v * r + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
  }
  // W_hh owners: k-steps [hw * U_hh, (hw + 1) * U_hh) of the stacked W_hh (hw = w - kUnitWGs)
  const long total_hh = (long)T3 * p.KH, hh0 = unit_wg ? total_hh : (long)(w - kUnitWGs) * p.U_hh;
  float bhh[3] = {0.f, 0.f, 0.f};
  int hoff[3][3];  // unit workgroups: offsets of the W_hh partials of this thread's gate rows
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int o = 0; o < 3; ++o) hoff[q][o] = -1;
  // The pool's fragments go straight from memory into LDS (no registers,
  // every load of a wave in flight at once): fragment f of wave f % kWaves,
  // lane ln's 16 bytes at pool + f KB + 16 ln.
  if (unit_wg) {
    // W1[:, d + w*units : d + (w+1)*units] as fragments of 16 rows x 32 columns
    for (int f = wave; f < (r / 16) * ksu; f += kWaves) {
      const int rt = f / ksu, ks = f - rt * ksu;
      const int row = rt * 16 + (lane & 15), c0 = ks * 32 + (lane >> 4) * 8;
      __builtin_amdgcn_global_load_lds((gptr_t)(p.w1 + (size_t)row * (p.d + H) + p.d + w * units + c0),
                                       (lptr_t)(pool + (size_t)f * 1024), 16, 0, 0);
    }
    if (tid < units && p.b_hh)
#pragma unroll
      for (int q = 0; q < 3; ++q) bhh[q] = bf16_to_f32(p.b_hh[q * H + w * units + tid]);
    if (tid < units)
#pragma unroll
      for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int o = 0; o < 3; ++o) hoff[q][o] = hh_partial_offset(p, q * H + w * units + tid, o, G);
  } else {
    // k-steps past the end of W_hh are zeros
    for (int f = wave; f < p.U_hh; f += kWaves) {
      const long gu = hh0 + f;
      if (gu < total_hh) {
        const int t = (int)(gu / p.KH), s = (int)(gu % p.KH);
        __builtin_amdgcn_global_load_lds(
            (gptr_t)(p.w_hh + (size_t)(t * 16 + (lane & 15)) * H + s * 32 + (lane >> 4) * 8),
            (lptr_t)(pool + (size_t)f * 1024), 16, 0, 0);
      } else {
        st16(pool + ((size_t)f * 64 + lane) * 16, u32x4{0, 0, 0, 0});
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // the direct-to-LDS loads have landed (the barrier below publishes them)
  const int nv = nt * 16;  // vocabulary entries of this workgroup: [t_lo * 16, t_lo * 16 + nv)
  for (int i = tid; i < nv; i += kThreads) {
    const int v = t_lo * 16 + i;
    b2s[i] = v < V && p.b2 ? bf16_to_f32(p.b2[v]) : 0.f;
  }
  for (int i = nv + tid; i < kMaxWgTiles * 16; i += kThreads) lbs[i] = -INFINITY;  // slots without a tile
  if (tid < 4) reinterpret_cast<uint32_t*>(smem + L.zero)[tid] = 0u;
  if (tid < kUnitMax) gs_prev[tid] = 0.f;
  __syncthreads();

  const int t_first_hh = (int)(hh0 / p.KH);
  const long hh_last = min(hh0 + p.U_hh, total_hh) - 1;
  const int t_last_hh = hh_last >= hh0 ? (int)(hh_last / p.KH) : -1;
  const int hw = w - kUnitWGs;
  // this wave's W_hh k-steps: hcount of them from global k-step hh0 + wave * UHW
  int hseg0 = 0, hs0 = 0, hcount = 0;
  if (!unit_wg) {
    const long g0 = hh0 + (long)wave * UHW;
    hcount = (int)max(0L, min((long)UHW, total_hh - g0));
    if (hcount > 0) {
      hseg0 = (int)(g0 / p.KH) - t_first_hh;
      hs0 = (int)(g0 % p.KH);
    }
  }
  bool ok = true;
  // Position i: unit workgroups run B(i) then C(i); the others run C(i) then
  // A(i+1).
  for (int step = 0; step < p.K; ++step) {
    const uint32_t tag = step + 1;
    const int par = step & 1;
    // base logits of this workgroup's vocabulary range at this position:
    // loaded now, stored to LDS (with b2 added) just before C needs them
    // (unit workgroups issue them after the key gather: a wave's loads
    // complete in order, so the gather's polls would wait for them)
    constexpr int kLbPer = (kMaxWgTiles * 16 + kThreads - 1) / kThreads;
    float lbr[kLbPer];
    auto load_base = [&]() {
      if constexpr (SKW > 0) return;
#pragma unroll
      for (int q = 0; q < kLbPer; ++q) {
        const int i = tid + q * kThreads, v = t_lo * 16 + i;
        lbr[q] = i < nv && v < V ? p.base[(size_t)step * V + v] : 0.f;
      }
    };
    if (!unit_wg) load_base();
    // Gumbel noise for this position (read in C, after two barriers)
    if (SAMPLED)
      for (int i = tid; i < nv; i += kThreads)
        gum[i] = gumbel_from_word(philox_word(p.seed, p.offset, p.rng_b, step, t_lo * 16 + i));

    if (unit_wg) {
      // ---------- B(i): unit workgroups ----------
      // W_hh g_{i-1} partials (published during the previous position): in
      // flight while the keys are gathered
      const unsigned long long* hsrc[9];
      unsigned long long hx[9];
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        const int off = hoff[q / 3][q % 3];
        hsrc[q] = tid < units && step > 0 && off >= 0 ? p.x_hh + (size_t)par * G * 32 + off : nullptr;
        hx[q] = hsrc[q] ? ld_word(hsrc[q]) : 0ull;
      }
      if (wave == kWaves - 1) {
        int tok;
        if (step == 0) {
          tok = p.x_t[0];
        } else {
          unsigned long long best;
          ok &= gather_keys(p.x_key + (size_t)(par ^ 1) * G, G, step, p.status, p.spin_limit, best);
          const int picked = key_index(best);
          if (w == 0 && lane == 0) p.tokens[step - 1] = picked;
          tok = p.teacher ? p.teacher[step - 1] : picked;
        }
        if (lane == 0) s_tok = min(max(tok, 0), V - 1);
      }
      if (__syncthreads_or(!ok)) {
        ok = false;
        break;
      }
      load_base();
      // unit workgroup w < S adds slice w of P = W1[:, :d] h_i + b1 to the
      // entries it publishes (lanes of row group 0 hold them); it arrives
      // while the gates are formed
      constexpr int kRtPerWave = 256 / 16 / kWaves;  // r / 16 / kWaves with r = 256
      float pslice[kRtPerWave];
#pragma unroll
      for (int i = 0; i < kRtPerWave; ++i) {
        const int row = (wave * kRtPerWave + i) * 16 + col;
        if constexpr (SKW > 0)  // rows w kPRows .. of P, formed in the stream
          pslice[i] = grp == 0 && row >= w * kPRows && row < (w + 1) * kPRows ? pxt[step * kPRows + row - w * kPRows]
                                                                              : 0.f;
        else
          pslice[i] = w < p.S && grp == 0 ? p.ppart[((size_t)w * p.K + step) * r + row] : 0.f;
      }
      if (tid < units) {
        const int j = w * units + tid;
        const float* trow = p.table + (size_t)s_tok * 3 * H;
        float a3[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) a3[q] = trow[q * H + j];
        ok &= settle_all(hsrc, tag, p.status, p.spin_limit, hx);
        float c3[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          float h = 0.f;
#pragma unroll
          for (int o = 0; o < 3; ++o)
            if (hsrc[q * 3 + o]) h += __uint_as_float((uint32_t)hx[q * 3 + o]);
          c3[q] = h + bhh[q];
        }
        const float rg = sigmoidf_(a3[0] + c3[0]);
        const float zg = sigmoidf_(a3[1] + c3[1]);
        const float ng = tanhf(a3[2] + rg * c3[2]);
        const float g = (1.f - zg) * ng + zg * gs_prev[tid];
        split_store(uhl, units, tid, g);
        gs_prev[tid] = g;
        p.states[(size_t)step * H + j] = g;
        put_f32(p.x_g + (size_t)par * H + j, g, tag);
      }
      if (__syncthreads_or(!ok)) {
        ok = false;
        break;
      }
      // this workgroup's share of W1[:, d:] g on the matrix cores: wave wv
      // owns bottleneck rows [wv * r / kWaves, (wv + 1) * r / kWaves)
      f32x4 acc[kRtPerWave];
#pragma unroll
      for (int i = 0; i < kRtPerWave; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      // (the plan admits H = kUnitWGs kUnitMax only, so ksu = kKsu) a
      // k-step's operand reads are all issued before its products: read one
      // at a time, each product waited out a read's latency (all k-steps'
      // reads at once would not fit in the registers left)
      constexpr int kKsu = kUnitMax / 32;
#pragma unroll
      for (int ks = 0; ks < kKsu; ++ks) {
        const u32x4 a = row_frag(uhl, units, ks * 32, col, grp, zero);
        u32x4 wf[kRtPerWave];
#pragma unroll
        for (int i = 0; i < kRtPerWave; ++i)
          wf[i] = ld16(pool + ((size_t)((wave * kRtPerWave + i) * kKsu + ks) * 64 + lane) * 16);
#pragma unroll
        for (int i = 0; i < kRtPerWave; ++i) acc[i] = mma16<Bf16>(acc[i], a, wf[i]);
        __builtin_amdgcn_sched_group_barrier(0x100, kRtPerWave + 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, kRtPerWave, 0);
      }
      if (grp == 0)
#pragma unroll
        for (int i = 0; i < kRtPerWave; ++i)
          put_f32(p.x_pu + ((size_t)par * kUnitWGs + w) * r + (wave * kRtPerWave + i) * 16 + col,
                  acc[i][0] + acc[i][1] + pslice[i], tag);
    }

    // ---------- C(i): u, W2 tiles, argmax ----------
    const bool do_hh = !unit_wg && step + 1 < p.K && hh0 < total_hh;
    if constexpr (SKW == 0)
#pragma unroll
      for (int q = 0; q < kLbPer; ++q)
        if (tid + q * kThreads < nv)
          lbs[tid + q * kThreads] = t_lo * 16 + tid + q * kThreads < V ? lbr[q] + b2s[tid + q * kThreads] : -INFINITY;
    if (wave == 0) ok &= wait_sentinels(p.x_pu + (size_t)par * kUnitWGs * r, kUnitWGs, r, tag, p.status, p.spin_limit);
    if (do_hh && wave == 1)
      ok &= wait_sentinels(p.x_g + (size_t)par * H, kUnitWGs, units, tag, p.status, p.spin_limit);
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    {
      // this thread's u entry (tid < r = kThreads) from the kUnitWGs shares and,
      // for a W_hh owner, its g_i entries for A(i+1) (published before the u
      // shares); all loads are issued before any is checked
      constexpr int kPer = 1024 / kThreads;  // H <= kPer * kThreads
      const unsigned long long* src[kUnitWGs + kPer];
      unsigned long long x[kUnitWGs + kPer];
#pragma unroll
      for (int q = 0; q < kUnitWGs; ++q) src[q] = tid < r ? p.x_pu + ((size_t)par * kUnitWGs + q) * r + tid : nullptr;
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        src[kUnitWGs + q] = do_hh && tid + q * kThreads < H ? p.x_g + (size_t)par * H + tid + q * kThreads : nullptr;
#pragma unroll
      for (int q = 0; q < kUnitWGs + kPer; ++q) x[q] = src[q] ? ld_word(src[q]) : 0ull;
      ok &= settle_all(src, tag, p.status, p.spin_limit, x);
      if (tid < r) {
        float s = 0.f;  // the shares carry P as well
#pragma unroll
        for (int q = 0; q < kUnitWGs; ++q) s += __uint_as_float((uint32_t)x[q]);
        split_store(utile, r, tid, s * sigmoidf_(s));
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (src[kUnitWGs + q]) split_store(ghl, H, tid + q * kThreads, __uint_as_float((uint32_t)x[kUnitWGs + q]));
    }
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    // u's hi / lo halves ride in rows 0 / 1 of the A operand (rows 2-15 read
    // zeros); its 8 k-step fragments are loaded once for all tiles.  Every
    // register slot is multiplied (a slot without a tile holds zeros) so the
    // tile loop is straight-line code; only live tiles reach the epilogue.
    u32x4 ua[RK];
#pragma unroll
    for (int k = 0; k < RK; ++k) ua[k] = row_frag(utile, r, k * 32, col, grp, zero);
    float bias[NR];  // Lb + b2 of the row-0 lanes' entries, read while the products run
#pragma unroll
    for (int s = 0; s < NR; ++s)
      bias[s] = (SKW > 0 ? lbt + step * kMaxWgTiles * 16 : lbs)[min((s * kWaves + wave) * 16 + col, kMaxWgTiles * 16 - 1)];
    f32x4 acc[NR];
#pragma unroll
    for (int s = 0; s < NR; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < RK; ++k)
#pragma unroll
      for (int s = 0; s < NR; ++s) acc[s] = mma16<Bf16>(acc[s], ua[k], w2r[s][k]);
    __builtin_amdgcn_sched_group_barrier(0x100, RK + NR, 0);  // every LDS read first,
    __builtin_amdgcn_sched_group_barrier(0x008, NR * RK, 0);  // then the products
    // branch-free over every slot and lane: only row-0 lanes (grp == 0) hold
    // results, the others and the slots without an entry (bias -inf) lose
    unsigned long long best = 0ull;
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      int i = (s * kWaves + wave) * 16 + col;
      // opaque here, so per-tile constants derived from i are not hoisted
      // out of the position loop (where they would be spilled)
      asm volatile("" : "+v"(i));
      const float L = acc[s][0] + acc[s][1] + bias[s];
      if constexpr (LOGITS)
        if (grp == 0 && i < nv && t_lo * 16 + i < V) p.logits[(size_t)step * V + t_lo * 16 + i] = L;
      const unsigned long long k = entry_key<SAMPLED>(L, p.inv_temp, SAMPLED ? gum[min(i, kMaxWgTiles * 16 - 1)] : 0.f,
                                                      (uint32_t)(t_lo * 16 + i), tag);
      best = grp == 0 && k > best ? k : best;
    }
    best = row_max16(best);  // the candidates are in row 0 (lanes 0-15)
    if (lane == 0) s_key[wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long k = s_key[0];
#pragma unroll
      for (int wv = 1; wv < kWaves; ++wv) k = s_key[wv] > k ? s_key[wv] : k;
      if (k == 0ull) k = (unsigned long long)(tag & 0xFFu) << 24;  // no tiles: a tagged lowest key
      put_word(p.x_key + (size_t)par * G + w, k);
    }

    // ---------- A(i+1): W_hh g_i (W_hh owners), from LDS only ----------
    if (do_hh) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      int seg = hseg0, s = hs0;  // this wave's first k-step: segment (tile - t_first_hh) and column step
#pragma unroll
      for (int q = 0; q < UHW; ++q) {
        if (q < hcount) {
          const u32x4 a = row_frag(ghl, H, s * 32, col, grp, zero);
          const u32x4 b = ld16(pool + ((size_t)(wave * UHW + q) * 64 + lane) * 16);
          if (seg == 0)
            acc0 = mma16<Bf16>(acc0, a, b);
          else
            acc1 = mma16<Bf16>(acc1, a, b);
        }
        if (++s == p.KH) {
          s = 0;
          ++seg;
        }
      }
      if (grp == 0) {
        red[(wave * 2 + 0) * 16 + col] = acc0[0] + acc0[1];
        red[(wave * 2 + 1) * 16 + col] = acc1[0] + acc1[1];
      }
      __syncthreads();
      if (tid < 32) {
        const int sg = tid >> 4, c = tid & 15;
        if (t_first_hh + sg <= t_last_hh) {
          float sum = 0.f;
#pragma unroll
          for (int wv = 0; wv < kWaves; ++wv) sum += red[(wv * 2 + sg) * 16 + c];
          put_f32(p.x_hh + (((size_t)(par ^ 1) * G + hw) * 2 + sg) * 16 + c, sum, tag + 1);
        }
      }
    }
  }

  if (ok && w == 0 && wave == kWaves - 1) {  // the token of the last position
    unsigned long long best;
    ok &= gather_keys(p.x_key + (size_t)((p.K - 1) & 1) * G, G, p.K, p.status, p.spin_limit, best);
    if (lane == 0 && ok) p.tokens[p.K - 1] = key_index(best);
  }
  if (!ok) {
    if (tid == 0) {
      atomicOr(p.status, 1u);
      atomicOr(p.call_status, 1u);
    }
    if (w == 0)
      for (int i = tid; i < p.K; i += kThreads) p.tokens[i] = -1;
  }
}

// Before the loop, one launch clears the argmax keys, the control words and
// the exchange words (no stale tag may survive from an earlier call) and
// writes P = W1[:, :d] h + b1 as S K-slice partials (launch_p_partials);
// unit workgroup s < S adds slice s of P into the share of W1[:, d:] g it
// publishes, so every workgroup's u = SiLU(sum of the shares).
struct PreArgs {
  const LoopArgs* a;
  PSplit shape;
};

static hipError_t launch_pre(const PreArgs& q, hipStream_t s) {
  const LoopArgs& a = *q.a;
  return launch_p_partials(a.hidden, a.K, a.d, a.w1, a.d + a.H, a.r, a.b1, a.ppart, q.shape, a.keys, a.clear_words,
                           a.xpart, (int)a.xwords, s);
}

// Checks that the loop kernel fits one workgroup per CU, then launches the
// pre-loop kernel and the loop, ordered after earlier loops of the device.
template <int UHW, int NR, int RK, bool SAMPLED, bool LOGITS, int SKW>
static hipError_t launch_t(const Params& p, int G, size_t lds, const PreArgs& q, hipStream_t s) {
  auto kern = draft_b1_kernel<UHW, NR, RK, SAMPLED, LOGITS, SKW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kThreads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorNotSupported;
  return LoopOrder::get().run(s, [&](hipEvent_t stop) -> hipError_t {
    // the loop that forms P itself needs only the clears before it
    hipError_t e2 = SKW > 0 ? launch_fill2_u64(q.a->keys, q.a->clear_words, q.a->xpart, (int)q.a->xwords, s)
                            : launch_pre(q, s);
    if (e2 != hipSuccess) return e2;
    hipExtLaunchKernelGGL(kern, dim3(G), dim3(kThreads), lds, s, nullptr, stop, 0, p);
    return hipGetLastError();
  });
}

template <int UHW, int NR, int RK, int SKW>
static hipError_t launch_flags(const Params& p, int G, size_t lds, const PreArgs& q, hipStream_t s) {
  if (p.sampled)
    return p.logits ? launch_t<UHW, NR, RK, true, true, SKW>(p, G, lds, q, s)
                    : launch_t<UHW, NR, RK, true, false, SKW>(p, G, lds, q, s);
  return p.logits ? launch_t<UHW, NR, RK, false, true, SKW>(p, G, lds, q, s)
                  : launch_t<UHW, NR, RK, false, false, SKW>(p, G, lds, q, s);
}

// skw: 64-B steps of a quarter of an LM-head row (0: the base logits are an input)
template <int UHW, int NR, int RK>
static hipError_t launch_skw(const Params& p, int skw, int G, size_t lds, const PreArgs& q, hipStream_t s) {
  switch (skw) {
    case 0: return launch_flags<UHW, NR, RK, 0>(p, G, lds, q, s);
    case kStreamKw4B: return launch_flags<UHW, NR, RK, kStreamKw4B>(p, G, lds, q, s);
    case kStreamKw8B: return launch_flags<UHW, NR, RK, kStreamKw8B>(p, G, lds, q, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace b1

size_t b1_exchange_words(int H, int r, int max_wg) {
  return 2 * ((size_t)max_wg * 2 * 16 + (size_t)H + (size_t)b1::kUnitWGs * r + (size_t)max_wg);
}

namespace b1 {
struct Plan {
  int G, KH, U_hh, ntiles, ut, skw;
  size_t lds;
};

// Host-side checks of the single-block loop; fills the launch plan.
static bool make_plan(const LoopArgs& a, Plan& pl) {
  constexpr int RK = 8;
  if (a.dtype != 1 || a.B != 1 || !a.table) return false;
  if (a.r != RK * 32 || a.H != kUnitWGs * kUnitMax) return false;  // 128 GRU units per unit workgroup
  PSplit pre;  // P arrives as S slices, one per unit workgroup at most
  if (!p_split_shape(a.d, a.r, pre) || pre.S > kUnitWGs) return false;
  pl.G = std::min(a.num_cu, std::min(a.max_wg, 256));
  if (pl.G <= kUnitWGs) return false;
  pl.KH = a.H / 32;
  const int T3 = 3 * a.H / 16;
  const long need = ((long)T3 * pl.KH + (pl.G - kUnitWGs) - 1) / (pl.G - kUnitWGs);  // over the W_hh owners
  pl.U_hh = (int)((need + 2 * kWaves - 1) / (2 * kWaves) * (2 * kWaves));           // UHW even
  if (pl.U_hh != kUHW * kWaves || pl.U_hh > pl.KH) return false;  // a range spans at most two tiles
  pl.ntiles = (a.V + 15) / 16;
  // the unit workgroups take ut tiles each, the others share the rest; every
  // workgroup's tiles must fit its waves' registers
  pl.ut = std::min(kWaves * kNR, pl.ntiles / pl.G);
  // forming the base logits, a unit workgroup also streams its kPRows rows of
  // W1's hidden half (as many bytes as kPRows / 16 LM-head tiles): it takes
  // that many fewer vocabulary tiles
  if (!a.base) pl.ut = std::max(0, pl.ut - kPRows / 16);
  const int rest = pl.ntiles - kUnitWGs * pl.ut;
  const int per_other = (rest + (pl.G - kUnitWGs) - 1) / (pl.G - kUnitWGs);
  if (per_other > kWaves * kNR) return false;
  // no base logits: the kernel forms them (LM-head widths it streams, a block
  // of at most kStreamPositions, a pool the stream's LDS fits in)
  pl.skw = 0;
  if (!a.base) {
    pl.skw = a.d * 2 / kWaves / 64;
    if (!a.lm_head || a.K > kStreamPositions || a.d % (kWaves * 32) != 0 ||
        (pl.skw != kStreamKw4B && pl.skw != kStreamKw8B))
      return false;
    if (lds_layout(pl.U_hh, a.H, a.r, true).ghl < stream_scratch_bytes()) return false;
  }
  pl.lds = (size_t)lds_layout(pl.U_hh, a.H, a.r, pl.skw > 0).total;
  return pl.lds <= 160 * 1024 - 256;
}
}  // namespace b1

bool b1_supported(const LoopArgs& a) {
  b1::Plan pl;
  return b1::make_plan(a, pl);
}

hipError_t launch_draft_b1(const LoopArgs& a, hipStream_t s) {
  using namespace b1;
  constexpr int NR = kNR, RK = 8;
  Plan pl;
  if (!make_plan(a, pl)) return hipErrorNotSupported;
  const int G = pl.G, KH = pl.KH, U_hh = pl.U_hh, ntiles = pl.ntiles, ut = pl.ut;
  Params p{};
  p.d = a.d;
  p.V = a.V;
  p.H = a.H;
  p.r = a.r;
  p.K = a.K;
  p.KH = KH;
  p.U_hh = U_hh;
  p.ntiles = ntiles;
  p.ut = ut;
  p.w_hh = static_cast<const uint16_t*>(a.w_hh);
  p.b_hh = static_cast<const uint16_t*>(a.b_hh);
  p.w1 = static_cast<const uint16_t*>(a.w1);
  p.w2 = static_cast<const uint16_t*>(a.w2);
  p.b2 = static_cast<const uint16_t*>(a.b2);
  p.b1 = static_cast<const uint16_t*>(a.b1);
  p.table = a.table;
  p.base = a.base;
  p.lm_head = static_cast<const uint16_t*>(a.lm_head);
  p.hidden = static_cast<const uint16_t*>(a.hidden);
  p.ppart = a.ppart;
  p.x_t = a.x_t;
  p.teacher = a.teacher;
  p.inv_temp = a.inv_temp;
  p.sampled = a.sampled;
  p.seed = a.seed;
  p.offset = a.offset;
  p.rng_b = a.rng_block;
  p.logits = a.logits;
  p.states = a.states;
  p.tokens = a.tokens;
  p.status = reinterpret_cast<unsigned int*>(a.keys + (size_t)a.K * a.B);
  p.call_status = a.call_status;
  p.spin_limit = a.spin_limit;
  unsigned long long* x = a.xpart;
  p.x_hh = x;
  x += 2 * (size_t)a.max_wg * 2 * 16;
  p.x_g = x;
  x += 2 * (size_t)a.H;
  p.x_pu = x;
  x += 2 * (size_t)kUnitWGs * a.r;
  p.x_key = x;
  PreArgs q{&a, {}};
  if (!p_split_shape(a.d, a.r, q.shape)) return hipErrorNotSupported;
  p.S = q.shape.S;
  return launch_skw<kUHW, NR, RK>(p, pl.skw, G, pl.lds, q, s);
}

}  // namespace domino
