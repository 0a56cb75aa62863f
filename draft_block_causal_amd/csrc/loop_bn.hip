// Draft loop for several blocks per launch (2 to 16) with the head's
// per-position weights held on chip ([notes] §二.1(2) items 1-3;
// [explainer] §四).
//
// Pages: [notes] "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn);
//        [explainer] the yhxrc.cn article on the Domino paper.
//
// One launch of G = #CU workgroups (256 threads, 4 waves, one workgroup per
// compute unit) runs all K positions of up to 16 blocks.  The workgroups take
// one of two roles and keep their weights resident for the whole loop:
//   * kUnitWGs "unit" workgroups, each owning kUnits GRU units: the W_hh rows
//     of those units' three gates in registers, the W1 columns of those units
//     (the GRU half of the first correction projection) in LDS;
//   * the other Gv = G - kUnitWGs "vocabulary" workgroups, each owning a
//     contiguous range of 16-row W2 tiles in registers.
// Matrix-core products take 8 blocks at a time: a block's float32 activation
// row is split into bf16 high and low rows, so 16 operand rows carry 8 blocks.
//
// Per position i (exchanged words are {tag = i + 1, payload}, double-buffered
// by the parity of i; see xchg.h):
//   unit workgroup u
//     A  tokens of position i - 1: the argmax keys of every vocabulary
//        workgroup for every block (x_t at i = 0; teacher tokens if given)
//     B  gates of its units for every block: GRU input row T[token] (the
//        per-head table W_ih E + b_ih), W_hh g_{i-1} + b_hh (formed in F of
//        the previous position) -> g_i (-> states, x_g)
//     D  its share of W1[:, d:] g_i for every block              -> x_pu
//     E  u rows [16u, 16u + 16): the shares of every unit workgroup plus
//        P_i = W1[:, :d] h_i + b1 (K-slice partials written before the loop),
//        SiLU                                                     -> x_u
//     F  W_hh g_i for position i + 1, from every unit workgroup's x_g words
//        (off the token-to-token path: it overlaps the vocabulary phase)
//   vocabulary workgroup
//     P  base logits + b2 of its range for every block at position i (and the
//        Gumbel noise when sampling), staged in LDS while it waits
//     W  u of every block from x_u
//     M  its W2 tiles times u on the matrix cores, 8 blocks per pass; scores;
//        one argmax key per block                                 -> x_key
// The exchanges on the token-to-token path are the key gather (A), the u
// shares (E) and u (W).  Every wait is bounded; a workgroup that gives up
// records it in `status` (and the call's status word), all others leave at
// their next poll, and the tokens are then -1.
//
// The workgroups wait on one another, so all G must be resident at once: the
// host checks that one workgroup fits per compute unit and orders the launch
// after every earlier on-chip loop of the process on the device (LoopOrder).
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include <hip/hip_ext.h>

#include "xchg.h"

namespace domino {
namespace bn {
using namespace xchg;

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
// s_waitcnt with only the vector-memory count limited (expcnt, lgkmcnt at max)
#define DOMINO_BN_WAIT_VM0() __builtin_amdgcn_s_waitcnt(0x0F70)
constexpr int kCoherentLoad = 16;  // cache policy of a global-to-LDS load: sc1, as agent-scope atomic loads

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kUnitWGs = 16;
constexpr int kH = 1024;                    // GRU width this loop takes
constexpr int kUnits = kH / kUnitWGs;       // GRU units per unit workgroup (64)
constexpr int kKH = kH / 32;                // 32-element k-steps of a W_hh row (32)
constexpr int kHhTiles = 3;                 // 16-row W_hh tiles per wave: 3 gates x 64 units / 16 / 4 waves
constexpr int kR = 256;                     // correction rank this loop takes
constexpr int kRK = kR / 32;                // k-steps of a W2 row (8)
constexpr int kNR = 10;                     // W2 tiles per wave of a vocabulary workgroup
constexpr int kMaxEntries = kNR * kWaves * 16;  // vocabulary entries of a vocabulary workgroup (640)
// LDS row stride (floats) of the per-block base-logit and noise tables: M reads
// blocks 2 g and 2 g + 2 in the same half-wave, and a stride of 8 mod 16 puts
// those rows on opposite halves of the 32 banks (640 put them on the same)
constexpr int kCombStride = kMaxEntries + 8;
constexpr int kGroup = 8;                   // blocks per matrix-core pass
constexpr int kMaxB = 16;                   // blocks per launch
constexpr int kUStride = kR + 8;            // u operand rows in LDS, bf16 (528 B: conflict-free 16-B reads)
constexpr int kHhStride = kH + 8;           // g operand rows for W_hh, bf16 (2064 B)
constexpr int kGStride = kUnits + 8;        // g operand rows for the W1 share, bf16 (144 B)
constexpr int kW1Frags = (kR / 16) * (kUnits / 32);  // W1 column fragments of a unit workgroup (32)

// g of two adjacent GRU units in one exchange word: {tag (16 bits), g_a, g_b}
// with each state rounded to its top 24 float32 bits (sign, exponent, 15
// mantissa bits; nearest).  The W_hh products take g as a bf16 high/low pair,
// whose two halves keep 16 significant bits together, and a 24-bit value's
// high and low halves are exact, so the products see the same precision from
// half the bytes: F's gather of every block's g is the largest read of a unit
// workgroup per position.
__device__ __forceinline__ uint32_t round_f24(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7Fu + ((u >> 8) & 1u)) >> 8;  // nearest, ties to even (|g| < 1: no overflow)
}
__device__ __forceinline__ unsigned long long pack_g2(float a, float b, uint32_t tag) {
  return ((unsigned long long)(tag & 0xFFFFu) << 48) | ((unsigned long long)round_f24(a) << 24) | round_f24(b);
}
__device__ __forceinline__ float unpack_g2_a(uint32_t lo, uint32_t hi) {
  return __uint_as_float(((hi & 0xFFFFu) << 16) | ((lo >> 24) << 8));
}
__device__ __forceinline__ float unpack_g2_b(uint32_t lo) { return __uint_as_float((lo & 0xFFFFFFu) << 8); }

struct Params {
  int B, K, V, d, ntiles, S, Gv;
  const uint16_t *w_hh, *b_hh, *w1, *w2, *b2;
  const float* table;   // [V][3H]: W_ih E[v] + b_ih
  const float* base;    // [B][K][V]
  const float* ppart;   // [S][B K][r]: P = W1[:, :d] h + b1 = sum over s of ppart[s] (b1 in s = 0)
  const int32_t *x_t, *teacher;
  float inv_temp;
  uint64_t seed;
  uint32_t offset;
  uint32_t rng_b;  // the first block's index in the sampler's counter
  float *logits, *states;
  int32_t* tokens;
  unsigned int* status;       // this launch's give-up flag
  unsigned int* call_status;  // the call's status word
  unsigned int spin_limit;
  unsigned long long* x_key;  // [2][B][Gv]
  unsigned long long* x_g;    // [2][B][H / 2]: g of two adjacent units per word (pack_g2)
  unsigned long long* x_pu;   // [2][kUnitWGs][B][r]
  unsigned long long* x_u;    // [2][B][r]
};

// LDS layout (bytes) of each role; the launch takes the larger.
struct UnitLds {
  int w1f, ghl, hha, stg, c, g, tok, total;
};
__host__ __device__ inline UnitLds unit_lds(int B) {
  const int ng = (B + kGroup - 1) / kGroup;
  UnitLds L{};
  int off = 0;
  L.w1f = off;
  off += kW1Frags * 64 * 16;  // W1[:, d + units] as matrix-core fragments
  L.ghl = off;
  off += ng * 16 * kGStride * 2;  // g_i of this workgroup's units, per group: 16 rows (block, hi | lo)
  L.hha = off;
  off += 16 * kHhStride * 2;  // g_i of every unit, one group at a time, for W_hh
  L.stg = off;
  off += ng * kGroup * kH * 4;  // the x_g words of every block, as loaded (tagged, two states a word)
  L.c = off;
  off += B * 3 * kUnits * 4;  // W_hh g + b_hh of this workgroup's gate rows [B][3][kUnits]
  L.g = off;
  off += B * kUnits * 4;  // the state of this workgroup's units [B][kUnits]
  L.tok = off;
  off += kMaxB * 4;
  L.total = off;
  return L;
}
struct VocabLds {
  int comb, noise, utile, b2s, total;
};
__host__ __device__ inline VocabLds vocab_lds(int B, bool noise) {
  const int ng = (B + kGroup - 1) / kGroup;
  VocabLds L{};
  int off = 0;
  L.comb = off;
  off += B * kCombStride * 4;  // base + b2 (scaled, + noise when sampling) per block and entry
  L.noise = off;
  off += noise ? B * kCombStride * 4 : 0;  // Gumbel noise kept apart when logits are written too
  L.utile = off;
  off += ng * 16 * kUStride * 2;  // u of every block, per group: 16 rows (block, hi | lo)
  L.b2s = off;
  off += kMaxEntries * 4;
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ unit role
template <int NG>
__device__ void unit_role(const Params& p, unsigned char* smem, bool& ok) {
  constexpr int kNB4 = (NG * kGroup + kWaves - 1) / kWaves;  // blocks per wave in the key gather / gates
  const int u = blockIdx.x;
  const int wave = wave_id();
  const int B = p.B, K = p.K, V = p.V, Gv = p.Gv;
  const int u0 = u * kUnits;
  const UnitLds L = unit_lds(B);
  unsigned char* w1f = smem + L.w1f;
  uint16_t* ghl = reinterpret_cast<uint16_t*>(smem + L.ghl);
  uint16_t* hha = reinterpret_cast<uint16_t*>(smem + L.hha);
  unsigned char* stg = smem + L.stg;
  float* cl = reinterpret_cast<float*>(smem + L.c);
  float* gl = reinterpret_cast<float*>(smem + L.g);
  int* s_tok = reinterpret_cast<int*>(smem + L.tok);

  int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  // ---- resident weights: W_hh rows of this workgroup's gates in registers.
  // Tile t = wave * kHhTiles + tt (of 12): gate q = t / 4, units
  // u0 + (t % 4) * 16 + col; k-step s covers inputs 32 s .. 32 s + 31.
  u32x4 whh[kHhTiles][kKH];
  float bhh[kHhTiles];
#pragma unroll
  for (int tt = 0; tt < kHhTiles; ++tt) {
    const int t = wave * kHhTiles + tt;
    const int row = (t >> 2) * kH + u0 + (t & 3) * 16 + col;
#pragma unroll
    for (int s = 0; s < kKH; ++s) whh[tt][s] = ld16(p.w_hh + (size_t)row * kH + s * 32 + grp * 8);
    bhh[tt] = p.b_hh ? bf16_to_f32(p.b_hh[row]) : 0.f;
  }
  // W1[:, d + u0 .. d + u0 + 63] as fragments (u-row tile rt, k-step ks),
  // straight from memory into LDS (every load of a wave in flight at once):
  // fragment f by wave f % kWaves, lane ln's 16 bytes at w1f + f KB + 16 ln
  for (int f = wave; f < kW1Frags; f += kWaves) {
    const int rt = f >> 1, ks = f & 1;
    __builtin_amdgcn_global_load_lds(
        (gptr_t)(p.w1 + (size_t)(rt * 16 + (lane & 15)) * (p.d + kH) + p.d + u0 + ks * 32 + (lane >> 4) * 8),
        (lptr_t)(w1f + (size_t)f * 1024), 16, 0, 0);
  }
  DOMINO_BN_WAIT_VM0();  // landed before the barrier below publishes them
  // position 0: g_{-1} = 0, so W_hh g + b_hh = b_hh
  for (int j = tid; j < B * 3 * kUnits; j += kThreads) {
    const int q = (j / kUnits) % 3, k = j % kUnits;
    cl[j] = p.b_hh ? bf16_to_f32(p.b_hh[q * kH + u0 + k]) : 0.f;
  }
  for (int j = tid; j < B * kUnits; j += kThreads) gl[j] = 0.f;
  for (int j = tid; j < NG * 16 * kGStride; j += kThreads) ghl[j] = 0;  // rows of absent blocks stay zero
  for (int j = tid; j < 16 * kHhStride; j += kThreads) hha[j] = 0;
  __syncthreads();

  for (int step = 0; step < K; ++step) {
    const uint32_t tag = step + 1;
    const int par = step & 1;
    // the lane's indices re-derived from an opaque copy at every position: the
    // addresses built from them are then recomputed where they are used
    // instead of being kept live (and spilled, with a wait at every reload)
    // across the loop next to the resident W_hh rows
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    grp = lane >> 4;
    col = lane & 15;
    // P_i = W1[:, :d] h_i + b1 for the u rows this workgroup adds up in E
    // (thread: row tid % 16 of blocks tid / 16 + 16 m): it does not depend on
    // the tokens, so its loads are issued before the key polls and are in
    // flight with them (issued after the gather, they added a second memory
    // round trip to every position)
    // The first kPReg slices are loaded into registers of their own (a
    // runtime trip count made the compiler wait for each load before the
    // next); they are added in slice order after the gather, then any further
    // slices (d > 4096) one by one.
    constexpr int kPairs = (NG * kGroup + 15) / 16;
    constexpr int kPReg = 8;
    float pr[kPairs][kPReg];
#pragma unroll
    for (int m = 0; m < kPairs; ++m) {
      const int b = (tid >> 4) + m * 16, row = u * 16 + (tid & 15);
#pragma unroll
      for (int sl = 0; sl < kPReg; ++sl)
        pr[m][sl] = b < B && sl < p.S ? p.ppart[((size_t)sl * B * K + (size_t)b * K + step) * kR + row] : 0.f;
    }
    // ---------- A: tokens of position step - 1 ----------
    if (step == 0) {
      for (int b = tid; b < B; b += kThreads) s_tok[b] = min(max(p.x_t[b], 0), V - 1);
    } else {
      // wave w takes blocks w, w + 4, ...; each lane 4 of the Gv keys of a block
      const unsigned long long* xk = p.x_key + (size_t)(par ^ 1) * B * Gv;
      unsigned long long k[kNB4][4];
#pragma unroll
      for (int m = 0; m < kNB4; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int b = wave + m * kWaves, v = lane + q * 64;
          k[m][q] = b < B && v < Gv ? ld_word(xk + (size_t)b * Gv + v) : 0ull;
        }
      unsigned int spins = 0;
      while (true) {
        bool done = true;
#pragma unroll
        for (int m = 0; m < kNB4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            done &= !(wave + m * kWaves < B && lane + q * 64 < Gv) || key_tagged(k[m][q], step);
        if (done && p.spin_limit != 0u) break;
        if (++spins > p.spin_limit || ((spins & 63u) == 0u && gave_up(p.status))) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int m = 0; m < kNB4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int b = wave + m * kWaves, v = lane + q * 64;
            if (b < B && v < Gv && !key_tagged(k[m][q], step)) k[m][q] = ld_word(xk + (size_t)b * Gv + v);
          }
      }
#pragma unroll
      for (int m = 0; m < kNB4; ++m) {
        const int b = wave + m * kWaves;
        unsigned long long best = 0ull;
#pragma unroll
        for (int q = 0; q < 4; ++q) best = k[m][q] > best ? k[m][q] : best;
        best = wave_max(best);
        if (b < B && lane == 0) {
          const int picked = key_index(best);
          if (u == 0) p.tokens[(size_t)b * K + step - 1] = picked;
          const int tk = p.teacher ? p.teacher[(size_t)b * K + step - 1] : picked;
          s_tok[b] = min(max(tk, 0), V - 1);
        }
      }
    }
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    float pv[kPairs];
#pragma unroll
    for (int m = 0; m < kPairs; ++m) {
      const int b = (tid >> 4) + m * 16, row = u * 16 + (tid & 15);
      float sum = 0.f;
#pragma unroll
      for (int sl = 0; sl < kPReg; ++sl) sum += pr[m][sl];  // slices past S are zero
      if (b < B)
        for (int sl = kPReg; sl < p.S; ++sl) sum += p.ppart[((size_t)sl * B * K + (size_t)b * K + step) * kR + row];
      pv[m] = sum;
    }
    // ---------- B: gates of this workgroup's units (thread: unit lane, blocks wave + 4 m) ----------
    {
      float a3[kNB4][3];
#pragma unroll
      for (int m = 0; m < kNB4; ++m) {
        const int b = wave + m * kWaves;
        const float* trow = p.table + (size_t)s_tok[min(b, B - 1)] * 3 * kH + u0 + lane;
#pragma unroll
        for (int q = 0; q < 3; ++q) a3[m][q] = b < B ? trow[q * kH] : 0.f;
      }
#pragma unroll
      for (int m = 0; m < kNB4; ++m) {
        const int b = wave + m * kWaves;
        if (b < B) {
          const float* c3 = cl + (size_t)b * 3 * kUnits + lane;
          const float rg = sigmoidf_(a3[m][0] + c3[0]);
          const float zg = sigmoidf_(a3[m][1] + c3[kUnits]);
          const float ng = tanhf(a3[m][2] + rg * c3[2 * kUnits]);
          const float g = (1.f - zg) * ng + zg * gl[b * kUnits + lane];
          gl[b * kUnits + lane] = g;
          p.states[((size_t)b * K + step) * kH + u0 + lane] = g;
          // even lanes publish their unit's and the next unit's g in one word
          const float g_next = __shfl_down(g, 1, 64);
          if ((lane & 1) == 0)
            put_word(p.x_g + ((size_t)par * B + b) * (kH / 2) + ((u0 + lane) >> 1), pack_g2(g, g_next, tag));
          uint16_t hi, lo;
          split_bf16(g, hi, lo);
          uint16_t* row = ghl + (size_t)((b >> 3) * 16 + 2 * (b & 7)) * kGStride + lane;
          row[0] = hi;
          row[kGStride] = lo;
        }
      }
    }
    __syncthreads();
    // ---------- D: this workgroup's share of W1[:, d:] g_i, 8 blocks per pass ----------
    // wave w: u-row tiles 4 w .. 4 w + 3
#pragma unroll
    for (int gb = 0; gb < NG; ++gb) {
      if (gb * kGroup < B) {
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        // every operand read is issued before the first product (read one
        // at a time, each product waited out a read's latency)
        u32x4 a[2], wf[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          a[ks] = ld16(reinterpret_cast<const unsigned char*>(ghl) + (size_t)(gb * 16 + col) * kGStride * 2 + ks * 64 +
                       grp * 16);
#pragma unroll
          for (int t = 0; t < 4; ++t) wf[ks][t] = ld16(w1f + ((size_t)((wave * 4 + t) * 2 + ks) * 64 + lane) * 16);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t] = mma16<Bf16>(acc[t], a[ks], wf[ks][t]);
        __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        const int b0 = gb * kGroup + 2 * grp;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = (wave * 4 + t) * 16 + col;
          if (b0 < B) put_f32(p.x_pu + (((size_t)par * kUnitWGs + u) * B + b0) * kR + row, acc[t][0] + acc[t][1], tag);
          if (b0 + 1 < B)
            put_f32(p.x_pu + (((size_t)par * kUnitWGs + u) * B + b0 + 1) * kR + row, acc[t][2] + acc[t][3], tag);
        }
      }
    }
    // ---------- E: u rows [16 u, 16 u + 16) of every block ----------
    // thread: row c = tid % 16 for blocks tid / 16 + 16 m (P loaded before B)
    {
      const int c = tid & 15, bb = tid >> 4;
      const int row = u * 16 + c;
      unsigned long long x[kPairs * kUnitWGs];
#pragma unroll
      for (int m = 0; m < kPairs; ++m)
#pragma unroll
        for (int o = 0; o < kUnitWGs; ++o) {
          const int b = bb + m * 16;
          x[m * kUnitWGs + o] = b < B ? ld_word(p.x_pu + (((size_t)par * kUnitWGs + o) * B + b) * kR + row) : 0ull;
        }
      unsigned int spins = 0;
      while (true) {
        bool done = true;
#pragma unroll
        for (int m = 0; m < kPairs; ++m)
#pragma unroll
          for (int o = 0; o < kUnitWGs; ++o)
            done &= bb + m * 16 >= B || (uint32_t)(x[m * kUnitWGs + o] >> 32) == tag;
        if (done && p.spin_limit != 0u) break;
        if (++spins > p.spin_limit || ((spins & 63u) == 0u && gave_up(p.status))) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int m = 0; m < kPairs; ++m)
#pragma unroll
          for (int o = 0; o < kUnitWGs; ++o) {
            const int b = bb + m * 16;
            if (b < B && (uint32_t)(x[m * kUnitWGs + o] >> 32) != tag)
              x[m * kUnitWGs + o] = ld_word(p.x_pu + (((size_t)par * kUnitWGs + o) * B + b) * kR + row);
          }
      }
      if (ok) {
#pragma unroll
        for (int m = 0; m < kPairs; ++m) {
          const int b = bb + m * 16;
          float s = pv[m];
#pragma unroll
          for (int o = 0; o < kUnitWGs; ++o) s += word_f32(x[m * kUnitWGs + o]);
          if (b < B) put_f32(p.x_u + ((size_t)par * B + b) * kR + row, s * sigmoidf_(s), tag);
        }
      }
    }
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    // ---------- F: W_hh g_i + b_hh for position step + 1, 8 blocks per pass ----------
    if (step + 1 < K) {
      // every block's x_g words straight into LDS at once (no registers): 1 KB
      // chunks, chunk j = block j / 4, words (j % 4) 128 .. + 127; wave w
      // loads chunks NG 8 w .. NG 8 w + NG 8 - 1 and loads again any chunk
      // that still holds a word without this position's tag
      constexpr int kCh = NG * 8;  // chunks per wave
      const unsigned long long* xg = p.x_g + (size_t)par * B * (kH / 2);
      unsigned int pending = 0;  // bit c: chunk kCh wave + c still to check
#pragma unroll
      for (int c = 0; c < kCh; ++c) {
        const int j = wave * kCh + c;
        if ((j >> 2) < B) {
          __builtin_amdgcn_global_load_lds((gptr_t)(xg + (size_t)j * 128 + lane * 2), (lptr_t)(stg + j * 1024), 16, 0,
                                           kCoherentLoad);
          pending |= 1u << c;
        }
      }
      unsigned int spins = 0;
      while (true) {
        DOMINO_BN_WAIT_VM0();
        unsigned int missing = 0;
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
          if (pending & (1u << c)) {
            const u32x4 w = ld16(stg + (wave * kCh + c) * 1024 + lane * 16);
            const bool bad = (w[1] >> 16) != (tag & 0xFFFFu) || (w[3] >> 16) != (tag & 0xFFFFu);
            if (__builtin_amdgcn_ballot_w64(bad) != 0ull) missing |= 1u << c;
          }
        }
        pending = missing;
        if (pending == 0u && p.spin_limit != 0u) break;
        if (++spins > p.spin_limit || ((spins & 63u) == 0u && gave_up(p.status))) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
          const int j = wave * kCh + c;
          if (pending & (1u << c))
            __builtin_amdgcn_global_load_lds((gptr_t)(xg + (size_t)j * 128 + lane * 2), (lptr_t)(stg + j * 1024), 16, 0,
                                             kCoherentLoad);
        }
      }
      if (__syncthreads_or(!ok)) {
        ok = false;
        break;
      }
#pragma unroll
      for (int gb = 0; gb < NG; ++gb) {
        if (gb * kGroup < B) {
          const int nb = min(kGroup, B - gb * kGroup);
          // float32 -> bf16 high and low rows: thread takes inputs 4 tid .. 4 tid + 3
#pragma unroll
          for (int bl = 0; bl < kGroup; ++bl) {
            if (bl < nb) {
              // words 2 tid, 2 tid + 1 of the block: units 4 tid .. 4 tid + 3
              const u32x4 w = ld16(stg + (size_t)(gb * kGroup + bl) * kH * 4 + tid * 16);
              const float x[4] = {unpack_g2_a(w[0], w[1]), unpack_g2_b(w[0]), unpack_g2_a(w[2], w[3]),
                                  unpack_g2_b(w[2])};
              uint16_t hi[4], lo[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) split_bf16(x[e], hi[e], lo[e]);
              uint16_t* rh = hha + (size_t)(2 * bl) * kHhStride + tid * 4;
              *reinterpret_cast<uint2*>(rh) = uint2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
              *reinterpret_cast<uint2*>(rh + kHhStride) =
                  uint2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
            }
          }
          __syncthreads();
          f32x4 acc[kHhTiles];
#pragma unroll
          for (int tt = 0; tt < kHhTiles; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
          auto rd = [&](int s) {
            return ld16(reinterpret_cast<const unsigned char*>(hha) + (size_t)col * kHhStride * 2 + s * 64 + grp * 16);
          };
          if constexpr (NG > 1) {
            // two groups: the state operand of k-step s + 3 is read while
            // step s is multiplied (order pinned by scheduling barriers;
            // 16 blocks: draft call 0.738 -> 0.724 ms; with one group the
            // pinned order measured slower, 0.552 -> 0.559 ms at 8 blocks)
            constexpr int kAhead = 3;
            u32x4 a[kKH];
#pragma unroll
            for (int s = 0; s < kAhead; ++s) a[s] = rd(s);
#pragma unroll
            for (int s = 0; s < kKH; ++s) {
              if (s + kAhead < kKH) a[s + kAhead] = rd(s + kAhead);
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int tt = 0; tt < kHhTiles; ++tt) acc[tt] = mma16<Bf16>(acc[tt], a[s], whh[tt][s]);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
            for (int s = 0; s < kKH; ++s) {
              const u32x4 a = rd(s);
#pragma unroll
              for (int tt = 0; tt < kHhTiles; ++tt) acc[tt] = mma16<Bf16>(acc[tt], a, whh[tt][s]);
            }
          }
          const int b0 = gb * kGroup + 2 * grp;
#pragma unroll
          for (int tt = 0; tt < kHhTiles; ++tt) {
            const int t = wave * kHhTiles + tt;
            const int q = t >> 2, j = (t & 3) * 16 + col;
            if (b0 < B) cl[((size_t)b0 * 3 + q) * kUnits + j] = acc[tt][0] + acc[tt][1] + bhh[tt];
            if (b0 + 1 < B) cl[((size_t)(b0 + 1) * 3 + q) * kUnits + j] = acc[tt][2] + acc[tt][3] + bhh[tt];
          }
          __syncthreads();  // hha is refilled by the next group
        }
      }
    }
  }

  if (ok && u == 0) {  // the tokens of the last position
    const int step = K;
    const unsigned long long* xk = p.x_key + (size_t)((K - 1) & 1) * B * Gv;
    for (int b = wave; b < B && ok; b += kWaves) {
      unsigned long long k[4];
      const unsigned long long* src[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        src[q] = lane + q * 64 < Gv ? xk + (size_t)b * Gv + lane + q * 64 : nullptr;
        k[q] = src[q] ? ld_word(src[q]) : 0ull;
      }
      unsigned int spins = 0;
      while (true) {
        bool done = true;
#pragma unroll
        for (int q = 0; q < 4; ++q) done &= !src[q] || key_tagged(k[q], step);
        if (done && p.spin_limit != 0u) break;
        if (++spins > p.spin_limit || ((spins & 63u) == 0u && gave_up(p.status))) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (src[q] && !key_tagged(k[q], step)) k[q] = ld_word(src[q]);
      }
      unsigned long long best = 0ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) best = k[q] > best ? k[q] : best;
      best = wave_max(best);
      if (ok && lane == 0) p.tokens[(size_t)b * K + K - 1] = key_index(best);
    }
  }
}

// ------------------------------------------------------------ vocabulary role
template <int NG, bool SAMPLED, bool LOGITS>
__device__ void vocab_role(const Params& p, unsigned char* smem, bool& ok) {
  __shared__ unsigned long long s_key[kWaves][kGroup];
  const int vw = blockIdx.x - kUnitWGs;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int B = p.B, K = p.K, V = p.V, Gv = p.Gv;
  constexpr bool kNoise = SAMPLED && LOGITS;
  const VocabLds L = vocab_lds(B, kNoise);
  float* comb = reinterpret_cast<float*>(smem + L.comb);
  float* noise = reinterpret_cast<float*>(smem + L.noise);
  unsigned char* utile = smem + L.utile;
  float* b2s = reinterpret_cast<float*>(smem + L.b2s);
  const int t_lo = (int)((long)vw * p.ntiles / Gv), t_hi = (int)((long)(vw + 1) * p.ntiles / Gv);
  const int nt = t_hi - t_lo;
  const int nv = nt * 16;
  const int v0 = t_lo * 16;

  // ---- resident weights: W2 tiles s * kWaves + wave of the range, 8 k-step fragments each
  u32x4 w2r[kNR][kRK];
#pragma unroll
  for (int s = 0; s < kNR; ++s) {
    const int j = s * kWaves + wave;
    const int v = min((t_lo + j) * 16 + col, V - 1);
#pragma unroll
    for (int k = 0; k < kRK; ++k)
      w2r[s][k] = j < nt ? ld16(p.w2 + (size_t)v * kR + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
  }
  for (int e = tid; e < kMaxEntries; e += kThreads) b2s[e] = e < nv && v0 + e < V && p.b2 ? bf16_to_f32(p.b2[v0 + e]) : 0.f;
  // slots past the range (or the vocabulary) never win: their combined bias is -inf
  for (int j = tid; j < B * kCombStride; j += kThreads) {
    comb[j] = -INFINITY;
    if (kNoise) noise[j] = 0.f;
  }
  for (int j = tid; j < NG * 16 * kUStride; j += kThreads) reinterpret_cast<uint16_t*>(utile)[j] = 0;
  __syncthreads();

  for (int step = 0; step < K; ++step) {
    const uint32_t tag = step + 1;
    const int par = step & 1;
    // ---------- P: base + b2 (+ noise) of the range at this position ----------
    // thread: 4 consecutive entries (one Philox block) of one block
    {
      const int quads = nv >> 2;
      for (int j = tid; j < B * quads; j += kThreads) {
        const int b = j / quads, e = (j - b * quads) * 4;
        const float* brow = p.base + ((size_t)b * K + step) * V + v0 + e;
        float lb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) lb[q] = v0 + e + q < V ? brow[q] : 0.f;
        u32x4 words = {0u, 0u, 0u, 0u};
        if constexpr (SAMPLED) words = philox4(p.seed, p.offset, p.rng_b + (uint32_t)b, (uint32_t)step, (uint32_t)((v0 + e) >> 2));
        // one 16-B store per thread and table (four 4-B stores 16 B apart
        // would put lanes l, l + 8, l + 16, l + 24 on one bank)
        f32x4 cv, nv4 = {0.f, 0.f, 0.f, 0.f};
        const f32x4 b2v = *reinterpret_cast<const f32x4*>(b2s + e);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool live = v0 + e + q < V;
          const float x = lb[q] + b2v[q];
          if constexpr (!SAMPLED) {
            cv[q] = live ? x : -INFINITY;
          } else if constexpr (kNoise) {
            cv[q] = live ? x : -INFINITY;
            nv4[q] = gumbel_from_word(words[q]);
          } else {
            cv[q] = live ? x * p.inv_temp + gumbel_from_word(words[q]) : -INFINITY;
          }
        }
        *reinterpret_cast<f32x4*>(comb + (size_t)b * kCombStride + e) = cv;
        if constexpr (kNoise) *reinterpret_cast<f32x4*>(noise + (size_t)b * kCombStride + e) = nv4;
      }
    }
    // ---------- W: u of every block ----------
    if (wave == 0)
      ok &= wait_sentinels(p.x_u + ((size_t)par * B + B - 1) * kR + 15, kUnitWGs, 16, tag, p.status, p.spin_limit);
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    {
      // thread: u entry tid (r = kThreads) of every block
      unsigned long long x[NG * kGroup];
      const unsigned long long* src = p.x_u + (size_t)par * B * kR + tid;
#pragma unroll
      for (int b = 0; b < NG * kGroup; ++b) x[b] = b < B ? ld_word(src + (size_t)b * kR) : 0ull;
      ok &= settle_strided(src, kR, B, tag, p.status, p.spin_limit, x);
#pragma unroll
      for (int b = 0; b < NG * kGroup; ++b) {
        if (b < B) {
          uint16_t hi, lo;
          split_bf16(word_f32(x[b]), hi, lo);
          uint16_t* row = reinterpret_cast<uint16_t*>(utile) + (size_t)((b >> 3) * 16 + 2 * (b & 7)) * kUStride + tid;
          row[0] = hi;
          row[kUStride] = lo;
        }
      }
    }
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    // ---------- M: W2 tiles x u, 8 blocks per pass; scores; keys ----------
#pragma unroll
    for (int gb = 0; gb < NG; ++gb) {
      if (gb * kGroup < B) {
        u32x4 ua[kRK];
#pragma unroll
        for (int k = 0; k < kRK; ++k)
          ua[k] = ld16(utile + (size_t)(gb * 16 + col) * kUStride * 2 + k * 64 + grp * 16);
        f32x4 acc[kNR];
#pragma unroll
        for (int s = 0; s < kNR; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kRK; ++k)
#pragma unroll
          for (int s = 0; s < kNR; ++s) acc[s] = mma16<Bf16>(acc[s], ua[k], w2r[s][k]);
        // lanes of row group grp hold blocks b0 = 2 grp and b0 + 1 of the pass
        const int b0 = gb * kGroup + 2 * grp;
        const int c0 = min(b0, B - 1), c1 = min(b0 + 1, B - 1);
        unsigned long long best0 = 0ull, best1 = 0ull;
#pragma unroll
        for (int s = 0; s < kNR; ++s) {
          int e = (s * kWaves + wave) * 16 + col;
          asm volatile("" : "+v"(e));  // keeps per-tile constants inside the position loop
          const uint32_t v = (uint32_t)(v0 + e);
          const float d0 = acc[s][0] + acc[s][1], d1 = acc[s][2] + acc[s][3];
          const float x0 = comb[(size_t)c0 * kCombStride + e], x1 = comb[(size_t)c1 * kCombStride + e];
          float s0, s1;
          if constexpr (!SAMPLED) {
            s0 = d0 + x0;
            s1 = d1 + x1;
          } else if constexpr (kNoise) {
            s0 = (d0 + x0) * p.inv_temp + noise[(size_t)c0 * kCombStride + e];
            s1 = (d1 + x1) * p.inv_temp + noise[(size_t)c1 * kCombStride + e];
          } else {
            s0 = d0 * p.inv_temp + x0;
            s1 = d1 * p.inv_temp + x1;
          }
          if constexpr (LOGITS) {
            if (e < nv && (int)v < V) {
              if (b0 < B) p.logits[((size_t)b0 * K + step) * V + v] = d0 + x0;
              if (b0 + 1 < B) p.logits[((size_t)(b0 + 1) * K + step) * V + v] = d1 + x1;
            }
          }
          const unsigned long long k0 = tagged_key(s0, v, tag), k1 = tagged_key(s1, v, tag);
          best0 = k0 > best0 ? k0 : best0;
          best1 = k1 > best1 ? k1 : best1;
        }
        best0 = row_max16(best0);
        best1 = row_max16(best1);
        if (col == 0) {
          s_key[wave][2 * grp] = best0;
          s_key[wave][2 * grp + 1] = best1;
        }
        __syncthreads();
        if (tid < kGroup && gb * kGroup + tid < B) {
          unsigned long long k = s_key[0][tid];
#pragma unroll
          for (int wv = 1; wv < kWaves; ++wv) k = s_key[wv][tid] > k ? s_key[wv][tid] : k;
          put_word(p.x_key + ((size_t)par * B + gb * kGroup + tid) * Gv + vw, k);
        }
        __syncthreads();  // s_key is reused by the next pass
      }
    }
  }
}

template <int NG, bool SAMPLED, bool LOGITS>
__global__ void __launch_bounds__(kThreads, 1) draft_bn_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bool ok = true;
  if ((int)blockIdx.x < kUnitWGs)
    unit_role<NG>(p, smem, ok);
  else
    vocab_role<NG, SAMPLED, LOGITS>(p, smem, ok);
  if (!ok) {
    if (threadIdx.x == 0) {
      atomicOr(p.status, 1u);
      atomicOr(p.call_status, 1u);
    }
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < p.B * p.K; i += kThreads) p.tokens[i] = -1;
  }
}

// Words of the exchange region for B blocks with Gv vocabulary workgroups.
inline size_t exchange_words(int B, int Gv) {
  return 2 * (size_t)B * ((size_t)Gv + kH / 2 + (size_t)kUnitWGs * kR + kR);
}

template <int NG, bool SAMPLED, bool LOGITS>
static hipError_t launch_t(const Params& p, int G, size_t lds, const LoopArgs& a, const PSplit& ps,
                           const void* hidden, int clear_words, size_t xwords, hipStream_t s) {
  auto kern = draft_bn_kernel<NG, SAMPLED, LOGITS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kThreads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorNotSupported;
  return LoopOrder::get().run(s, [&](hipEvent_t stop) -> hipError_t {
    // before the loop: the key region's words that must start at zero (this
    // launch's status word, and for the first launch of a call the call's
    // status word), the exchange words, and P as K-slice partials
    hipError_t e2 = launch_p_partials(hidden, p.B * p.K, a.d, a.w1, a.d + kH, kR, a.b1, a.ppart, ps, a.keys,
                                      clear_words, a.xpart, (int)xwords, s);
    if (e2 != hipSuccess) return e2;
    hipExtLaunchKernelGGL(kern, dim3(G), dim3(kThreads), lds, s, nullptr, stop, 0, p);
    return hipGetLastError();
  });
}

template <bool SAMPLED, bool LOGITS>
static hipError_t launch_ng(int ng, const Params& p, int G, size_t lds, const LoopArgs& a, const PSplit& ps,
                            const void* hidden, int clear_words, size_t xwords, hipStream_t s) {
  switch (ng) {
    case 1: return launch_t<1, SAMPLED, LOGITS>(p, G, lds, a, ps, hidden, clear_words, xwords, s);
    case 2: return launch_t<2, SAMPLED, LOGITS>(p, G, lds, a, ps, hidden, clear_words, xwords, s);
    default: return hipErrorNotSupported;
  }
}

// Blocks per launch: at most kMaxB; the launches of a call are about equal.
inline int chunk_blocks(const LoopArgs& a) {
  const int cap = kMaxB;
  const int n = (a.B + cap - 1) / cap;
  return (a.B + n - 1) / n;
}

inline int vocab_wgs(const LoopArgs& a) { return std::min(a.num_cu, std::min(a.max_wg, 256)) - kUnitWGs; }

}  // namespace bn

size_t bn_exchange_words(int batch, int max_wg, int H, int r) {
  if (H != bn::kH || r != bn::kR || batch < 2) return 0;
  return bn::exchange_words(std::min(batch, bn::kMaxB), max_wg - bn::kUnitWGs);
}

// Host-side checks of the several-block loop (no HIP call).
bool bn_supported(const LoopArgs& a) {
  using namespace bn;
  if (a.dtype != 1 || a.B < 2 || !a.table) return false;
  if (a.H != kH || a.r != kR) return false;
  PSplit ps;
  if (!p_split_shape(a.d, a.r, ps)) return false;
  const int Gv = vocab_wgs(a);
  if (Gv < 1) return false;
  const int ntiles = (a.V + 15) / 16;
  if ((ntiles + Gv - 1) / Gv > kNR * kWaves) return false;  // every range fits its waves' registers
  const int bc = chunk_blocks(a);
  const size_t lds = std::max((size_t)unit_lds(bc).total, (size_t)vocab_lds(bc, a.sampled && a.logits).total);
  if (lds > 160 * 1024 - 512) return false;
  return exchange_words(bc, Gv) <= a.xwords;
}

hipError_t launch_draft_bn(const LoopArgs& a, hipStream_t s) {
  using namespace bn;
  if (!bn_supported(a)) return hipErrorNotSupported;
  PSplit ps;
  p_split_shape(a.d, a.r, ps);
  const int G = std::min(a.num_cu, std::min(a.max_wg, 256));
  const int Gv = G - kUnitWGs;
  const int bc = chunk_blocks(a);
  const bool noise = a.sampled && a.logits;
  for (int c0 = 0; c0 < a.B; c0 += bc) {
    const int nb = std::min(bc, a.B - c0);
    const size_t K = (size_t)a.K;
    Params p{};
    p.B = nb;
    p.K = a.K;
    p.V = a.V;
    p.d = a.d;
    p.ntiles = (a.V + 15) / 16;
    p.S = ps.S;
    p.Gv = Gv;
    p.w_hh = static_cast<const uint16_t*>(a.w_hh);
    p.b_hh = static_cast<const uint16_t*>(a.b_hh);
    p.w1 = static_cast<const uint16_t*>(a.w1);
    p.w2 = static_cast<const uint16_t*>(a.w2);
    p.b2 = static_cast<const uint16_t*>(a.b2);
    p.table = a.table;
    p.base = a.base + c0 * K * a.V;
    p.ppart = a.ppart;
    p.x_t = a.x_t + c0;
    p.teacher = a.teacher ? a.teacher + c0 * K : nullptr;
    p.inv_temp = a.inv_temp;
    p.seed = a.seed;
    p.offset = a.offset;
    p.rng_b = a.rng_block + (uint32_t)c0;
    p.logits = a.logits ? a.logits + c0 * K * a.V : nullptr;
    p.states = a.states + c0 * K * a.H;
    p.tokens = a.tokens + c0 * K;
    p.status = reinterpret_cast<unsigned int*>(a.keys);
    p.call_status = a.call_status;
    p.spin_limit = a.spin_limit;
    const size_t xw = exchange_words(nb, Gv);
    unsigned long long* x = a.xpart;
    p.x_key = x;
    x += 2 * (size_t)nb * Gv;
    p.x_g = x;
    x += 2 * (size_t)nb * (kH / 2);
    p.x_pu = x;
    x += 2 * (size_t)kUnitWGs * nb * kR;
    p.x_u = x;
    const size_t lds = std::max((size_t)unit_lds(nb).total, (size_t)vocab_lds(nb, noise).total);
    // the first launch clears the whole key region (the call's status word
    // included); later ones only this launch's status word
    const int clear = c0 == 0 ? a.clear_words : 1;
    const void* hidden = static_cast<const uint16_t*>(a.hidden) + c0 * K * a.d;
    const int ng = (nb + kGroup - 1) / kGroup;
    hipError_t e;
    if (a.sampled)
      e = a.logits ? launch_ng<true, true>(ng, p, G, lds, a, ps, hidden, clear, xw, s)
                   : launch_ng<true, false>(ng, p, G, lds, a, ps, hidden, clear, xw, s);
    else
      e = a.logits ? launch_ng<false, true>(ng, p, G, lds, a, ps, hidden, clear, xw, s)
                   : launch_ng<false, false>(ng, p, G, lds, a, ps, hidden, clear, xw, s);
    if (e != hipSuccess) return e == hipErrorNotSupported && c0 > 0 ? hipErrorUnknown : e;
  }
  return hipSuccess;
}

}  // namespace domino
