// Single-block (B = 1) draft loop with the head's per-position weights held
// on chip ([notes] §二.1(2) items 1-3; [explainer] §四).
//
// Pages: [notes] "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn);
//        [explainer] the yhxrc.cn article on the Domino paper.
//
// One cooperative launch of G = #CU workgroups (512 threads, 8 waves each)
// runs the whole K-position loop.  Re-reading W2 and W_hh from HBM at every
// position would cost ~85 MB per position; each workgroup instead loads its
// share once and keeps it resident:
//   * W2:   a contiguous range of 16-row vocabulary tiles, NR per wave in
//           registers and the rest in LDS;
//   * W_hh: a contiguous range of U_hh "k-steps" (16 gate rows x 32 inputs)
//           of the stacked [3H, H] matrix, in registers;
//   * W1[:, d:] (the GRU half of the first correction projection): the
//           kUnitWGs "unit" workgroups hold the columns of their H / kUnitWGs
//           GRU units in LDS, in place of some of their W2 tiles.
// The GRU input term W_ih e(y) + b_ih is read from the per-head table
// T[y] = W_ih E[y] + b_ih (domino_prepare_gru_table): one row gather per
// position instead of a 25 MB matrix-vector product.
//
// Per position i (every exchanged word is {tag = i + 1, payload}, written and
// polled with relaxed agent-scope atomics, double-buffered by the parity of i):
//   A. every workgroup: W_hh g_{i-1} partials of its k-range         -> x_hh
//   B. unit workgroups: y_{i-1} from the G argmax keys, T[y_{i-1}] for their
//      units, gates, new state (-> states, x_g), their share of
//      W1[:, d:] g                                                    -> x_pu
//   C. every workgroup: u = SiLU(P_i + sum of the shares), its W2 tiles on the
//      matrix cores, + b2 + base logits (+ Gumbel), argmax            -> x_key
// Every wait is bounded: a workgroup that gives up records it in `status`
// and all others leave at their next poll; the tokens are then -1.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace domino {
namespace b1 {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kUnitWGs = 8;
constexpr int kUnitMax = 128;  // GRU units per unit workgroup (H <= 1024)
constexpr unsigned int kSpinLimit = 1u << 20;

struct Params {
  int d, V, H, r, K;
  int KH;      // 32-element k-steps per W_hh row: H / 32
  int U_hh;    // W_hh k-steps per workgroup (multiple of kWaves)
  int ntiles;  // ceil(V / 16)
  int nl;      // W2 tiles kept in LDS by an ordinary workgroup
  int nl_unit; // ... by a unit workgroup (the rest of its LDS pool holds its W1 columns)
  int ut;      // W2 tiles of a unit workgroup (the others share the remainder evenly)
  const uint16_t *w_hh, *b_hh, *w1, *w2, *b2;
  const float* table;     // [V][3H]: W_ih E[v] + b_ih
  const float *base, *P;  // base [K][V], P [K][r] (includes b1)
  const int32_t *x_t, *teacher;
  float inv_temp;
  int sampled;
  uint64_t seed;
  uint32_t offset;
  float *logits, *states;
  int32_t* tokens;
  unsigned int* status;
  unsigned long long* x_hh;   // [2][G][2 segments][16]
  unsigned long long* x_g;    // [2][H]
  unsigned long long* x_pu;   // [2][kUnitWGs][r]
  unsigned long long* x_key;  // [2][G]
};

__device__ __forceinline__ unsigned long long ld_word(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_word(unsigned long long* p, unsigned long long w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_f32(unsigned long long* p, float v, uint32_t tag) {
  put_word(p, ((unsigned long long)tag << 32) | __float_as_uint(v));
}
__device__ __forceinline__ bool gave_up(const unsigned int* status) {
  return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Polls *p until it carries `tag` in its high word (bounded); w is the last value read.
__device__ __forceinline__ bool settle(const unsigned long long* p, uint32_t tag, const unsigned int* status,
                                      unsigned long long& w) {
  unsigned int spins = 0;
  while ((uint32_t)(w >> 32) != tag) {
    if (++spins > kSpinLimit || ((spins & 63u) == 0u && gave_up(status))) return false;
    __builtin_amdgcn_s_sleep(1);
    w = ld_word(p);
  }
  return true;
}

// Argmax key carrying the position tag: score (32) | tag (8) | 0xFFFFFF - v (24).
__device__ __forceinline__ unsigned long long b1_key(float s, uint32_t v, uint32_t tag) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | ((unsigned long long)(tag & 0xFFu) << 24) |
         (unsigned long long)(0xFFFFFFu - v);
}
__device__ __forceinline__ bool key_tagged(unsigned long long k, uint32_t tag) {
  return k != 0ull && ((uint32_t)(k >> 24) & 0xFFu) == (tag & 0xFFu);
}
__device__ __forceinline__ int key_index(unsigned long long k) { return (int)(0xFFFFFFu - (uint32_t)(k & 0xFFFFFFull)); }

// Max over the G keys published for one position, on one wave; every load of a
// lane is in flight before the first is checked.
__device__ __forceinline__ bool gather_keys(const unsigned long long* keys, int G, uint32_t tag,
                                            const unsigned int* status, unsigned long long& best) {
  constexpr int kMaxPer = 4;  // G <= 256
  const int lane = threadIdx.x & 63;
  unsigned long long k[kMaxPer];
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) k[q] = lane + q * 64 < G ? ld_word(keys + lane + q * 64) : 0ull;
  bool ok = true;
  best = 0ull;
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    if (lane + q * 64 < G) {
      unsigned int spins = 0;
      while (!key_tagged(k[q], tag)) {
        if (++spins > kSpinLimit || ((spins & 63u) == 0u && gave_up(status))) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        k[q] = ld_word(keys + lane + q * 64);
      }
      best = k[q] > best ? k[q] : best;
    }
  }
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const unsigned long long o = __shfl_xor(best, sh, 64);
    best = o > best ? o : best;
  }
  return ok;
}

// The o-th W_hh partial of gate row `row` (workgroups whose k-step range covers
// the row's tile, each holding it in segment 0 (its first tile) or 1), or
// nullptr when the tile has fewer owners.
__device__ __forceinline__ const unsigned long long* hh_partial(const Params& p, int row, int o, int par, int G) {
  const int t = row >> 4, c = row & 15;
  const int lo = (t * p.KH) / p.U_hh, hi = (t * p.KH + p.KH - 1) / p.U_hh;
  const int ow = lo + o;
  if (ow > hi) return nullptr;
  const int seg = ((ow * p.U_hh) / p.KH == t) ? 0 : 1;
  return p.x_hh + (((size_t)par * G + ow) * 2 + seg) * 16 + c;
}

// L_i[v] = base + (W2 u)[v] + b2[v] for the lane's vocabulary entry (row 0 of
// the accumulator); returns the running argmax key.
__device__ __forceinline__ unsigned long long tile_epilogue(const Params& p, float dl, int v, int step, uint32_t tag,
                                                            float lbv, float bbv, unsigned long long best) {
  if (v < p.V) {
    const float Lv = lbv + (dl + bbv);
    if (p.logits) p.logits[(size_t)step * p.V + v] = Lv;
    float sc = Lv;
    if (p.sampled) sc = Lv * p.inv_temp + gumbel_from_word(philox_word(p.seed, p.offset, 0u, step, v));
    const unsigned long long k = b1_key(sc, v, tag);
    best = k > best ? k : best;
  }
  return best;
}

struct Lds {
  int w2l, w1u, gst, utile, pu, gs_new, gs_prev, red, total;
};

// The W2 pool is shared: ordinary workgroups keep nl tiles there; unit
// workgroups keep nl_unit tiles followed by their W1 columns (r x units bf16).
__host__ __device__ inline Lds lds_layout(int nl, int nl_unit, int RK, int H, int r) {
  Lds L{};
  int off = 0;
  L.w2l = off;
  L.w1u = nl_unit * RK * 1024;
  const int unit_pool = L.w1u + r * (H / kUnitWGs) * 2;
  const int pool = nl * RK * 1024;
  off += pool > unit_pool ? pool : unit_pool;
  L.gst = off;
  off += H * 4;
  L.utile = off;
  off += r * 4;  // hi then lo, r bf16 each
  L.pu = off;
  off += 2 * r * 4;
  L.gs_new = off;
  off += kUnitMax * 4;
  L.gs_prev = off;
  off += kUnitMax * 4;
  L.red = off;
  off += kWaves * 2 * 16 * 4;
  L.total = off;
  return L;
}

template <int UHW, int NR, int RK>
__global__ void __launch_bounds__(kThreads, 1) draft_b1_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ unsigned long long s_key[kWaves];
  __shared__ int s_tok;
  const int w = blockIdx.x, G = gridDim.x;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int H = p.H, V = p.V, r = p.r;
  const int T3 = (3 * H) >> 4;
  const Lds L = lds_layout(p.nl, p.nl_unit, RK, H, r);
  unsigned char* w2l = smem + L.w2l;
  const uint16_t* w1u = reinterpret_cast<const uint16_t*>(smem + L.w1u);
  float* gst = reinterpret_cast<float*>(smem + L.gst);
  uint16_t* utile = reinterpret_cast<uint16_t*>(smem + L.utile);
  float* pu = reinterpret_cast<float*>(smem + L.pu);
  float* gs_new = reinterpret_cast<float*>(smem + L.gs_new);
  float* gs_prev = reinterpret_cast<float*>(smem + L.gs_prev);
  float* red = reinterpret_cast<float*>(smem + L.red);
  const int units = H / kUnitWGs;
  const bool unit_wg = w < kUnitWGs;
  constexpr int kLdsSlots = 2;  // LDS W2 tiles a wave can own: nl <= kLdsSlots * kWaves
  const int my_nl = unit_wg ? p.nl_unit : p.nl;

  // ---------------- resident weights ----------------
  const long total_hh = (long)T3 * p.KH, hh0 = (long)w * p.U_hh;
  u32x4 whh[UHW];
#pragma unroll
  for (int q = 0; q < UHW; ++q) {
    const long gu = hh0 + wave * UHW + q;
    whh[q] = u32x4{0, 0, 0, 0};
    if (gu < total_hh) {
      const int t = (int)(gu / p.KH), s = (int)(gu % p.KH);
      whh[q] = ld16(p.w_hh + (size_t)(t * 16 + col) * H + s * 32 + grp * 8);
    }
  }
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
  u32x4 w2r[NR][RK];
#pragma unroll
  for (int s = 0; s < NR; ++s) {
    const int j = s * kWaves + wave;
    const int v = min((t_lo + j) * 16 + col, V - 1);
#pragma unroll
    for (int k = 0; k < RK; ++k)
      w2r[s][k] = j < nt ? ld16(p.w2 + (size_t)v * r + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
  }
  for (int j = tid; j < my_nl * RK * 64; j += kThreads) {
    const int l = j / (RK * 64), k = (j / 64) % RK, ln = j & 63;
    const int lt = kWaves * NR + l;
    u32x4 v = {0, 0, 0, 0};
    if (lt < nt) {
      const int vv = min((t_lo + lt) * 16 + (ln & 15), V - 1);
      v = ld16(p.w2 + (size_t)vv * r + k * 32 + (ln >> 4) * 8);
    }
    st16(w2l + ((size_t)l * RK + k) * 1024 + ln * 16, v);
  }
  // unit workgroups: W1[:, d + w*units : d + (w+1)*units] as [r][units] bf16 in LDS
  const int urow = tid % r, uhalf = tid / r;
  const int half_units = units / 2;
  if (unit_wg) {
    const int chunks = units / 8;
    for (int j = tid; j < r * chunks; j += kThreads) {
      const int row = j / chunks, c = j - row * chunks;
      st16(smem + L.w1u + ((size_t)row * units + c * 8) * 2, ld16(p.w1 + (size_t)row * (p.d + H) + p.d + w * units + c * 8));
    }
  }
  if (tid < kUnitMax) gs_prev[tid] = 0.f;
  __syncthreads();

  const int t_first_hh = (int)(hh0 / p.KH);
  const long hh_last = min(hh0 + p.U_hh, total_hh) - 1;
  const int t_last_hh = hh_last >= hh0 ? (int)(hh_last / p.KH) : -1;
  bool ok = true;
  for (int step = 0; step < p.K; ++step) {
    const uint32_t tag = step + 1;
    const int par = step & 1;
    // base logits and b2 of this wave's tiles at this position (lanes of row 0 only)
    float lb[NR + kLdsSlots], bb[NR + kLdsSlots];
#pragma unroll
    for (int s = 0; s < NR + kLdsSlots; ++s) {
      const int l = (s - NR) * kWaves + wave;
      const int j = s < NR ? s * kWaves + wave : kWaves * NR + l;
      const int v = (t_lo + j) * 16 + col;
      const bool live = grp == 0 && j < nt && (s < NR || l < my_nl) && v < V;
      lb[s] = live ? p.base[(size_t)step * V + v] : 0.f;
      bb[s] = live && p.b2 ? bf16_to_f32(p.b2[v]) : 0.f;
    }

    // ---------- A: W_hh g_{i-1} ----------
    if (step > 0) {
      {
        constexpr int kPer = 2;  // H <= kPer * kThreads
        const unsigned long long* src = p.x_g + (size_t)(par ^ 1) * H;
        unsigned long long x[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) x[q] = tid + q * kThreads < H ? ld_word(src + tid + q * kThreads) : 0ull;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int j = tid + q * kThreads;
          if (j < H) {
            ok &= settle(src + j, step, p.status, x[q]);
            gst[j] = __uint_as_float((uint32_t)x[q]);
          }
        }
      }
      if (__syncthreads_or(!ok)) {
        ok = false;
        break;
      }
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < UHW; ++q) {
        const long gu = hh0 + wave * UHW + q;
        if (gu < total_hh) {
          const int t = (int)(gu / p.KH), s = (int)(gu % p.KH);
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = col == 0 ? gst[s * 32 + grp * 8 + e] : 0.f;
          ActFrag<Bf16> a;
          a.from_f32(x);
          if (t == t_first_hh)
            acc0 = a.mma(acc0, whh[q]);
          else
            acc1 = a.mma(acc1, whh[q]);
        }
      }
      if (grp == 0) {
        red[(wave * 2 + 0) * 16 + col] = acc0[0];
        red[(wave * 2 + 1) * 16 + col] = acc1[0];
      }
      __syncthreads();
      if (tid < 32) {
        const int seg = tid >> 4, c = tid & 15;
        if (t_first_hh + seg <= t_last_hh) {
          float sum = 0.f;
#pragma unroll
          for (int wv = 0; wv < kWaves; ++wv) sum += red[(wv * 2 + seg) * 16 + c];
          put_f32(p.x_hh + (((size_t)par * G + w) * 2 + seg) * 16 + c, sum, tag);
        }
      }
    }

    // ---------- B: unit workgroups ----------
    if (unit_wg) {
      if (wave == 0) {
        int tok;
        if (step == 0) {
          tok = p.x_t[0];
        } else {
          unsigned long long best;
          ok &= gather_keys(p.x_key + (size_t)(par ^ 1) * G, G, step, p.status, best);
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
      if (tid < units) {
        const int j = w * units + tid;
        const float* trow = p.table + (size_t)s_tok * 3 * H;
        float a3[3];
        unsigned long long x[3][3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          a3[q] = trow[q * H + j];
#pragma unroll
          for (int o = 0; o < 3; ++o) {
            const unsigned long long* src = step > 0 ? hh_partial(p, q * H + j, o, par, G) : nullptr;
            x[q][o] = src ? ld_word(src) : 0ull;
          }
        }
        float c3[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          float h = 0.f;
#pragma unroll
          for (int o = 0; o < 3; ++o) {
            const unsigned long long* src = step > 0 ? hh_partial(p, q * H + j, o, par, G) : nullptr;
            if (src) {
              ok &= settle(src, tag, p.status, x[q][o]);
              h += __uint_as_float((uint32_t)x[q][o]);
            }
          }
          c3[q] = h + (p.b_hh ? bf16_to_f32(p.b_hh[q * H + j]) : 0.f);
        }
        const float rg = sigmoidf_(a3[0] + c3[0]);
        const float zg = sigmoidf_(a3[1] + c3[1]);
        const float ng = tanhf(a3[2] + rg * c3[2]);
        const float g = (1.f - zg) * ng + zg * gs_prev[tid];
        gs_new[tid] = g;
        gs_prev[tid] = g;
        p.states[(size_t)step * H + j] = g;
        put_f32(p.x_g + (size_t)par * H + j, g, tag);
      }
      if (__syncthreads_or(!ok)) {
        ok = false;
        break;
      }
      if (uhalf < 2) {
        // bottleneck row urow, units [uhalf * half_units, (uhalf + 1) * half_units)
        float s = 0.f;
        const uint16_t* wr = w1u + (size_t)urow * units + uhalf * half_units;
        for (int k = 0; k < half_units; k += 8) {
          const u32x4 wb = ld16(wr + k);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s += bf16_to_f32((uint16_t)(wb[e] & 0xFFFFu)) * gs_new[uhalf * half_units + k + 2 * e];
            s += bf16_to_f32((uint16_t)(wb[e] >> 16)) * gs_new[uhalf * half_units + k + 2 * e + 1];
          }
        }
        pu[uhalf * r + urow] = s;
      }
      __syncthreads();
      if (tid < r) put_f32(p.x_pu + ((size_t)par * kUnitWGs + w) * r + tid, pu[tid] + pu[r + tid], tag);
    }

    // ---------- C: u, W2 tiles, argmax ----------
    if (tid < r) {
      const unsigned long long* src = p.x_pu + (size_t)par * kUnitWGs * r + tid;
      unsigned long long x[kUnitWGs];
#pragma unroll
      for (int q = 0; q < kUnitWGs; ++q) x[q] = ld_word(src + (size_t)q * r);
      float s = p.P[(size_t)step * r + tid];
#pragma unroll
      for (int q = 0; q < kUnitWGs; ++q) {
        ok &= settle(src + (size_t)q * r, tag, p.status, x[q]);
        s += __uint_as_float((uint32_t)x[q]);
      }
      const float uv = s * sigmoidf_(s);
      const uint32_t hb = __float_as_uint(uv) & 0xFFFF0000u;
      utile[tid] = (uint16_t)(hb >> 16);
      utile[r + tid] = (uint16_t)f32_to_bf16_rne(uv - __uint_as_float(hb));
    }
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    unsigned long long best = 0ull;
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const int j = s * kWaves + wave;
      if (j < nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < RK; ++k) {
          const u32x4 ahi = col == 0 ? ld16(utile + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
          const u32x4 alo = col == 0 ? ld16(utile + r + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
          acc = mma16<Bf16>(acc, ahi, w2r[s][k]);
          acc = mma16<Bf16>(acc, alo, w2r[s][k]);
        }
        if (grp == 0) best = tile_epilogue(p, acc[0], (t_lo + j) * 16 + col, step, tag, lb[s], bb[s], best);
      }
    }
#pragma unroll
    for (int s = 0; s < kLdsSlots; ++s) {
      const int l = s * kWaves + wave;
      const int j = kWaves * NR + l;
      if (l < my_nl && j < nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < RK; ++k) {
          const u32x4 wv = ld16(w2l + ((size_t)l * RK + k) * 1024 + lane * 16);
          const u32x4 ahi = col == 0 ? ld16(utile + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
          const u32x4 alo = col == 0 ? ld16(utile + r + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
          acc = mma16<Bf16>(acc, ahi, wv);
          acc = mma16<Bf16>(acc, alo, wv);
        }
        if (grp == 0)
          best = tile_epilogue(p, acc[0], (t_lo + j) * 16 + col, step, tag, lb[NR + s], bb[NR + s], best);
      }
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const unsigned long long o = __shfl_xor(best, sh, 64);
      best = o > best ? o : best;
    }
    if (lane == 0) s_key[wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long k = s_key[0];
#pragma unroll
      for (int wv = 1; wv < kWaves; ++wv) k = s_key[wv] > k ? s_key[wv] : k;
      if (k == 0ull) k = (unsigned long long)(tag & 0xFFu) << 24;  // no tiles: a tagged lowest key
      put_word(p.x_key + (size_t)par * G + w, k);
    }
  }

  if (ok && w == 0 && wave == 0) {  // the token of the last position
    unsigned long long best;
    ok &= gather_keys(p.x_key + (size_t)((p.K - 1) & 1) * G, G, p.K, p.status, best);
    if (lane == 0 && ok) p.tokens[p.K - 1] = key_index(best);
  }
  if (!ok) {
    if (tid == 0) atomicOr(p.status, 1u);
    if (w == 0)
      for (int i = tid; i < p.K; i += kThreads) p.tokens[i] = -1;
  }
}

template <int UHW, int NR, int RK>
static hipError_t launch_t(const Params& p, int G, size_t lds, hipStream_t s) {
  auto kern = draft_b1_kernel<UHW, NR, RK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kThreads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorNotSupported;
  Params pp = p;
  void* args[] = {&pp};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(G), dim3(kThreads), args,
                                    (unsigned)lds, s);
}

}  // namespace b1

size_t b1_exchange_words(int H, int r, int max_wg) {
  return 2 * ((size_t)max_wg * 2 * 16 + (size_t)H + (size_t)b1::kUnitWGs * r + (size_t)max_wg);
}

hipError_t launch_draft_b1(const LoopArgs& a, hipStream_t s) {
  using namespace b1;
  constexpr int NR = 3, RK = 8;
  if (a.dtype != 1 || a.B != 1 || !a.table) return hipErrorNotSupported;
  if (a.r != RK * 32 || a.H % (2 * kUnitWGs) || a.H / kUnitWGs > kUnitMax || a.H > 2 * kThreads)
    return hipErrorNotSupported;
  const int G = std::min(a.num_cu, std::min(a.max_wg, 256));
  if (G < kUnitWGs) return hipErrorNotSupported;
  const int KH = a.H / 32, T3 = 3 * a.H / 16;
  const long need = ((long)T3 * KH + G - 1) / G;
  const int U_hh = (int)((need + kWaves - 1) / kWaves * kWaves);
  if (U_hh > KH) return hipErrorNotSupported;  // a range spans at most two tiles
  const int ntiles = (a.V + 15) / 16;
  const int units = a.H / kUnitWGs;
  const int w1_bytes = a.r * units * 2;
  constexpr int kSlots = 2;  // LDS W2 tiles per wave
  // unit workgroups give up LDS tiles for their W1 columns; the others take the rest
  const int nl_max = kSlots * kWaves;
  const int nl_unit = std::max(0, (nl_max * RK * 1024 - w1_bytes) / (RK * 1024));
  const int ut = std::min(kWaves * NR + nl_unit, ntiles / G);
  const int rest = ntiles - kUnitWGs * ut;
  const int per_other = (rest + (G - kUnitWGs) - 1) / (G - kUnitWGs);
  const int nl = std::max(0, per_other - kWaves * NR);
  if (nl > nl_max || G <= kUnitWGs) return hipErrorNotSupported;
  const Lds L = lds_layout(nl, nl_unit, RK, a.H, a.r);
  if (L.total > 160 * 1024 - 256) return hipErrorNotSupported;
  Params p{};
  p.d = a.d;
  p.V = a.V;
  p.H = a.H;
  p.r = a.r;
  p.K = a.K;
  p.KH = KH;
  p.U_hh = U_hh;
  p.ntiles = ntiles;
  p.nl = nl;
  p.nl_unit = nl_unit;
  p.ut = ut;
  p.w_hh = static_cast<const uint16_t*>(a.w_hh);
  p.b_hh = static_cast<const uint16_t*>(a.b_hh);
  p.w1 = static_cast<const uint16_t*>(a.w1);
  p.w2 = static_cast<const uint16_t*>(a.w2);
  p.b2 = static_cast<const uint16_t*>(a.b2);
  p.table = a.table;
  p.base = a.base;
  p.P = a.P;
  p.x_t = a.x_t;
  p.teacher = a.teacher;
  p.inv_temp = a.inv_temp;
  p.sampled = a.sampled;
  p.seed = a.seed;
  p.offset = a.offset;
  p.logits = a.logits;
  p.states = a.states;
  p.tokens = a.tokens;
  p.status = reinterpret_cast<unsigned int*>(a.keys + (size_t)a.K * a.B);
  unsigned long long* x = a.xpart;
  p.x_hh = x;
  x += 2 * (size_t)a.max_wg * 2 * 16;
  p.x_g = x;
  x += 2 * (size_t)a.H;
  p.x_pu = x;
  x += 2 * (size_t)kUnitWGs * a.r;
  p.x_key = x;
  const int UHW = U_hh / kWaves;
  switch (UHW) {
    case 1: return launch_t<1, NR, RK>(p, G, L.total, s);
    case 2: return launch_t<2, NR, RK>(p, G, L.total, s);
    case 3: return launch_t<3, NR, RK>(p, G, L.total, s);
    case 4: return launch_t<4, NR, RK>(p, G, L.total, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace domino
