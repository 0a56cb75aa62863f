// Single-block (B = 1) draft loop with the head's per-position weights held
// on chip ([notes] §二.1(2) items 1-3; [explainer] §四).
//
// Pages: [notes] "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn);
//        [explainer] the yhxrc.cn article on the Domino paper.
//
// One cooperative launch of G = #CU workgroups (256 threads each) runs the
// whole K-position loop.  Re-reading W2, W_ih, W_hh and W1 from HBM at every
// position would cost ~110 MB per position; instead each workgroup loads its
// share once and keeps it resident:
//   * W_ih: a contiguous range of U_ih "k-steps" (16 gate rows x 32 inputs,
//     1 KB) of the stacked [3H, d] matrix, in LDS;
//   * W_hh: a contiguous range of U_hh k-steps of [3H, H], in registers;
//   * W2:   a contiguous range of 16-row vocabulary tiles, 4*NR in registers
//     (NR per wave) and the rest in LDS;
//   * W1[:, d:] (the GRU half of the first correction projection): workgroups
//     0..kUnitWGs-1 each hold the columns of their H/kUnitWGs GRU units.
// Per position i (tags are i + 1; every exchanged word is {tag, payload}
// written and polled with relaxed agent-scope atomics, double-buffered by the
// parity of i):
//   A1. W_hh g_{i-1} partials of each workgroup's k-range       -> x_hh
//   A2. token y_{i-1} from the G argmax keys, the token's embedding
//       row staged in LDS, W_ih e partials                       -> x_ih
//   B.  unit workgroups: gate pre-activations from the partials,
//       new GRU state for their units (-> states, x_g) and their
//       share of W1[:, d:] g                                      -> x_pu
//   C.  every workgroup: u = SiLU(P_i + sum of the shares), its W2 tiles on
//       the matrix cores, + b2 + base logits (+ Gumbel), argmax   -> x_key
// A1 runs while the keys of position i-1 are still arriving.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace domino {
namespace b1 {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kUnitWGs = 8;
constexpr unsigned int kSpinLimit = 1u << 20;

struct Params {
  int d, V, H, r, K;
  int KI, KH;      // 32-element k-steps per gate row: d / 32, H / 32
  int U_ih, U_hh;  // k-steps of W_ih / W_hh per workgroup (multiples of kWaves)
  int ntiles;      // ceil(V / 16)
  int nl;          // W2 tiles per workgroup kept in LDS (capacity)
  const uint16_t *embed, *w_ih, *w_hh, *b_ih, *b_hh, *w1, *w2, *b2;
  const float *base, *P;  // base [K][V], P [K][r] (includes b1)
  const int32_t *x_t, *teacher;
  float inv_temp;
  int sampled;
  uint64_t seed;
  uint32_t offset;
  float *logits, *states;
  int32_t* tokens;
  unsigned int* status;
  unsigned long long *x_ih, *x_hh;  // [2][G][2 segments][16]
  unsigned long long* x_g;          // [2][H]
  unsigned long long* x_pu;         // [2][kUnitWGs][r]
  unsigned long long* x_key;        // [2][G]
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
__device__ __forceinline__ bool has_tag(unsigned long long w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// Polls *p until it carries `tag` (bounded); w holds the last value read.
__device__ __forceinline__ bool settle(const unsigned long long* p, uint32_t tag, const unsigned int* status,
                                      unsigned long long& w) {
  unsigned int spins = 0;
  while (!has_tag(w, tag)) {
    if (++spins > kSpinLimit ||
        ((spins & 63u) == 0u && __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
    w = ld_word(p);
  }
  return true;
}

// Argmax key with the position tag in the low word: score (32) | tag (8) | 0xFFFFFF - v (24).
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

// Max over the G argmax keys published for one position (tag), on one wave.
// The loads of a lane are all in flight before any is checked.
__device__ __forceinline__ bool gather_keys(const unsigned long long* keys, int G, uint32_t tag,
                                            const unsigned int* status, unsigned long long& best) {
  constexpr int kMaxPer = 4;  // G <= 4 * 64
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
        if (++spins > kSpinLimit ||
            ((spins & 63u) == 0u && __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
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

// Workgroups whose k-step range covers gate-row tile t (contiguous ranges of
// U k-steps over tiles of KT k-steps), and the segment (0: the workgroup's
// first tile, 1: its second) that holds tile t.
__device__ __forceinline__ void tile_owners(int t, int KT, int U, int& w_lo, int& w_hi) {
  w_lo = (t * KT) / U;
  w_hi = (t * KT + KT - 1) / U;
}
__device__ __forceinline__ int tile_segment(int w, int t, int KT, int U) { return ((w * U) / KT == t) ? 0 : 1; }

// Address of the o-th partial (kind 0: W_ih e, 1: W_hh g) of gate row `row`,
// or nullptr when the tile has fewer owners (or no W_hh term at step 0).
__device__ __forceinline__ const unsigned long long* partial_ptr(const Params& p, int kind, int row, int o, int par,
                                                                 int G, int step) {
  const int t = row >> 4, c = row & 15;
  const int KT = kind ? p.KH : p.KI, U = kind ? p.U_hh : p.U_ih;
  if (kind && step == 0) return nullptr;
  int lo, hi;
  tile_owners(t, KT, U, lo, hi);
  const int ow = lo + o;
  if (ow > hi) return nullptr;
  const unsigned long long* base = kind ? p.x_hh : p.x_ih;
  return base + (((size_t)par * G + ow) * 2 + tile_segment(ow, t, KT, U)) * 16 + c;
}

// bf16 hi/lo operand fragment of 8 floats (lanes whose batch row is empty pass zeros).
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
  ActFrag<Bf16> a;
  a.from_f32(x);
  hi = a.hi;
  lo = a.lo;
}

// L_i[v] = base + (W2 u)[v] + b2[v] for the lane's vocabulary entry v (row 0
// of the accumulator); returns the running argmax key.
__device__ __forceinline__ unsigned long long tile_epilogue(const Params& p, f32x4 acc, int v, int step, uint32_t tag,
                                                            float lbv, float bbv, unsigned long long best) {
  if (v < p.V) {
    const float Lv = lbv + (acc[0] + bbv);
    if (p.logits) p.logits[(size_t)step * p.V + v] = Lv;
    float sc = Lv;
    if (p.sampled) sc = Lv * p.inv_temp + gumbel_from_word(philox_word(p.seed, p.offset, 0u, step, v));
    const unsigned long long k = b1_key(sc, v, tag);
    best = k > best ? k : best;
  }
  return best;
}

struct Lds {
  // byte offsets into dynamic LDS
  int ihw, w2l, erow, gst, utile, red, gs_new, gs_prev, kred, total;
};

__host__ __device__ inline Lds lds_layout(int U_ih, int nl, int RK, int d, int H, int r) {
  Lds L{};
  int off = 0;
  L.ihw = off;
  off += U_ih * 1024;
  L.w2l = off;
  off += nl * RK * 1024;
  L.erow = off;
  off += d * 2;
  L.gst = off;
  off += H * 4;
  L.utile = off;
  off += r * 4;  // hi then lo, r bf16 each
  L.red = off;
  off += kWaves * 2 * 16 * 4;
  L.gs_new = off;
  off += (H / kUnitWGs) * 4;
  L.gs_prev = off;
  off += (H / kUnitWGs) * 4;
  L.kred = off;
  off += 64;
  L.total = off;
  return L;
}

template <int UIW, int UHW, int NR, int RK>
__global__ void __launch_bounds__(kThreads, 1) draft_b1_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_tok;
  __shared__ int s_fail;
  const int w = blockIdx.x, G = gridDim.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int H = p.H, d = p.d, V = p.V, r = p.r;
  const int rows3 = 3 * H;
  const int T3 = rows3 >> 4;
  const Lds L = lds_layout(p.U_ih, p.nl, RK, d, H, r);
  unsigned char* ihw = smem + L.ihw;
  unsigned char* w2l = smem + L.w2l;
  const uint16_t* erow = reinterpret_cast<const uint16_t*>(smem + L.erow);
  float* gst = reinterpret_cast<float*>(smem + L.gst);
  uint16_t* utile = reinterpret_cast<uint16_t*>(smem + L.utile);
  float* red = reinterpret_cast<float*>(smem + L.red);
  float* gs_new = reinterpret_cast<float*>(smem + L.gs_new);
  float* gs_prev = reinterpret_cast<float*>(smem + L.gs_prev);
  unsigned long long* kred = reinterpret_cast<unsigned long long*>(smem + L.kred);
  const int units = H / kUnitWGs;  // GRU units per unit workgroup
  const bool unit_wg = w < kUnitWGs;

  // ---------------- load the resident weights ----------------
  const long total_ih = (long)T3 * p.KI, total_hh = (long)T3 * p.KH;
  const long ih0 = (long)w * p.U_ih, hh0 = (long)w * p.U_hh;
  for (int j = tid; j < p.U_ih * 64; j += kThreads) {
    const int lu = j >> 6, ln = j & 63;
    const long gu = ih0 + lu;
    u32x4 v = {0, 0, 0, 0};
    if (gu < total_ih) {
      const int t = (int)(gu / p.KI), s = (int)(gu % p.KI);
      v = ld16(p.w_ih + (size_t)(t * 16 + (ln & 15)) * d + s * 32 + (ln >> 4) * 8);
    }
    st16(ihw + (size_t)lu * 1024 + ln * 16, v);
  }
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
  // W2 tiles [t_lo, t_hi): local j < 4*NR in registers (wave j%4, slot j/4), the rest in LDS
  const int t_lo = (int)((long)w * p.ntiles / G), t_hi = (int)((long)(w + 1) * p.ntiles / G);
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
  for (int j = tid; j < p.nl * RK * 64; j += kThreads) {
    const int l = j / (RK * 64), k = (j / 64) % RK, ln = j & 63;
    const int lt = kWaves * NR + l;
    u32x4 v = {0, 0, 0, 0};
    if (lt < nt) {
      const int vv = min((t_lo + lt) * 16 + (ln & 15), V - 1);
      v = ld16(p.w2 + (size_t)vv * r + k * 32 + (ln >> 4) * 8);
    }
    st16(w2l + ((size_t)l * RK + k) * 1024 + ln * 16, v);
  }
  // unit workgroups: their columns of W1[:, d:] for bottleneck row `tid`
  constexpr int UW = 16;  // 16-byte chunks of the unit slice (128 units / 8)
  u32x4 w1g[UW];
  if (unit_wg && tid < r) {
#pragma unroll
    for (int c = 0; c < UW; ++c)
      w1g[c] = (c * 8 < units) ? ld16(p.w1 + (size_t)tid * (d + H) + d + w * units + c * 8) : u32x4{0, 0, 0, 0};
  }
  if (tid < units) gs_prev[tid] = 0.f;
  __syncthreads();

  const int t_first_ih = (int)(ih0 / p.KI), t_first_hh = (int)(hh0 / p.KH);
  bool ok = true;
  for (int step = 0; step < p.K; ++step) {
    const uint32_t tag = step + 1;
    const int par = step & 1;
    // prefetch the base logits (and b2) this workgroup's tiles need at this position
    float lb[NR + 4], bb[NR + 4];
#pragma unroll
    for (int s = 0; s < NR + 4; ++s) {
      const int l = (s - NR) * kWaves + wave;  // LDS slot (s >= NR)
      const int j = s < NR ? s * kWaves + wave : kWaves * NR + l;
      const int v = (t_lo + j) * 16 + col;
      const bool live = j < nt && (s < NR || l < p.nl) && v < V && grp == 0;
      lb[s] = live ? p.base[(size_t)step * V + v] : 0.f;
      bb[s] = live && p.b2 ? bf16_to_f32(p.b2[v]) : 0.f;
    }

    // ---------- A1: W_hh g_{i-1} ----------
    if (step > 0) {
      {
        constexpr int kMaxPer = 4;  // H <= 4 * kThreads
        const unsigned long long* src = p.x_g + (size_t)(par ^ 1) * H;
        unsigned long long x[kMaxPer];
#pragma unroll
        for (int q = 0; q < kMaxPer; ++q) {
          const int j = tid + q * kThreads;
          x[q] = j < H ? ld_word(src + j) : 0ull;
        }
#pragma unroll
        for (int q = 0; q < kMaxPer; ++q) {
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
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int q = 0; q < UHW; ++q) {
        const long gu = hh0 + wave * UHW + q;
        if (gu < total_hh) {
          const int t = (int)(gu / p.KH), s = (int)(gu % p.KH);
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = col == 0 ? gst[s * 32 + grp * 8 + e] : 0.f;
          u32x4 hi, lo;
          split8(x, hi, lo);
          const int seg = t == t_first_hh ? 0 : 1;
          if (seg == 0) {
            acc[0] = mma16<Bf16>(acc[0], hi, whh[q]);
            acc[0] = mma16<Bf16>(acc[0], lo, whh[q]);
          } else {
            acc[1] = mma16<Bf16>(acc[1], hi, whh[q]);
            acc[1] = mma16<Bf16>(acc[1], lo, whh[q]);
          }
        }
      }
      if (grp == 0) {
        red[(wave * 2 + 0) * 16 + col] = acc[0][0];
        red[(wave * 2 + 1) * 16 + col] = acc[1][0];
      }
      __syncthreads();
      if (tid < 32) {
        const int seg = tid >> 4, c = tid & 15;
        const long last = min(hh0 + p.U_hh, total_hh) - 1;
        const int t_last = last >= hh0 ? (int)(last / p.KH) : -1;
        if (t_first_hh + seg <= t_last) {
          float sum = 0.f;
#pragma unroll
          for (int wv = 0; wv < kWaves; ++wv) sum += red[(wv * 2 + seg) * 16 + c];
          put_f32(p.x_hh + (((size_t)par * G + w) * 2 + seg) * 16 + c, sum, tag);
        }
      }
      __syncthreads();
    }

    // ---------- A2: the previous token, its embedding row, W_ih e ----------
    if (wave == 0) {
      int tok;
      if (step == 0) {
        tok = p.x_t[0];
      } else {
        unsigned long long best;
        ok &= gather_keys(p.x_key + (size_t)(par ^ 1) * G, G, step, p.status, best);
        const int picked = (int)(0xFFFFFFu - (uint32_t)(best & 0xFFFFFFull));
        if (w == 0 && lane == 0) p.tokens[step - 1] = picked;
        tok = p.teacher ? p.teacher[step - 1] : picked;
      }
      if (lane == 0) s_tok = min(max(tok, 0), V - 1);
    }
    if (__syncthreads_or(!ok)) {
      ok = false;
      break;
    }
    {
      const uint16_t* e = p.embed + (size_t)s_tok * d;
      for (int j = tid; j < d / 8; j += kThreads)
        st16(smem + L.erow + j * 16, ld16(e + j * 8));
    }
    __syncthreads();
    {
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int q = 0; q < UIW; ++q) {
        const int lu = wave * UIW + q;
        const long gu = ih0 + lu;
        if (gu < total_ih) {
          const int t = (int)(gu / p.KI), s = (int)(gu % p.KI);
          const u32x4 wv = ld16(ihw + (size_t)lu * 1024 + lane * 16);
          const u32x4 a = col == 0 ? ld16(erow + s * 32 + grp * 8) : u32x4{0, 0, 0, 0};
          if (t == t_first_ih)
            acc[0] = mma16<Bf16>(acc[0], a, wv);
          else
            acc[1] = mma16<Bf16>(acc[1], a, wv);
        }
      }
      if (grp == 0) {
        red[(wave * 2 + 0) * 16 + col] = acc[0][0];
        red[(wave * 2 + 1) * 16 + col] = acc[1][0];
      }
      __syncthreads();
      if (tid < 32) {
        const int seg = tid >> 4, c = tid & 15;
        const long last = min(ih0 + p.U_ih, total_ih) - 1;
        const int t_last = last >= ih0 ? (int)(last / p.KI) : -1;
        if (t_first_ih + seg <= t_last) {
          float sum = 0.f;
#pragma unroll
          for (int wv = 0; wv < kWaves; ++wv) sum += red[(wv * 2 + seg) * 16 + c];
          put_f32(p.x_ih + (((size_t)par * G + w) * 2 + seg) * 16 + c, sum, tag);
        }
      }
      __syncthreads();
    }

    // ---------- B: unit workgroups -> new state of their units, share of W1[:, d:] g ----------
    if (unit_wg) {
      if (tid < units) {
        const int j = w * units + tid;
        // every partial this unit needs: 3 gate rows x (<= 3 W_ih owners + <= 3 W_hh owners);
        // all loads are issued before any is checked
        constexpr int kOwn = 3;
        unsigned long long x[3][2][kOwn];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const int row = q * H + j;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const unsigned long long* ptr = nullptr;
#pragma unroll
            for (int o = 0; o < kOwn; ++o) {
              ptr = partial_ptr(p, k, row, o, par, G, step);
              x[q][k][o] = ptr ? ld_word(ptr) : 0ull;
            }
          }
        }
        float pre[3], hpre[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const int row = q * H + j;
          float acc2[2] = {0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int o = 0; o < kOwn; ++o) {
              const unsigned long long* ptr = partial_ptr(p, k, row, o, par, G, step);
              if (ptr) {
                ok &= settle(ptr, tag, p.status, x[q][k][o]);
                acc2[k] += __uint_as_float((uint32_t)x[q][k][o]);
              }
            }
          pre[q] = acc2[0] + (p.b_ih ? bf16_to_f32(p.b_ih[row]) : 0.f);
          hpre[q] = acc2[1] + (p.b_hh ? bf16_to_f32(p.b_hh[row]) : 0.f);
        }
        const float rg = sigmoidf_(pre[0] + hpre[0]);
        const float zg = sigmoidf_(pre[1] + hpre[1]);
        const float ng = tanhf(pre[2] + rg * hpre[2]);
        const float g = (1.f - zg) * ng + zg * gs_prev[tid];
        gs_new[tid] = g;
        p.states[(size_t)step * H + j] = g;
        put_f32(p.x_g + (size_t)par * H + j, g, tag);
      }
      if (__syncthreads_or(!ok)) {
        ok = false;
        break;
      }
      if (tid < r) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < UW; ++c) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wbits = w1g[c][e];
            const int k = c * 8 + e * 2;
            if (k < units) {
              s += bf16_to_f32((uint16_t)(wbits & 0xFFFFu)) * gs_new[k];
              s += bf16_to_f32((uint16_t)(wbits >> 16)) * gs_new[k + 1];
            }
          }
        }
        put_f32(p.x_pu + ((size_t)par * kUnitWGs + w) * r + tid, s, tag);
      }
      if (tid < units) gs_prev[tid] = gs_new[tid];
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
        best = tile_epilogue(p, acc, grp == 0 ? (t_lo + j) * 16 + col : V, step, tag, lb[s], bb[s], best);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int l = s * kWaves + wave;
      const int j = kWaves * NR + l;
      if (l < p.nl && j < nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < RK; ++k) {
          const u32x4 wv = ld16(w2l + ((size_t)l * RK + k) * 1024 + lane * 16);
          const u32x4 ahi = col == 0 ? ld16(utile + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
          const u32x4 alo = col == 0 ? ld16(utile + r + k * 32 + grp * 8) : u32x4{0, 0, 0, 0};
          acc = mma16<Bf16>(acc, ahi, wv);
          acc = mma16<Bf16>(acc, alo, wv);
        }
        best = tile_epilogue(p, acc, grp == 0 ? (t_lo + j) * 16 + col : V, step, tag, lb[NR + s], bb[NR + s], best);
      }
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const unsigned long long o = __shfl_xor(best, sh, 64);
      best = o > best ? o : best;
    }
    if (lane == 0) kred[wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long k = kred[0];
#pragma unroll
      for (int wv = 1; wv < kWaves; ++wv) k = kred[wv] > k ? kred[wv] : k;
      if (k == 0ull) k = (unsigned long long)(tag & 0xFFu) << 24;  // no tiles: a valid lowest key
      put_word(p.x_key + (size_t)par * G + w, k);
    }
  }

  if (ok && w == 0 && wave == 0) {
    // the token of the last position
    const int step = p.K;
    unsigned long long best;
    ok &= gather_keys(p.x_key + (size_t)((step - 1) & 1) * G, G, step, p.status, best);
    if (lane == 0 && ok) p.tokens[step - 1] = (int)(0xFFFFFFu - (uint32_t)(best & 0xFFFFFFull));
  }
  if (!ok) {
    if (tid == 0) atomicOr(p.status, 1u);
    if (w == 0)
      for (int i = tid; i < p.K; i += kThreads) p.tokens[i] = -1;
  }
}

template <int UIW, int UHW, int NR, int RK>
static hipError_t launch_t(const Params& p, int G, size_t lds, hipStream_t s) {
  auto kern = draft_b1_kernel<UIW, UHW, NR, RK>;
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
  return 2 * ((size_t)max_wg * 2 * 16 * 2 + (size_t)H + (size_t)b1::kUnitWGs * r + (size_t)max_wg);
}

hipError_t launch_draft_b1(const LoopArgs& a, hipStream_t s) {
  using namespace b1;
  constexpr int NR = 8;
  if (a.dtype != 1 || a.B != 1) return hipErrorNotSupported;
  if (a.d % 32 || a.H % 32 || a.r != 256 || a.H % kUnitWGs || a.H / kUnitWGs > 128 || a.r > kThreads)
    return hipErrorNotSupported;
  const int G = std::min(a.num_cu, a.max_wg);
  const int KI = a.d / 32, KH = a.H / 32, T3 = 3 * a.H / 16;
  auto round4 = [](long x) { return (int)((x + kWaves - 1) / kWaves * kWaves); };
  const int U_ih = round4(((long)T3 * KI + G - 1) / G);
  const int U_hh = round4(((long)T3 * KH + G - 1) / G);
  if (U_ih > KI || U_hh > KH) return hipErrorNotSupported;  // a range must span at most two tiles
  const int ntiles = (a.V + 15) / 16;
  const int per_wg = (ntiles + G - 1) / G;
  const int nl = std::max(0, per_wg - kWaves * NR);
  if (nl > 4 * kWaves) return hipErrorNotSupported;
  constexpr int RK = 8;
  const Lds L = lds_layout(U_ih, nl, RK, a.d, a.H, a.r);
  if (L.total > 160 * 1024) return hipErrorNotSupported;
  if (G < kUnitWGs) return hipErrorNotSupported;
  Params p{};
  p.d = a.d;
  p.V = a.V;
  p.H = a.H;
  p.r = a.r;
  p.K = a.K;
  p.KI = KI;
  p.KH = KH;
  p.U_ih = U_ih;
  p.U_hh = U_hh;
  p.ntiles = ntiles;
  p.nl = nl;
  p.embed = static_cast<const uint16_t*>(a.embed);
  p.w_ih = static_cast<const uint16_t*>(a.w_ih);
  p.w_hh = static_cast<const uint16_t*>(a.w_hh);
  p.b_ih = static_cast<const uint16_t*>(a.b_ih);
  p.b_hh = static_cast<const uint16_t*>(a.b_hh);
  p.w1 = static_cast<const uint16_t*>(a.w1);
  p.w2 = static_cast<const uint16_t*>(a.w2);
  p.b2 = static_cast<const uint16_t*>(a.b2);
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
  p.x_ih = x;
  x += 2 * (size_t)a.max_wg * 2 * 16;
  p.x_hh = x;
  x += 2 * (size_t)a.max_wg * 2 * 16;
  p.x_g = x;
  x += 2 * (size_t)a.H;
  p.x_pu = x;
  x += 2 * (size_t)kUnitWGs * a.r;
  p.x_key = x;
  const int UIW = U_ih / kWaves, UHW = U_hh / kWaves;
  if (UIW == 24 && UHW == 6) return launch_t<24, 6, NR, RK>(p, G, L.total, s);  // d = 4096, H = 1024, 256 CUs
  if (UIW == 15 && UHW == 6) return launch_t<15, 6, NR, RK>(p, G, L.total, s);  // d = 2560, H = 1024, 256 CUs
  return hipErrorNotSupported;
}

}  // namespace domino
