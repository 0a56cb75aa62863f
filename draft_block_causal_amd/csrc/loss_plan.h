// Launch shape and workspace layout of the curriculum loss (host-only
// arithmetic, shared by the launcher and the argument checks).
#pragma once

#include <stddef.h>

namespace domino {

constexpr int kMaxLossBlock = 1024;     // positions per block
constexpr int kMaxLossBatch = 1 << 20;  // blocks per call

struct LossPlan {
  int S;         // vocabulary slices per row
  size_t stats;  // byte offset of the [B K][S] float4 partials (base max, sum; final max, sum)
  size_t lse;    // byte offset of the [B K][2] float log-normalisers (base, final)
  size_t contrib;  // byte offset of the [B K] float weighted per-position terms
  size_t total;  // workspace bytes
};

// About 2048 workgroups per pass, each slice at least 2048 entries long, and
// at most 32 slices per row (one thread merges a row's partials in order).
inline LossPlan loss_plan(int B, int K, int V) {
  auto align256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  LossPlan p{};
  const long rows = (long)B * K;
  long S = (2048 + rows - 1) / rows;
  long smax = V / 2048 > 1 ? V / 2048 : 1;
  smax = smax > 32 ? 32 : smax;
  S = S < 1 ? 1 : S > smax ? smax : S;
  p.S = (int)S;
  p.stats = 0;
  p.lse = align256((size_t)rows * p.S * 16);
  p.contrib = align256(p.lse + (size_t)rows * 8);
  p.total = align256(p.contrib + (size_t)rows * 4);
  return p;
}

}  // namespace domino
