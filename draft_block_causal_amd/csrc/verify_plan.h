// Launch shape and workspace layout of the sampled-draft verification
// (host-only arithmetic, shared by the launcher and the argument checks).
#pragma once

#include <stddef.h>

namespace domino {

constexpr int kMaxVerifyBlock = 255;      // drafted positions per block
constexpr int kMaxVerifyBatch = 1 << 20;  // blocks per call

struct VerifyPlan {
  int S1;        // vocabulary slices per logit row in the normaliser pass
  int S2;        // vocabulary slices per block in the draw pass
  size_t stats;  // byte offset of the [B][K + 1][S1] float4 partials
  size_t keys;   // byte offset of the [B] 64-bit draw keys
  size_t total;  // workspace bytes
};

// About 2048 workgroups in the normaliser pass and 1024 in the draw pass,
// each slice at least 2048 (1024) entries long; at most 32 normaliser slices
// per row (the draw pass merges a row's partials in order, one thread a row).
inline VerifyPlan verify_plan(int B, int K, int V) {
  auto clampi = [](long x, long lo, long hi) { return (int)(x < lo ? lo : x > hi ? hi : x); };
  auto align256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  VerifyPlan p{};
  const long rows = (long)B * (K + 1);
  const long s1max = V / 2048 > 1 ? (V / 2048 < 32 ? V / 2048 : 32) : 1;
  p.S1 = clampi((2048 + rows - 1) / rows, 1, s1max);
  p.S2 = clampi((1024 + (long)B - 1) / B, 1, V / 1024 > 1 ? V / 1024 : 1);
  p.stats = 0;
  p.keys = align256((size_t)rows * p.S1 * 16);
  p.total = align256(p.keys + (size_t)B * 8);
  return p;
}

}  // namespace domino
