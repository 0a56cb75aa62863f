// K-slicing of the hidden half of the first correction projection,
// P = A W1[:, :d]^T + b1, into partial sums (host logic shared by the
// launchers and the workspace layout; no HIP).
#pragma once

namespace domino {

constexpr int kMaxPSlices = 16;

// waves: waves per workgroup, each taking 512 B of K of a bf16 row;
// S: slices (workgroup K ranges) that P is split into.
struct PSplit {
  int waves, S;
};

// False unless d * 2 (bf16 bytes of a row) is a multiple of 512 and r of 16.
inline bool p_split_shape(int d, int r, PSplit& ps) {
  const int row = d * 2;
  if (d <= 0 || row % 512 || r <= 0 || r % 16) return false;
  const int chunks = row / 512;
  ps.waves = chunks % 4 == 0 ? 4 : chunks % 2 == 0 ? 2 : 1;
  ps.S = chunks / ps.waves;
  return ps.S <= kMaxPSlices;
}

}  // namespace domino
