// Split-K bf16 MFMA path of the few-row quantized GEMV (gfx950).
//
// Prior art on the pages: the few-row MMA kernels of "metal : few-row MMA
// mat-mul and batched copies for speculative decoding" (Overview: 8x8
// simdgroup matrices, each weight dequantized once for all rows, the
// simdgroups of a threadgroup split K) and the split-K MMA variants on the
// MLX quantized_matmul small-M verify kernels page (Facts: dequantize per
// quantization group rather than per MMA tile; split K across the
// simdgroups; load the activation operand straight from device bf16).
//
// CDNA4 design:
// * One v_mfma_f32_16x16x32_bf16 computes a 16(m) x 16(n) tile over 32 k.
//   A = activations (rows m >= M are zero and never loaded), B = weights as
//   exact bf16 values 128+q.  A workgroup owns NT tiles of 16 output columns
//   over the whole of K; its waves split K into "bias blocks" of 4 groups.
// * Lane (col = lane%16, kb = lane/16) loads 16 contiguous bytes of row
//   n = col at byte 16*kb of each 64-byte super-chunk, so 16 rows x 64 B are
//   read per load instruction.  A 4x4 transpose of dwords across the four
//   16-lane rows (v_permlane32_swap + v_permlane16_swap) then gives every
//   MFMA step 32 consecutive-in-K codes from one chunk, i.e. from one group.
// * The group's partial product is accumulated by gs/32 MFMAs and folded with
//   the group scale once: acc += s * acc_g (4 FMAs per lane per group).
// * Bias and the 128 code offset: sum_g (b - 128 s)[n,g] * xsum[m,g] is a
//   tiny product over groups.  xsum is produced by an extra MFMA per step
//   with an indicator A operand (row r is all ones iff r/4 is the step's
//   group within the block), which leaves xsum[m][g0 + lane/16] in exactly
//   the A layout of v_mfma_f32_16x16x4_f32; one such MFMA per block and tile
//   adds the bias term.
// * Partial tiles of the waves are summed through LDS in a fixed wave order
//   (deterministic, no atomics) and rows m < M are stored.

#include "qgemv_device.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

// activation units (16 bytes) staged per thread by the LDS variant
constexpr int kMfmaLdsUnitsPerThread = 8;
// The LDS-staged variant measured slower than direct fragment loads on the
// square 4096x4096 shapes (its staging barrier serializes the waves); it is
// kept for shapes where that may change but not selected.
constexpr bool kMfmaUseLdsStaging = false;

template <int BITS, int GS, int NT, int MAXT, int SPI>
__global__ __launch_bounds__(MAXT) void qgemv_mfma_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *__restrict__ y,
    int M, int N, int K) {
  constexpr int CW = 128 / BITS;       // weights per 16-byte chunk
  constexpr int SCW = 4 * CW;          // weights per 64-byte super-chunk
  constexpr int BLKW = 4 * GS;         // weights per bias block (4 groups)
  constexpr int BSC = BLKW / SCW;      // super-chunks per block
  constexpr int STEPS_SC = SCW / 32;   // MFMA steps per super-chunk
  constexpr int STEPS_G = GS / 32;     // MFMA steps per group
  constexpr int XW = BITS == 4 ? 4 : 8;  // 16-byte activation loads per lane per super-chunk
  // A wave walks its K-slice in batches of UNR super-chunks (whole blocks):
  // all loads of a batch are issued together, in the order they are
  // consumed, then the batch is computed.  UNR is compile-time so positions
  // within a block and register slots are static.
  constexpr int UNR = SPI > BSC ? SPI : BSC;
  constexpr int BPB = UNR / BSC;       // blocks per batch
  static_assert(BSC >= 1 && BLKW % SCW == 0 && UNR % BSC == 0, "block layout");

  __shared__ float red[MAXT / 64][NT][4][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int col = lane & 15;
  const int kb = lane >> 4;
  const int n_base = blockIdx.x * 16 * NT;
  const int NBLK = K / BLKW;
  // K-slice of this wave.  The slice order is rotated per workgroup (by
  // blockIdx/8: workgroups are dealt round-robin over the 8 XCDs) so that the
  // CUs sharing an L2 do not all read the same activation lines at the same
  // moment.  Partials are reduced in slice order, so results do not depend
  // on the rotation.
  const int slice = (wave + (int)(blockIdx.x >> 3)) % waves;
  const int b_begin = (slice * NBLK) / waves;
  const int b_end = ((slice + 1) * NBLK) / waves;
  const size_t RB = (size_t)K * BITS / 8;
  const int G = K / GS;
  // Rows m >= M and columns n >= N only feed outputs that are never stored,
  // so their lanes read valid clamped addresses instead of branching around
  // the loads (a branch would force a wait on every load).
  const uint16_t *xr = x + (size_t)(col < M ? col : M - 1) * K + kb * (CW / 4);
  const uint8_t *crow[NT];
  const uint16_t *srow[NT];
  const uint16_t *brow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = min(n_base + 16 * t + col, N - 1);
    crow[t] = codes + (size_t)n * RB + kb * 16;
    srow[t] = scales + (size_t)n * G;
    brow[t] = biases + (size_t)n * G;
  }
  const uint32_t offset_pair = opaque_u32(kOffsetPair);

  // indicator operands: A row r = col is all ones iff r/4 == j
  u32x4_t ind[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = ((col >> 2) == j) ? 0x3F803F80u : 0u;
    ind[j] = u32x4_t{v, v, v, v};
  }

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int blk0 = b_begin; blk0 < b_end; blk0 += BPB) {
    const int nb = min(BPB, b_end - blk0);  // blocks in this batch (uniform)
    // ---- issue: activations, codes and metadata of the batch
    u32x4_t xv[UNR][XW];
    u32x4_t cv[UNR][NT];
    uint2 s4[BPB][NT], b4[BPB][NT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC < nb) {
        const int gsc = blk0 * BSC + u;
#pragma unroll
        for (int i = 0; i < XW; ++i) {
          const int c = BITS == 4 ? i : (i >> 1);
          const int k0 = gsc * SCW + c * CW + (BITS == 4 ? 0 : 8 * (i & 1));
          xv[u][i] = *reinterpret_cast<const u32x4_t *>(xr + k0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
          cv[u][t] = load_stream_u32x4(crow[t] + (size_t)gsc * 64);
        if (u % BSC == 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            s4[u / BSC][t] = *reinterpret_cast<const uint2 *>(srow[t] + (size_t)(gsc / BSC) * 4);
            b4[u / BSC][t] = *reinterpret_cast<const uint2 *>(brow[t] + (size_t)(gsc / BSC) * 4);
          }
        }
      }
    }

    // ---- compute, super-chunk by super-chunk in load order
    f32x4_t xsacc = zero4;
    f32x4_t accg[NT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC >= nb) break;
      const int scb = u % BSC;  // super-chunk within its block
      uint32_t cur[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        cur[t][0] = cv[u][t][0];
        cur[t][1] = cv[u][t][1];
        cur[t][2] = cv[u][t][2];
        cur[t][3] = cv[u][t][3];
        transpose_rows4(cur[t]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int h = 0; h < (BITS == 4 ? 1 : 2); ++h) {
          const int st = scb * STEPS_SC + (BITS == 4 ? c : 2 * c + h);  // step within block
          const int j = st / STEPS_G;                                      // group within block
          const bool gfirst = (st % STEPS_G) == 0;
          const bool glast = (st % STEPS_G) == STEPS_G - 1;
          u32x4_t xa;
          if constexpr (BITS == 4) {
            xa = xv[u][c];
          } else {
            const uint32_t X[8] = {xv[u][2 * c][0],     xv[u][2 * c][1],     xv[u][2 * c][2],
                                   xv[u][2 * c][3],     xv[u][2 * c + 1][0], xv[u][2 * c + 1][1],
                                   xv[u][2 * c + 1][2], xv[u][2 * c + 1][3]};
            xa = u32x4_t{xpair_stride8(X, 4 * h + 0), xpair_stride8(X, 4 * h + 1),
                         xpair_stride8(X, 4 * h + 2), xpair_stride8(X, 4 * h + 3)};
          }
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xa);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            u32x4_t bw;
            if constexpr (BITS == 4) {
              bw = unpack4_natural_quad(cur[t][c], offset_pair);
            } else {
              bw = unpack2_split_quad(cur[t][c], h, offset_pair);
            }
            accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, bw), gfirst ? zero4 : accg[t], 0, 0, 0);
          }
          xsacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ind[j]), a,
                                                          st == 0 ? zero4 : xsacc, 0, 0, 0);
          if (glast) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const uint32_t sw = (j < 2) ? s4[u / BSC][t].x : s4[u / BSC][t].y;
              const float s = half_bits_to_float((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(s, accg[t][i], acc[t][i]);
            }
          }
        }
      }
      if (scb == BSC - 1) {
        // bias (with the 128 offset): acc += xsum[m][g0+j] * (b - 128 s)[n][g0+j]
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint32_t sw = (kb < 2) ? s4[u / BSC][t].x : s4[u / BSC][t].y;
          const uint32_t bw = (kb < 2) ? b4[u / BSC][t].x : b4[u / BSC][t].y;
          const float s = half_bits_to_float((kb & 1) ? (sw >> 16) : (sw & 0xFFFFu));
          const float b = half_bits_to_float((kb & 1) ? (bw >> 16) : (bw & 0xFFFFu));
          const float bo = fmaf(-128.f, s, b);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsacc[0], bo, acc[t], 0, 0, 0);
        }
      }
    }
  }

  // split-K reduction over the slices, fixed order
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[slice][t][i][lane] = acc[t][i];
  __syncthreads();
  for (int o = threadIdx.x; o < NT * 256; o += blockDim.x) {
    const int t = o >> 8;
    const int i = (o >> 6) & 3;
    const int l = o & 63;
    float s = 0.f;
    for (int w = 0; w < waves; ++w) s += red[w][t][i][l];
    const int m = 4 * (l >> 4) + i;
    const int n = n_base + 16 * t + (l & 15);
    if (m < M && n < N) y[(size_t)m * N + n] = s;
  }
}

// Same path with the activations staged once per workgroup in LDS.
//
// Every workgroup needs all M*K activations (its 16*NT output columns span
// the whole of K), so with one tile per CU the activation reads through L2
// grow with M and overtake the weight stream at M ~ 8.  Staging them once per
// workgroup with full-line 16-byte loads (issued before the code loads, so
// the staging never waits for HBM) halves the L2 requests of the per-lane
// fragment loads and lets lanes of rows m >= M skip memory entirely.  The
// per-group activation sums are formed during the staging (8-element partial
// sums reduced over the gs/8 lanes that hold one group), which replaces the
// indicator MFMAs of the direct kernel.
//
// LDS: x rows at a pitch of 2K+16 bytes (the 16-byte pad puts the 16 rows of
// an A fragment on distinct bank groups), the group sums [M][K/gs] fp32 and
// the split-K reduction buffer.
template <int BITS, int GS, int NT, int MAXT, int SPI>
__global__ __launch_bounds__(MAXT) void qgemv_mfma_lds_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *__restrict__ y,
    int M, int N, int K) {
  constexpr int CW = 128 / BITS;
  constexpr int SCW = 4 * CW;
  constexpr int BLKW = 4 * GS;
  constexpr int BSC = BLKW / SCW;
  constexpr int STEPS_SC = SCW / 32;
  constexpr int STEPS_G = GS / 32;
  constexpr int UNR = SPI > BSC ? SPI : BSC;
  constexpr int BPB = UNR / BSC;
  constexpr int UPG = GS / 8;          // 16-byte activation units per group
  constexpr int XUNITS = kMfmaLdsUnitsPerThread;
  static_assert(BSC >= 1 && BLKW % SCW == 0 && UNR % BSC == 0, "block layout");

  extern __shared__ uint4 lds_u4[];
  uint8_t *lds = reinterpret_cast<uint8_t *>(lds_u4);
  const int XP = 2 * K + 16;  // bytes per staged row
  const int G = K / GS;
  float *xsl = reinterpret_cast<float *>(lds + (size_t)M * XP);  // [M][G]
  float *red = xsl + (size_t)M * G;                              // [waves][NT][4][64]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int col = lane & 15;
  const int kb = lane >> 4;
  const int n_base = blockIdx.x * 16 * NT;
  const int NBLK = K / BLKW;
  const int slice = (wave + (int)(blockIdx.x >> 3)) % waves;  // rotated as in the direct kernel
  const int b_begin = (slice * NBLK) / waves;
  const int b_end = ((slice + 1) * NBLK) / waves;
  const size_t RB = (size_t)K * BITS / 8;

  // ---- 1. activation staging loads: 16-byte units, row after row
  const int upr = K / 8;
  const int units = M * upr;
  uint4 xu[XUNITS];
#pragma unroll
  for (int i = 0; i < XUNITS; ++i) {
    if (i * (int)blockDim.x < units) {  // uniform
      const int u = min((int)threadIdx.x + i * (int)blockDim.x, units - 1);
      xu[i] = reinterpret_cast<const uint4 *>(x)[u];  // row-major [M][K]: unit u = row u/upr
    }
  }

  // ---- 2. codes and metadata of the first batch
  const uint8_t *crow[NT];
  const uint16_t *srow[NT];
  const uint16_t *brow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = min(n_base + 16 * t + col, N - 1);
    crow[t] = codes + (size_t)n * RB + kb * 16;
    srow[t] = scales + (size_t)n * G;
    brow[t] = biases + (size_t)n * G;
  }
  u32x4_t cv[UNR][NT];
  uint2 s4[BPB][NT], b4[BPB][NT];
  auto issue_batch = [&](int blk0, int nb) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC < nb) {
        const int gsc = blk0 * BSC + u;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          cv[u][t] = load_stream_u32x4(crow[t] + (size_t)gsc * 64);
        if (u % BSC == 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            s4[u / BSC][t] = *reinterpret_cast<const uint2 *>(srow[t] + (size_t)(gsc / BSC) * 4);
            b4[u / BSC][t] = *reinterpret_cast<const uint2 *>(brow[t] + (size_t)(gsc / BSC) * 4);
          }
        }
      }
    }
  };
  if (b_begin < b_end) issue_batch(b_begin, min(BPB, b_end - b_begin));

  // ---- 3. write the staged activations and their group sums to LDS
#pragma unroll
  for (int i = 0; i < XUNITS; ++i) {
    if (i * (int)blockDim.x < units) {  // uniform
      const int u = (int)threadIdx.x + i * (int)blockDim.x;
      const int m = u / upr;
      const int jj = u - m * upr;
      const uint4 v = xu[i];
      float part = dot2_bf16(v.x, 0x3F803F80u, 0.f);
      part = dot2_bf16(v.y, 0x3F803F80u, part);
      part = dot2_bf16(v.z, 0x3F803F80u, part);
      part = dot2_bf16(v.w, 0x3F803F80u, part);
      // the UPG lanes of one group are consecutive and aligned
#pragma unroll
      for (int off = 1; off < UPG; off <<= 1) part += __shfl_xor(part, off, 64);
      if (u < units) {
        *reinterpret_cast<uint4 *>(lds + (size_t)m * XP + (size_t)jj * 16) = v;
        if (jj % UPG == 0) xsl[m * G + jj / UPG] = part;
      }
    }
  }
  __syncthreads();

  // ---- 4. split-K MFMA over this wave's blocks
  const int mrow = col < M ? col : M - 1;  // rows >= M repeat a real row; never stored
  const uint8_t *xrow = lds + (size_t)mrow * XP + kb * (CW / 4) * 2;
  const float *xsrow = xsl + (size_t)mrow * G;
  const uint32_t offset_pair = opaque_u32(kOffsetPair);
  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int blk0 = b_begin; blk0 < b_end; blk0 += BPB) {
    const int nb = min(BPB, b_end - blk0);
    if (blk0 != b_begin) issue_batch(blk0, nb);
    f32x4_t accg[NT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC >= nb) break;
      const int gsc = blk0 * BSC + u;
      const int scb = u % BSC;
      // A fragments of this super-chunk from LDS
      u32x4_t xa4[BITS == 4 ? 4 : 8];
#pragma unroll
      for (int i = 0; i < (BITS == 4 ? 4 : 8); ++i) {
        const int c = BITS == 4 ? i : (i >> 1);
        const int k0 = gsc * SCW + c * CW + (BITS == 4 ? 0 : 8 * (i & 1));
        xa4[i] = *reinterpret_cast<const u32x4_t *>(xrow + (size_t)k0 * 2);
      }
      uint32_t cur[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        cur[t][0] = cv[u][t][0];
        cur[t][1] = cv[u][t][1];
        cur[t][2] = cv[u][t][2];
        cur[t][3] = cv[u][t][3];
        transpose_rows4(cur[t]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int h = 0; h < (BITS == 4 ? 1 : 2); ++h) {
          const int st = scb * STEPS_SC + (BITS == 4 ? c : 2 * c + h);
          const int j = st / STEPS_G;
          const bool gfirst = (st % STEPS_G) == 0;
          const bool glast = (st % STEPS_G) == STEPS_G - 1;
          u32x4_t xa;
          if constexpr (BITS == 4) {
            xa = xa4[c];
          } else {
            const uint32_t X[8] = {xa4[2 * c][0],     xa4[2 * c][1],     xa4[2 * c][2],
                                   xa4[2 * c][3],     xa4[2 * c + 1][0], xa4[2 * c + 1][1],
                                   xa4[2 * c + 1][2], xa4[2 * c + 1][3]};
            xa = u32x4_t{xpair_stride8(X, 4 * h + 0), xpair_stride8(X, 4 * h + 1),
                         xpair_stride8(X, 4 * h + 2), xpair_stride8(X, 4 * h + 3)};
          }
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xa);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            u32x4_t bw;
            if constexpr (BITS == 4) {
              bw = unpack4_natural_quad(cur[t][c], offset_pair);
            } else {
              bw = unpack2_split_quad(cur[t][c], h, offset_pair);
            }
            accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, bw), gfirst ? zero4 : accg[t], 0, 0, 0);
          }
          if (glast) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const uint32_t sw = (j < 2) ? s4[u / BSC][t].x : s4[u / BSC][t].y;
              const float s = half_bits_to_float((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(s, accg[t][i], acc[t][i]);
            }
          }
        }
      }
      if (scb == BSC - 1) {
        // bias with the 128 offset: acc += xsum[m][g0+kb] * (b - 128 s)[n][g0+kb]
        const int blk = gsc / BSC;
        const float xsv = xsrow[blk * 4 + kb];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint32_t sw = (kb < 2) ? s4[u / BSC][t].x : s4[u / BSC][t].y;
          const uint32_t bw = (kb < 2) ? b4[u / BSC][t].x : b4[u / BSC][t].y;
          const float s = half_bits_to_float((kb & 1) ? (sw >> 16) : (sw & 0xFFFFu));
          const float b = half_bits_to_float((kb & 1) ? (bw >> 16) : (bw & 0xFFFFu));
          const float bo = fmaf(-128.f, s, b);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsv, bo, acc[t], 0, 0, 0);
        }
      }
    }
  }

  // ---- 5. split-K reduction over the waves, fixed order
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((slice * NT + t) * 4 + i) * 64 + lane] = acc[t][i];
  __syncthreads();
  for (int o = threadIdx.x; o < NT * 256; o += blockDim.x) {
    const int t = o >> 8;
    const int i = (o >> 6) & 3;
    const int l = o & 63;
    float sum = 0.f;
    for (int w = 0; w < waves; ++w) sum += red[((w * NT + t) * 4 + i) * 64 + l];
    const int m = 4 * (l >> 4) + i;
    const int n = n_base + 16 * t + (l & 15);
    if (m < M && n < N) y[(size_t)m * N + n] = sum;
  }
}

// waves per workgroup: spread the bias blocks evenly over at most max_waves
int pick_waves(int nblk, int max_waves) {
  if (nblk <= max_waves) return nblk;
  int best = max_waves;
  double best_eff = 0.0;
  for (int w = max_waves; w >= max_waves / 2; --w) {
    const int per = (nblk + w - 1) / w;
    const double eff = (double)nblk / (double)(per * w);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = w;
    }
  }
  return best;
}

// Per-variant launch shape: thread cap (waves per workgroup) and the number of
// super-chunks in flight per wave, chosen to keep every variant within the
// register budget of its thread cap without spills.
template <int BITS, int GS, int NT>
struct MfmaShape {
  static constexpr int SPI = (BITS == 4 && GS == 128) ? 4 : 2;
  static constexpr int MAXT = (BITS == 4 && NT == 1 && GS <= 64) ? 1024 : 512;
};

size_t mfma_lds_bytes(int M, int K, int group_size, int waves, int nt) {
  return (size_t)M * (2 * (size_t)K + 16) + (size_t)M * (K / group_size) * 4 +
         (size_t)waves * nt * 4 * 64 * 4;
}

template <int BITS, int GS, int NT>
int launch_mfma_t(const QgemvArgs &a, hipStream_t stream) {
  constexpr int MAXT = MfmaShape<BITS, GS, NT>::MAXT;
  constexpr int SPI = MfmaShape<BITS, GS, NT>::SPI;
  const int nblk = a.K / (4 * GS);
  const int waves = pick_waves(nblk, MAXT / 64);
  const int tiles = (a.N + 15) / 16;
  const int blocks = (tiles + NT - 1) / NT;
  const size_t lds = mfma_lds_bytes(a.M, a.K, GS, waves, NT);
  const bool staged = kMfmaUseLdsStaging && lds <= kLdsMax &&
                      (size_t)a.M * a.K / 8 <= (size_t)kMfmaLdsUnitsPerThread * 64 * waves;
  if (staged) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&qgemv_mfma_lds_kernel<BITS, GS, NT, MAXT, SPI>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (attr != hipSuccess) return QGEMV_EHIP;
    hipLaunchKernelGGL((qgemv_mfma_lds_kernel<BITS, GS, NT, MAXT, SPI>), dim3(blocks),
                       dim3(64 * waves), lds, stream, a.codes, a.scales, a.biases, a.x, a.y, a.M,
                       a.N, a.K);
  } else {
    hipLaunchKernelGGL((qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI>), dim3(blocks), dim3(64 * waves),
                       0, stream, a.codes, a.scales, a.biases, a.x, a.y, a.M, a.N, a.K);
  }
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

template <int BITS, int GS>
int launch_mfma_gs(const QgemvArgs &a, hipStream_t stream) {
  const int tiles = (a.N + 15) / 16;
  if (tiles >= 512) return launch_mfma_t<BITS, GS, 2>(a, stream);
  return launch_mfma_t<BITS, GS, 1>(a, stream);
}

}  // namespace

bool mfma_supports(int K, int bits, int group_size) {
  if (bits == 2 && group_size < 64) return false;
  const int scw = bits == 4 ? 128 : 256;
  return K % scw == 0 && K % (4 * group_size) == 0;
}

int launch_mfma(const QgemvArgs &a, hipStream_t stream) {
  if (!mfma_supports(a.K, a.bits, a.group_size)) return QGEMV_EUNSUPPORTED;
  if (a.bits == 4) {
    switch (a.group_size) {
      case 32: return launch_mfma_gs<4, 32>(a, stream);
      case 64: return launch_mfma_gs<4, 64>(a, stream);
      case 128: return launch_mfma_gs<4, 128>(a, stream);
    }
  } else {
    switch (a.group_size) {
      case 64: return launch_mfma_gs<2, 64>(a, stream);
      case 128: return launch_mfma_gs<2, 128>(a, stream);
    }
  }
  return QGEMV_EUNSUPPORTED;
}

}  // namespace qgemv
