// Single-pass split-K bf16 MFMA path of the few-row quantized GEMV (gfx950).
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
//   A = activations (rows m >= M repeat row M-1 and are never stored),
//   B = weights as exact bf16 values 128+q (2/4-bit) or q (8-bit, two code
//   dwords per MFMA step).  A workgroup owns NT tiles of
//   16 output columns over the whole of K; its waves split K into
//   contiguous slices of "bias blocks" (4 groups).
// * Lane (col = lane%16, kb = lane/16) loads 16 contiguous bytes of row
//   n = col at byte 16*kb of each 64-byte super-chunk, so 16 rows x 64 B are
//   read per load instruction.  A partial exchange of dwords across the four
//   16-lane rows (none, v_permlane32_swap, or the full 4x4 transpose with
//   v_permlane16_swap, as the group size requires) gives every MFMA step 32
//   codes of one quantization group.
// * The group's partial product is accumulated by gs/32 MFMAs and folded with
//   the group scale once: acc += s * acc_g (4 FMAs per lane per group).
// * Bias and the 128 code offset: sum_g (b - 128 s)[n,g] * xsum[m,g] over the
//   4 groups of a block is one v_mfma_f32_16x16x4_f32, with the per-group
//   activation sums xsum (dot2 against ones, then a row transpose-reduce)
//   formed while the codes are still in flight.
// * Partial tiles of the waves are summed through LDS in slice order
//   (deterministic, no atomics) and rows m < M are stored.
// * Fused residual sum (ADD, "metal : few-row MMA mat-mul and batched copies
//   for speculative decoding", Overview: MUL_MAT + ADD writes the residual
//   sum from the store): each thread loads the residual of the outputs it
//   will store at the start of its tile group and adds it in the store, so
//   y = fl(product + r), bit for bit the plain call and a separate fp32 add.
// Shapes with more 16-column tiles than CUs go to the persistent kernel
// (qgemv_persist.hip) unless K is too long for its register-resident
// activations.

#include "qgemv_device.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {


// Bit pattern that y holds, before a K-split launch with the residual sum,
// until the first half of K lands.  A NaN payload that no partial sum can
// carry: partials derive from bf16 and fp16 inputs, whose NaNs have zero low
// 13 bits in fp32, and fresh NaNs are the canonical 0x7FC00000.
constexpr uint32_t kSplitSentinel = 0x7FC0DEADu;

// y and res may be the same buffer (in-place residual sum): neither is
// declared restrict; every element is read before it is written, by the same
// thread.
// FMT: kAffine, or a block-scaled FP format (one scale byte per block in
// `scales`, no bias, elements decoded in natural order): kMxfp4 and kMxfp8
// (32-element blocks, GS = 32, scale folded per block in fp32) or kNvfp4
// (16-element blocks, laid out as GS = 32; each element is multiplied by its
// block scale before the MFMA, exactly, so B holds the weights themselves).
template <int BITS, int GS, int NT, int MAXT, int SPI, int KS, bool PERSIST, bool ADD, int FMT>
__global__ __launch_bounds__(MAXT) void qgemv_mfma_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *y,
    const float *res, int M, int N, int K, int ngroups) {
  constexpr int CW = 128 / BITS;       // codes per 16-byte chunk
  constexpr int SCW = 4 * CW;          // codes per 64-byte super-chunk
  constexpr int DW = CW / 4;           // codes per dword
  constexpr int HS = BITS == 2 ? 2 : 1;  // MFMA steps per code dword (8-bit: one per two dwords)
  // activation operands per super-chunk: one per code register (2/4-bit) or
  // per pair of code registers (8-bit)
  constexpr int XR = BITS == 8 ? 2 : 4;
  constexpr bool HAS_BIAS = FMT == kAffine;
  constexpr int BLKW = 4 * GS;         // codes per bias block (4 groups)
  constexpr int BSC = BLKW / SCW;      // super-chunks per block
  constexpr int CPG = GS / CW;         // chunks per group (1, 2 or 4)
  constexpr int GPS = 4 / CPG;         // groups per super-chunk
  // how far the four chunk rows are exchanged so that a register holds one group
  constexpr int LVL = CPG >= 4 ? 0 : (CPG == 2 ? 1 : 2);
  constexpr int REGS_G = CPG;          // registers (of one super-chunk) per group
  // A wave walks its K-slice in batches of UNR super-chunks (whole blocks):
  // activations, codes and metadata of a batch are issued together, then the
  // activation work is done while the codes are in flight, then the codes
  // are consumed in load order.  UNR is compile-time so positions within a
  // block and register slots are static.
  constexpr int UNR = SPI > BSC ? SPI : BSC;
  constexpr int BPB = UNR / BSC;       // blocks per batch
  static_assert(BSC >= 1 && BLKW % SCW == 0 && UNR % BSC == 0 && CPG >= 1, "block layout");

  __shared__ float red[MAXT / 64][NT][4][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int col = lane & 15;
  const int kb = lane >> 4;
  const int NBLK = K / BLKW;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t offset_pair = opaque_u32(kOffsetPair);
  // element offset, within a super-chunk, of the codes register i holds in
  // this lane's row after the partial transpose
  int xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xoff[i] = lvl_chunk<LVL>(i, kb) * CW + lvl_dword<LVL>(i, kb) * DW;

  // One tile group (16*NT output columns over all of K) per call of `group`.
  auto group = [&](const int tg) {
  // group tg = (tile group, part of K); with KS = 2 the two halves of K of a
  // tile group are separate groups whose results are added into y
  const int kpart = KS == 1 ? 0 : (tg & 1);
  const int n_base = (KS == 1 ? tg : tg >> 1) * 16 * NT;
  const int p_lo = KS == 1 ? 0 : (kpart ? NBLK >> 1 : 0);
  const int nbp = KS == 1 ? NBLK : (kpart ? NBLK - (NBLK >> 1) : NBLK >> 1);
  // K-slice of this wave.  The slice order is rotated per workgroup (by
  // blockIdx/8: workgroups are dealt round-robin over the 8 XCDs) so that the
  // CUs sharing an L2 do not all read the same activation lines at the same
  // moment.  Partials are reduced in slice order, so results do not depend
  // on the rotation.
  const int slice = (wave + (tg >> 3)) % waves;
  const int b_begin = p_lo + (slice * nbp) / waves;
  const int b_end = p_lo + ((slice + 1) * nbp) / waves;
  const size_t RB = (size_t)K * BITS / 8;
  const int G = FMT == kNvfp4 ? K / 16 : K / GS;  // scale (or scale-and-bias) entries per row
  // Rows m >= M and columns n >= N only feed outputs that are never stored,
  // so their lanes read valid clamped addresses instead of branching around
  // the loads (a branch would force a wait on every load).
  const uint16_t *xr = x + (size_t)(col < M ? col : M - 1) * K;
  const uint8_t *crow[NT];
  const uint16_t *srow[NT];
  const uint16_t *brow[NT];
  const uint8_t *srow8[NT];  // FP formats: scale bytes
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = min(n_base + 16 * t + col, N - 1);
    crow[t] = codes + (size_t)n * RB + kb * 16;
    srow[t] = scales + (size_t)n * G;
    brow[t] = biases + (size_t)n * G;
    srow8[t] = reinterpret_cast<const uint8_t *>(scales) + (size_t)n * G;
  }

  // residual of the outputs this thread stores in its first NT reduction
  // steps (all of them when the workgroup has at least 4 waves), loaded ahead
  // of the weight stream; clamped indices read a valid element, never used
  float rpre[NT];
  if constexpr (ADD) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int o = min((int)threadIdx.x + j * (int)blockDim.x, NT * 256 - 1);
      const int l = o & 63;
      const int m = min(4 * (l >> 4) + ((o >> 6) & 3), M - 1);
      const int n = min(n_base + 16 * (o >> 8) + (l & 15), N - 1);
      rpre[j] = res[(size_t)m * N + n];
    }
  }

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = zero4;

  for (int blk0 = b_begin; blk0 < b_end; blk0 += BPB) {
    const int nb = min(BPB, b_end - blk0);  // blocks in this batch (uniform)
    // ---- issue: activations first (L2), then codes (HBM), then metadata
    u32x4_t xv[UNR][XR][HS];
    u32x4_t cv[UNR][NT];
    uint2 s4[BPB][NT], b4[BPB][NT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC < nb) {
        const int k0 = (blk0 * BSC + u) * SCW;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
          for (int l = 0; l < HS; ++l)
            xv[u][i][l] = *reinterpret_cast<const u32x4_t *>(
                xr + k0 + (BITS == 8 ? xoff[2 * i] : xoff[i]) + 8 * l);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC < nb) {
        const int gsc = blk0 * BSC + u;
#pragma unroll
        for (int t = 0; t < NT; ++t) cv[u][t] = load_stream_u32x4(crow[t] + (size_t)gsc * 64);
      }
    }
#pragma unroll
    for (int bb = 0; bb < BPB; ++bb) {
      if (bb < nb) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (HAS_BIAS) {
            s4[bb][t] = *reinterpret_cast<const uint2 *>(srow[t] + (size_t)(blk0 + bb) * 4);
            b4[bb][t] = *reinterpret_cast<const uint2 *>(brow[t] + (size_t)(blk0 + bb) * 4);
          } else if constexpr (FMT == kNvfp4) {
            // the 8 scale bytes of the block's 128 elements
            s4[bb][t] = *reinterpret_cast<const uint2 *>(srow8[t] + (size_t)(blk0 + bb) * 8);
          } else {
            // the block's 4 scale bytes
            s4[bb][t].x = *reinterpret_cast<const uint32_t *>(srow8[t] + (size_t)(blk0 + bb) * 4);
          }
        }
      }
    }
    // keep the whole batch of loads ahead of the compute: without this the
    // scheduler may sink later loads below the first waits and serialize them
    __builtin_amdgcn_sched_barrier(0);

    // ---- activation work, overlapping the code loads: re-pair x to the
    // code pairing and form the per-group activation sums.  xsum of group
    // g0 + j ends up in row j of this lane's column, i.e. in the A layout of
    // v_mfma_f32_16x16x4_f32 for the bias product.
    float xsum[BPB];
#pragma unroll
    for (int bb = 0; bb < BPB; ++bb) {
      float P[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int uu = 0; uu < BSC; ++uu) {
        const int u = bb * BSC + uu;
        if constexpr (!HAS_BIAS) continue;  // FP formats: natural order, no bias sums
        if constexpr (BITS == 8) {
          // natural order: only the group sums; step e of the super-chunk
          // holds 8 codes of group (uu*SCW + 32e)/GS of the block
#pragma unroll
          for (int e = 0; e < XR; ++e) {
            const int j = (uu * SCW + 32 * e) / GS;
#pragma unroll
            for (int c = 0; c < 4; ++c) P[j] = dot2_bf16(xv[u][e][0][c], 0x3F803F80u, P[j]);
          }
          continue;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = uu * GPS + i / REGS_G;  // group within the block
#pragma unroll
          for (int l = 0; l < HS; ++l)
#pragma unroll
            for (int e = 0; e < 4; ++e) P[j] = dot2_bf16(xv[u][i][l][e], 0x3F803F80u, P[j]);
          if constexpr (BITS == 4) {
            const uint32_t X[4] = {xv[u][i][0][0], xv[u][i][0][1], xv[u][i][0][2], xv[u][i][0][3]};
            xv[u][i][0] = u32x4_t{xpair_stride4(X, 0), xpair_stride4(X, 1), xpair_stride4(X, 2),
                                  xpair_stride4(X, 3)};
          } else {
            const uint32_t X[8] = {xv[u][i][0][0], xv[u][i][0][1], xv[u][i][0][2], xv[u][i][0][3],
                                   xv[u][i][1][0], xv[u][i][1][1], xv[u][i][1][2], xv[u][i][1][3]};
#pragma unroll
            for (int h = 0; h < 2; ++h)
              xv[u][i][h] = u32x4_t{xpair_stride8(X, 4 * h + 0), xpair_stride8(X, 4 * h + 1),
                                    xpair_stride8(X, 4 * h + 2), xpair_stride8(X, 4 * h + 3)};
          }
        }
      }
      if constexpr (HAS_BIAS) xsum[bb] = rows_transpose_reduce4(P);
    }

    // ---- codes, super-chunk by super-chunk in load order
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
        transpose_rows_lvl<LVL>(cur[t]);
      }
      if constexpr (BITS == 8) {
        // MFMA step e takes code registers 2e, 2e+1 (8 consecutive codes of
        // this lane's row; the activations at xoff[2e]..+7)
#pragma unroll
        for (int e = 0; e < XR; ++e) {
          const int kk = scb * SCW + 32 * e;  // first code of the step within the block
          const int j = kk / GS;              // its group within the block
          const bool gfirst = kk % GS == 0;
          const bool glast = (kk + 32) % GS == 0;
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xv[u][e][0]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            u32x4_t bw;
            if constexpr (FMT == kMxfp8) {
              bw = u32x4_t{fp8_pair<false>(cur[t][2 * e]), fp8_pair<true>(cur[t][2 * e]),
                           fp8_pair<false>(cur[t][2 * e + 1]), fp8_pair<true>(cur[t][2 * e + 1])};
            } else {
              bw = unpack8_quad(cur[t][2 * e], cur[t][2 * e + 1]);
            }
            accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, bw), gfirst ? zero4 : accg[t], 0, 0, 0);
          }
          if (glast) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              float sc;
              if constexpr (HAS_BIAS) {
                const uint32_t sw = (j < 2) ? s4[u / BSC][t].x : s4[u / BSC][t].y;
                sc = half_bits_to_float((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
              } else {
                sc = fp_scale_to_float<FMT>(s4[u / BSC][t].x >> (8 * j));
              }
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[t][q] = fmaf(sc, accg[t][q], acc[t][q]);
            }
          }
        }
      }
      if constexpr (FMT == kNvfp4) {
        // register i holds elements 8kb..8kb+7 of chunk i (4x4 transpose), i.e.
        // 16-element block 2i + kb/2 of the super-chunk: scale them exactly and
        // accumulate straight into acc
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 2 * i + (kb >> 1);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xv[u][i][0]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint32_t sw = b < 4 ? s4[u / BSC][t].x : s4[u / BSC][t].y;
            const float sc = e4m3_to_float(sw >> (8 * (b & 3)));
            const u32x4_t bw = u32x4_t{fp4_pair_scaled<0>(cur[t][i], sc), fp4_pair_scaled<1>(cur[t][i], sc),
                                       fp4_pair_scaled<2>(cur[t][i], sc), fp4_pair_scaled<3>(cur[t][i], sc)};
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bw),
                                                              acc[t], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < (BITS == 8 || FMT == kNvfp4 ? 0 : 4); ++i) {
        const int j = scb * GPS + i / REGS_G;  // group within the block
#pragma unroll
        for (int h = 0; h < HS; ++h) {
          const bool gfirst = (i % REGS_G) == 0 && h == 0;
          const bool glast = (i % REGS_G) == REGS_G - 1 && h == HS - 1;
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xv[u][i][h]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            u32x4_t bw;
            if constexpr (FMT == kMxfp4) {
              // 8 elements of one dword, natural order
              bw = u32x4_t{fp4_pair<0>(cur[t][i]), fp4_pair<1>(cur[t][i]), fp4_pair<2>(cur[t][i]),
                           fp4_pair<3>(cur[t][i])};
            } else if constexpr (BITS == 4) {
              bw = unpack4_split_quad(cur[t][i], offset_pair);
            } else {
              bw = unpack2_split_quad(cur[t][i], h, offset_pair);
            }
            accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, bw), gfirst ? zero4 : accg[t], 0, 0, 0);
          }
          if (glast) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              float sc;
              if constexpr (HAS_BIAS) {
                const uint32_t sw = (j < 2) ? s4[u / BSC][t].x : s4[u / BSC][t].y;
                sc = half_bits_to_float((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
              } else {
                sc = fp_scale_to_float<FMT>(s4[u / BSC][t].x >> (8 * j));
              }
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[t][q] = fmaf(sc, accg[t][q], acc[t][q]);
            }
          }
        }
      }
      if (HAS_BIAS && scb == BSC - 1) {
        // bias with the 128 offset: acc += xsum[m][g0+kb] * (b - 128 s)[n][g0+kb]
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint32_t sw = (kb < 2) ? s4[u / BSC][t].x : s4[u / BSC][t].y;
          const uint32_t bw = (kb < 2) ? b4[u / BSC][t].x : b4[u / BSC][t].y;
          const float sc = half_bits_to_float((kb & 1) ? (sw >> 16) : (sw & 0xFFFFu));
          const float b = half_bits_to_float((kb & 1) ? (bw >> 16) : (bw & 0xFFFFu));
          const float bo = BITS == 8 ? b : fmaf(-128.f, sc, b);  // 2/4-bit: remove the 128 offset
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsum[u / BSC], bo, acc[t], 0, 0, 0);
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
  // output o of the tile group: sum over the slices, then store (pre: the
  // residual rv was prefetched)
  auto finish = [&](const int o, const bool pre, float rv) {
    const int t = o >> 8;
    const int i = (o >> 6) & 3;
    const int l = o & 63;
    float s = 0.f;
    for (int w = 0; w < waves; ++w) s += red[w][t][i][l];
    const int m = 4 * (l >> 4) + i;
    const int n = n_base + 16 * t + (l & 15);
    if (m < M && n < N) {
      float *dst = y + (size_t)m * N + n;
      if constexpr (ADD) {
        if (!pre) rv = res[(size_t)m * N + n];
      }
      if constexpr (KS == 1) {
        *dst = ADD ? s + rv : s;
      } else if constexpr (!ADD) {
        // y was zeroed before the launch and receives exactly two addends:
        // 0 + a + b equals 0 + b + a bit for bit, whichever half lands first
        unsafeAtomicAdd(dst, s);
      } else {
        // y held kSplitSentinel: the first half leaves its partial there, the
        // second finds it and stores (a + b) + r.  a + b and b + a are the same
        // float, so the result is the plain product's plus r, whichever half
        // lands first.
        const float old = atomicExch(dst, s);
        if (__builtin_bit_cast(uint32_t, old) != kSplitSentinel) *dst = (old + s) + rv;
      }
    }
  };
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int o = threadIdx.x + j * blockDim.x;
    if (o < NT * 256) finish(o, true, ADD ? rpre[j] : 0.f);
  }
  for (int o = threadIdx.x + NT * blockDim.x; o < NT * 256; o += blockDim.x) finish(o, false, 0.f);
  };

  if constexpr (PERSIST) {
    // Persistent workgroups: the grid holds as many workgroups as the device
    // runs at once, and each walks tile groups tg, tg + gridDim.x, ... so that
    // no partial last round of workgroups is left for a few CUs.
    for (int tg = blockIdx.x; tg < ngroups; tg += gridDim.x) {
      if (tg != (int)blockIdx.x) __syncthreads();  // reduction buffer drained
      group(tg);
    }
  } else {
    // one tile group per workgroup (all groups resident at once)
    group(blockIdx.x);
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
  static constexpr int SPI = (BITS == 4 && GS == 128 && NT == 1) ? 4 : 2;
  static constexpr int MAXT = (BITS == 4 && NT == 1 && GS <= 64) ? 1024 : 512;
};




// y[0..n) = v (bit pattern): zero before a K-split launch, kSplitSentinel
// before one with the residual sum
__global__ __launch_bounds__(256) void fill_kernel(uint32_t *__restrict__ y, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) y[i] = v;
}

template <int BITS, int GS, int NT, bool ADD, int FMT>
int launch_mfma_t(const QgemvArgs &a, hipStream_t stream) {
  constexpr int MAXT = MfmaShape<BITS, GS, NT>::MAXT;
  constexpr int SPI = MfmaShape<BITS, GS, NT>::SPI;
  const auto kern = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 1, true, ADD, FMT>;
  const auto kern1 = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 1, false, ADD, FMT>;
  const auto kern_s = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 2, true, ADD, FMT>;
  const auto kern1_s = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 2, false, ADD, FMT>;
  const int nblk = a.K / (4 * GS);
  const int tiles = (a.N + 15) / 16;
  const int cus = device_cu_count();
  // Few tile groups for the CUs: split K in two halves across workgroups
  // (added into y), for long K when there are under two groups per CU, and
  // for any K of at least 2048 when groups cover at most a quarter of the CUs.
  // Not for an in-place residual sum: y must be prefilled, which would erase
  // the residual.
  const int tgroups = (tiles + NT - 1) / NT;
  const bool in_place = ADD && static_cast<const void *>(a.res) == static_cast<const void *>(a.y);
  const int ksplit =
      !in_place && ((tgroups < 2 * cus && a.K >= 8192) || (4 * tgroups <= cus && a.K >= 2048)) ? 2
                                                                                                : 1;
  const int waves = pick_waves(nblk / ksplit, MAXT / 64);
  const int groups = (tiles + NT - 1) / NT * ksplit;
  if (ksplit == 2) {
    const size_t n = (size_t)a.M * a.N;
    const int fb = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(fill_kernel, dim3(fb), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t *>(a.y), n, ADD ? kSplitSentinel : 0u);
  }
  // workgroups resident at once for this block size (cached per wave count)
  static int occ_cache[MAXT / 64 + 1] = {0};
  int occ = occ_cache[waves];
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void *>(kern),
                                                     64 * waves, 0) != hipSuccess ||
        occ <= 0)
      occ = 1;
    occ_cache[waves] = occ;
  }
  const int slots = occ * cus;
  const bool single = groups <= slots;
  const auto k = ksplit == 1 ? (single ? kern1 : kern) : (single ? kern1_s : kern_s);
  hipLaunchKernelGGL(k, dim3(single ? groups : slots), dim3(64 * waves), 0, stream, a.codes,
                     a.scales, a.biases, a.x, a.y, a.res, a.M, a.N, a.K, groups);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

template <int BITS, int GS, int FMT = kAffine>
int launch_mfma_gs(const QgemvArgs &a, hipStream_t stream) {
  // more output columns per workgroup on wide matrices: every workgroup reads
  // all M*K activations, so wider groups cut that traffic per weight byte
  const int tiles = (a.N + 15) / 16;
  const int cus = device_cu_count();
  if (a.res) {
    if (tiles >= 2 * cus) return launch_mfma_t<BITS, GS, 2, true, FMT>(a, stream);
    return launch_mfma_t<BITS, GS, 1, true, FMT>(a, stream);
  }
  if (tiles >= 2 * cus) return launch_mfma_t<BITS, GS, 2, false, FMT>(a, stream);
  return launch_mfma_t<BITS, GS, 1, false, FMT>(a, stream);
}

}  // namespace

bool mfma_supports_fp(int K, int fmt) {
  (void)fmt;
  return K % 128 == 0;  // one 128-element block of bias blocks per super-chunk
}

bool mfma_supports(int K, int bits, int group_size) {
  if (bits == 2 && group_size < 64) return false;
  // 8-bit gs128: a bias block (4 groups) would be 8 super-chunks per batch,
  // beyond the register budget
  if (bits == 8 && group_size > 64) return false;
  const int scw = 512 / bits;  // codes per 64-byte super-chunk
  return K % scw == 0 && K % (4 * group_size) == 0;
}

int launch_mfma(const QgemvArgs &a, hipStream_t stream) {
  if (a.fmt != kAffine) {
    if (!mfma_supports_fp(a.K, a.fmt)) return QGEMV_EUNSUPPORTED;
    if (a.fmt == kMxfp4) return launch_mfma_gs<4, 32, kMxfp4>(a, stream);
    if (a.fmt == kNvfp4) return launch_mfma_gs<4, 32, kNvfp4>(a, stream);
    return launch_mfma_gs<8, 32, kMxfp8>(a, stream);
  }
  if (!mfma_supports(a.K, a.bits, a.group_size)) return QGEMV_EUNSUPPORTED;
  // more tiles than CUs: the persistent kernel streams several tiles per CU;
  // otherwise one tile group per workgroup in a single pass
  if ((a.N + 15) / 16 > device_cu_count()) {
    const int st = launch_persist(a, stream);
    if (st != QGEMV_EUNSUPPORTED) return st;
  }
  if (a.bits == 8) {
    switch (a.group_size) {
      case 32: return launch_mfma_gs<8, 32>(a, stream);
      case 64: return launch_mfma_gs<8, 64>(a, stream);
    }
  } else if (a.bits == 4) {
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
