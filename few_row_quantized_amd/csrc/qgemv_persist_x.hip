// Persistent bf16 MFMA path of the few-row quantized GEMV for long K
// (gfx950): activations staged in LDS, K split in two halves.
//
// Prior art on the pages: the few-row MMA kernels of "metal : few-row MMA
// mat-mul and batched copies for speculative decoding" (Overview: each weight
// dequantized once for all rows, K split across the simdgroups) and the
// split-K MMA variants on the MLX quantized_matmul small-M verify kernels page
// (Facts: dequantize per quantization group rather than per MMA tile; split K
// across the simdgroups).
//
// Why a third MFMA kernel: every 16-column tile needs all M*K activations.
// The single-pass kernel reads them from L2 again for every tile, which on
// the long down projections (K = 17408) moves more bytes into the CUs than
// the weights themselves once M reaches 4-8.  The register-resident
// persistent kernel reads them once per CU, but a wave holds at most one or
// two bias blocks of activations in registers, so K beyond ~6144 does not fit.
// Here the activations of one half of K live in LDS (160 KiB per CU on
// gfx950), read once per CU and re-read from LDS for every tile.
//
// CDNA4 design:
// * A persistent grid of one workgroup per CU.  Workgroup b takes half
//   b & 1 of the bias blocks (4 groups) of K and the contiguous range
//   [g*T/GP, (g+1)*T/GP) of the T 16-column tiles, g = b >> 1, GP = grid/2.
// * Prologue: the first tile's codes and metadata are requested, then the
//   workgroup copies its half of x (M rows) into LDS, already re-paired to
//   the code pairing of the MFMA operand (elements (e, e+4) of each 8 for
//   4-bit codes, (e, e+8) of each 16 for 2-bit codes), and forms the
//   activation sum of every group of that half from the registers: the
//   lanes holding a group's units reduce their sums by a fixed butterfly
//   (summing a group from LDS instead, one lane per group, put every lane of
//   a wave on the same bank: row offsets of GS*2 bytes).
// * Wave w owns the bias blocks w, w+W, ... of the half.  For each tile its
//   codes and metadata come through a register ring of S slots (the next
//   tile's loads are in flight while the current one is multiplied); the
//   activation operand of each v_mfma_f32_16x16x32_bf16 is one 16-byte LDS
//   read per lane (rows m >= M read row M-1: their outputs are never
//   stored).  Unpack, scale fold and the bias product
//   (v_mfma_f32_16x16x4_f32 against the group sums) are those of the other
//   MFMA kernels.
// * Every S tiles the waves' partial tiles are summed through LDS in block
//   order and each half is added into y with a float atomic; y was zeroed
//   before the launch and receives exactly two addends, so 0 + a + b and
//   0 + b + a are the same float: deterministic, and row m of an M-row call
//   equals the M = 1 call bit for bit.
// * Fused residual sum (ADD, "metal : few-row MMA mat-mul and batched copies
//   for speculative decoding", Overview: MUL_MAT + ADD writes the residual
//   sum from the store): y is prefilled with kSplitSentinel; the first half
//   to land leaves its partial, the second stores (a + b) + r.

#include "qgemv_device.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

constexpr int kXMaxWaves = 12;  // register budget: 768-thread workgroups
constexpr int kXRing = 2;       // slots of the code prefetch ring

template <int BITS, int GS, int BPW, bool ADD>
__global__ __launch_bounds__(64 * kXMaxWaves) void qgemv_persist_x_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *__restrict__ y,
    const float *__restrict__ res, int M, int N, int K) {
  constexpr int S = kXRing;
  constexpr int CW = 128 / BITS;         // codes per 16-byte chunk
  constexpr int SCW = 4 * CW;            // codes per 64-byte super-chunk
  constexpr int DW = CW / 4;             // codes per dword
  constexpr int HS = BITS == 4 ? 1 : 2;  // MFMA steps per code dword
  constexpr int BLKW = 4 * GS;           // codes per bias block
  constexpr int BSC = BLKW / SCW;        // super-chunks per block
  constexpr int CPG = GS / CW;           // chunks per group
  constexpr int GPS = 4 / CPG;           // groups per super-chunk
  constexpr int LVL = CPG >= 4 ? 0 : (CPG == 2 ? 1 : 2);
  constexpr int REGS_G = CPG;
  constexpr int UE = BITS == 4 ? 8 : 16;  // elements of one re-pairing unit
  constexpr int GU = GS / UE;             // units per group (a power of two <= 16)
  // staging units per thread per round: their registers are live next to
  // ring slot 0, so at most 32 VGPRs, 16 when the slot holds 8 super-chunks
  constexpr int XU = (BPW * BSC >= 8 ? 4 : 8) / (UE / 8);
  static_assert(BSC >= 1 && BLKW % SCW == 0 && CPG >= 1 && (BITS == 2 || BITS == 4), "layout");
  static_assert(GU >= 1 && GU <= 64 && (GU & (GU - 1)) == 0, "group lanes");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int col = lane & 15;
  const int kb = lane >> 4;
  const int NBLK = K / BLKW;
  const size_t RB = (size_t)K * BITS / 8;
  const int NG = K / GS;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t offset_pair = opaque_u32(kOffsetPair);

  // half of K and tile range of this workgroup (products stay below 2^31:
  // the grid is at most twice the CU count and T <= 2^18)
  const int part = (int)(blockIdx.x & 1u);
  const int GP = (int)(gridDim.x >> 1);
  const int gp = (int)(blockIdx.x >> 1);
  const int p_lo = part ? NBLK >> 1 : 0;
  const int nbp = part ? NBLK - (NBLK >> 1) : NBLK >> 1;  // blocks of this half
  const int nbp_max = NBLK - (NBLK >> 1);
  const int T = (N + 15) >> 4;
  const int t_first = (int)((unsigned)gp * (unsigned)T / (unsigned)GP);
  const int ntile = (int)((unsigned)(gp + 1) * (unsigned)T / (unsigned)GP) - t_first;

  // LDS: x rows of the half (re-paired bf16, padded pitch), group sums, and
  // the partial tiles of the waves
  extern __shared__ uint4 lds[];
  const int pitch = nbp_max * BLKW * 2 + 16;  // bytes per activation row
  const int gpr = nbp_max * 4;                // group sums per row
  uint8_t *xl = reinterpret_cast<uint8_t *>(lds);
  float *xs = reinterpret_cast<float *>(xl + (size_t)M * pitch);
  float *red = xs + (size_t)M * gpr;  // [S][W][4][64]

  int xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xoff[i] = lvl_chunk<LVL>(i, kb) * CW + lvl_dword<LVL>(i, kb) * DW;

  // owned blocks (index within the half); a wave past the last block loads a
  // valid block and skips the arithmetic
  int lb[BPW];
  bool own[BPW];
#pragma unroll
  for (int k = 0; k < BPW; ++k) {
    own[k] = wave + k * W < nbp;
    lb[k] = own[k] ? wave + k * W : nbp - 1;
  }

  // ---- prefetch ring of codes and metadata.  Issues past the last tile are
  // still made (a branch around loads would make the compiler wait for every
  // load in flight), but then read the first line of the workgroup's first
  // tile: one cached line per instruction.
  u32x4_t cv[S][BPW][BSC];
  uint2 s4[S][BPW], b4[S][BPW];
  const uint64_t crow_dead = (uint64_t)(16 * t_first) * RB;
  const uint64_t mrow_dead = (uint64_t)(16 * t_first) * NG;
  int it = 0;  // tile step of the next issue
  auto issue = [&](const int slot) {
    const uint64_t m64 = 0ull - (uint64_t)(it < ntile);  // all-ones while live
    const int n = min(16 * (t_first + it) + col, N - 1);
    const uint64_t crow = (((uint64_t)n * RB + kb * 16) & m64) | (crow_dead & ~m64);
    const uint64_t mrow = (((uint64_t)n * NG) & m64) | (mrow_dead & ~m64);
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
#pragma unroll
      for (int u = 0; u < BSC; ++u)
        cv[slot][k][u] = load_stream_u32x4(codes + crow + (size_t)((p_lo + lb[k]) * BSC + u) * 64);
    }
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      s4[slot][k] = *reinterpret_cast<const uint2 *>(scales + mrow + (p_lo + lb[k]) * 4);
      b4[slot][k] = *reinterpret_cast<const uint2 *>(biases + mrow + (p_lo + lb[k]) * 4);
    }
    ++it;
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);

  // ---- stage x of the half into LDS, re-paired, XU units per thread at a
  // time (all loads of a round issued before any is used; clamped indices
  // read a valid unit and are not stored)
  {
    const int upr = nbp * BLKW / UE;  // units per row
    const int units = M * upr;
    const uint16_t *xh = x + (size_t)p_lo * BLKW;
    const int rot = 0;  // unit order (a whole number of groups)
    auto unit_of = [&](int uu) { return uu + rot < units ? uu + rot : uu + rot - units; };
    for (int u0 = 0; u0 < units; u0 += XU * (int)blockDim.x) {
      u32x4_t v[XU][UE / 8];
#pragma unroll
      for (int j = 0; j < XU; ++j) {
        const int u = unit_of(min(u0 + j * (int)blockDim.x + (int)threadIdx.x, units - 1));
        const int m = u / upr;
        const int c = u - m * upr;
#pragma unroll
        for (int h = 0; h < UE / 8; ++h)
          v[j][h] = *reinterpret_cast<const u32x4_t *>(xh + (size_t)m * K + (size_t)c * UE + 8 * h);
      }
#pragma unroll
      for (int j = 0; j < XU; ++j) {
        const int uu = u0 + j * (int)blockDim.x + (int)threadIdx.x;
        // activation sum of the unit, then of its group: units are dealt to
        // consecutive lanes, so the GU lanes of a group add their sums in a
        // fixed butterfly (every lane of the wave takes part)
        float p = 0.f;
#pragma unroll
        for (int h = 0; h < UE / 8; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) p = dot2_bf16(v[j][h][e], 0x3F803F80u, p);
#pragma unroll
        for (int off = 1; off < GU; off <<= 1) p += __shfl_xor(p, off);
        if (uu < units) {
          const int u = unit_of(uu);
          const int m = u / upr;
          const int c = u - m * upr;
          if ((threadIdx.x & (GU - 1)) == 0) xs[m * gpr + c / GU] = p;
          u32x4_t *dst = reinterpret_cast<u32x4_t *>(xl + (size_t)m * pitch + (size_t)c * UE * 2);
          if constexpr (BITS == 4) {
            const uint32_t X[4] = {v[j][0][0], v[j][0][1], v[j][0][2], v[j][0][3]};
            dst[0] = u32x4_t{xpair_stride4(X, 0), xpair_stride4(X, 1), xpair_stride4(X, 2),
                             xpair_stride4(X, 3)};
          } else {
            const uint32_t X[8] = {v[j][0][0], v[j][0][1], v[j][0][2], v[j][0][3],
                                   v[j][1][0], v[j][1][1], v[j][1][2], v[j][1][3]};
#pragma unroll
            for (int h = 0; h < 2; ++h)
              dst[h] = u32x4_t{xpair_stride8(X, 4 * h + 0), xpair_stride8(X, 4 * h + 1),
                               xpair_stride8(X, 4 * h + 2), xpair_stride8(X, 4 * h + 3)};
          }
        }
      }
    }
    __syncthreads();
  }

  // this lane's activation row in LDS (rows m >= M read row M-1)
  const uint8_t *xrow = xl + (size_t)(col < M ? col : M - 1) * pitch;
  const float *xsrow = xs + (col < M ? col : M - 1) * gpr;

  // ---- groups of S tile steps (the unrolled ring); a range always has a
  // tile (do-while: no guard branch that would let the compiler sink the
  // prologue loads)
  int j0 = 0;
  do {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (j0 + s >= ntile) break;
      issue((s + S - 1) % S);
      __builtin_amdgcn_sched_barrier(0);

      f32x4_t acc = zero4;
#pragma unroll
      for (int k = 0; k < BPW; ++k) {
        if (!own[k]) continue;  // uniform per wave
        f32x4_t accg;
#pragma unroll
        for (int u = 0; u < BSC; ++u) {
          uint32_t cur[4] = {cv[s][k][u][0], cv[s][k][u][1], cv[s][k][u][2], cv[s][k][u][3]};
          transpose_rows_lvl<LVL>(cur);
          const int k0 = (lb[k] * BSC + u) * SCW;  // first element of the super-chunk in the half
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jg = u * GPS + i / REGS_G;  // group within the block
#pragma unroll
            for (int h = 0; h < HS; ++h) {
              const bool gfirst = (i % REGS_G) == 0 && h == 0;
              const bool glast = (i % REGS_G) == REGS_G - 1 && h == HS - 1;
              const u32x4_t av = *reinterpret_cast<const u32x4_t *>(xrow + (size_t)(k0 + xoff[i] + 8 * h) * 2);
              u32x4_t bw;
              if constexpr (BITS == 4) {
                bw = unpack4_split_quad(cur[i], offset_pair);
              } else {
                bw = unpack2_split_quad(cur[i], h, offset_pair);
              }
              accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                            __builtin_bit_cast(bf16x8_t, bw),
                                                            gfirst ? zero4 : accg, 0, 0, 0);
              if (glast) {
                const uint32_t sw = (jg < 2) ? s4[s][k].x : s4[s][k].y;
                const float scl = half_bits_to_float((jg & 1) ? (sw >> 16) : (sw & 0xFFFFu));
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = fmaf(scl, accg[q], acc[q]);
              }
            }
          }
        }
        // bias with the 128 offset: acc += xsum[m][g0+kb] * (b - 128 s)[n][g0+kb]
        const uint32_t sw = (kb < 2) ? s4[s][k].x : s4[s][k].y;
        const uint32_t bw = (kb < 2) ? b4[s][k].x : b4[s][k].y;
        const float scl = half_bits_to_float((kb & 1) ? (sw >> 16) : (sw & 0xFFFFu));
        const float b = half_bits_to_float((kb & 1) ? (bw >> 16) : (bw & 0xFFFFu));
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsrow[lb[k] * 4 + kb], fmaf(-128.f, scl, b), acc,
                                                   0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((s * W + wave) * 4 + i) * 64 + lane] = acc[i];
    }

    // ---- sum the partial tiles over the waves in block order and add this
    // half into y
    __syncthreads();
    const int nj = min(S, ntile - j0);
    for (int o = threadIdx.x; o < nj * 256; o += blockDim.x) {
      const int s = o >> 8, i = (o >> 6) & 3, l = o & 63;
      float v = 0.f;
      for (int w = 0; w < W; ++w) v += red[((s * W + w) * 4 + i) * 64 + l];
      const int m = 4 * (l >> 4) + i;
      const int n = 16 * (t_first + j0 + s) + (l & 15);
      if (m < M && n < N) {
        float *dst = y + (size_t)m * N + n;
        if constexpr (!ADD) {
          unsafeAtomicAdd(dst, v);
        } else {
          const float old = atomicExch(dst, v);
          if (__builtin_bit_cast(uint32_t, old) != kSplitSentinel) *dst = (old + v) + res[(size_t)m * N + n];
        }
      }
    }
    __syncthreads();  // red is rewritten by the next group
    j0 += S;
  } while (j0 < ntile);
}

// Blocks owned per wave: 4 super-chunks per ring slot, or 8 where a block is
// 4 super-chunks (4-bit gs128: still within the register budget; with
// smaller blocks 8 super-chunks bring twice the metadata registers and
// spill).  Halves of K that need more waves take the single-pass kernel.
template <int BITS, int GS>
struct PersistXShape {
  static constexpr int BSC = 4 * GS / (512 / BITS);
  static constexpr int BPW_NARROW = BSC >= 4 ? 1 : 4 / BSC;
  static constexpr int BPW_WIDE = BSC == 4 ? 2 : BPW_NARROW;
};

template <int BITS, int GS, int BPW, bool ADD>
int launch_persist_x_k(const QgemvArgs &a, int waves, int grid, size_t lds, hipStream_t stream) {
  const auto kern = qgemv_persist_x_kernel<BITS, GS, BPW, ADD>;
  if (!allow_max_dynamic_lds(reinterpret_cast<const void *>(kern))) return QGEMV_EHIP;
  const int st = launch_fill(a.y, (size_t)a.M * a.N, ADD ? kSplitSentinel : 0u, stream);
  if (st != QGEMV_OK) return st;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), lds, stream, a.codes, a.scales, a.biases, a.x,
                     a.y, a.res, a.M, a.N, a.K);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

template <int BITS, int GS, bool ADD>
int launch_persist_x_t(const QgemvArgs &a, hipStream_t stream) {
  using Sh = PersistXShape<BITS, GS>;
  const int nblk = a.K / (4 * GS);
  if (nblk < 2) return QGEMV_EUNSUPPORTED;
  const int nbp_max = nblk - nblk / 2;
  const int tiles = (a.N + 15) / 16;
  const int cus = device_cu_count();
  if (tiles < cus) return QGEMV_EUNSUPPORTED;
  const bool narrow = (nbp_max + Sh::BPW_NARROW - 1) / Sh::BPW_NARROW <= kXMaxWaves;
  const int bpw = narrow ? Sh::BPW_NARROW : Sh::BPW_WIDE;
  const int waves = (nbp_max + bpw - 1) / bpw;
  if (waves > kXMaxWaves) return QGEMV_EUNSUPPORTED;
  const size_t pitch = (size_t)nbp_max * 4 * GS * 2 + 16;
  const size_t lds = (size_t)a.M * pitch + (size_t)a.M * nbp_max * 4 * sizeof(float) +
                     (size_t)kXRing * waves * 256 * sizeof(float);
  if (lds > kLdsMax) return QGEMV_EUNSUPPORTED;
  // one workgroup per CU, half of them per half of K (every workgroup has
  // at least one tile: tiles >= CUs)
  const int grid = 2 * (cus / 2);
  if (narrow) return launch_persist_x_k<BITS, GS, Sh::BPW_NARROW, ADD>(a, waves, grid, lds, stream);
  return launch_persist_x_k<BITS, GS, Sh::BPW_WIDE, ADD>(a, waves, grid, lds, stream);
}

template <int BITS, int GS>
int launch_persist_x_gs(const QgemvArgs &a, hipStream_t stream) {
  return a.res ? launch_persist_x_t<BITS, GS, true>(a, stream) : launch_persist_x_t<BITS, GS, false>(a, stream);
}

}  // namespace

int launch_persist_x(const QgemvArgs &a, hipStream_t stream) {
  if (a.fmt != kAffine || !mfma_supports(a.K, a.bits, a.group_size)) return QGEMV_EUNSUPPORTED;
  // an in-place residual sum cannot be prefilled
  if (a.res && static_cast<const void *>(a.res) == static_cast<const void *>(a.y)) return QGEMV_EUNSUPPORTED;
  if (a.bits == 4) {
    switch (a.group_size) {
      case 32: return launch_persist_x_gs<4, 32>(a, stream);
      case 64: return launch_persist_x_gs<4, 64>(a, stream);
      case 128: return launch_persist_x_gs<4, 128>(a, stream);
    }
  } else if (a.bits == 2) {
    switch (a.group_size) {
      case 64: return launch_persist_x_gs<2, 64>(a, stream);
      case 128: return launch_persist_x_gs<2, 128>(a, stream);
    }
  }
  return QGEMV_EUNSUPPORTED;
}

}  // namespace qgemv
