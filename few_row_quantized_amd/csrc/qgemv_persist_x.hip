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
// gfx950), read once per CU and re-read from LDS for every tile; when a half
// does not fit (M above 7 at K = 17408), the half is walked in P phases,
// each restaging its share of the activations.
//
// CDNA4 design:
// * A persistent grid of one workgroup per CU.  Workgroup b takes half
//   b & 1 of the bias blocks (4 groups) of K and the contiguous range
//   [g*T/GP, (g+1)*T/GP) of the T 16-column tiles, g = b >> 1, GP = grid/2.
// * Phase q covers the blocks [q*nb/P, (q+1)*nb/P) of the half; wave w owns
//   its blocks lo+w, lo+w+W, ... and reads activations only from their LDS
//   columns.  So each wave stages its own blocks (prologue and each phase
//   change, after the next step's codes and metadata are requested): the M
//   rows of its blocks are copied into LDS, already re-paired to the code
//   pairing of the MFMA operand (elements (0,2), (1,3), (4,6), (5,7) of each
//   8 for 4-bit codes, (e, e+4) of each 8 for 2-bit codes), with the
//   activation sum of every group formed from the registers (the lanes
//   holding a group's units reduce their sums by a fixed butterfly; summing
//   a group from LDS instead, one lane per group, put every lane of a wave
//   on the same bank: row offsets of GS*2 bytes).  No workgroup barrier
//   orders the staging: a wave starts its first step as soon as its own
//   blocks are staged and restages its columns when it leaves a phase (27B
//   down projection, K = 17408: 19.3 -> 17.9 us at M = 1, 25.9 -> 21.6 at
//   M = 8, 31.2 -> 24.3 at M = 12, against a workgroup-wide staging with a
//   barrier at each phase change).
// * The workgroup walks (phase, tile) steps in
//   phase-major order; each step's codes and metadata come through a
//   register ring of S slots (the next step's loads are in flight while the
//   current one is multiplied, also across a phase change; codes as whole
//   128-byte lines where a bias block holds an even number of 64-byte
//   super-chunks, as in the register-resident persistent kernel); the
//   activation operand of each v_mfma_f32_16x16x32_bf16 is one 16-byte LDS
//   read per lane (rows m >= M read row M-1: their outputs are never
//   stored).  Unpack, scale fold, the bias product (v_mfma_f32_16x16x4_f32
//   against the group sums) and the zero-weight flags are those of the
//   other MFMA kernels.
// * Each wave adds its partial 16x16 tile of a step into an LDS slot of its
//   own per tile (no barrier between steps); after the last step the slots
//   are summed over the waves in block order and each half is added into y
//   with a float atomic.  y was zeroed before the launch and receives exactly
//   two addends, so 0 + a + b and 0 + b + a are the same float:
//   deterministic, and row m of an M-row call equals the M = 1 call bit for
//   bit whenever both take the same number of phases (the phase count and
//   the waves' blocks depend on M through the LDS budget).
// * Fused residual sum (ADD, "metal : few-row MMA mat-mul and batched copies
//   for speculative decoding", Overview: MUL_MAT + ADD writes the residual
//   sum from the store): y is prefilled with kSplitSentinel; the first half
//   to land leaves its partial, the second stores (a + b) + r.

#include <type_traits>

#include "qgemv_device.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

constexpr int kXMaxWaves = 12;  // register budget: 768-thread workgroups
constexpr int kXRing = 2;       // slots of the code prefetch ring
// passes over the half of K (activations restaged per pass): a third pass
// was slower than the single-pass kernel (4-bit down projection, M = 16:
// 36.6 against 35.8 us)
constexpr int kXMaxPhases = 2;

template <int BITS, int GS, int BPW, bool ADD>
__global__ __launch_bounds__(64 * kXMaxWaves) void qgemv_persist_x_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *__restrict__ y,
    const float *__restrict__ res, int M, int N, int K, int P, int ntile_max) {
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
  // metadata loads in the quad-row layout: measured faster for 4-bit codes
  // with groups of 32 or 64 (FFN-up 4096x12288: 14.2 -> 13.2 us and
  // 11.3 -> 10.6 us at M = 8), slower by 1-5% with groups of 128 and for
  // 2-bit codes, where metadata loads are few
  constexpr bool MQ = BITS == 4 && GS <= 64;
  constexpr int UE = BITS == 4 ? 8 : 16;  // elements of one re-pairing unit
  constexpr int GU = GS / UE;             // units per group (a power of two <= 16)
  static_assert(BSC >= 1 && BLKW % SCW == 0 && CPG >= 1 && (BITS == 2 || BITS == 4), "layout");
  // codes of two consecutive super-chunks as whole 128-byte lines (8 rows per
  // load, pair_to_operand_lanes) where a block has an even number of them;
  // otherwise lane quads on 64 bytes (to_operand_lanes)
  constexpr bool LINES = BSC % 2 == 0;
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

  // half of K and tile range of this workgroup (products stay below 2^31:
  // the grid is at most twice the CU count and T <= 2^18)
  const int part = (int)(blockIdx.x & 1u);
  const int GP = (int)(gridDim.x >> 1);
  const int gp = (int)(blockIdx.x >> 1);
  const int p_lo = part ? NBLK >> 1 : 0;
  const int nbp = part ? NBLK - (NBLK >> 1) : NBLK >> 1;  // blocks of this half
  const int nbp_max = NBLK - (NBLK >> 1);
  const int nbq_max = (nbp_max + P - 1) / P;  // blocks of the longest phase
  const int T = (N + 15) >> 4;
  const int t_first = (int)((unsigned)gp * (unsigned)T / (unsigned)GP);
  const int ntile = (int)((unsigned)(gp + 1) * (unsigned)T / (unsigned)GP) - t_first;
  const int steps = P * ntile;  // (phase, tile) steps, phase-major

  // LDS: x rows of the phase (re-paired bf16, padded pitch), its group sums,
  // and one partial 16x16 tile per (tile, wave), added to over the phases
  extern __shared__ uint4 lds[];
  const int pitch = nbq_max * BLKW * 2 + 16;  // bytes per activation row
  const int gpr = nbq_max * 4;                // group sums per row
  uint8_t *xl = reinterpret_cast<uint8_t *>(lds);
  float *xs = reinterpret_cast<float *>(xl + (size_t)M * pitch);
  float *pacc = xs + (size_t)M * gpr;  // [ntile_max][W][4][64]

  int xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xoff[i] = lvl_chunk<LVL>(i, kb) * CW + lvl_dword<LVL>(i, kb) * DW;

  // phase q takes the blocks [q*nbp/P, (q+1)*nbp/P) of the half; slot k of a
  // wave is its block lo + wave + k*W (a wave past the phase's last block
  // loads a valid block and skips the arithmetic)
  auto phase_lo = [&](int q) { return q * nbp / P; };
  auto owned = [&](int q, int k, int &blk) {
    const int lo = phase_lo(q);
    const int nbq = phase_lo(q + 1) - lo;
    const bool o = wave + k * W < nbq;
    blk = lo + (o ? wave + k * W : nbq - 1);
    return o;
  };

  // ---- prefetch ring of codes and metadata, one (phase, tile) step per
  // slot.  Issues past the last step are still made (a branch around loads
  // would make the compiler wait for every load in flight), but then read
  // the first line of the workgroup's first tile: one cached line per
  // instruction.
  u32x4_t cv[S][BPW][BSC];
  uint2 s4[S][BPW], b4[S][BPW];
  const uint64_t crow_dead = (uint64_t)(16 * t_first) * RB;
  const uint64_t mrow_dead = (uint64_t)(16 * t_first) * NG;
  int it = 0;  // step of the next issue
  auto issue = [&](const int slot) {
    const bool live = it < steps;
    const int q = live ? it / ntile : 0;
    const int tt = live ? it - q * ntile : 0;
    const uint64_t m64 = 0ull - (uint64_t)live;  // all-ones while live
    // codes: whole 128-byte lines (LINES: lane L on piece L%8 of row L/8,
    // rows 8-15 in a second load) or lane quads (piece L%4 of row L/4, see
    // quad_row_lane); metadata in lane quads where groups are small (MQ),
    // else per column
    const int nq = min(16 * (t_first + tt) + (lane >> 2), N - 1);
    const int nl = min(16 * (t_first + tt) + (lane >> 3), N - 1);      // LINES: rows 0-7
    const int nl8 = min(16 * (t_first + tt) + 8 + (lane >> 3), N - 1);  // rows 8-15
    const uint64_t crow = LINES ? (((uint64_t)nl * RB + (lane & 7) * 16) & m64) | (crow_dead & ~m64)
                                : (((uint64_t)nq * RB + (lane & 3) * 16) & m64) | (crow_dead & ~m64);
    const uint64_t crow8 = (((uint64_t)nl8 * RB + (lane & 7) * 16) & m64) | (crow_dead & ~m64);
    const int nm = MQ ? nq : min(16 * (t_first + tt) + col, N - 1);
    const uint64_t mrow = (((uint64_t)nm * NG) & m64) | (mrow_dead & ~m64);
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      int blk;
      owned(q, k, blk);
#pragma unroll
      for (int u = 0; u < BSC; ++u) {
        if constexpr (LINES)
          cv[slot][k][u] =
              load_stream_u32x4(codes + ((u & 1) ? crow8 : crow) + (size_t)((p_lo + blk) * BSC + (u & ~1)) * 64);
        else
          cv[slot][k][u] = load_stream_u32x4(codes + crow + (size_t)((p_lo + blk) * BSC + u) * 64);
      }
      s4[slot][k] = *reinterpret_cast<const uint2 *>(scales + mrow + (p_lo + blk) * 4);
      b4[slot][k] = *reinterpret_cast<const uint2 *>(biases + mrow + (p_lo + blk) * 4);
    }
    ++it;
  };

  // ---- stage this wave's blocks of phase q into LDS (every row), re-paired,
  // with the activation sum of every group; the other waves neither read nor
  // write these columns, so no workgroup barrier is needed.  The wave's units
  // (block, row, unit) are taken 64 at a time, XB rounds per batch (then
  // smaller batches for the rest); a group's units are on consecutive lanes.
  constexpr int UPB = BLKW / UE;                      // units per block row
  // rounds per batch: their registers are live next to one ring slot (32
  // VGPRs, 16 with 4-block slots)
  constexpr int XB = (BPW >= 4 ? 4 : 8) / (UE / 8);
  auto stage_wave = [&](const int q) {
    const int lo = phase_lo(q);
    const int nbq = phase_lo(q + 1) - lo;
    int kown = 0;  // blocks of this wave in the phase (a prefix of its slots)
#pragma unroll
    for (int k = 0; k < BPW; ++k) kown += wave + k * W < nbq ? 1 : 0;
    const int per_blk = M * UPB;
    const int units = kown * per_blk;
    const int rounds = (units + 63) >> 6;
    const uint16_t *xh = x + (size_t)(p_lo + lo) * BLKW;
    // unit t -> LDS unit column c of row m (slot k's block is lq = wave + k*W)
    auto locate = [&](const int t, int &m, int &c) {
      int rem = t, k = 0;
#pragma unroll
      for (int kk = 1; kk < BPW; ++kk) {
        if (rem >= per_blk) {
          rem -= per_blk;
          ++k;
        }
      }
      m = rem / UPB;
      c = (wave + k * W) * UPB + (rem - m * UPB);
    };
    auto batch = [&](auto nb_tag, const int r0) {
      constexpr int NB = decltype(nb_tag)::value;
      u32x4_t v[NB][UE / 8];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        int m, c;
        locate(min((r0 + j) * 64 + lane, units - 1), m, c);
#pragma unroll
        for (int h = 0; h < UE / 8; ++h)
          v[j][h] = *reinterpret_cast<const u32x4_t *>(xh + (size_t)m * K + (size_t)c * UE + 8 * h);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int t = (r0 + j) * 64 + lane;
        float pp = 0.f;
#pragma unroll
        for (int h = 0; h < UE / 8; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) pp = dot2_bf16(v[j][h][e], 0x3F803F80u, pp);
#pragma unroll
        for (int off = 1; off < GU; off <<= 1) pp += __shfl_xor(pp, off);
        if (t < units) {
          int m, c;
          locate(t, m, c);
          if ((lane & (GU - 1)) == 0) xs[m * gpr + c / GU] = pp;
          u32x4_t *dst = reinterpret_cast<u32x4_t *>(xl + (size_t)m * pitch + (size_t)c * UE * 2);
#pragma unroll
          for (int h = 0; h < UE / 8; ++h) dst[h] = pair_activations<BITS>(v[j][h]);
        }
      }
    };
    int r = 0;
    for (; r + XB <= rounds; r += XB) batch(std::integral_constant<int, XB>{}, r);
    if constexpr (XB > 4) {
      if (r + 4 <= rounds) {
        batch(std::integral_constant<int, 4>{}, r);
        r += 4;
      }
    }
    if constexpr (XB > 2) {
      if (r + 2 <= rounds) {
        batch(std::integral_constant<int, 2>{}, r);
        r += 2;
      }
    }
    if (r < rounds) batch(std::integral_constant<int, 1>{}, r);
  };

  // this lane's activation row in LDS (rows m >= M read row M-1)
  const uint8_t *xrow = xl + (size_t)(col < M ? col : M - 1) * pitch;
  const float *xsrow = xs + (col < M ? col : M - 1) * gpr;

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);

  // ---- the steps, S at a time (the unrolled ring); a workgroup always has a
  // step (do-while: no guard branch that would let the compiler sink the
  // prologue loads)
  int j0 = 0;
  do {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int step = j0 + s;
      if (step >= steps) break;
      const int q = step / ntile;
      const int tt = step - q * ntile;
      if (tt == 0) stage_wave(q);
      issue((s + S - 1) % S);
      __builtin_amdgcn_sched_barrier(0);

      const int lo = phase_lo(q);
      f32x4_t acc = zero4;
      // traces of nonzero weights in this lane's quarter of the column (see
      // zero weights in qgemv_device.h)
      uint32_t nz = 0u;
      if constexpr (MQ) {
#pragma unroll
        for (int k = 0; k < BPW; ++k) {
          s4[s][k] = to_operand_lanes(s4[s][k]);
          b4[s][k] = to_operand_lanes(b4[s][k]);
        }
      }
#pragma unroll
      for (int k = 0; k < BPW; ++k) {
        int blk;
        if (!owned(q, k, blk)) continue;  // uniform per wave
        const int lq = blk - lo;          // block within the phase
        f32x4_t accg;
        uint32_t zc0 = 0u;  // the current group's first code word
#pragma unroll
        for (int u = 0; u < BSC; ++u) {
          uint32_t cur[4];
          if constexpr (LINES) {
            if (u & 1)
              pair_to_operand_lanes<1>(cv[s][k][u & ~1], cv[s][k][u | 1], cur);
            else
              pair_to_operand_lanes<0>(cv[s][k][u & ~1], cv[s][k][u | 1], cur);
          } else {
            to_operand_lanes(cv[s][k][u], cur);
          }
          transpose_rows_lvl<LVL>(cur);
          const int k0 = (lq * BSC + u) * SCW;  // first element of the super-chunk in the phase
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jg = u * GPS + i / REGS_G;  // group within the block
#pragma unroll
            for (int h = 0; h < HS; ++h) {
              const bool gfirst = (i % REGS_G) == 0 && h == 0;
              const bool glast = (i % REGS_G) == REGS_G - 1 && h == HS - 1;
              const u32x4_t av = *reinterpret_cast<const u32x4_t *>(xrow + (size_t)(k0 + xoff[i] + 8 * h) * 2);
              if (h == 0) {
                // zero-weight traces: code words against the group's first,
                // then the group's weight s*c + b at its last word
                if (gfirst) {
                  zc0 = cur[i];
                  nz |= fields_spread<BITS>(cur[i]);
                } else {
                  nz |= cur[i] ^ zc0;
                }
                pin(nz);
                if ((i % REGS_G) == REGS_G - 1) {
                  const uint2 sw_v = s4[s][k];
                  const uint2 bw16_v = b4[s][k];
                  nz |= weight_trace(half_bits_to_float(field16(sw_v, jg)), low_field<BITS>(zc0),
                                     half_bits_to_float(field16(bw16_v, jg)));
                }
              }
              const u32x4_t bw = BITS == 4 ? unpack4_quad(cur[i]) : unpack2_quad(cur[i], h);
              accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                            __builtin_bit_cast(bf16x8_t, bw),
                                                            gfirst ? zero4 : accg, 0, 0, 0);
              if (glast) {
                const uint2 sw_v = s4[s][k];
                const float scl = half_bits_to_float(field16(sw_v, jg));
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) acc[qq] = fmaf(scl, accg[qq], acc[qq]);
              }
            }
          }
        }
        // bias: acc += xsum[m][g0+kb] * b[n][g0+kb]
        const uint2 bw_v = b4[s][k];
        const float b = half_bits_to_float(field16(bw_v, kb));
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsrow[lq * 4 + kb], b, acc, 0, 0, 0);
      }
      // this wave's partial of tile tt: its own LDS slot, added to over the
      // phases in phase order
      float *pa = pacc + (size_t)((tt * W + wave) * 4) * 64 + lane;
      // a partial whose column held only zero weights is exactly 0
      const uint32_t keep = keep_mask(column_or(nz));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = unless_zero(acc[i], keep);
        pa[i * 64] = q == 0 ? a : pa[i * 64] + a;
      }
    }
    j0 += S;
  } while (j0 < steps);

  // ---- sum each tile's partials over the waves in block order and add this
  // half into y
  __syncthreads();
  for (int o = threadIdx.x; o < ntile * 256; o += blockDim.x) {
    const int t = o >> 8, i = (o >> 6) & 3, l = o & 63;
    float v = 0.f;
    for (int w = 0; w < W; ++w) v += pacc[((t * W + w) * 4 + i) * 64 + l];
    const int m = 4 * (l >> 4) + i;
    const int n = 16 * (t_first + t) + (l & 15);
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
}

// Blocks owned per wave: 4 super-chunks per ring slot, or 8 where a block is
// 4 super-chunks (4-bit gs128: still within the register budget; with
// smaller blocks 8 super-chunks bring twice the metadata registers and
// spill), or 2 where a block is one super-chunk.  The launcher takes the
// fewest blocks per wave (the most waves) that stay within kXMaxWaves.
template <int BITS, int GS>
struct PersistXShape {
  static constexpr int BSC = 4 * GS / (512 / BITS);
  static constexpr int BPW_SMALL = BSC >= 2 ? 1 : 2;
  static constexpr int BPW_NARROW = BSC >= 4 ? 1 : 4 / BSC;
  static constexpr int BPW_WIDE = BSC == 4 ? 2 : BPW_NARROW;
};

template <int BITS, int GS, int BPW, bool ADD>
int launch_persist_x_k(const QgemvArgs &a, int waves, int grid, size_t lds, int phases, int ntile_max,
                       hipStream_t stream) {
  const auto kern = qgemv_persist_x_kernel<BITS, GS, BPW, ADD>;
  if (!allow_max_dynamic_lds(reinterpret_cast<const void *>(kern))) return QGEMV_EHIP;
  const int st = launch_fill(a.y, (size_t)a.M * a.N, ADD ? kSplitSentinel : 0u, stream);
  if (st != QGEMV_OK) return st;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), lds, stream, a.codes, a.scales, a.biases, a.x,
                     a.y, a.res, a.M, a.N, a.K, phases, ntile_max);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

template <int BITS, int GS, bool ADD>
int launch_persist_x_t(const QgemvArgs &a, hipStream_t stream) {
  using Sh = PersistXShape<BITS, GS>;
  const int nblk = a.K / (4 * GS);
  if (nblk < 2) return QGEMV_EUNSUPPORTED;
  const int nbp_min = nblk / 2, nbp_max = nblk - nblk / 2;
  const int tiles = (a.N + 15) / 16;
  const int cus = device_cu_count();
  if (tiles < cus) return QGEMV_EUNSUPPORTED;
  // one workgroup per CU, half of them per half of K (every workgroup has
  // at least one tile: tiles >= CUs)
  const int grid = 2 * (cus / 2);
  const int ntile_max = (tiles + grid / 2 - 1) / (grid / 2);
  // fewest phases, then fewest blocks per wave, whose activations, group
  // sums and partial tiles fit the LDS
  const int bpws[3] = {Sh::BPW_SMALL, Sh::BPW_NARROW, Sh::BPW_WIDE};
  for (int phases = 1; phases <= kXMaxPhases && phases <= nbp_min; ++phases) {
    const int nbq_max = (nbp_max + phases - 1) / phases;
    for (int variant = 0; variant < 3; ++variant) {
      // two passes with the 8-super-chunk slots (5 waves on the 4-bit gs128
      // down projection) were slower than the single-pass kernel: 40.5
      // against 34.8 us at M = 15
      if (phases > 1 && variant == 2 && Sh::BPW_WIDE != Sh::BPW_NARROW) continue;
      const int bpw = bpws[variant];
      const int waves = (nbq_max + bpw - 1) / bpw;
      if (waves > kXMaxWaves) continue;
      const size_t pitch = (size_t)nbq_max * 4 * GS * 2 + 16;
      const size_t lds = (size_t)a.M * pitch + (size_t)a.M * nbq_max * 4 * sizeof(float) +
                         (size_t)ntile_max * waves * 256 * sizeof(float);
      if (lds > kLdsMax) continue;
      if (variant == 0)
        return launch_persist_x_k<BITS, GS, Sh::BPW_SMALL, ADD>(a, waves, grid, lds, phases, ntile_max, stream);
      if (variant == 1)
        return launch_persist_x_k<BITS, GS, Sh::BPW_NARROW, ADD>(a, waves, grid, lds, phases, ntile_max, stream);
      return launch_persist_x_k<BITS, GS, Sh::BPW_WIDE, ADD>(a, waves, grid, lds, phases, ntile_max, stream);
    }
  }
  return QGEMV_EUNSUPPORTED;
}

template <int BITS, int GS>
int launch_persist_x_gs(const QgemvArgs &a, hipStream_t stream) {
  return a.res ? launch_persist_x_t<BITS, GS, true>(a, stream) : launch_persist_x_t<BITS, GS, false>(a, stream);
}

}  // namespace

int launch_persist_x(const QgemvArgs &a, hipStream_t stream) {
  if (a.fmt != kAffine || !mfma_supports(a.K, a.bits, a.group_size) || !mfma_whole_blocks(a.K, a.group_size))
    return QGEMV_EUNSUPPORTED;
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
