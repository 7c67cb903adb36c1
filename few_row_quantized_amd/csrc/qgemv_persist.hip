// Persistent bf16 MFMA path of the few-row quantized GEMV (gfx950), for
// shapes whose weight stream spans many tiles per CU.
//
// Prior art on the pages: the few-row MMA kernels of "metal : few-row MMA
// mat-mul and batched copies for speculative decoding" (Overview: each weight
// dequantized once for all rows, the simdgroups of a threadgroup split K) and
// the split-K MMA variants on the MLX quantized_matmul small-M verify kernels
// page (Facts: dequantize per quantization group rather than per MMA tile;
// split K across the simdgroups).
//
// CDNA4 design:
// * A persistent grid of one workgroup per CU; workgroup g owns the
//   contiguous range of 16-column tiles [g*T/G, (g+1)*T/G) over the whole of K.
// * Its W waves split K into bias blocks (4 groups): wave w owns the blocks
//   vw, vw+W, ... (vw = w rotated per workgroup) for every tile, so its
//   activation operands and the per-group activation sums of the bias term
//   are loaded, re-paired and summed once and then stay in registers while
//   the workgroup walks its tiles (up to 4 or 8 rows in compact loads, each
//   row filling 4 or 2 MFMA rows: compact_pick in qgemv_device.h).
// * Codes and group metadata of the next tile are prefetched into a ring of
//   S register slots while the current tile is unpacked and multiplied, so a
//   CU keeps weight bytes in flight from its first tile to its last.  Codes
//   come as whole 128-byte lines (8 rows per load) where a bias block holds
//   an even number of 64-byte super-chunks (pair_to_operand_lanes).
// * Every S tiles the waves' partial 16x16 tiles are summed through LDS in
//   block order (deterministic, no atomics) and rows m < M are stored.  Two
//   LDS buffers alternate between groups of S tiles, so a group needs one
//   workgroup barrier, not two (27B gate 5120 x 17408: 15.6 -> 14.3 us at
//   M = 1, 16.1 -> 15.6 at M = 8).
// * Fused residual sum (ADD, "metal : few-row MMA mat-mul and batched copies
//   for speculative decoding", Overview: MUL_MAT + ADD writes the residual
//   sum from the store): the residual of the S tiles' outputs a thread stores
//   is loaded when their first tile starts and added in the store, so
//   y = fl(product + r), bit for bit the plain call and a separate fp32 add.
// * 8-bit codes (groups of 32 or 64; MLX page, Facts: the int8 M = 8
//   speedup) take two code registers per MFMA step in natural order, as in
//   the single-pass kernel.  With more than 16 bias blocks (K > 4096 at
//   groups of 64) two blocks per wave spill registers, so K is split in two
//   halves over two workgroups instead (KS = 2: workgroup b takes half b & 1
//   of the blocks for tile range b >> 1; each half is added into y, zeroed
//   before the launch, which receives exactly two addends, so the result does
//   not depend on which lands first; with the residual sum y is prefilled
//   with kSplitSentinel and the second half stores (a + b) + r).  Measured in
//   graph chains against the single-pass kernel: 8-bit 15360 x 3840 19.4 ->
//   15.0 us at M = 1, 20.0 -> 15.8 at M = 8; 8-bit 17408 x 5120 (split)
//   33.5 -> 22.3 us at M = 1, 35.2 -> 23.8 at M = 8.  The split is slower
//   for every other format here (27B gate 5120 x 17408 4-bit gs128 15.5 ->
//   19.3 us at M = 8, FFN-up gs64 10.4 -> 12.7, 2-bit gate/up 15.7 -> 16.1,
//   the 8-bit 15360 x 3840 shape 15.9 -> 18.7), so only those rows take it.
// * Gathered verify (GATHER; MLX page, Facts: MoE gather_qmm verify): every
//   workgroup resolves the device routing (gather_route), cuts each expert's
//   pairs into chunks of at most 16 (4 or 8 with compact activation loads)
//   and takes a contiguous range of the (chunk, tile) items in chunk-major
//   order, so consecutive items are adjacent tiles of one expert and stream
//   through the same prefetch ring; a step entering a new chunk reloads the
//   activation set (its pairs' rows) and stores to its pairs' rows of y.
// The inner MFMA step (code layout, partial lane transpose, unpack to exact
// bf16 q, per-group scale fold, bias product by v_mfma_f32_16x16x4_f32,
// zero-weight flags) is the one of the single-pass kernel.

#include <atomic>

#include "qgemv_device.h"
#include "qgemv_gather_route.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

// y and res may be the same buffer (in-place residual sum): neither is
// declared restrict; every element is read before it is written, by the same
// thread.
template <int BITS, int GS, int BPW, int S, int MAXW, bool ADD, bool PAIRK, int XC, int KS, bool GATHER = false>
__global__ __launch_bounds__(64 * MAXW) void qgemv_persist_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *y,
    const float *res, int M, int N, int K, GatherArgs ga) {
  constexpr int CW = 128 / BITS;         // codes per 16-byte chunk
  constexpr int SCW = 4 * CW;            // codes per 64-byte super-chunk
  constexpr int DW = CW / 4;             // codes per dword
  constexpr int HS = BITS == 2 ? 2 : 1;  // MFMA steps per code dword (8-bit: one per two dwords)
  // activation operands per super-chunk and HS: one per code register
  // (2/4-bit) or per pair of code registers (8-bit)
  constexpr int XR = BITS == 8 ? 2 : 4;
  constexpr int BLKW = 4 * GS;           // codes per bias block
  constexpr int BSC = BLKW / SCW;        // super-chunks per block
  constexpr int CPG = GS / CW;           // chunks per group
  constexpr int GPS = 4 / CPG;           // groups per super-chunk
  constexpr int LVL = CPG >= 4 ? 0 : (CPG == 2 ? 1 : 2);
  constexpr int REGS_G = CPG;
  // codes of two consecutive super-chunks as whole 128-byte lines (8 rows per
  // load, pair_to_operand_lanes): the two halves of a block where a block has
  // an even number of them, or (PAIRK: one super-chunk per block, two blocks
  // per wave, an even block count) the wave's two blocks, which PAIRK makes
  // adjacent; otherwise lane quads on 64 bytes (to_operand_lanes).  The
  // wave's super-chunks j = k * BSC + u then pair as (j & ~1, j | 1).
  static_assert(!PAIRK || (BPW == 2 && BSC == 1), "block pairs need two one-super-chunk blocks per wave");
  constexpr bool LINES = BSC % 2 == 0 || PAIRK;
  // metadata loads in the quad-row layout: measured faster for 4-bit codes
  // with groups of 32 or 64 (FFN-up 4096x12288: 14.2 -> 13.2 us and
  // 11.3 -> 10.6 us at M = 8), slower by 1-5% with groups of 128 and for
  // 2-bit codes, where metadata loads are few
  constexpr bool MQ = BITS == 4 && GS <= 64;
  static_assert(BSC >= 1 && BLKW % SCW == 0 && CPG >= 1 && GPS >= 1, "block layout");
  // compact activation loads (XC = 4 or 8 rows, M <= XC; see compact_pick):
  // XG operands per load; a load covers part of one super-chunk (LPU loads
  // each) or whole super-chunks (SPL each), NLB loads per block
  static_assert(XC == 0 || XC == 4 || XC == 8, "compact activation rows");
  constexpr int XG = XC ? 16 / (XC ? XC : 1) : 1;
  constexpr int OPS = XR * HS;  // activation operands per super-chunk
  constexpr int LPU = OPS >= XG ? OPS / XG : 1;
  constexpr int SPL = OPS >= XG ? 1 : XG / OPS;
  constexpr int NLB = BSC * OPS / XG;
  static_assert((OPS % XG == 0 || XG % OPS == 0) && (BSC * OPS) % XG == 0, "compact activation layout");

  __shared__ float red[2][S][MAXW][4][64];
  // gathered verify (GATHER): the routing (gather_route), and its slots cut
  // into chunks of at most CH pairs (16, or XC with compact activation
  // loads), each one activation set
  static_assert(!GATHER || (!ADD && KS == 1), "gathered variant");
  constexpr int CH = XC ? XC : 16;
  __shared__ int gexp[GATHER ? kMaxPairs : 1], gxr[GATHER ? kMaxPairs : 1], gsorted[GATHER ? kMaxPairs : 1];
  __shared__ int gstart[GATHER ? kMaxPairs + 1 : 1], gslot_exp[GATHER ? kMaxPairs : 1];
  __shared__ int gcs[GATHER ? kMaxPairs + 1 : 1];  // first sorted position of each chunk
  __shared__ int gce[GATHER ? kMaxPairs : 1];      // expert of each chunk
  __shared__ int gmeta[2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int col = lane & 15;
  const int kb = lane >> 4;
  // Block ownership is rotated per workgroup (workgroups are dealt
  // round-robin over the 8 XCDs, so blockIdx/8 differs between the CUs that
  // share an L2): without it every CU asks for the same activation lines at
  // the same moment.  Partials are summed in block order, so results do not
  // depend on the rotation.
  const int rot = (int)((blockIdx.x >> 3) % (unsigned)W);
  const int vw = wave + rot < W ? wave + rot : wave + rot - W;
  const int nblk = K / BLKW;
  const size_t RB = (size_t)K * BITS / 8;
  const int NG = K / GS;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  // activation loads in the quad-row layout once several rows are distinct
  // (results do not depend on the choice; from M = 5 for every group size
  // here: 27B q at M = 7, 9.44 -> 8.91 us); set with each activation set
  bool xquad = false;
  int xoff[4];

  // Gathered verify: resolve the routing, then cut each slot's pairs into
  // chunks of at most CH (wave 0: a scan of the chunk counts over the slots)
  if constexpr (GATHER) {
    gather_route(ga, gexp, gxr, gsorted, gstart, gslot_exp, gmeta);
    const int nslots = gmeta[0];
    if (wave == 0) {
      int base = 0;
      for (int s0 = 0; s0 < nslots; s0 += 64) {
        const int sl = s0 + lane;
        const int cnt = sl < nslots ? gstart[sl + 1] - gstart[sl] : 0;
        const int nch = (cnt + CH - 1) / CH;
        int inc = nch;  // inclusive scan over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int v = __shfl_up(inc, d);
          if (lane >= d) inc += v;
        }
        const int first = base + inc - nch;
        for (int j = 0; j < nch; ++j) {
          gcs[first + j] = gstart[sl] + CH * j;
          gce[first + j] = gslot_exp[sl];
        }
        base += __shfl(inc, 63);
      }
      if (lane == 0) {
        gmeta[1] = base;
        gcs[base] = gstart[nslots];
      }
    }
    __syncthreads();
  }

  // tile range of this workgroup (the products stay below 2^31: the grid is
  // at most the CU count and T <= 2^18); with K split in two (KS = 2),
  // workgroup b takes half b & 1 of the bias blocks for tile range b >> 1.
  // Gathered: a range of the items (chunk, tile) in chunk-major order
  // (T tiles per chunk); a workgroup without items has nothing to do.
  const int T = (N + 15) >> 4;
  const int part = KS == 2 ? (int)(blockIdx.x & 1u) : 0;
  const unsigned gi = KS == 2 ? blockIdx.x >> 1 : blockIdx.x;
  const unsigned GPn = KS == 2 ? gridDim.x >> 1 : gridDim.x;
  const uint64_t items = GATHER ? (uint64_t)gmeta[1] * (uint64_t)T : (uint64_t)T;
  const int t_first = (int)((uint64_t)gi * items / GPn);
  const int ntile = (int)((uint64_t)(gi + 1) * items / GPn) - t_first;
  if constexpr (GATHER) {
    if (ntile <= 0) return;  // uniform for the workgroup
  }
  // chunk and tile of item step j of this workgroup
  auto item_chunk = [&](const int j) -> int { return GATHER ? (t_first + j) / T : 0; };
  // activation set in registers: its first sorted position and pair count
  // (gathered); rows a >= the count read the last row, never stored
  int cur_ch = -1, gcs0 = 0, gcnt = M;
  auto xrow_at = [&](const int a) -> size_t {
    const int m = min(a, gcnt - 1);
    if constexpr (GATHER) return (size_t)gxr[gsorted[gcs0 + m]];
    return (size_t)m;
  };
  const int p_lo = part ? nblk >> 1 : 0;                                  // first block of the part
  const int nbp = KS == 1 ? nblk : (part ? nblk - (nblk >> 1) : nblk >> 1);  // its blocks

  // owned blocks of the part (vw, vw + W, ...; PAIRK: vw*BPW, vw*BPW + 1,
  // adjacent); a wave past the last block loads a valid block and skips the
  // arithmetic
  int blk[BPW];
  bool own[BPW];
#pragma unroll
  for (int k = 0; k < BPW; ++k) {
    const int b = PAIRK ? vw * BPW + k : vw + k * W;
    own[k] = b < nbp;
    blk[k] = p_lo + (own[k] ? b : nbp - 1);
  }

  // ---- activations of the owned blocks (rows m >= M read row M-1: their
  // outputs are never stored), later re-paired to the code pairing and
  // summed per group into the A layout of the bias MFMA
  u32x4_t xv[BPW][BSC][XR][HS];
  float xsum[BPW];
  // compact loads: load ld of a block carries its operands ld*XG ..
  // ld*XG + XG-1 (operand (u, i, l) -> (u*XR + i)*HS + l); this lane holds
  // operand ld*XG + lane%XG of row (lane%16)/XG at its K-part kb, at element
  // (ld / LPU)*SPL*SCW + xlp[ld % LPU] of the block
  u32x4_t cx[XC ? BPW : 1][XC ? NLB : 1];
  auto acts_load = [&]() {
  xquad = XC == 0 && gcnt >= 5;
  const int xkb = xquad ? (lane & 3) : kb;
#pragma unroll
  for (int i = 0; i < 4; ++i) xoff[i] = lvl_chunk<LVL>(i, xkb) * CW + lvl_dword<LVL>(i, xkb) * DW;
  const uint16_t *xr = x + xrow_at(xquad ? (lane >> 2) : col) * K;
  if constexpr (XC != 0) {
    const uint16_t *xrc = x + xrow_at((lane & 15) / XG) * K;
    int xlp[LPU];
#pragma unroll
    for (int p = 0; p < LPU; ++p) {
      const int f = p * XG + (lane & (XG - 1));
      const int u = f / OPS, i = (f % OPS) / HS, l = f % HS;
      const int ii = BITS == 8 ? 2 * i : i;
      xlp[p] = u * SCW + lvl_chunk<LVL>(ii, kb) * CW + lvl_dword<LVL>(ii, kb) * DW + 8 * l;
    }
#pragma unroll
    for (int k = 0; k < BPW; ++k)
#pragma unroll
      for (int ld = 0; ld < NLB; ++ld)
        cx[k][ld] = *reinterpret_cast<const u32x4_t *>(xrc + blk[k] * BSC * SCW + (ld / LPU) * SPL * SCW +
                                                        xlp[ld % LPU]);
  } else {
#pragma unroll
    for (int k = 0; k < BPW; ++k)
#pragma unroll
      for (int u = 0; u < BSC; ++u) {
        const int k0 = (blk[k] * BSC + u) * SCW;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
          for (int l = 0; l < HS; ++l)
            xv[k][u][i][l] =
                *reinterpret_cast<const u32x4_t *>(xr + k0 + (BITS == 8 ? xoff[2 * i] : xoff[i]) + 8 * l);
      }
  }
  };
  if constexpr (GATHER) {
    cur_ch = item_chunk(0);
    gcs0 = gcs[cur_ch];
    gcnt = gcs[cur_ch + 1] - gcs0;
  }
  acts_load();

  // ---- prefetch ring of codes and metadata.  Issues past the last tile are
  // still made (a branch around loads would make the compiler wait for every
  // load in flight), but all lanes of the wave then read the first line of
  // the wave's own first-tile data: one cached line per instruction, and a
  // different line for every wave of the device.
  u32x4_t cv[S][BPW][BSC];
  uint2 s4[S][BPW], b4[S][BPW];
  // item step j's tile: its first column, and the first row of its matrix
  // among the rows of all experts (gathered: the chunk's expert, N rows each)
  auto item_col0 = [&](const int j) -> int { return 16 * (t_first + j - item_chunk(j) * T); };
  auto item_mat = [&](const int j) -> uint64_t {
    if constexpr (GATHER) return (uint64_t)gce[item_chunk(j)] * (uint64_t)N;
    return 0ull;
  };
  const uint64_t crow_dead = (item_mat(0) + (uint64_t)item_col0(0)) * RB;
  const uint64_t mrow_dead = (item_mat(0) + (uint64_t)item_col0(0)) * NG;
  int it = 0;  // tile step of the next issue
  auto issue = [&](const int slot) {
    const uint64_t m64 = 0ull - (uint64_t)(it < ntile);  // all-ones while live
    // codes: whole 128-byte lines (LINES: lane L on piece L%8 of row L/8,
    // rows 8-15 in a second load) or lane quads (piece L%4 of row L/4, see
    // quad_row_lane); metadata in lane quads where groups are small (MQ),
    // else per column.  Rows past N (a ragged last tile) read row N-1 of the
    // same matrix.
    const int jl = GATHER ? min(it, ntile - 1) : it;  // gathered: a live item (chunk table bounds)
    const int c0 = item_col0(jl);
    const uint64_t rb = item_mat(jl);
    const uint64_t nq = rb + (uint64_t)min(c0 + (lane >> 2), N - 1);
    const uint64_t nl = rb + (uint64_t)min(c0 + (lane >> 3), N - 1);      // LINES: rows 0-7
    const uint64_t nl8 = rb + (uint64_t)min(c0 + 8 + (lane >> 3), N - 1);  // rows 8-15
    const uint64_t crow = LINES ? ((nl * RB + (lane & 7) * 16) & m64) | (crow_dead & ~m64)
                                : ((nq * RB + (lane & 3) * 16) & m64) | (crow_dead & ~m64);
    const uint64_t crow8 = ((nl8 * RB + (lane & 7) * 16) & m64) | (crow_dead & ~m64);
    const uint64_t nm = MQ ? nq : rb + (uint64_t)min(c0 + col, N - 1);
    const uint64_t mrow = ((nm * NG) & m64) | (mrow_dead & ~m64);
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
#pragma unroll
      for (int u = 0; u < BSC; ++u) {
        if constexpr (LINES)
          cv[slot][k][u] = load_stream_u32x4(codes + (((k * BSC + u) & 1) ? crow8 : crow) +
                                             (size_t)((blk[k] * BSC + u) & ~1) * 64);
        else
          cv[slot][k][u] = load_stream_u32x4(codes + crow + (size_t)(blk[k] * BSC + u) * 64);
      }
    }
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      s4[slot][k] = *reinterpret_cast<const uint2 *>(scales + mrow + blk[k] * 4);
      b4[slot][k] = *reinterpret_cast<const uint2 *>(biases + mrow + blk[k] * 4);
    }
    ++it;
  };

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  // keep the code loads ahead of the activation work that waits for x
  __builtin_amdgcn_sched_barrier(0);

  auto acts_finish = [&]() {
  if constexpr (XC != 0) {
#pragma unroll
    for (int k = 0; k < BPW; ++k)
#pragma unroll
      for (int u = 0; u < BSC; ++u)
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
          for (int l = 0; l < HS; ++l) {
            const int f = (u * XR + i) * HS + l;
            xv[k][u][i][l] = compact_pick<XG>(cx[k][f / XG], f % XG);
          }
  } else if (xquad) {
#pragma unroll
    for (int k = 0; k < BPW; ++k)
#pragma unroll
      for (int u = 0; u < BSC; ++u)
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
          for (int l = 0; l < HS; ++l) xv[k][u][i][l] = to_operand_lanes(xv[k][u][i][l]);
  }

#pragma unroll
  for (int k = 0; k < BPW; ++k) {
    float P[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < BSC; ++u) {
      if constexpr (BITS == 8) {
        // natural order: only the group sums; step e of the super-chunk
        // holds 8 codes of group (u*SCW + 32e)/GS of the block
#pragma unroll
        for (int e = 0; e < XR; ++e) {
          const int j = (u * SCW + 32 * e) / GS;
#pragma unroll
          for (int c = 0; c < 4; ++c) P[j] = dot2_bf16(xv[k][u][e][0][c], 0x3F803F80u, P[j]);
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = u * GPS + i / REGS_G;
#pragma unroll
        for (int l = 0; l < HS; ++l)
#pragma unroll
          for (int e = 0; e < 4; ++e) P[j] = dot2_bf16(xv[k][u][i][l][e], 0x3F803F80u, P[j]);
#pragma unroll
        for (int l = 0; l < HS; ++l) xv[k][u][i][l] = pair_activations<BITS>(xv[k][u][i][l]);
      }
    }
    xsum[k] = rows_transpose_reduce4(P);
  }
  };
  acts_finish();

  // ---- groups of S tile steps (the unrolled ring); a range always has a
  // tile (do-while: no guard branch that would let the compiler sink the
  // prologue loads below the activation work)
  int j0 = 0;
  int rb = 0;  // reduction buffer of this group
  do {
    // residual of the outputs this thread stores for these S tiles (its first
    // S reduction steps: all of them with at least 4 waves); clamped indices
    // read a valid element and are never used
    float rpre[S];
    if constexpr (ADD) {
#pragma unroll
      for (int j = 0; j < S; ++j) {
        const int o = min((int)threadIdx.x + j * (int)blockDim.x, S * 256 - 1);
        const int l = o & 63;
        const int m = min((4 * (l >> 4) + ((o >> 6) & 3)) / XG, M - 1);
        const int n = min(16 * (t_first + j0 + (o >> 8)) + (l & 15), N - 1);
        rpre[j] = res[(size_t)m * N + n];
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (j0 + s >= ntile) break;
      // gathered: a step that enters a new chunk loads its activation set
      // first (ahead of the next step's codes, so that waiting for it does
      // not wait for them)
      bool fresh = false;
      if constexpr (GATHER) {
        const int ch = item_chunk(j0 + s);
        if (ch != cur_ch) {
          cur_ch = ch;
          gcs0 = gcs[ch];
          gcnt = gcs[ch + 1] - gcs0;
          acts_load();
          fresh = true;
        }
      }
      issue((s + S - 1) % S);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (GATHER) {
        if (fresh) acts_finish();
      }

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
        if (!own[k]) continue;  // uniform per wave
        f32x4_t accg;
        uint32_t zc0 = 0u;  // the current group's first code word
#pragma unroll
        for (int u = 0; u < BSC; ++u) {
          uint32_t cur[4];
          if constexpr (LINES) {
            const int ja = (k * BSC + u) & ~1, jb = (k * BSC + u) | 1;  // the pair's two super-chunks
            if ((k * BSC + u) & 1)
              pair_to_operand_lanes<1>(cv[s][ja / BSC][ja % BSC], cv[s][jb / BSC][jb % BSC], cur);
            else
              pair_to_operand_lanes<0>(cv[s][ja / BSC][ja % BSC], cv[s][jb / BSC][jb % BSC], cur);
          } else {
            to_operand_lanes(cv[s][k][u], cur);
          }
          transpose_rows_lvl<LVL>(cur);
          if constexpr (BITS == 8) {
            // MFMA step e takes code registers 2e, 2e+1 (8 consecutive codes
            // of this lane's row; the activations at xoff[2e]..+7)
#pragma unroll
            for (int e = 0; e < XR; ++e) {
              const int kk = u * SCW + 32 * e;  // first code of the step within the block
              const int jg = kk / GS;           // its group within the block
              const bool gfirst = kk % GS == 0;
              const bool glast = (kk + 32) % GS == 0;
              // zero-weight traces: code words against the group's first,
              // then the group's weight s*c + b at its last step
              if (gfirst) {
                zc0 = cur[2 * e];
                nz |= fields_spread<BITS>(cur[2 * e]);
              } else {
                nz |= cur[2 * e] ^ zc0;
              }
              nz |= cur[2 * e + 1] ^ zc0;
              pin(nz);
              if (glast) {
                const uint2 sw_v = s4[s][k];
                const uint2 bw16_v = b4[s][k];
                nz |= weight_trace(half_bits_to_float(field16(sw_v, jg)), low_field<BITS>(zc0),
                                   half_bits_to_float(field16(bw16_v, jg)));
              }
              const u32x4_t bw = unpack8_quad(cur[2 * e], cur[2 * e + 1]);
              accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, xv[k][u][e][0]), __builtin_bit_cast(bf16x8_t, bw),
                  gfirst ? zero4 : accg, 0, 0, 0);
              if (glast) {
                const uint2 sw_v = s4[s][k];
                const float scl = half_bits_to_float(field16(sw_v, jg));
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = fmaf(scl, accg[q], acc[q]);
              }
            }
            continue;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jg = u * GPS + i / REGS_G;  // group within the block
#pragma unroll
            for (int h = 0; h < HS; ++h) {
              const bool gfirst = (i % REGS_G) == 0 && h == 0;
              const bool glast = (i % REGS_G) == REGS_G - 1 && h == HS - 1;
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
              accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, xv[k][u][i][h]), __builtin_bit_cast(bf16x8_t, bw),
                  gfirst ? zero4 : accg, 0, 0, 0);
              if (glast) {
                const uint2 sw_v = s4[s][k];
                const float scl = half_bits_to_float(field16(sw_v, jg));
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = fmaf(scl, accg[q], acc[q]);
              }
            }
          }
        }
        // bias: acc += xsum[m][g0+kb] * b[n][g0+kb]
        const uint2 bw_v = b4[s][k];
        const float b = half_bits_to_float(field16(bw_v, kb));
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsum[k], b, acc, 0, 0, 0);
      }
      // a partial whose column held only zero weights is exactly 0
      const uint32_t keep = keep_mask(column_or(nz));
#pragma unroll
      for (int i = 0; i < 4; ++i) red[rb][s][wave][i][lane] = unless_zero(acc[i], keep);
    }

    // ---- sum the group's partial tiles over the waves in block order
    __syncthreads();
    const int nj = min(S, ntile - j0);
    auto finish = [&](const int o, const bool pre, float rv) {
      const int s = o >> 8, i = (o >> 6) & 3, l = o & 63;
      float v = 0.f;
      for (int w = 0; w < W; ++w) {
        const int pw = w >= rot ? w - rot : w - rot + W;  // wave acting as virtual wave w
        v += red[rb][s][pw][i][l];
      }
      // MFMA row a holds activation row a / XG (compact loads: each row XG
      // times); gathered: pair a of the item's chunk, output row that pair
      const int a = 4 * (l >> 4) + i;
      int m = a % XG == 0 ? a / XG : M;
      int rows = M;
      size_t yr = (size_t)m;
      if constexpr (GATHER) {
        const int ch = item_chunk(j0 + s);
        rows = gcs[ch + 1] - gcs[ch];
        yr = (size_t)gsorted[gcs[ch] + min(m, rows - 1)];
      }
      const int n = item_col0(j0 + s) + (l & 15);
      if (m < rows && n < N) {
        float *dst = y + yr * N + n;
        if constexpr (ADD) {
          if (!pre) rv = res[(size_t)m * N + n];
        }
        if constexpr (KS == 1) {
          *dst = ADD ? v + rv : v;
        } else if constexpr (!ADD) {
          // y was zeroed before the launch and receives exactly two addends:
          // 0 + a + b equals 0 + b + a bit for bit, whichever half lands first
          unsafeAtomicAdd(dst, v);
        } else {
          // y held kSplitSentinel: the first half leaves its partial there,
          // the second finds it and stores (a + b) + r
          const float old = atomicExch(dst, v);
          if (__builtin_bit_cast(uint32_t, old) != kSplitSentinel) *dst = (old + v) + rv;
        }
      }
    };
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int o = threadIdx.x + j * blockDim.x;
      if (o < nj * 256) finish(o, true, ADD ? rpre[j] : 0.f);
    }
    for (int o = threadIdx.x + S * blockDim.x; o < nj * 256; o += blockDim.x) finish(o, false, 0.f);
    // the next group writes the other buffer; the group after it waits at
    // that group's barrier, by which every thread has finished reading this one
    rb ^= 1;
    j0 += S;
  } while (j0 < ntile);
}

// Per-format launch shape: blocks owned per wave (activation registers stay
// within 64 VGPRs), the wave cap whose register budget the kernel fits, and
// the depth S of the prefetch ring.
template <int BITS, int GS>
struct PersistShape {
  static constexpr int BPW = (BITS != 2 && GS == 32) || (BITS == 2 && GS == 64) ? 2 : 1;
  static constexpr int MAXW = (BITS != 2 && GS <= 64) ? 16 : 12;
  static constexpr int S = 2;
};

template <int BITS, int GS, int BPW, int MAXW, int KS, bool ADD, int XC>
int launch_persist_k(const QgemvArgs &a, hipStream_t stream) {
  constexpr int S = PersistShape<BITS, GS>::S;
  const int nblk = a.K / (4 * GS);
  const int nbh = nblk - (KS == 2 ? nblk >> 1 : 0);  // blocks of the longer part
  if (nbh > MAXW * BPW) return QGEMV_EUNSUPPORTED;   // activations would not fit the registers
  const int waves = (nbh + BPW - 1) / BPW;
  const int tiles = (a.N + 15) / 16;
  const int cus = device_cu_count();
  const int G = KS * (tiles < cus / KS ? tiles : cus / KS);
  if constexpr (KS == 2) {
    // the halves are added into y, prefilled here; not for an in-place
    // residual sum, whose residual the prefill would erase
    if (ADD && static_cast<const void *>(a.res) == static_cast<const void *>(a.y)) return QGEMV_EUNSUPPORTED;
    const int st = launch_fill(a.y, (size_t)a.M * a.N, ADD ? kSplitSentinel : 0u, stream);
    if (st != QGEMV_OK) return st;
  }
  // the wave's two one-super-chunk blocks as whole lines where every wave has
  // two (an even block count)
  constexpr bool CAN_PAIRK = KS == 1 && BPW == 2 && 4 * GS * BITS == 512;
  if (CAN_PAIRK && nblk % 2 == 0) {
    hipLaunchKernelGGL((qgemv_persist_kernel<BITS, GS, BPW, S, MAXW, ADD, CAN_PAIRK, XC, KS>), dim3(G),
                       dim3(64 * waves), 0, stream, a.codes, a.scales, a.biases, a.x, a.y, a.res, a.M, a.N, a.K,
                       GatherArgs{});
    return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
  }
  hipLaunchKernelGGL((qgemv_persist_kernel<BITS, GS, BPW, S, MAXW, ADD, false, XC, KS>), dim3(G),
                     dim3(64 * waves), 0, stream, a.codes, a.scales, a.biases, a.x, a.y, a.res, a.M, a.N, a.K,
                       GatherArgs{});
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

template <int BITS, int GS, bool ADD, int XC>
int launch_persist_t(const QgemvArgs &a, hipStream_t stream) {
  using Sh = PersistShape<BITS, GS>;
  // 8-bit codes in groups of 64 with more than 16 bias blocks: K split in two
  // halves over two workgroups (two blocks per wave spill registers)
  if constexpr (BITS == 8 && GS == 64) {
    if (a.K / (4 * GS) > Sh::MAXW * Sh::BPW) return launch_persist_k<BITS, GS, 1, 16, 2, ADD, XC>(a, stream);
  }
  return launch_persist_k<BITS, GS, Sh::BPW, Sh::MAXW, 1, ADD, XC>(a, stream);
}

template <int BITS, int GS, int XC>
int launch_persist_c(const QgemvArgs &a, hipStream_t stream) {
  return a.res ? launch_persist_t<BITS, GS, true, XC>(a, stream) : launch_persist_t<BITS, GS, false, XC>(a, stream);
}

// Activations of up to 4 or 8 rows in compact loads (compact_pick): 4 or 2
// times fewer activation load instructions in the prologue.  The arithmetic
// is the same either way.
template <int BITS, int GS>
int launch_persist_gs(const QgemvArgs &a, hipStream_t stream) {
  if (a.M <= 4) return launch_persist_c<BITS, GS, 4>(a, stream);
  if (a.M <= 8) return launch_persist_c<BITS, GS, 8>(a, stream);
  return launch_persist_c<BITS, GS, 0>(a, stream);
}

// Gathered verify on the persistent kernel (called for 3 or more activation
// rows): as many workgroups as are resident at once, each taking a
// contiguous range of the (chunk, tile) items, where the chunks are the
// union's experts' pairs 16 at a time (4 or 8 with compact activation loads).
// The grid decides only which workgroup takes which item; the wave split
// follows the shape only (as in the dense kernel), so a pair's row does not
// depend on the other pairs of the call.  Resident workgroups rather than
// one per CU: 128-expert top-8 2048 -> 1536 gate/up 12.99 -> 12.59 us at
// M = 2, 19.27 -> 17.94 at M = 4.
// At most 8 waves (the activation reload inside the tile loop needs the
// register budget of 512-thread workgroups: at 16 waves the 4-bit gs64
// variant spilled).
template <int BITS, int GS, int XC>
int launch_persist_gather_t(const QgemvArgs &a, const GatherArgs &ga, hipStream_t stream) {
  using Sh = PersistShape<BITS, GS>;
  constexpr int BPW = Sh::BPW, MAXW = 8, S = Sh::S;
  const int nblk = a.K / (4 * GS);
  if (nblk > MAXW * BPW) return QGEMV_EUNSUPPORTED;  // activations would not fit the registers
  const int waves = (nblk + BPW - 1) / BPW;
  constexpr bool CAN_PAIRK = BPW == 2 && 4 * GS * BITS == 512;
  const bool pairk = CAN_PAIRK && nblk % 2 == 0;
  static std::atomic<int> occ_cache[2][MAXW + 1];  // per kernel and wave count
  int occ = occ_cache[pairk][waves].load(std::memory_order_relaxed);
  if (occ == 0) {
    const void *k =
        pairk ? reinterpret_cast<const void *>(qgemv_persist_kernel<BITS, GS, BPW, S, MAXW, false, CAN_PAIRK, XC, 1, true>)
              : reinterpret_cast<const void *>(qgemv_persist_kernel<BITS, GS, BPW, S, MAXW, false, false, XC, 1, true>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, 64 * waves, 0) != hipSuccess || occ < 1) occ = 1;
    occ_cache[pairk][waves].store(occ, std::memory_order_relaxed);
  }
  const int G = device_cu_count() * occ;
  if (pairk) {
    hipLaunchKernelGGL((qgemv_persist_kernel<BITS, GS, BPW, S, MAXW, false, CAN_PAIRK, XC, 1, true>), dim3(G),
                       dim3(64 * waves), 0, stream, a.codes, a.scales, a.biases, a.x, a.y,
                       static_cast<const float *>(nullptr), 16, a.N, a.K, ga);
    return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
  }
  hipLaunchKernelGGL((qgemv_persist_kernel<BITS, GS, BPW, S, MAXW, false, false, XC, 1, true>), dim3(G),
                     dim3(64 * waves), 0, stream, a.codes, a.scales, a.biases, a.x, a.y,
                     static_cast<const float *>(nullptr), 16, a.N, a.K, ga);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

// Activation rows in compact loads (compact_pick) when there are at most 4
// or 8 of them, with chunks of as many pairs (an expert with more pairs gets
// several chunks); the arithmetic of a pair's row is the same either way.
template <int BITS, int GS>
int launch_persist_gather_x(const QgemvArgs &a, const GatherArgs &ga, hipStream_t stream) {
  if (ga.X <= 4) return launch_persist_gather_t<BITS, GS, 4>(a, ga, stream);
  if (ga.X <= 8) return launch_persist_gather_t<BITS, GS, 8>(a, ga, stream);
  return launch_persist_gather_t<BITS, GS, 0>(a, ga, stream);
}

}  // namespace

int launch_persist_gather(const QgemvArgs &a, const GatherArgs &ga, hipStream_t stream) {
  if (a.fmt != 0 || !mfma_supports(a.K, a.bits, a.group_size) || !mfma_whole_blocks(a.K, a.group_size))
    return QGEMV_EUNSUPPORTED;
  if (a.bits == 4) {
    switch (a.group_size) {
      case 32: return launch_persist_gather_x<4, 32>(a, ga, stream);
      case 64: return launch_persist_gather_x<4, 64>(a, ga, stream);
      case 128: return launch_persist_gather_x<4, 128>(a, ga, stream);
    }
  } else if (a.bits == 2) {
    switch (a.group_size) {
      case 64: return launch_persist_gather_x<2, 64>(a, ga, stream);
      case 128: return launch_persist_gather_x<2, 128>(a, ga, stream);
    }
  } else {
    switch (a.group_size) {
      case 32: return launch_persist_gather_x<8, 32>(a, ga, stream);
      case 64: return launch_persist_gather_x<8, 64>(a, ga, stream);
    }
  }
  return QGEMV_EUNSUPPORTED;
}

int launch_persist(const QgemvArgs &a, hipStream_t stream) {
  if (!mfma_supports(a.K, a.bits, a.group_size) || !mfma_whole_blocks(a.K, a.group_size)) return QGEMV_EUNSUPPORTED;
  if (a.bits == 8) {
    // groups of 128 span two super-chunks: the single-pass kernel
    switch (a.group_size) {
      case 32: return launch_persist_gs<8, 32>(a, stream);
      case 64: return launch_persist_gs<8, 64>(a, stream);
    }
    return QGEMV_EUNSUPPORTED;
  }
  if (a.bits == 4) {
    switch (a.group_size) {
      case 32: return launch_persist_gs<4, 32>(a, stream);
      case 64: return launch_persist_gs<4, 64>(a, stream);
      case 128: return launch_persist_gs<4, 128>(a, stream);
    }
  } else {
    switch (a.group_size) {
      case 64: return launch_persist_gs<2, 64>(a, stream);
      case 128: return launch_persist_gs<2, 128>(a, stream);
    }
  }
  return QGEMV_EUNSUPPORTED;
}

}  // namespace qgemv
