// Single-pass split-K bf16 MFMA kernel of the few-row quantized GEMV
// (gfx950): the kernel template and its launch-shape helpers, shared by the
// dense launchers (qgemv_mfma.hip) and the gathered MoE launcher
// (qgemv_gather.hip).  The design is described in qgemv_mfma.hip.
#pragma once

#include <type_traits>

#include "qgemv_device.h"
#include "qgemv_gather_route.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

// y and res may be the same buffer (in-place residual sum): neither is
// declared restrict; every element is read before it is written, by the same
// thread.
// FMT: kAffine, or a block-scaled FP format (one scale byte per block in
// `scales`, no bias, elements decoded in natural order): kMxfp4 and kMxfp8
// (32-element blocks, GS = 32, scale folded per block in fp32) or kNvfp4
// (16-element blocks, laid out as GS = 32; each element is multiplied by its
// block scale before the MFMA, exactly, so B holds the weights themselves).
// GATHER: the rows of a (slot, tile group) item are the pairs routed to the
// slot's expert (slots: the union of e_idx in ascending id order; pairs in
// ascending order, 16 at a time, or XC with compact rows), gathered from x
// and scattered to y[pair].
// With one tile per workgroup the grid walks the items with its stride;
// with two, workgroup b serves item b and exits if its slot is past the
// union.  (KS = 1, not PERSIST, affine codes.)
template <int BITS, int GS, int NT, int MAXT, int SPI, int KS, bool PERSIST, bool ADD, int FMT,
          bool GATHER = false, int XC = 0, bool XDYN = false, bool PB = false>
__global__ __launch_bounds__(MAXT) void qgemv_mfma_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *y,
    const float *res, int M, int N, int K, int ngroups, GatherArgs ga) {
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
  // compact activation rows (XC: 4 or 8; XDYN, gathered verify: 4 for the
  // chunks of at most 4 rows, none for the others)
  static_assert(XC == 0 || XC == 4 || XC == 8, "compact activation rows");
  static_assert(!XDYN || (GATHER && XC == 0), "per-chunk compact rows");

  __shared__ float red[MAXT / 64][NT][4][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // floor(a / waves) for 0 <= a <= 65536 through a reciprocal, in scalar
  // registers: the true quotient's fraction is a multiple of 1/waves, so a
  // half-step margin (>= 1/32 for waves <= 16) absorbs the reciprocal's and
  // the product's rounding (< 0.02 at these sizes).  Used for the slice
  // rotation (tile group / 8 <= 65536) and the slice bounds (<= 16 * 1024).
  const float rwaves = __builtin_amdgcn_rcpf((float)(blockDim.x >> 6));
  auto div_waves = [&](const int a) -> int {
    return __builtin_amdgcn_readfirstlane((int)(((float)a + 0.5f) * rwaves));
  };
  const int waves = blockDim.x >> 6;
  const int col = lane & 15;
  const int kb = lane >> 4;
  // Bias blocks of 4 groups; with PB the last one is partial (affine 2/4-bit
  // codes: K a whole number of super-chunks and of groups, at least 4
  // groups).  Its missing super-chunks load the row's last real one (valid
  // addresses) with their activations set to zero, and its metadata load is
  // moved back inside the row and shifted, so the missing groups carry scale
  // and bias 0: they add exactly nothing.  (A compile-time variant: the
  // clamps cost whole-block shapes 5-20% in the single-pass kernel.)
  static_assert(!PB || (FMT == kAffine && BITS != 8), "partial blocks: affine 2/4-bit codes");
  const int NBLK = PB ? (K + BLKW - 1) / BLKW : K / BLKW;
  const int NSC = K / SCW;  // real super-chunks per row
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  // element offset, within a super-chunk, of the codes register i holds in
  // this lane's row after the partial transpose

  // Gathered verify.  The routing is read once per workgroup into LDS.
  // GSORT (one tile per workgroup): the valid pairs are ordered by
  // (expert, pair) with a stable rank sort, the runs of equal experts (the
  // union in ascending id order) become slots, and the workgroup walks the
  // (slot, tile group) items with the grid stride.  Otherwise (two tiles per
  // workgroup, short K): workgroup b serves slot b / ngroups alone, found as
  // the slot-th set bit of a union bitmap, and compacts that expert's pairs.
  // Either way a slot's pairs are in ascending order, so each expert sees the
  // same 16-row chunks.
  constexpr bool GSORT = GATHER && NT == 1;
  __shared__ uint32_t gbits[GATHER && !GSORT ? kMaxExperts / 32 : 1];
  __shared__ int gexp[GATHER ? kMaxPairs : 1];        // expert of each pair, -1 if invalid
  __shared__ int gxr[GATHER ? kMaxPairs : 1];         // activation row of each pair
  __shared__ int gsorted[GATHER ? kMaxPairs : 1];     // pairs of the slots, in slot order
  __shared__ int gstart[GSORT ? kMaxPairs + 1 : 1];   // first position of each slot
  __shared__ int gslot_exp[GSORT ? kMaxPairs : 1];    // expert of each slot
  __shared__ int gmeta[2];
  int c0 = 0;     // first pair of the current chunk of 16 rows
  int pbase = 0;  // first position in gsorted of the current slot
  const uint8_t *const codes0 = codes;
  const uint16_t *const scales0 = scales;
  const uint16_t *const biases0 = biases;
  if constexpr (GATHER) {
    static_assert(KS == 1 && !PERSIST && !ADD && FMT == kAffine, "gather variant");
    if constexpr (GSORT) {
      gather_route(ga, gexp, gxr, gsorted, gstart, gslot_exp, gmeta);
    } else {
      const int words = (ga.E + 31) >> 5;
      for (int i = threadIdx.x; i < words; i += blockDim.x) gbits[i] = 0u;
      __syncthreads();
      for (int p = threadIdx.x; p < ga.P; p += blockDim.x) {
        const int e = ga.e_idx[p], xi = ga.x_idx[p];
        const bool valid = e >= 0 && e < ga.E && xi >= 0 && xi < ga.X;
        gexp[p] = valid ? e : -1;
        gxr[p] = xi;
        if (valid) atomicOr(&gbits[e >> 5], 1u << (e & 31));
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        // the slot-th set bit of the union bitmap
        const int slot = (int)blockIdx.x / ngroups;
        int seen = 0, expert = -1;
        for (int w = 0; w < words && expert < 0; ++w) {
          uint32_t b = gbits[w];
          const int c = __popc(b);
          if (seen + c > slot) {
            for (int k = slot - seen; k > 0; --k) b &= b - 1;  // drop the lower set bits
            expert = 32 * w + __ffs(b) - 1;
          }
          seen += c;
        }
        gmeta[0] = expert;
      }
      __syncthreads();
      const int expert = gmeta[0];
      if (expert < 0) return;  // slot past the union (uniform for the workgroup)
      if (wave == 0) {
        // pairs of this expert in ascending order (ballot compaction)
        int base = 0;
        for (int p0 = 0; p0 < ga.P; p0 += 64) {
          const int p = p0 + lane;
          const bool hit = p < ga.P && gexp[p] == expert;
          const uint64_t bal = __ballot(hit);
          if (hit) gsorted[base + __popcll(bal & ((1ull << lane) - 1ull))] = p;
          base += __popcll(bal);
        }
        if (lane == 0) gmeta[1] = base;
      }
      __syncthreads();
      const size_t G_ = (size_t)(K / GS);
      codes = codes0 + (size_t)expert * N * ((size_t)K * BITS / 8);
      scales = scales0 + (size_t)expert * N * G_;
      biases = biases0 + (size_t)expert * N * G_;
    }
  }
  // activation row of row m of the current chunk, and its output row
  auto xrow = [&](const int m) -> size_t { return GATHER ? (size_t)gxr[gsorted[pbase + c0 + m]] : (size_t)m; };
  auto yrow = [&](const int m) -> size_t { return GATHER ? (size_t)gsorted[pbase + c0 + m] : (size_t)m; };

  // One tile group (16*NT output columns over all of K) per call of `group`.
  auto group_x = [&](auto xc_tag, const int tg) {
  // compact activation loads: XG operands per load, NLD loads per batch; a
  // load holds operands of one block, and the operands of a load cover part
  // of one super-chunk (LPU loads each) or whole super-chunks (SPL each)
  constexpr int XCV = decltype(xc_tag)::value;
  constexpr int XG = XCV ? 16 / (XCV ? XCV : 1) : 1;
  constexpr int OPS = XR * HS;        // activation operands per super-chunk
  constexpr int NGR = UNR * OPS;      // activation operands per batch
  constexpr int NLD = NGR / XG;
  constexpr int LPU = OPS >= XG ? OPS / XG : 1;
  constexpr int SPL = OPS >= XG ? 1 : XG / OPS;
  static_assert(NGR % XG == 0 && (OPS % XG == 0 || XG % OPS == 0) && (BSC * OPS) % XG == 0,
                "compact activation layout");
  // Activation loads in the quad-row layout (lane L: what lane (L/4, L%4)
  // needs) once several rows are distinct; with few rows most lanes read the
  // same row anyway and the move to the operand lanes would only cost (the
  // data each lane ends up with is the same either way, so results do not
  // depend on the choice).  Thresholds measured on the square shapes; M is
  // the rows of this group (a gathered expert's chunk of pairs).
  const bool xquad = XCV == 0 && (FMT != kAffine || M >= (BITS == 8 ? 3 : (LVL == 0 ? 8 : 5)));
  const int xkb = xquad ? (lane & 3) : kb;
  int xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xoff[i] = lvl_chunk<LVL>(i, xkb) * CW + lvl_dword<LVL>(i, xkb) * DW;
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
  const int rot = (tg >> 3) - div_waves(tg >> 3) * waves;
  const int slice = wave + rot < waves ? wave + rot : wave + rot - waves;
  const int b_begin = p_lo + div_waves(slice * nbp);
  const int b_end = p_lo + div_waves((slice + 1) * nbp);
  const size_t RB = (size_t)K * BITS / 8;
  const int G = FMT == kNvfp4 ? K / 16 : K / GS;  // scale (or scale-and-bias) entries per row
  // Rows m >= M and columns n >= N only feed outputs that are never stored,
  // so their lanes read valid clamped addresses instead of branching around
  // the loads (a branch would force a wait on every load).
  const uint16_t *xr = x + xrow(min(xquad ? (lane >> 2) : col, M - 1)) * K;
  // Compact activation loads (XCV = 4 or 8 rows, M <= XCV; see compact_pick):
  // load ld of a batch carries operands ld*XG .. ld*XG + XG-1 of the batch,
  // numbered (u, i, l) -> (u*OPS + i*HS + l); this lane holds operand
  // ld*XG + lane%XG of row (lane%16)/XG at its K-part kb.  Its element
  // offset within the batch is (ld / LPU)*SPL*SCW + xlp[ld % LPU].
  const uint16_t *xrc = x + xrow(min((lane & 15) / XG, M - 1)) * K;
  int xlp[LPU];
  if constexpr (XCV != 0) {
#pragma unroll
    for (int p = 0; p < LPU; ++p) {
      const int f = p * XG + (lane & (XG - 1));  // operand within the load's first super-chunk
      const int u = f / OPS, i = (f % OPS) / HS, l = f % HS;
      const int ii = BITS == 8 ? 2 * i : i;
      xlp[p] = u * SCW + lvl_chunk<LVL>(ii, kb) * CW + lvl_dword<LVL>(ii, kb) * DW + 8 * l;
    }
  }
  const uint8_t *crow[NT];
  const uint16_t *srow[NT];
  const uint16_t *brow[NT];
  const uint8_t *srow8[NT];  // FP formats: scale bytes
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // codes and metadata: lane L reads for row L/4 (codes: 16-byte piece L%4;
    // see quad_row_lane); moved to the operand lanes before use
    const int nq = min(n_base + 16 * t + (lane >> 2), N - 1);
    crow[t] = codes + (size_t)nq * RB + (lane & 3) * 16;
    srow[t] = scales + (size_t)nq * G;
    brow[t] = biases + (size_t)nq * G;
    srow8[t] = reinterpret_cast<const uint8_t *>(scales) + (size_t)nq * G;
  }

  // residual of the outputs this thread stores in its first NT reduction
  // steps (all of them when the workgroup has at least 4 waves), loaded ahead
  // of the weight stream; clamped indices read a valid element, never used
  float rpre[NT];
  auto load_res = [&]() {
    if constexpr (ADD) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int o = min((int)threadIdx.x + j * (int)blockDim.x, NT * 256 - 1);
        const int l = o & 63;
        const int m = min((4 * (l >> 4) + ((o >> 6) & 3)) / XG, M - 1);
        const int n = min(n_base + 16 * (o >> 8) + (l & 15), N - 1);
        rpre[j] = res[yrow(m) * N + n];
      }
    }
  };

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = zero4;
  // Zero weights (affine codes): nz[t] collects traces of nonzero weights in
  // this lane's quarter of tile t's groups (see zero weights in
  // qgemv_device.h); zc0 is the current group's first code word.  The FP
  // formats never need it.
  uint32_t nz[NT], zc0[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    nz[t] = HAS_BIAS ? 0u : 1u;
    zc0[t] = 0u;
  }

  for (int blk0 = b_begin; blk0 < b_end; blk0 += BPB) {
    const int nb = min(BPB, b_end - blk0);  // blocks in this batch (uniform)
    // ---- issue: activations first (L2), then codes (HBM), then metadata
    u32x4_t xv[UNR][XR][HS];
    u32x4_t cx[XCV ? NLD : 1];
    u32x4_t cv[UNR][NT];
    uint2 s4[BPB][NT], b4[BPB][NT];
    if constexpr (XCV != 0) {
      // a load of a block past the batch reads the batch's first operands
      // (never used)
      const uint16_t *xb = xrc + (size_t)blk0 * BSC * SCW;
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld) {
        const int blk = ld * XG / (BSC * OPS);
        const bool in = blk < nb && (!PB || blk0 * BSC + (ld / LPU) * SPL < NSC);
        cx[ld] = *reinterpret_cast<const u32x4_t *>(xb + (in ? (ld / LPU) * SPL * SCW + xlp[ld % LPU] : xlp[0]));
      }
    } else {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (u / BSC < nb) {
          const int k0 = (PB ? min(blk0 * BSC + u, NSC - 1) : blk0 * BSC + u) * SCW;
#pragma unroll
          for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int l = 0; l < HS; ++l)
              xv[u][i][l] = *reinterpret_cast<const u32x4_t *>(
                  xr + k0 + (BITS == 8 ? xoff[2 * i] : xoff[i]) + 8 * l);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC < nb) {
        const int gsc = PB ? min(blk0 * BSC + u, NSC - 1) : blk0 * BSC + u;
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
            const int gm = PB ? min((blk0 + bb) * 4, G - 4) : (blk0 + bb) * 4;  // inside the row (G >= 4)
            s4[bb][t] = *reinterpret_cast<const uint2 *>(srow[t] + (size_t)gm);
            b4[bb][t] = *reinterpret_cast<const uint2 *>(brow[t] + (size_t)gm);
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
    // the residual is read after the first batch's loads, so that the
    // batch's first wait does not wait for it too
    if constexpr (ADD) {
      if (blk0 == b_begin) load_res();
    }
    // keep the whole batch of loads ahead of the compute: without this the
    // scheduler may sink later loads below the first waits and serialize them
    __builtin_amdgcn_sched_barrier(0);

    // ---- a partial last block (uniform): activations of its missing
    // super-chunks are zero (their metadata fields are moved below, where
    // the metadata is first used: the metadata loads are the batch's last)
    if constexpr (PB) {
      if ((blk0 + nb) * BSC > NSC) {
        if constexpr (XCV != 0) {
#pragma unroll
          for (int ld = 0; ld < NLD; ++ld)
            if (blk0 * BSC + (ld / LPU) * SPL >= NSC) cx[ld] = u32x4_t{0u, 0u, 0u, 0u};
        } else {
#pragma unroll
          for (int u = 0; u < UNR; ++u)
            if (blk0 * BSC + u >= NSC)
#pragma unroll
              for (int i = 0; i < XR; ++i)
#pragma unroll
                for (int l = 0; l < HS; ++l) xv[u][i][l] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }

    // ---- activation work, overlapping the code loads: re-pair x to the
    // code pairing and form the per-group activation sums.  xsum of group
    // g0 + j ends up in row j of this lane's column, i.e. in the A layout of
    // v_mfma_f32_16x16x4_f32 for the bias product.
    if constexpr (XCV != 0) {
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
          for (int l = 0; l < HS; ++l) {
            const int f = (u * XR + i) * HS + l;
            xv[u][i][l] = compact_pick<XG>(cx[f / XG], f % XG);
          }
    } else if (xquad) {
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
          for (int l = 0; l < HS; ++l) xv[u][i][l] = to_operand_lanes(xv[u][i][l]);
    }
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
#pragma unroll
          for (int l = 0; l < HS; ++l) xv[u][i][l] = pair_activations<BITS>(xv[u][i][l]);
        }
      }
      if constexpr (HAS_BIAS) xsum[bb] = rows_transpose_reduce4(P);
    }

    // a partial last block's metadata fields move down to their groups (its
    // missing groups get scale and bias 0)
    if constexpr (PB) {
      if ((blk0 + nb) * BSC > NSC) {
#pragma unroll
        for (int bb = 0; bb < BPB; ++bb) {
          const int sh = (blk0 + bb) * 4 - min((blk0 + bb) * 4, G - 4);  // 0..3 inside K
          if (bb < nb && sh > 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const uint64_t sv = ((uint64_t)s4[bb][t].y << 32 | s4[bb][t].x) >> (16 * sh);
              const uint64_t bv = ((uint64_t)b4[bb][t].y << 32 | b4[bb][t].x) >> (16 * sh);
              s4[bb][t] = make_uint2((uint32_t)sv, (uint32_t)(sv >> 32));
              b4[bb][t] = make_uint2((uint32_t)bv, (uint32_t)(bv >> 32));
            }
          }
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < BPB; ++bb)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        s4[bb][t] = to_operand_lanes(s4[bb][t]);
        if constexpr (HAS_BIAS) b4[bb][t] = to_operand_lanes(b4[bb][t]);
      }
    // zero-weight traces of group j: the step's code words against the
    // group's first (and that word's own spread), then the group's weight
    // s*c + b (c: the first code) at its last step
    auto zero_step = [&](const bool gfirst, const uint32_t (&w)[NT], const int nw, const uint32_t (&w2)[NT]) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (gfirst) {
          zc0[t] = w[t];
          nz[t] |= fields_spread<BITS>(w[t]);
        } else {
          nz[t] |= w[t] ^ zc0[t];
        }
        if (nw == 2) nz[t] |= w2[t] ^ zc0[t];
        pin(nz[t]);
      }
    };
    auto zero_group = [&](const int bb, const int j) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint2 sw_v = s4[bb][t];
        const uint2 bw_v = b4[bb][t];
        nz[t] |= weight_trace(half_bits_to_float(field16(sw_v, j)), low_field<BITS>(zc0[t]),
                              half_bits_to_float(field16(bw_v, j)));
      }
    };
    // ---- codes, super-chunk by super-chunk in load order
    f32x4_t accg[NT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u / BSC >= nb) break;
      const int scb = u % BSC;  // super-chunk within its block
      uint32_t cur[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        to_operand_lanes(cv[u][t], cur[t]);
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
          if constexpr (HAS_BIAS) {
            uint32_t w[NT], w2[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              w[t] = cur[t][2 * e];
              w2[t] = cur[t][2 * e + 1];
            }
            zero_step(gfirst, w, 2, w2);
            if (glast) zero_group(u / BSC, j);
          }
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
                const uint2 sw_v = s4[u / BSC][t];
                sc = half_bits_to_float(field16(sw_v, j));
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
          if constexpr (HAS_BIAS) {
            uint32_t w[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) w[t] = cur[t][i];
            if (h == 0) zero_step(gfirst, w, 1, w);
            if (glast) zero_group(u / BSC, j);
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            u32x4_t bw;
            if constexpr (FMT == kMxfp4) {
              // 8 elements of one dword, natural order
              bw = u32x4_t{fp4_pair<0>(cur[t][i]), fp4_pair<1>(cur[t][i]), fp4_pair<2>(cur[t][i]),
                           fp4_pair<3>(cur[t][i])};
            } else if constexpr (BITS == 4) {
              bw = unpack4_quad(cur[t][i]);
            } else {
              bw = unpack2_quad(cur[t][i], h);
            }
            accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, bw), gfirst ? zero4 : accg[t], 0, 0, 0);
          }
          if (glast) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              float sc;
              if constexpr (HAS_BIAS) {
                const uint2 sw_v = s4[u / BSC][t];
                sc = half_bits_to_float(field16(sw_v, j));
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
        // bias: acc += xsum[m][g0+kb] * b[n][g0+kb]
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint2 bw_v = b4[u / BSC][t];
          const float b = half_bits_to_float(field16(bw_v, kb));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsum[u / BSC], b, acc[t], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (ADD) {
    if (b_begin >= b_end) load_res();  // a wave without blocks
  }

  // split-K reduction over the slices, fixed order; a partial whose column
  // held only zero weights (no trace in any of its four lanes) is exactly 0
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t keep = keep_mask(column_or(nz[t]));
#pragma unroll
    for (int i = 0; i < 4; ++i) red[slice][t][i][lane] = unless_zero(acc[t][i], keep);
  }
  __syncthreads();
  // output o of the tile group: sum over the slices, then store (pre: the
  // residual rv was prefetched)
  auto finish = [&](const int o, const bool pre, float rv) {
    const int t = o >> 8;
    const int i = (o >> 6) & 3;
    const int l = o & 63;
    float s = 0.f;
    for (int w = 0; w < waves; ++w) s += red[w][t][i][l];
    // MFMA row a holds activation row a / XG (compact loads: each row XG times)
    const int a = 4 * (l >> 4) + i;
    const int m = a % XG == 0 ? a / XG : M;
    const int n = n_base + 16 * t + (l & 15);
    if (m < M && n < N) {
      float *dst = y + yrow(m) * N + n;
      if constexpr (ADD) {
        if (!pre) rv = res[yrow(m) * N + n];
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
  auto group = [&](const int tg) {
    if constexpr (XDYN) {
      if (M <= 4) group_x(std::integral_constant<int, 4>{}, tg);
      else group_x(std::integral_constant<int, 0>{}, tg);
    } else {
      group_x(std::integral_constant<int, XC>{}, tg);
    }
  };

  // rows per chunk of a gathered expert's pairs: 16, or the compact row
  // count (the launcher takes it at least the activation rows, so a routing
  // with at most one pair per expert and row still gives one chunk per expert)
  constexpr int CH = XC ? XC : 16;
  if constexpr (GSORT) {
    // items (slot, tile group) in slot-major order, walked with the grid
    // stride; each slot's pairs are taken CH rows at a time
    const int items = gmeta[0] * ngroups;
    const size_t G_ = (size_t)(K / GS);
    bool first = true;
    for (int w = blockIdx.x; w < items; w += gridDim.x) {
      const int slot = w / ngroups;
      const int expert = gslot_exp[slot];
      codes = codes0 + (size_t)expert * N * ((size_t)K * BITS / 8);
      scales = scales0 + (size_t)expert * N * G_;
      biases = biases0 + (size_t)expert * N * G_;
      pbase = gstart[slot];
      const int pairs = gstart[slot + 1] - pbase;
      for (c0 = 0; c0 < pairs; c0 += CH) {
        M = min(CH, pairs - c0);
        if (!first) __syncthreads();  // reduction buffer drained
        first = false;
        group(w - slot * ngroups);
      }
    }
  } else if constexpr (GATHER) {
    // the expert's pairs, CH rows at a time
    const int pairs = gmeta[1];
    for (c0 = 0; c0 < pairs; c0 += CH) {
      M = min(CH, pairs - c0);
      if (c0 != 0) __syncthreads();  // reduction buffer drained
      group((int)blockIdx.x % ngroups);
    }
  } else if constexpr (PERSIST) {
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




}  // namespace

}  // namespace qgemv
