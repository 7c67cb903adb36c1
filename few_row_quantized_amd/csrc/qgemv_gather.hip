// Gathered (MoE) verify: y[p] = x[x_idx[p]] . dequant(W[e_idx[p]])^T over
// (activation row, expert) pairs, the MoE form of the verify product (MLX
// page, Facts: dense and MoE gather_qmm verify, whose expert-union cost per
// verify row is named as unstudied).
//
// Every expert in the union of e_idx is read from HBM once per call, for all
// the pairs routed to it.  With 3 or more activation rows (X) and a shape the
// persistent MFMA kernel takes, that kernel does it (GATHER variant in
// qgemv_persist.hip: contiguous ranges of the (chunk, tile) items per
// workgroup, streamed through its code prefetch ring).  Otherwise the
// single-pass MFMA kernel (GATHER variant in qgemv_mfma_impl.h) does, as
// follows.  The work is the (expert slot, 16-column tile group)
// items, slots being the union's experts in ascending id order, each with its
// pairs in ascending order taken 16 rows at a time (4 when there are at most
// 4 activation rows; a chunk of at most 4 pairs loads its activations in the
// compact form either way).  The host does not know the union size (the
// routing stays on the device), so it plans for min(P, E) slots:
// * one tile per workgroup: a grid of the workgroups resident at once, each
//   sorting the routing once and walking the items with the grid stride
//   (measured on the 128-expert top-8 1536 x 2048 gate/up shape: 80.7 ->
//   70.4 us at M = 16, 44.6 -> 40.3 at M = 8, 9.9 -> 8.9 at M = 1, against
//   one workgroup per item with the routing prologue in each);
// * two tiles per workgroup (short K): one workgroup per item, which finds
//   its slot's expert from a bitmap of the union and exits when the slot is
//   past it (there the per-workgroup rank sort cost more than it saved:
//   2048 x 768 +8 to +17%).

#include <atomic>

#include "qgemv_mfma_impl.h"

namespace qgemv {

namespace {

constexpr int kGatherWideTiles = 64;

template <int BITS, int GS, int NT, int XC, bool XDYN, bool PB = false>
int launch_gather_nt(const QgemvArgs &a, const GatherArgs &ga, hipStream_t stream) {
  constexpr int MAXT = MfmaShape<BITS, GS, NT>::MAXT;
  constexpr int SPI = MfmaShape<BITS, GS, NT>::SPI;
  const auto kern = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 1, false, false, kAffine, true, XC, XDYN, PB>;
  const int nblk = (a.K + 4 * GS - 1) / (4 * GS);  // the last block may be partial
  // at most 4 waves (K-slices) per item: more workgroups resident per CU, so
  // more items' loads in flight (128-expert top-8 1536 x 2048 gate/up: 70.3 ->
  // 60.2 us at M = 16, 40.0 -> 33.8 at M = 8, 8.74 -> 8.75 at M = 1; 2 waves:
  // 56.5 at M = 16 but 9.75 at M = 1).  Fixed by the shape, so a pair's row
  // does not depend on the other pairs of the call.
  const int waves = pick_waves(nblk, MAXT / 64 < 4 ? MAXT / 64 : 4);
  const int groups = ((a.N + 15) / 16 + NT - 1) / NT;
  const int slots = ga.P < ga.E ? ga.P : ga.E;
  // at most kMaxPairs * 2^18 (slot, tile group) items: within the grid limit.
  // One tile per workgroup: at most the workgroups resident at once, each
  // walking the items with the grid stride (the routing is sorted once per
  // workgroup); two tiles: one workgroup per item.
  unsigned blocks = (unsigned)slots * (unsigned)groups;
  if constexpr (NT == 1) {
    static std::atomic<int> occ_cache[MAXT / 64 + 1];
    int occ = occ_cache[waves].load(std::memory_order_relaxed);
    if (occ == 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void *>(kern),
                                                       64 * waves, 0) != hipSuccess ||
          occ <= 0)
        occ = 1;
      occ_cache[waves].store(occ, std::memory_order_relaxed);
    }
    const unsigned cap = (unsigned)occ * (unsigned)device_cu_count();
    if (blocks > cap) blocks = cap;
  }
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * waves), 0, stream, a.codes, a.scales, a.biases,
                     a.x, a.y, static_cast<const float *>(nullptr), 16, a.N, a.K, groups, ga);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

// Two 16-column tiles per workgroup when K is short (at most 4 bias blocks,
// so at most 4 waves) and the expert has at least 64 tiles: the routing
// prologue and the activation loads are then shared by twice the weight
// bytes.  Measured on the 128-expert top-8 shapes at M = 16: 2048 x 768
// 37.5 -> 29.0 us; 1536 x 2048 (8 blocks) 84.2 -> 87.0 us, so it stays at one.
template <int BITS, int GS>
int launch_gather_t(const QgemvArgs &a, const GatherArgs &ga, hipStream_t stream) {
  // experts with a partial last bias block: the single-pass kernel's variant
  // for them, one tile per workgroup
  constexpr bool CAN_PB = BITS != 8 && 4 * GS > 512 / BITS;
  if (a.K % (4 * GS) != 0) {
    if constexpr (CAN_PB) {
      if (ga.X <= 4) return launch_gather_nt<BITS, GS, 1, 4, false, true>(a, ga, stream);
      return launch_gather_nt<BITS, GS, 1, 0, true, true>(a, ga, stream);
    }
    return QGEMV_EUNSUPPORTED;
  }
  if ((a.N + 15) / 16 >= kGatherWideTiles && a.K / (4 * GS) <= 4)
    return launch_gather_nt<BITS, GS, 2, 0, false>(a, ga, stream);
  // from 3 activation rows, the persistent kernel over (chunk, tile) ranges,
  // where a shape fits it (the 128-expert top-8 2048 -> 1536 gate/up: 17.4
  // -> 16.6 us at M = 3, 33.3 -> 28.7 at M = 8, 58.2 -> 48.5 at M = 16, one
  // run; at M = 1 and 2 it measured 8.35 -> 8.88 and 12.00 -> 12.75, its
  // few items per workgroup not paying for the routing prologue)
  if (ga.X >= 3) {
    const int st = launch_persist_gather(a, ga, stream);
    if (st != QGEMV_EUNSUPPORTED) return st;
  }
  // activation rows in compact loads (compact_pick) when there are at most 4
  // of them: a valid routing then sends each expert at most 4 pairs, one
  // chunk (128-expert top-8 2048 -> 1536 gate/up: 8.89 -> 8.46 us at M = 1,
  // 20.98 -> 20.06 at M = 4; with 8 rows at M = 5..8 within 1%); with more
  // rows, each chunk of at most 4 pairs takes them (the same shape: 25.7 ->
  // 25.1 us at M = 5, 60.3 -> 58.3 at M = 16; with two tiles per workgroup
  // neither helped: 2048 x 768 +1% at M = 5..16)
  if (ga.X <= 4) return launch_gather_nt<BITS, GS, 1, 4, false>(a, ga, stream);
  return launch_gather_nt<BITS, GS, 1, 0, true>(a, ga, stream);
}

}  // namespace

int launch_gather(const QgemvArgs &a, const int32_t *x_idx, const int32_t *e_idx, int P, int X,
                  int E, hipStream_t stream) {
  if (!mfma_supports(a.K, a.bits, a.group_size)) return QGEMV_EUNSUPPORTED;
  const GatherArgs ga{x_idx, e_idx, P, X, E};
  if (a.bits == 4) {
    switch (a.group_size) {
      case 32: return launch_gather_t<4, 32>(a, ga, stream);
      case 64: return launch_gather_t<4, 64>(a, ga, stream);
      case 128: return launch_gather_t<4, 128>(a, ga, stream);
    }
  } else if (a.bits == 2) {
    switch (a.group_size) {
      case 64: return launch_gather_t<2, 64>(a, ga, stream);
      case 128: return launch_gather_t<2, 128>(a, ga, stream);
    }
  } else {
    switch (a.group_size) {
      case 32: return launch_gather_t<8, 32>(a, ga, stream);
      case 64: return launch_gather_t<8, 64>(a, ga, stream);
      case 128: return launch_gather_t<8, 128>(a, ga, stream);
    }
  }
  return QGEMV_EUNSUPPORTED;
}

}  // namespace qgemv
