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
//   A = activations (rows m >= M repeat row M-1 and are never stored; with
//   at most 4 or 8 rows each row fills 4 or 2 MFMA rows, loaded compactly:
//   compact_pick in qgemv_device.h),
//   B = weights as exact bf16 code values q (2/4-bit: one code dword per
//   step or half-step; 8-bit: two code dwords per MFMA step).  A workgroup owns NT tiles of
//   16 output columns over the whole of K; its waves split K into
//   contiguous slices of "bias blocks" (4 groups).
// * Lane (col = lane%16, kb = lane/16) needs 16 contiguous bytes of row
//   n = col at byte 16*kb of each 64-byte super-chunk (16 rows x 64 B per
//   load instruction).  The load itself is made with lane L reading piece
//   L%4 of row L/4, so that each lane quad reads 64 contiguous bytes, and
//   ds_bpermute moves the dwords to their operand lanes (to_operand_lanes).
//   A partial exchange of dwords across the four 16-lane rows (none,
//   v_permlane32_swap, or the full 4x4 transpose with v_permlane16_swap, as
//   the group size requires) then gives every MFMA step 32 codes of one
//   quantization group.
// * The group's partial product is accumulated by gs/32 MFMAs and folded with
//   the group scale once: acc += s * acc_g (4 FMAs per lane per group).
// * Bias: sum_g b[n,g] * xsum[m,g] over the 4 groups of a block is one
//   v_mfma_f32_16x16x4_f32, with the per-group activation sums xsum (dot2
//   against ones, then a row transpose-reduce) formed while the codes are
//   still in flight.
// * Zero weights: a lane's column of a tile whose groups so far all held
//   zero weights (codes all equal to c in the column's four lanes and
//   s*c + b exactly 0) keeps a flag; a flagged partial is stored as exactly 0,
//   its exact value, so a row of zero weights gives y = 0 (the factored sum
//   would leave a rounding residue of the size of s*c*sum(x)).  The test runs
//   only while some lane of the wave is flagged.
// * Partial tiles of the waves are summed through LDS in slice order
//   (deterministic, no atomics) and rows m < M are stored.
// * Fused residual sum (ADD, "metal : few-row MMA mat-mul and batched copies
//   for speculative decoding", Overview: MUL_MAT + ADD writes the residual
//   sum from the store): each thread loads the residual of the outputs it
//   will store right after its wave's first batch of loads (ahead of them, it
//   sat in front of the batch's first wait: square 4096^2 M = 3 fused
//   5.60 -> 5.34 us against 5.25 plain) and adds it in the store, so
//   y = fl(product + r), bit for bit the plain call and a separate fp32 add.
// Shapes with more 16-column tiles than CUs go to the persistent kernel
// (qgemv_persist.hip) unless K is too long for its register-resident
// activations.

#include <atomic>

#include "qgemv_mfma_impl.h"

namespace qgemv {

namespace {

__global__ __launch_bounds__(256) void fill_kernel(uint32_t *__restrict__ y, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) y[i] = v;
}

// Workgroups of `waves` waves of kernel `kern` resident on one CU (cached per
// kernel and wave count: the same on every MI355X; concurrent first calls
// store the same value).
template <const void *(*KERN)()>
int resident_per_cu(int waves, std::atomic<int> (&cache)[17]) {
  int occ = cache[waves].load(std::memory_order_relaxed);
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, KERN(), 64 * waves, 0) != hipSuccess || occ <= 0)
      occ = 1;
    cache[waves].store(occ, std::memory_order_relaxed);
  }
  return occ;
}

template <int BITS, int GS, int NT, bool ADD, int FMT, int XC, int KS, bool PERSIST, bool PB>
const void *mfma_kernel_ptr() {
  constexpr int MAXT = MfmaShape<BITS, GS, NT>::MAXT;
  constexpr int SPI = MfmaShape<BITS, GS, NT>::SPI;
  return reinterpret_cast<const void *>(
      qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, KS, PERSIST, ADD, FMT, false, XC, false, PB>);
}

// Launch with XC compact activation rows (0: none).  The persistent grid
// takes no compact variant.
template <int BITS, int GS, int NT, bool ADD, int FMT, int XC, bool PB>
int launch_mfma_k(const QgemvArgs &a, int ksplit, bool single, int waves, int grid, int groups,
                  hipStream_t stream) {
  constexpr int MAXT = MfmaShape<BITS, GS, NT>::MAXT;
  constexpr int SPI = MfmaShape<BITS, GS, NT>::SPI;
  const auto kern = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 1, XC == 0, ADD, FMT, false, XC, false, PB>;
  const auto kern1 = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 1, false, ADD, FMT, false, XC, false, PB>;
  const auto kern_s = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 2, XC == 0, ADD, FMT, false, XC, false, PB>;
  const auto kern1_s = qgemv_mfma_kernel<BITS, GS, NT, MAXT, SPI, 2, false, ADD, FMT, false, XC, false, PB>;
  const auto k = ksplit == 1 ? (single ? kern1 : kern) : (single ? kern1_s : kern_s);
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * waves), 0, stream, a.codes, a.scales, a.biases, a.x,
                     a.y, a.res, a.M, a.N, a.K, groups, GatherArgs{});
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

template <int BITS, int GS, int NT, bool ADD, int FMT, bool PB>
int launch_mfma_t(const QgemvArgs &a, hipStream_t stream) {
  constexpr int MAXT = MfmaShape<BITS, GS, NT>::MAXT;
  static_assert(MAXT / 64 <= 16, "wave cap");
  const int nblk = (a.K + 4 * GS - 1) / (4 * GS);  // the last block may be partial
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
  // one tile group per workgroup when all are resident at once, else the
  // persistent grid (one per resident workgroup, walking the groups)
  static std::atomic<int> occ0[17], occ4[2][17], occ8[2][17];
  const int slots = resident_per_cu<mfma_kernel_ptr<BITS, GS, NT, ADD, FMT, 0, 1, true, PB>>(waves, occ0) * cus;
  const bool single = groups <= slots;
  if (ksplit == 2) {
    const int st = launch_fill(a.y, (size_t)a.M * a.N, ADD ? kSplitSentinel : 0u, stream);
    if (st != QGEMV_OK) return st;
  }
  const int grid = single ? groups : slots;
  // Activations of up to 4 or 8 rows in compact loads (compact_pick: 4 or 2
  // times fewer activation load instructions per batch; square 4096^2 M = 2:
  // 4-bit 5.55 -> 5.39 us, 8-bit 6.95 -> 6.54, mxfp4 5.55 -> 5.25, nvfp4
  // 5.91 -> 5.37; 27B k 6.79 -> 6.63), with one tile per workgroup and only
  // where all the workgroups of the compact variant, which holds more
  // registers, are resident at once.  Two tiles per workgroup measured slower
  // with them (8-bit 3840 x 15360 at M = 2: 19.6 -> 23.2 us).  The arithmetic
  // is the same either way.
  if constexpr (NT == 1) {
    auto fits = [&](const int occ) { return groups <= occ * cus; };
    if (single && a.M <= 4 &&
        fits(ksplit == 1 ? resident_per_cu<mfma_kernel_ptr<BITS, GS, NT, ADD, FMT, 4, 1, false, PB>>(waves, occ4[0])
                         : resident_per_cu<mfma_kernel_ptr<BITS, GS, NT, ADD, FMT, 4, 2, false, PB>>(waves, occ4[1])))
      return launch_mfma_k<BITS, GS, NT, ADD, FMT, 4, PB>(a, ksplit, single, waves, grid, groups, stream);
    // (not with a partial last block: there the 8-row form measured slower
    // than the full one, 11008 x 4096 at M = 8: 18.7 against 14.6 us)
    if (!PB && single && a.M <= 8 &&
        fits(ksplit == 1 ? resident_per_cu<mfma_kernel_ptr<BITS, GS, NT, ADD, FMT, 8, 1, false, PB>>(waves, occ8[0])
                         : resident_per_cu<mfma_kernel_ptr<BITS, GS, NT, ADD, FMT, 8, 2, false, PB>>(waves, occ8[1])))
      return launch_mfma_k<BITS, GS, NT, ADD, FMT, 8, PB>(a, ksplit, single, waves, grid, groups, stream);
  }
  return launch_mfma_k<BITS, GS, NT, ADD, FMT, 0, PB>(a, ksplit, single, waves, grid, groups, stream);
}

template <int BITS, int GS, int FMT = kAffine>
int launch_mfma_gs(const QgemvArgs &a, hipStream_t stream) {
  // more output columns per workgroup on wide matrices: every workgroup reads
  // all M*K activations, so wider groups cut that traffic per weight byte.
  // The choice depends on the shape only: the two-tile kernel has half the
  // thread cap, so it splits K into other wave slices, and a choice by M
  // would make the rows of an M-row call differ in the last bits from the
  // single-row calls.  (Two tiles on long K once M > 8 measured 36.0 against
  // 39.6 us at M = 16 on the 17408-long down projection where the
  // persistent kernels do not run, and slower than one tile below M = 8.)
  const int tiles = (a.N + 15) / 16;
  const int cus = device_cu_count();
  const bool wide = tiles >= 2 * cus;
  // a partial last bias block: its own variant (affine 2/4-bit codes whose
  // blocks span more than one super-chunk)
  constexpr bool CAN_PB = FMT == kAffine && BITS != 8 && 4 * GS > 512 / BITS;
  if constexpr (CAN_PB) {
    if (a.K % (4 * GS) != 0) {
      if (a.res) {
        if (wide) return launch_mfma_t<BITS, GS, 2, true, FMT, true>(a, stream);
        return launch_mfma_t<BITS, GS, 1, true, FMT, true>(a, stream);
      }
      if (wide) return launch_mfma_t<BITS, GS, 2, false, FMT, true>(a, stream);
      return launch_mfma_t<BITS, GS, 1, false, FMT, true>(a, stream);
    }
  }
  if (a.K % (4 * GS) != 0) return QGEMV_EUNSUPPORTED;
  if (a.res) {
    if (wide) return launch_mfma_t<BITS, GS, 2, true, FMT, false>(a, stream);
    return launch_mfma_t<BITS, GS, 1, true, FMT, false>(a, stream);
  }
  if (wide) return launch_mfma_t<BITS, GS, 2, false, FMT, false>(a, stream);
  return launch_mfma_t<BITS, GS, 1, false, FMT, false>(a, stream);
}

}  // namespace

int launch_fill(float *y, size_t n, uint32_t v, hipStream_t stream) {
  const int fb = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(fill_kernel, dim3(fb), dim3(256), 0, stream, reinterpret_cast<uint32_t *>(y), n, v);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

bool mfma_supports_fp(int K, int fmt) {
  (void)fmt;
  return K % 128 == 0;  // one 128-element block of bias blocks per super-chunk
}

// Whole 64-byte super-chunks and whole groups; bias blocks of 4 groups, of
// which the single-pass kernel also takes a partial last one (2- and 4-bit
// codes, at least 4 groups in K); the persistent kernels need whole blocks
// (mfma_whole_blocks).
bool mfma_supports(int K, int bits, int group_size) {
  if (bits == 2 && group_size < 64) return false;
  const int scw = 512 / bits;  // codes per 64-byte super-chunk
  if (K % scw != 0 || K % group_size != 0) return false;
  return K % (4 * group_size) == 0 || (bits != 8 && K / group_size >= 4);
}

bool mfma_whole_blocks(int K, int group_size) { return K % (4 * group_size) == 0; }

int launch_mfma(const QgemvArgs &a, hipStream_t stream) {
  if (a.fmt != kAffine) {
    if (!mfma_supports_fp(a.K, a.fmt)) return QGEMV_EUNSUPPORTED;
    if (a.fmt == kMxfp4) return launch_mfma_gs<4, 32, kMxfp4>(a, stream);
    if (a.fmt == kNvfp4) return launch_mfma_gs<4, 32, kNvfp4>(a, stream);
    return launch_mfma_gs<8, 32, kMxfp8>(a, stream);
  }
  if (!mfma_supports(a.K, a.bits, a.group_size)) return QGEMV_EUNSUPPORTED;
  // more tiles than CUs: the persistent kernel streams several tiles per CU,
  // with the activations in registers, or, for K too long for them, in LDS
  // (one half of K per workgroup); otherwise one tile group per workgroup in
  // a single pass
  if ((a.N + 15) / 16 > device_cu_count() && mfma_whole_blocks(a.K, a.group_size)) {
    int st = launch_persist(a, stream);
    if (st != QGEMV_EUNSUPPORTED) return st;
    st = launch_persist_x(a, stream);
    if (st != QGEMV_EUNSUPPORTED) return st;
  }
  if (a.bits == 8) {
    switch (a.group_size) {
      case 32: return launch_mfma_gs<8, 32>(a, stream);
      case 64: return launch_mfma_gs<8, 64>(a, stream);
      case 128: return launch_mfma_gs<8, 128>(a, stream);
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
