// Multi-row dot path of the few-row quantized GEMV (gfx950).
//
// Design (MI355X-first restatement of the "dequantize once, reuse across the
// rows" idea: specgate-metal README, the mul_mv_ext rows 2..5 kernels; MLX
// quantized_matmul small-M verify kernels, Facts: qmv_wide dequantizes each
// group once into registers and reuses it across the M rows of a tile):
//
// * A workgroup is 4 waves; each wave owns a tile of R consecutive output rows
//   n.  The 64 lanes of a wave split K: lane l takes 16-byte code chunks
//   l, l+64, l+128, ... of every row in its tile, so each load instruction of
//   the wave reads 1 KiB of one row contiguously (128-bit loads, fully
//   coalesced).  Codes are read from HBM exactly once per call.
// * The M activation rows are staged in LDS once per workgroup, already
//   re-paired to match the code pairing (elements (0,2), (1,3), (4,6), (5,7)
//   of each 8 for 4-bit codes, (e, e+4) of each 8 for 2-bit codes), together
//   with the activation sum of every lane chunk.  K is staged in pieces when
//   M*K does not fit the LDS budget.
// * Each code dword is unpacked once into exact bf16 pairs q (no offset) and
//   used for all M rows with v_dot2c_f32_bf16.  The group's scale and bias
//   are applied once per lane chunk and row: acc += s*d + b*sum(x), i.e. the
//   scale is folded out of the inner loop (MLX page, Facts: the qmv_wide
//   tuning bullet) and metadata is read directly per group, not cached across
//   lanes (same page: the scale-caching patch regressed).
// * Zero weights: a lane whose chunks of row r all hold zero weights (every
//   code equal to c and fma(s, c, b) == 0) contributes exactly 0 for that
//   row (see zero_weights in qgemv_device.h), so a row of zero weights gives
//   y = 0 exactly.
// * The R*M per-lane partial sums are reduced across the wave with
//   permlane32/permlane16 swaps and a DPP butterfly, then stored.
// * Fused residual sum (ADD): the residual elements a lane will store are
//   loaded at the start, ahead of the weight stream, and added to the reduced
//   product in the store ("metal : few-row MMA mat-mul and batched copies for
//   speculative decoding", Overview: MUL_MAT + ADD writes the residual sum
//   from the store), so y = fl(product + r): bit for bit the plain call
//   followed by a separate fp32 add.
//
// Per-row accumulation order depends only on K and the lane mapping, never on
// M, so row m of an M-row call equals the M=1 call bitwise.

#pragma once

#include "qgemv_device.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

constexpr int kDotThreads = 256;
constexpr int kDotWaves = kDotThreads / 64;
constexpr int kMaxPasses = 3;  // lane passes (of 64 chunks) per LDS stage, at most

// ADD: y = product + res (the fused residual sum); res may equal y (each
// element is read and then written by the same lane), so neither pointer is
// declared restrict.
// FMT: kAffine (fp16 scale and bias per group) or a block-scaled FP format
// (kMxfp4, kNvfp4, kMxfp8: one scale byte per block in `scales`, no bias).
// XR: with one activation row (two for 8-bit codes and the FP formats, when
// they fit 16 registers of x per lane), each lane loads the x chunks of its
// own code chunks straight into registers and pairs them there (no LDS
// staging, no workgroup barrier; the same arithmetic in the same order as the
// staging, so results are bit for bit those of the staged kernel).  Used
// where the grid has at most two workgroups per CU: it needs more registers,
// which costs occupancy on larger grids (measured: square 4096^2 4-bit 4.83 ->
// 4.56 us at M = 1, 27B gate 13.3 -> 15.2 us).  At M = 2 on the 4096^2
// matrices: 8-bit 7.54 -> 6.86 us, mxfp4 5.02 -> 4.69, nvfp4 5.33 -> 5.17,
// mxfp8 6.80 -> 6.21, but 4-bit affine 5.15 -> 5.29, which keeps the staging.
template <int BITS, int M, int R, int NSUB, int P, bool ADD, int FMT, bool XR = false>
__global__ __launch_bounds__(kDotThreads) void qgemv_dot_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x, float *y,
    const float *res, int N, int K, int gs, int kch) {
  constexpr int CW = 128 / BITS;        // weights per 16-byte code chunk
  constexpr int QUADS = CW / 8;         // 16-byte units of paired x per (row m, chunk)
  constexpr int QPS = QUADS / NSUB;     // quads per metadata sub-chunk
  constexpr int SUBW = CW / NSUB;       // weights per sub-chunk
  constexpr int V = ((R * M + 3) / 4) * 4;
  // activations in memory order (8-bit codes, FP elements) or re-paired to
  // the split pairing in which the 2/4-bit codes are decoded
  constexpr bool NATURAL = BITS == 8 || FMT != kAffine;
  constexpr bool HAS_BIAS = FMT == kAffine;
  constexpr bool XREG = XR && (M == 1 || (M == 2 && !(FMT == kAffine && BITS == 4))) &&
                        M * (CW / 8) * P <= 16;
  const uint8_t *scales8 = reinterpret_cast<const uint8_t *>(scales);

  extern __shared__ uint4 lds[];
  uint4 *xl = lds;                                              // [M][QUADS][kch]
  float *xsl = reinterpret_cast<float *>(lds + M * QUADS * kch);  // [M][NSUB][kch]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kDotWaves + wave) * R;
  const int NC = K / CW;
  const int G = K / gs;
  const size_t RB = (size_t)K * BITS / 8;

  // Residual of the outputs this lane stores (lane 16*rho stores value
  // indices 4j + row_value_index(rho)), loaded before the weight stream so its
  // latency is hidden; lanes and indices without an output read a clamped
  // valid element and never use it.
  float rres[V / 4];
  if constexpr (ADD) {
    const int rv = row_value_index(lane >> 4);
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const int idx = min(4 * j + rv, R * M - 1);
      const int n = min(row0 + idx / M, N - 1);
      rres[j] = res[(size_t)(idx % M) * N + n];
    }
  }

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
  // traces of nonzero weights in row r's chunks of this lane (affine codes;
  // see zero weights in qgemv_device.h); the FP formats never need them
  uint32_t nz[R];
#pragma unroll
  for (int r = 0; r < R; ++r) nz[r] = HAS_BIAS ? 0u : 1u;

  for (int c0 = 0; c0 < NC; c0 += kch) {
    const int nc = min(kch, NC - c0);

    // 1. activations for staging, first units: loaded before the codes so that
    //    writing them to LDS does not wait for HBM.  Loads never sit behind a
    //    per-lane branch (that would force a wait right after each load):
    //    lanes past the end read a valid clamped address and ignore the data.
    const int units = M * nc;
    const int npass = (nc + 63) >> 6;  // uniform
    if (!XREG && c0 != 0) __syncthreads();  // previous stage fully consumed
    // Units are visited in an order rotated per workgroup (by blockIdx/8:
    // workgroups are dealt round-robin over the 8 XCDs) so that the CUs sharing
    // an L2 do not all read the same activation lines at the same moment.
    const int rot = (int)(((blockIdx.x >> 3) * 64u) % (unsigned)units);
    auto unit_of = [&](int uu) { return uu + rot < units ? uu + rot : uu + rot - units; };
    // staging units per thread loaded ahead: a stage holds at most 64*P
    // chunks, i.e. M*64*P units, so one unit per thread while M*P <= 4, two
    // otherwise (the launcher keeps M*kch within two units per thread)
    constexpr int JU = XREG ? 0 : (M * P <= 4 ? 1 : 2);
    uint4 xa[JU > 0 ? JU : 1][CW / 8];
    // XREG: the x chunks of this lane's pass t, row m (clamped past the end)
    uint4 xg[XREG ? P : 1][XREG ? M : 1][CW / 8];
    if constexpr (XREG) {
#pragma unroll
      for (int t = 0; t < P; ++t) {
        const int c = min(lane + 64 * t, nc - 1);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int i = 0; i < CW / 8; ++i)
            xg[t][m][i] = reinterpret_cast<const uint4 *>(x + (size_t)m * K + (size_t)(c0 + c) * CW)[i];
      }
    }
#pragma unroll
    for (int j = 0; j < JU; ++j) {
      const int u = unit_of(min((int)threadIdx.x + kDotThreads * j, units - 1));
      const int m = u / nc;
      const int cl = u - m * nc;
#pragma unroll
      for (int i = 0; i < CW / 8; ++i)
        xa[j][i] = reinterpret_cast<const uint4 *>(x + (size_t)m * K + (size_t)(c0 + cl) * CW)[i];
    }

    // 2. code and metadata loads for this stage, in the order they are consumed
    uint4 cw[P][R];
    uint32_t sr[P][R][NSUB], br[P][R][NSUB];
#pragma unroll
    for (int t = 0; t < P; ++t) {
      if (t < npass) {
        const int c = min(lane + 64 * t, nc - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int n = min(row0 + r, N - 1);
          const u32x4_t v = load_stream_u32x4(codes + (size_t)n * RB + (size_t)(c0 + c) * 16);
          cw[t][r] = make_uint4(v[0], v[1], v[2], v[3]);
#pragma unroll
          for (int s = 0; s < NSUB; ++s) {
            const int g = ((c0 + c) * CW + s * SUBW) / gs;
            if constexpr (HAS_BIAS) {
              sr[t][r][s] = scales[(size_t)n * G + g];
              br[t][r][s] = biases[(size_t)n * G + g];
            } else {
              sr[t][r][s] = scales8[(size_t)n * G + g];
            }
          }
        }
      }
    }

    // all loads of the stage stay ahead of the staging and compute
    __builtin_amdgcn_sched_barrier(0);

    // 3. stage x: paired layout + per-sub-chunk sums (units beyond the first
    //    two per thread are loaded here, which only happens for large M)
    auto stage_unit = [&](int u, const uint4 (&xv)[CW / 8]) {
      const int m = u / nc;
      const int cl = u - m * nc;
      uint32_t X[CW / 2];
#pragma unroll
      for (int i = 0; i < CW / 8; ++i) {
        X[4 * i] = xv[i].x;
        X[4 * i + 1] = xv[i].y;
        X[4 * i + 2] = xv[i].z;
        X[4 * i + 3] = xv[i].w;
      }
      float ssum[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) ssum[s] = 0.f;
      if constexpr (HAS_BIAS) {
#pragma unroll
        for (int i = 0; i < CW / 2; ++i)
          ssum[(2 * i) / SUBW] = dot2_bf16(X[i], 0x3F803F80u, ssum[(2 * i) / SUBW]);
      }
      if constexpr (NATURAL) {
        // natural pairs: quad d holds elements 8d..8d+7 in memory order
#pragma unroll
        for (int d = 0; d < QUADS; ++d)
          xl[(m * QUADS + d) * kch + cl] = make_uint4(X[4 * d], X[4 * d + 1], X[4 * d + 2], X[4 * d + 3]);
      } else if constexpr (BITS == 4) {
        // code dword d covers elements 8d..8d+7; pairs (0,2), (1,3), (4,6), (5,7)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t Xd[4] = {X[4 * d], X[4 * d + 1], X[4 * d + 2], X[4 * d + 3]};
          uint4 q;
          q.x = xpair4(Xd, 0);
          q.y = xpair4(Xd, 1);
          q.z = xpair4(Xd, 2);
          q.w = xpair4(Xd, 3);
          xl[(m * QUADS + d) * kch + cl] = q;
        }
      } else {
        // code dword d covers elements 16d..16d+15; quad (d, h) holds half h,
        // elements 16d+8h..16d+8h+7, paired (e, e+4)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t Xd[4] = {X[8 * d + 4 * h], X[8 * d + 4 * h + 1], X[8 * d + 4 * h + 2],
                                    X[8 * d + 4 * h + 3]};
            uint4 q;
            q.x = xpair_stride4(Xd, 0);
            q.y = xpair_stride4(Xd, 1);
            q.z = xpair_stride4(Xd, 2);
            q.w = xpair_stride4(Xd, 3);
            xl[(m * QUADS + 2 * d + h) * kch + cl] = q;
          }
        }
      }
      if constexpr (HAS_BIAS) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s) xsl[(m * NSUB + s) * kch + cl] = ssum[s];
      }
    };
#pragma unroll
    for (int j = 0; j < JU; ++j) {
      const int uu = threadIdx.x + kDotThreads * j;
      if (uu < units) stage_unit(unit_of(uu), xa[j]);
    }
    for (int uu = threadIdx.x + JU * kDotThreads; !XREG && uu < units; uu += kDotThreads) {
      const int u = unit_of(uu);
      const int m = u / nc;
      const int cl = u - m * nc;
      uint4 xv[CW / 8];
#pragma unroll
      for (int i = 0; i < CW / 8; ++i)
        xv[i] = reinterpret_cast<const uint4 *>(x + (size_t)m * K + (size_t)(c0 + cl) * CW)[i];
      stage_unit(u, xv);
    }
    // XREG: pairs and sums of the lane's own chunks, as stage_unit forms them
    uint4 xq[XREG ? P : 1][XREG ? M : 1][QUADS];
    float xsm[XREG ? P : 1][XREG ? M : 1][NSUB];
    if constexpr (XREG) {
#pragma unroll
      for (int t = 0; t < P; ++t)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        uint32_t X[CW / 2];
#pragma unroll
        for (int i = 0; i < CW / 8; ++i) {
          X[4 * i] = xg[t][m][i].x;
          X[4 * i + 1] = xg[t][m][i].y;
          X[4 * i + 2] = xg[t][m][i].z;
          X[4 * i + 3] = xg[t][m][i].w;
        }
#pragma unroll
        for (int s = 0; s < NSUB; ++s) xsm[t][m][s] = 0.f;
        if constexpr (HAS_BIAS) {
#pragma unroll
          for (int i = 0; i < CW / 2; ++i)
            xsm[t][m][(2 * i) / SUBW] = dot2_bf16(X[i], 0x3F803F80u, xsm[t][m][(2 * i) / SUBW]);
        }
        if constexpr (NATURAL) {
#pragma unroll
          for (int d = 0; d < QUADS; ++d) xq[t][m][d] = make_uint4(X[4 * d], X[4 * d + 1], X[4 * d + 2], X[4 * d + 3]);
        } else if constexpr (BITS == 4) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t Xd[4] = {X[4 * d], X[4 * d + 1], X[4 * d + 2], X[4 * d + 3]};
            xq[t][m][d] = make_uint4(xpair4(Xd, 0), xpair4(Xd, 1), xpair4(Xd, 2), xpair4(Xd, 3));
          }
        } else {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t Xd[4] = {X[8 * d + 4 * h], X[8 * d + 4 * h + 1], X[8 * d + 4 * h + 2],
                                      X[8 * d + 4 * h + 3]};
              xq[t][m][2 * d + h] = make_uint4(xpair_stride4(Xd, 0), xpair_stride4(Xd, 1),
                                               xpair_stride4(Xd, 2), xpair_stride4(Xd, 3));
            }
          }
        }
      }
    } else {
      __syncthreads();
    }

    // 4. multi-row dot products over this stage, in load order
#pragma unroll
    for (int t = 0; t < P; ++t) {
      const int c = lane + 64 * t;
      if (t >= npass || c >= nc) continue;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        float d[R][M];
        uint32_t zc0[R];  // first code dword of the sub-chunk, row r
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < M; ++m) d[r][m] = 0.f;
#pragma unroll
        for (int qq = 0; qq < QPS; ++qq) {
          const int q = s * QPS + qq;
          uint32_t pr[R][4];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t cd[4] = {cw[t][r].x, cw[t][r].y, cw[t][r].z, cw[t][r].w};
            if constexpr (HAS_BIAS) {
              // quad q reads code dword q (4-bit), q >> 1 (2-bit) or 2q, 2q + 1
              // (8-bit): traces of their differences from the sub-chunk's
              // first word, and of that word's own spread
              const int dq = BITS == 8 ? 2 * q : (BITS == 4 ? q : (q >> 1));
              if (qq == 0) {
                zc0[r] = cd[dq];
                nz[r] |= fields_spread<BITS>(cd[dq]);
              } else if (BITS != 2 || (q & 1) == 0) {
                nz[r] |= cd[dq] ^ zc0[r];
              }
              if constexpr (BITS == 8) nz[r] |= cd[dq + 1] ^ zc0[r];
            }
            if constexpr (FMT == kMxfp4 || FMT == kNvfp4) {
              // quad q = code dword q (elements 8q..8q+7, natural pairs)
              unpack_fp4_pairs(cd[q], pr[r]);
            } else if constexpr (FMT == kMxfp8) {
              uint32_t lo[2], hi[2];
              unpack_fp8_pairs(cd[2 * q], lo);
              unpack_fp8_pairs(cd[2 * q + 1], hi);
              pr[r][0] = lo[0];
              pr[r][1] = lo[1];
              pr[r][2] = hi[0];
              pr[r][3] = hi[1];
            } else if constexpr (BITS == 8) {
              // quad q = code dwords 2q, 2q+1 (codes 8q..8q+7, natural pairs)
              uint32_t lo[2], hi[2];
              unpack8_pairs(cd[2 * q], lo);
              unpack8_pairs(cd[2 * q + 1], hi);
              pr[r][0] = lo[0];
              pr[r][1] = lo[1];
              pr[r][2] = hi[0];
              pr[r][3] = hi[1];
            } else if constexpr (BITS == 4) {
              unpack4_pairs(cd[q], pr[r]);
            } else {
              uint32_t p8[8];
              unpack2_pairs(cd[q >> 1], p8);
#pragma unroll
              for (int e = 0; e < 4; ++e) pr[r][e] = p8[4 * (q & 1) + e];
            }
          }
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const uint4 xv = XREG ? xq[t][m][q] : xl[(m * QUADS + q) * kch + c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              float a = d[r][m];
              a = dot2_bf16(pr[r][0], xv.x, a);
              a = dot2_bf16(pr[r][1], xv.y, a);
              a = dot2_bf16(pr[r][2], xv.z, a);
              a = dot2_bf16(pr[r][3], xv.w, a);
              d[r][m] = a;
            }
          }
        }
        // fold the scale (and, for affine codes, the bias) once per sub-chunk
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if constexpr (!HAS_BIAS) {
            const float sc = fp_scale_to_float<FMT>(sr[t][r][s]);
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = fmaf(sc, d[r][m], acc[r][m]);
          } else {
            const float sc = half_bits_to_float(sr[t][r][s]);
            const float bo = half_bits_to_float(br[t][r][s]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const float xs = XREG ? xsm[t][m][s] : xsl[(m * NSUB + s) * kch + c];
              acc[r][m] = fmaf(sc, d[r][m], fmaf(bo, xs, acc[r][m]));
            }
            // trace of the sub-chunk's weight s*c + b (c: its first code)
            nz[r] |= weight_trace(sc, low_field<BITS>(zc0[r]), bo);
          }
        }
      }
    }
  }

  // 5. reduce over the 64 lanes and store y[m][row0 + r]
  float v[V];
  uint32_t keep[R];
#pragma unroll
  for (int r = 0; r < R; ++r) keep[r] = keep_mask(nz[r]);
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? unless_zero(acc[i / M][i % M], keep[i / M]) : 0.f;
  float red[V / 4];
  wave_reduce_multi<V>(v, red);
  const int rho = lane >> 4;
  if ((lane & 15) == 0) {
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const int idx = 4 * j + row_value_index(rho);
      if (idx < R * M) {
        const int r = idx / M, m = idx % M;
        const int n = row0 + r;
        if (n < N) y[(size_t)m * N + n] = ADD ? red[j] + rres[j] : red[j];
      }
    }
  }
}

template <int BITS, int M, int R, int NSUB, int P, bool ADD, int FMT, bool XR = false>
int launch_dot_tp(const QgemvArgs &a, hipStream_t stream) {
  constexpr int CW = 128 / BITS;
  constexpr int QUADS = CW / 8;
  const int NC = a.K / CW;
  // Stages always hold whole multiples of 64 chunks, so lane l processes
  // chunks l, l+64, l+128, ... in the same order for every M (row results do
  // not depend on M).  Up to P*64 chunks per stage, within the LDS budget;
  // 64 chunks always fit (at most 139 KiB for M = 16, 2-bit codes).
  const size_t per_chunk = (size_t)M * (QUADS * 16 + NSUB * 4);
  int kch = 64 * (int)(kDotLdsBudget / (64 * per_chunk));
  // at most two staging units per thread (loaded ahead of the codes)
  const int kch_units = 64 * ((2 * kDotThreads / M) / 64);
  if (kch > kch_units) kch = kch_units;
  if (kch < 64) kch = 64;
  if (kch > 64 * P) kch = 64 * P;
  if (kch > NC) kch = NC;  // one stage holds the whole row
  constexpr bool XREG = XR && (M == 1 || (M == 2 && !(FMT == kAffine && BITS == 4))) &&
                        M * (CW / 8) * P <= 16;  // no LDS then
  const size_t lds = XREG ? 0 : per_chunk * (size_t)kch;
  if (lds > kLdsMax) return QGEMV_EUNSUPPORTED;
  if (!allow_max_dynamic_lds(
          reinterpret_cast<const void *>(&qgemv_dot_kernel<BITS, M, R, NSUB, P, ADD, FMT, XR>)))
    return QGEMV_EHIP;
  const int rows_per_block = kDotWaves * R;
  const int blocks = (a.N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((qgemv_dot_kernel<BITS, M, R, NSUB, P, ADD, FMT, XR>), dim3(blocks), dim3(kDotThreads),
                     lds, stream, a.codes, a.scales, a.biases, a.x, a.y, a.res, a.N, a.K,
                     a.group_size, kch);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

// Lane passes per stage: two when a row has at most 128 chunks (K <= 4096 at
// 4 bits), which keeps fewer code registers live; three otherwise.  Only for
// M <= 4, where the dot path is the one that runs.
template <int BITS, int M, int R, int NSUB, bool ADD, int FMT>
int launch_dot_t(const QgemvArgs &a, hipStream_t stream) {
  if constexpr (M == 1 || (M == 2 && !(FMT == kAffine && BITS == 4))) {
    // activation rows in registers where the grid has at most two
    // workgroups per CU (see the kernel's XR)
    const int blocks = (a.N + kDotWaves * R - 1) / (kDotWaves * R);
    if (blocks <= 2 * device_cu_count()) {
      if (a.K / (128 / BITS) <= 128) return launch_dot_tp<BITS, M, R, NSUB, 2, ADD, FMT, true>(a, stream);
      return launch_dot_tp<BITS, M, R, NSUB, kMaxPasses, ADD, FMT, true>(a, stream);
    }
  }
  if constexpr (M <= 4) {
    if (a.K / (128 / BITS) <= 128) return launch_dot_tp<BITS, M, R, NSUB, 2, ADD, FMT>(a, stream);
  }
  return launch_dot_tp<BITS, M, R, NSUB, kMaxPasses, ADD, FMT>(a, stream);
}

// rows per wave for each M: enough rows to share each x read (LDS traffic per
// code byte ~ 4M/R), few enough to keep R*M accumulators in registers.
// 8-bit codes fill twice the code registers per row (16 codes per 16-byte
// chunk), so they take fewer rows per wave.
template <int BITS, int M>
constexpr int dot_rows_per_wave() {
  if constexpr (BITS == 8) return M <= 8 ? 2 : 1;
  return M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 8 ? 2 : 1));
}

template <int BITS, int M, int R, bool ADD, int FMT>
int launch_dot_r(const QgemvArgs &a, hipStream_t stream) {
  if constexpr (FMT == kNvfp4) {
    return launch_dot_t<4, M, R, 2, ADD, FMT>(a, stream);  // two 16-element blocks per chunk
  } else if constexpr (BITS == 8) {
    return launch_dot_t<8, M, R, 1, ADD, FMT>(a, stream);  // a 16-code chunk never spans two groups
  } else if constexpr (BITS == 2) {
    if (a.group_size == 32) return launch_dot_t<2, M, R, 2, ADD, FMT>(a, stream);
    return launch_dot_t<2, M, R, 1, ADD, FMT>(a, stream);
  } else {
    return launch_dot_t<4, M, R, 1, ADD, FMT>(a, stream);
  }
}

template <int BITS, int M, bool ADD, int FMT>
int launch_dot_m(const QgemvArgs &a, hipStream_t stream) {
  constexpr int R = dot_rows_per_wave<BITS, M>();
  // Few rows (small N): fewer rows per wave, so that every CU gets a
  // workgroup.  The row-to-lane arithmetic is the same for every R, so
  // results do not depend on this choice.
  const int cus = device_cu_count();
  if constexpr (R == 4) {
    if (a.N / (kDotWaves * 4) < cus) {
      if (a.N / (kDotWaves * 2) >= cus) return launch_dot_r<BITS, M, 2, ADD, FMT>(a, stream);
      return launch_dot_r<BITS, M, 1, ADD, FMT>(a, stream);
    }
  } else if constexpr (R == 2) {
    if (a.N / (kDotWaves * 2) < cus) return launch_dot_r<BITS, M, 1, ADD, FMT>(a, stream);
  }
  return launch_dot_r<BITS, M, R, ADD, FMT>(a, stream);
}

template <int BITS, bool ADD, int FMT = kAffine>
int launch_dot_bits(const QgemvArgs &a, hipStream_t stream) {
  switch (a.M) {
    case 1: return launch_dot_m<BITS, 1, ADD, FMT>(a, stream);
    case 2: return launch_dot_m<BITS, 2, ADD, FMT>(a, stream);
    case 3: return launch_dot_m<BITS, 3, ADD, FMT>(a, stream);
    case 4: return launch_dot_m<BITS, 4, ADD, FMT>(a, stream);
    case 5: return launch_dot_m<BITS, 5, ADD, FMT>(a, stream);
    case 6: return launch_dot_m<BITS, 6, ADD, FMT>(a, stream);
    case 7: return launch_dot_m<BITS, 7, ADD, FMT>(a, stream);
    case 8: return launch_dot_m<BITS, 8, ADD, FMT>(a, stream);
    case 9: return launch_dot_m<BITS, 9, ADD, FMT>(a, stream);
    case 10: return launch_dot_m<BITS, 10, ADD, FMT>(a, stream);
    case 11: return launch_dot_m<BITS, 11, ADD, FMT>(a, stream);
    case 12: return launch_dot_m<BITS, 12, ADD, FMT>(a, stream);
    case 13: return launch_dot_m<BITS, 13, ADD, FMT>(a, stream);
    case 14: return launch_dot_m<BITS, 14, ADD, FMT>(a, stream);
    case 15: return launch_dot_m<BITS, 15, ADD, FMT>(a, stream);
    case 16: return launch_dot_m<BITS, 16, ADD, FMT>(a, stream);
    default: return QGEMV_EINVAL;
  }
}

// The instantiations of the 2- and 4-bit codes for one value of ADD; the
// 8-bit ones are launch_dot_bits<8, ADD>, the FP formats'
// launch_dot_bits<BITS, ADD, FMT> (each translation unit that includes this
// header compiles one set, so they build in parallel).
template <bool ADD>
int launch_dot_impl(const QgemvArgs &a, hipStream_t stream) {
  return a.bits == 4 ? launch_dot_bits<4, ADD>(a, stream) : launch_dot_bits<2, ADD>(a, stream);
}

}  // namespace

}  // namespace qgemv
