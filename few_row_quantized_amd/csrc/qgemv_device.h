// Device helpers for the few-row quantized GEMV kernels (gfx950, wave64).
//
// 2- and 4-bit codes become bf16 values 128+q: for 0 <= q < 128 the bf16 bit
// pattern of 128+q is 0x4300 | q (exponent of 2^7, q in the 7 mantissa bits),
// so one AND-OR places two codes into the two halves of a dword as an exact
// bf16 pair.  Dot products of these pairs with bf16 activations are exact per
// product in fp32; the 128 offset is removed once per group through the
// group's activation sum (128 * sum x), folded together with the bias.
// 8-bit codes (0..255) do not fit that pattern; they are converted exactly
// without an offset (unpack8_pairs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgemv {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kOffsetPair = 0x43004300u;  // bf16(128) in both halves

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// a.lo*b.lo + a.hi*b.hi + c, bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// v_perm_b32: bytes of {hi_src, lo_src} selected by `sel` (0-3: lo_src, 4-7: hi_src, 0x0c: zero).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// 16-byte load of data read exactly once per call (the weight codes):
// non-temporal, so the stream does not push the activations (reused by every
// workgroup) out of the caches.
__device__ __forceinline__ u32x4_t load_stream_u32x4(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

// A value the compiler cannot see through, kept in a VGPR.  Used for the
// OR operand of the unpack so that AND+OR fuse into one v_and_or_b32 (a VOP3
// instruction on gfx9 takes at most one literal/SGPR operand).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// ---------------------------------------------------------------- code unpack
//
// 4-bit "offset" pairing (dot path): dword w holds codes j = 0..7 (nibble j).
// Pair p (p = 0..3) = codes (p, p+4).
// `off` holds kOffsetPair (pass opaque_u32(kOffsetPair) for a fused AND-OR).
__device__ __forceinline__ void unpack4_split_pairs(uint32_t w, uint32_t (&o)[4],
                                                    uint32_t off = kOffsetPair) {
  o[0] = (w & 0x000F000Fu) | off;
  o[1] = ((w >> 4) & 0x000F000Fu) | off;
  o[2] = ((w >> 8) & 0x000F000Fu) | off;
  o[3] = ((w >> 12) & 0x000F000Fu) | off;
}

// 4-bit "natural" pairing (MFMA path): pair p = codes (2p, 2p+1), i.e. the two
// nibbles of byte p, so the activation operand keeps its memory order.
__device__ __forceinline__ void unpack4_natural_pairs(uint32_t w, uint32_t (&o)[4]) {
  const uint32_t h = w >> 4;
  // byte p of w -> byte 0, byte p of (w >> 4) -> byte 2, zeros elsewhere.
  o[0] = (perm_b32(h, w, 0x0c040c00u) & 0x000F000Fu) | kOffsetPair;
  o[1] = (perm_b32(h, w, 0x0c050c01u) & 0x000F000Fu) | kOffsetPair;
  o[2] = (perm_b32(h, w, 0x0c060c02u) & 0x000F000Fu) | kOffsetPair;
  o[3] = (perm_b32(h, w, 0x0c070c03u) & 0x000F000Fu) | kOffsetPair;
}

// Same, as the 4-dword MFMA operand; `off` holds kOffsetPair (opaque_u32).
__device__ __forceinline__ u32x4_t unpack4_natural_quad(uint32_t w, uint32_t off) {
  const uint32_t h = w >> 4;
  u32x4_t o;
  o[0] = (perm_b32(h, w, 0x0c040c00u) & 0x000F000Fu) | off;
  o[1] = (perm_b32(h, w, 0x0c050c01u) & 0x000F000Fu) | off;
  o[2] = (perm_b32(h, w, 0x0c060c02u) & 0x000F000Fu) | off;
  o[3] = (perm_b32(h, w, 0x0c070c03u) & 0x000F000Fu) | off;
  return o;
}

// 2-bit pairing (both paths): dword w holds codes j = 0..15 (crumb j).
// Pair j (j = 0..7) = codes (j, j+8).
__device__ __forceinline__ void unpack2_split_pairs(uint32_t w, uint32_t (&o)[8],
                                                    uint32_t off = kOffsetPair) {
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = ((w >> (2 * j)) & 0x00030003u) | off;
}

// 4-bit split pairing as the 4-dword MFMA operand (pairs (p, p+4)).
__device__ __forceinline__ u32x4_t unpack4_split_quad(uint32_t w, uint32_t off) {
  u32x4_t o;
  o[0] = (w & 0x000F000Fu) | off;
  o[1] = ((w >> 4) & 0x000F000Fu) | off;
  o[2] = ((w >> 8) & 0x000F000Fu) | off;
  o[3] = ((w >> 12) & 0x000F000Fu) | off;
  return o;
}

// Half h (h = 0, 1) of the 2-bit pairing as an MFMA operand: pairs 4h..4h+3.
__device__ __forceinline__ u32x4_t unpack2_split_quad(uint32_t w, int h, uint32_t off) {
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = ((w >> (2 * (4 * h + e))) & 0x00030003u) | off;
  return o;
}

// 8-bit codes: byte j of dword w is code j (0..255).  Every code is exact in
// bf16 (at most 8 significant bits), so no offset is needed: each byte is
// converted to fp32 (v_cvt_f32_ubyte0..3, exact), whose upper half is the
// bf16 pattern of the same value, and v_perm packs two such halves.  Pairs are
// the natural ones, codes (0, 1) and (2, 3): the activations keep their memory
// order.
__device__ __forceinline__ uint32_t bf16_pair_of(float lo, float hi) {
  return perm_b32(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}

__device__ __forceinline__ void unpack8_pairs(uint32_t w, uint32_t (&o)[2]) {
  o[0] = bf16_pair_of((float)(w & 0xFFu), (float)((w >> 8) & 0xFFu));
  o[1] = bf16_pair_of((float)((w >> 16) & 0xFFu), (float)(w >> 24));
}

// Two code dwords (8 codes) as the 4-dword MFMA operand, natural order.
__device__ __forceinline__ u32x4_t unpack8_quad(uint32_t w0, uint32_t w1) {
  uint32_t a[2], b[2];
  unpack8_pairs(w0, a);
  unpack8_pairs(w1, b);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

// ---------------------------------------------------------------- block-scaled FP elements
//
// FP4 (E2M1) and FP8 (E4M3) elements are exact in bf16, so each is decoded with
// gfx950's conversion instructions at scale 1.0 (the scale is applied per block
// in fp32, like the affine scale): one instruction per two elements, natural
// pair order (the activations keep their memory order).
enum FpFormat { kAffine = 0, kMxfp4 = 1, kNvfp4 = 2, kMxfp8 = 3 };

// FP4 elements of byte `sel` of w (elements 2*sel, 2*sel+1) as a bf16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// FP8 elements of half `hi` of w (elements 2*hi, 2*hi+1) as a bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// One code dword as bf16 pairs in natural order: 4 pairs (FP4) or 2 (FP8).
__device__ __forceinline__ void unpack_fp4_pairs(uint32_t w, uint32_t (&o)[4]) {
  o[0] = fp4_pair<0>(w);
  o[1] = fp4_pair<1>(w);
  o[2] = fp4_pair<2>(w);
  o[3] = fp4_pair<3>(w);
}
__device__ __forceinline__ void unpack_fp8_pairs(uint32_t w, uint32_t (&o)[2]) {
  o[0] = fp8_pair<false>(w);
  o[1] = fp8_pair<true>(w);
}

// FP4 elements of byte SEL of w times a block scale, as a bf16 pair.  The
// conversion's own scale operand takes only the power of two of its argument,
// so the product is formed in fp32; for an E4M3 scale it has at most 6
// significant bits and lies within [2^-10, 2688], so the bf16 truncation is
// exact (the nvfp4 weights themselves).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair_scaled(uint32_t w, float sc) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return bf16_pair_of(f[0] * sc, f[1] * sc);
}

// Block scales: E8M0 (2^(e-127), 0xFF NaN) and E4M3, to fp32 (exact).
__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
  e &= 0xFFu;
  const uint32_t b = e == 0u ? 0x00400000u : (e == 255u ? 0x7FC00000u : e << 23);
  return __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float e4m3_to_float(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v & 0xFFu, 1.0f, false)[0];
}
template <int FMT>
__device__ __forceinline__ float fp_scale_to_float(uint32_t byte) {
  if constexpr (FMT == kNvfp4) return e4m3_to_float(byte);
  return e8m0_to_float(byte);
}

// ---------------------------------------------------------------- activation pairing
//
// Activations are re-paired to match the code pairing.  X[i] holds bf16
// elements (2i, 2i+1) of a run of consecutive activations.
//
// pair of elements (e, e+4) from X[0..3] (4-bit offset pairing), e = 0..3
__device__ __forceinline__ uint32_t xpair_stride4(const uint32_t (&X)[4], int e) {
  return (e & 1) ? perm_b32(X[(e >> 1) + 2], X[e >> 1], 0x07060302u)
                 : perm_b32(X[(e >> 1) + 2], X[e >> 1], 0x05040100u);
}

// pair of elements (e, e+8) from X[0..7] (2-bit pairing), e = 0..7
__device__ __forceinline__ uint32_t xpair_stride8(const uint32_t (&X)[8], int e) {
  return (e & 1) ? perm_b32(X[(e >> 1) + 4], X[e >> 1], 0x07060302u)
                 : perm_b32(X[(e >> 1) + 4], X[e >> 1], 0x05040100u);
}

// ---------------------------------------------------------------- lane exchange
//
// 4x4 transpose of dwords between the four 16-lane rows of a wave:
// on entry row g holds r[c] = T[g][c]; on exit row g holds r[c] = T[c][g].
// Uses v_permlane32_swap (upper 32 lanes of the first operand <-> lower 32
// lanes of the second) and v_permlane16_swap (odd rows of the first operand
// <-> even rows of the second).
__device__ __forceinline__ void transpose_rows4(uint32_t (&r)[4]) {
  {
    auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
    r[0] = a[0];
    r[2] = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
    r[1] = b[0];
    r[3] = b[1];
  }
  {
    auto a = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
    r[0] = a[0];
    r[1] = a[1];
    auto b = __builtin_amdgcn_permlane16_swap(r[2], r[3], false, false);
    r[2] = b[0];
    r[3] = b[1];
  }
}

// Partial transpose for the MFMA path.  On entry row g (lanes 16g..16g+15)
// holds the 4 dwords of chunk g of a 64-byte super-chunk in r[0..3].  LVL
// selects how far the dwords are exchanged so that each register holds codes
// of one quantization group:
//   LVL 0 (no exchange):  r[i] in row g = dword i of chunk g
//   LVL 1 (permlane32):   r[i] in row g = dword (i&1) + 2(g>>1) of chunk (g&1) + 2(i>>1)
//   LVL 2 (full 4x4):     r[i] in row g = dword g of chunk i
template <int LVL>
__device__ __forceinline__ void transpose_rows_lvl(uint32_t (&r)[4]) {
  if constexpr (LVL == 1) {
    auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
    r[0] = a[0];
    r[2] = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
    r[1] = b[0];
    r[3] = b[1];
  } else if constexpr (LVL == 2) {
    transpose_rows4(r);
  }
}
template <int LVL>
__device__ __forceinline__ int lvl_chunk(int i, int g) {
  return LVL == 0 ? g : (LVL == 1 ? (g & 1) + 2 * (i >> 1) : i);
}
template <int LVL>
__device__ __forceinline__ int lvl_dword(int i, int g) {
  return LVL == 0 ? i : (LVL == 1 ? (i & 1) + 2 * (g >> 1) : g);
}

// MFMA operand lanes and code loads.  The 16x16 MFMA layouts put output
// column n = lane % 16 in lane n, n+16, n+32, n+48, so a load in that layout
// (lane (n, c) reading 16-byte piece c of row n's 64-byte super-chunk) has
// every group of 4 consecutive lanes read 4 different rows; the address
// unit then spends about four times longer per instruction than on a
// contiguous read (rocprofv3 TA_BUSY: ~40 against ~16 cycles per load).
// The MFMA kernels therefore load with lane L reading piece L%4 of row L/4
// (each lane quad reads 64 contiguous bytes) and move every dword to its
// operand lane with ds_bpermute: lane (n, c) takes lane 4n + c's data.
// The same holds for the per-row metadata and, in the single-pass kernel,
// for the activation operand (row m = lane % 16) once several rows are
// distinct.  Measured on MI355X: codes alone took the square 4-bit MFMA path
// from 6.82 to 6.51 us at M = 8 and the 4-bit FFN-up gs64 persistent kernel
// from 11.98 to 11.26 us; metadata and activations then took the square path
// to 5.57 us at M = 8 and from 7.77 to 5.86 us at M = 16.
__device__ __forceinline__ int quad_row_lane(int lane) { return 4 * (lane & 15) + (lane >> 4); }

__device__ __forceinline__ void to_operand_lanes(const u32x4_t &loaded, uint32_t (&cur)[4]) {
  const int src = quad_row_lane((int)(threadIdx.x & 63)) * 4;
#pragma unroll
  for (int d = 0; d < 4; ++d) cur[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)loaded[d]);
}

__device__ __forceinline__ u32x4_t to_operand_lanes(const u32x4_t &v) {
  uint32_t c[4];
  to_operand_lanes(v, c);
  return u32x4_t{c[0], c[1], c[2], c[3]};
}

__device__ __forceinline__ uint2 to_operand_lanes(const uint2 &v) {
  const int src = quad_row_lane((int)(threadIdx.x & 63)) * 4;
  return make_uint2((uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.x),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.y));
}

// P[j] is a per-lane partial for value j (j = 0..3) that must be summed over
// the four 16-lane rows.  Returns, in row j, the total of value j (lane
// positions within a row are kept).  Two swap stages, three adds.
__device__ __forceinline__ float rows_transpose_reduce4(const float (&P)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, P[0]),
                                            __builtin_bit_cast(uint32_t, P[2]), false, false);
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, P[1]),
                                            __builtin_bit_cast(uint32_t, P[3]), false, false);
  const float u02 = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
  const float u13 = __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
  auto c = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, u02),
                                            __builtin_bit_cast(uint32_t, u13), false, false);
  return __builtin_bit_cast(float, (uint32_t)c[0]) + __builtin_bit_cast(float, (uint32_t)c[1]);
}

__device__ __forceinline__ float dpp_row_sum16(float v) {
  // butterfly inside each 16-lane row: mirror, half-mirror, quad swaps
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  return v;
}

// Sum V per-lane values over all 64 lanes (V % 4 == 0).  On exit out[j]
// holds, in every lane of row rho (lanes 16*rho .. 16*rho+15), the total of
// value index 4*j + kRowValue[rho], kRowValue = {0, 2, 1, 3}.
// Each swap stage halves the number of live registers, so the cost is
// ~2.5 instructions per value instead of ~6-12 for independent reductions.
template <int V>
__device__ __forceinline__ void wave_reduce_multi(const float (&v)[V], float (&out)[V / 4]) {
  static_assert(V % 4 == 0, "pad to a multiple of 4");
  float h[V / 2];
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[2 * i]),
                                              __builtin_bit_cast(uint32_t, v[2 * i + 1]), false,
                                              false);
    h[i] = __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
  }
#pragma unroll
  for (int j = 0; j < V / 4; ++j) {
    auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, h[2 * j]),
                                              __builtin_bit_cast(uint32_t, h[2 * j + 1]), false,
                                              false);
    out[j] = dpp_row_sum16(__builtin_bit_cast(float, (uint32_t)p[0]) +
                           __builtin_bit_cast(float, (uint32_t)p[1]));
  }
}

__device__ __forceinline__ int row_value_index(int rho) {
  // {0, 2, 1, 3}
  return ((rho & 1) << 1) | (rho >> 1);
}

}  // namespace qgemv
