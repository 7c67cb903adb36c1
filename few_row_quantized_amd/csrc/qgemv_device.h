// Device helpers for the few-row quantized GEMV kernels (gfx950, wave64).
//
// Codes become exact bf16 values q with no offset.  A byte 0000qqqq read as
// an FP8 E4M3 number is q * 2^-9 for every q in 0..15 (exponent field 0 holds
// 0..7 as subnormals m * 2^-9, field 1 holds 8..15 as (8 + m) * 2^-9), so the
// gfx950 scaled conversion FP8 -> bf16 at scale 2^9 turns two such bytes into
// the exact bf16 pair (q_a, q_b) in one instruction: 2- and 4-bit fields are
// first spread into bytes with one shift-and-mask per four fields.  Dot
// products of these pairs with bf16 activations are exact per product in
// fp32, and the bias is applied through the group's activation sum with no
// offset to remove.  8-bit codes (0..255) are converted exactly through fp32
// (unpack8_pairs).
//
// Zero weights are exact (zero_weights): each lane tracks whether every group
// it has folded dequantizes to exactly zero and then returns exactly 0, so a
// row of zero weights gives y = 0 whatever the fp32 rounding of the factored
// sum s * sum(q x) + b * sum(x) would leave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgemv {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// 16-bit field f (0..3) of the 64 bits {v.x, v.y} (the fp16 scales or biases
// of a block's 4 groups), for a lane-dependent f: a bit-field select of the
// word and a shift, all in registers (written as a ?: on the vector members,
// the compiler may go through private memory).
__device__ __forceinline__ uint32_t field16(uint2 v, int f) {
  const uint32_t m = 0u - (uint32_t)(f < 2);  // all ones for fields 0 and 1
  const uint32_t w = (v.x & m) | (v.y & ~m);  // one bit-field insert
  return (w >> (16 * (f & 1))) & 0xFFFFu;
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

// ---------------------------------------------------------------- code unpack
//
// Two codes held in bytes 2*HI and 2*HI+1 of `bytes` (each 0..15) as the
// exact bf16 pair (code of the lower byte in the low half).
constexpr float kCodeScale = 512.0f;  // 2^9: E4M3 byte q -> q
template <bool HI>
__device__ __forceinline__ uint32_t code_pair(uint32_t bytes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bytes, kCodeScale, HI));
}

// 4-bit codes: dword w holds codes j = 0..7 (nibble j, low nibble first).
// Pairs (0, 2), (1, 3), (4, 6), (5, 7): the low nibbles of the four bytes are
// codes 0, 2, 4, 6 and the high nibbles 1, 3, 5, 7.  Seven instructions per
// eight codes.  The activations are paired to match (xpair4).
__device__ __forceinline__ u32x4_t unpack4_quad(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
  return u32x4_t{code_pair<false>(lo), code_pair<false>(hi), code_pair<true>(lo), code_pair<true>(hi)};
}
__device__ __forceinline__ void unpack4_pairs(uint32_t w, uint32_t (&o)[4]) {
  const u32x4_t v = unpack4_quad(w);
  o[0] = v[0];
  o[1] = v[1];
  o[2] = v[2];
  o[3] = v[3];
}

// 2-bit codes: dword w holds codes j = 0..15 (crumb j, lowest crumb first).
// (w >> 2e) & 0x03030303 holds codes e, e+4, e+8, e+12 in bytes 0..3, so half
// h (codes 8h..8h+7) is the pairs (8h + e, 8h + e + 4), e = 0..3.  Fifteen
// instructions per sixteen codes.  The activations of each half are paired
// to match (xpair_stride4).
__device__ __forceinline__ u32x4_t unpack2_quad(uint32_t w, int h) {
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t c = (w >> (2 * e)) & 0x03030303u;
    o[e] = h ? code_pair<true>(c) : code_pair<false>(c);
  }
  return o;
}
__device__ __forceinline__ void unpack2_pairs(uint32_t w, uint32_t (&o)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t c = (w >> (2 * e)) & 0x03030303u;
    o[e] = code_pair<false>(c);
    o[4 + e] = code_pair<true>(c);
  }
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

// ---------------------------------------------------------------- zero weights
//
// A group whose codes all equal c and whose fma(s, c, b) is exactly 0 holds
// only zero weights: its exact contribution is 0.  The kernels fold such
// groups like any other (s * sum(q x) + b * sum(x) leaves an fp32 rounding
// residue of the size of s * c * sum(x)), but each lane ORs into a word `nz`
// every trace of a nonzero weight it folds: the differences between its code
// words and the group's first (and between that word and itself rotated by
// one field), and the magnitude bits of s*c + b.  A partial whose nz is still
// 0 at the end held only zero weights and is stored as exactly 0, its exact
// value.  Plain bitwise ORs, no comparisons: the optimizer keeps the loops as
// they are (a chain of boolean tests made it branch around the accumulation,
// at a large register cost).

// Makes v opaque at this point: the trace of each code word is then formed
// while the word is in hand (left free, the optimizer gathers a group's
// traces at its end and keeps all of its code words live until then).
__device__ __forceinline__ void pin(uint32_t &v) { asm volatile("" : "+v"(v)); }

// Trace of non-uniform BITS-bit fields within w (0 iff all fields equal).
template <int BITS>
__device__ __forceinline__ uint32_t fields_spread(uint32_t w) {
  return w ^ __builtin_amdgcn_alignbit(w, w, BITS);
}

// The value of the lowest BITS-bit field of w.
template <int BITS>
__device__ __forceinline__ float low_field(uint32_t w) {
  return (float)(w & ((1u << BITS) - 1u));
}

// Trace of a nonzero group weight s*c + b (its magnitude bits).
__device__ __forceinline__ uint32_t weight_trace(float s, float c, float b) {
  return __builtin_bit_cast(uint32_t, fmaf(s, c, b)) & 0x7FFFFFFFu;
}

// acc where nz != 0, else exactly 0.  The mask passes through an empty asm
// statement so that the select stays a select.
__device__ __forceinline__ uint32_t keep_mask(uint32_t nz) {
  uint32_t m = nz != 0u ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  return m;
}
__device__ __forceinline__ float unless_zero(float acc, uint32_t keep) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, acc) & keep);
}

// MFMA operand layout: lanes 16*rho + c (rho = 0..3) hold the four quarters of
// column c's codes.  The OR of nz over the column's four lanes, in each of
// them (two row swaps).
__device__ __forceinline__ uint32_t column_or(uint32_t nz) {
  auto a = __builtin_amdgcn_permlane32_swap(nz, nz, false, false);
  const uint32_t h = a[0] | a[1];
  auto b = __builtin_amdgcn_permlane16_swap(h, h, false, false);
  return b[0] | b[1];
}

// ---------------------------------------------------------------- activation pairing
//
// Activations are re-paired to match the code pairing.  X[i] holds bf16
// elements (2i, 2i+1) of a run of consecutive activations.
//
// 4-bit pairing: pair e of (0, 2), (1, 3), (4, 6), (5, 7) from X[0..3]
__device__ __forceinline__ uint32_t xpair4(const uint32_t (&X)[4], int e) {
  return (e & 1) ? perm_b32(X[2 * (e >> 1) + 1], X[2 * (e >> 1)], 0x07060302u)
                 : perm_b32(X[2 * (e >> 1) + 1], X[2 * (e >> 1)], 0x05040100u);
}

// 2-bit pairing of one half: pair (e, e+4) from X[0..3], e = 0..3
__device__ __forceinline__ uint32_t xpair_stride4(const uint32_t (&X)[4], int e) {
  return (e & 1) ? perm_b32(X[(e >> 1) + 2], X[e >> 1], 0x07060302u)
                 : perm_b32(X[(e >> 1) + 2], X[e >> 1], 0x05040100u);
}

// The four pairs of 8 consecutive activations (one u32x4 in memory order)
// in the pairing of BITS-bit codes (2 or 4).
template <int BITS>
__device__ __forceinline__ u32x4_t pair_activations(const u32x4_t &v) {
  const uint32_t X[4] = {v[0], v[1], v[2], v[3]};
  if constexpr (BITS == 4) return u32x4_t{xpair4(X, 0), xpair4(X, 1), xpair4(X, 2), xpair4(X, 3)};
  return u32x4_t{xpair_stride4(X, 0), xpair_stride4(X, 1), xpair_stride4(X, 2), xpair_stride4(X, 3)};
}

constexpr uint32_t kOnesPair = 0x3F803F80u;  // bf16 (1.0, 1.0)

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

// Codes loaded as whole 128-byte lines: load A has lane L on 16-byte piece
// L%8 of row L/8 (rows 0-7 of a tile), load B the same for rows 8-15; the
// two 64-byte halves of each row's 128 bytes are two consecutive
// super-chunks.  For half h, operand lane (n, c) takes piece 4h + c of row
// n: first a row shift by 4 lanes merges the pieces of rows 8-15 that half h
// needs into the lanes of A it does not need (one DPP move and a select per
// dword), then one ds_bpermute per dword as in to_operand_lanes.  Full-line
// loads measured 8-12% faster than lane quads on 64 contiguous bytes on the
// persistent kernel's large matrices (FFN-up 4096 x 12288 gs64 at M = 8:
// 11.69 -> 10.50 us; 27B gate: 17.56 -> 15.44 us).
template <int H>
__device__ __forceinline__ void pair_to_operand_lanes(const u32x4_t &a, const u32x4_t &b, uint32_t (&cur)[4]) {
  const int lane = (int)(threadIdx.x & 63);
  const int n = lane & 15, c = lane >> 4;
  const int src = 4 * (n < 8 ? 8 * n + 4 * H + c : 8 * (n - 8) + 4 * (1 - H) + c);
  // lanes whose piece of A half H uses; the others take B moved by 4 lanes
  // (row_shr:4 for half 0, row_shl:4 for half 1: always from the same row of 16)
  const bool keep_a = H == 0 ? (lane & 7) < 4 : (lane & 7) >= 4;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int moved = __builtin_amdgcn_mov_dpp((int)b[d], H == 0 ? 0x114 : 0x104, 0xF, 0xF, false);
    const int merged = keep_a ? (int)a[d] : moved;
    cur[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, merged);
  }
}

__device__ __forceinline__ u32x4_t to_operand_lanes(const u32x4_t &v) {
  uint32_t c[4];
  to_operand_lanes(v, c);
  return u32x4_t{c[0], c[1], c[2], c[3]};
}

// Compact activation operands for few rows.  With R = 16 / XG distinct rows
// (R = 4 or 8), one 16-byte load per lane carries XG operands: lane
// 16*kb + XG*q + g holds operand g's piece for K-part kb of row q.  One DPP
// quad permutation per dword then gives operand g to every lane of the
// 16-lane row kb: lane (kb, a) takes lane 16*kb + XG*(a / XG) + g, i.e. row
// a / XG.  The MFMA row a thus holds activation row a / XG (each row XG
// times), and output row a is stored as row a / XG when a % XG == 0.  A
// quad permutation never leaves its row of 16 lanes and moves no data
// through LDS, so XG operands cost one load instruction and 4 VALU moves
// instead of XG loads (and, in the quad-row layout, 4*XG ds_bpermutes).
template <int XG, int G>
__device__ __forceinline__ uint32_t compact_pick_dword(uint32_t v) {
  static_assert((XG == 2 || XG == 4) && G >= 0 && G < XG, "compact operand");
  // quad_perm selectors: [G, G, G, G] (XG = 4) or [G, G, 2 + G, 2 + G] (XG = 2)
  constexpr int ctrl = XG == 4 ? G * 0x55 : G * 0x55 + 0xA0;
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
}

template <int XG>
__device__ __forceinline__ u32x4_t compact_pick(const u32x4_t &v, const int g) {
  u32x4_t r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // g is a compile-time constant once the caller's loops are unrolled
    if (g == 0) r[d] = compact_pick_dword<XG, 0>(v[d]);
    else if (g == 1) r[d] = compact_pick_dword<XG, 1>(v[d]);
    else if (g == 2) r[d] = compact_pick_dword<XG, XG == 4 ? 2 : 0>(v[d]);
    else r[d] = compact_pick_dword<XG, XG == 4 ? 3 : 1>(v[d]);
  }
  return r;
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
