/*
 * qgemv.h -- few-row quantized GEMV for AMD Instinct MI355X (gfx950).
 *
 *   y[M,N] = x[M,K] . dequant(W[N,K])^T,   1 <= M <= 16
 *
 * The verify step of speculative / multi-token-prediction decoding runs a
 * weight matrix against a handful of activation rows ("metal : few-row MMA
 * mat-mul and batched copies for speculative decoding", Overview: 2..16 src1
 * rows; "MLX quantized_matmul small-M verify kernels", Facts: the M=2..12
 * window between qmv and qmm).  This library reads and dequantizes every
 * weight group once per call and reuses it for all M rows, instead of
 * streaming the weights once per row.
 *
 * Weight format (affine group quantization, the "affine" mode of the MLX
 * page's Facts on qmv_wide; 4 B of fp16 scale+bias per group, Facts: the
 * group-size mechanism):
 *   w[n,k] = s[n, k/gs] * q[n,k] + b[n, k/gs]
 *   codes   uint8 [N][K*bits/8], row-major, no padding between rows.
 *           bits = 4: two codes per byte, column k in bits 4*(k%2).. (low
 *           nibble first).  bits = 2: four codes per byte, column k in bits
 *           2*(k%4).. (lowest crumb first).  bits = 8: one code per byte,
 *           the unsigned byte (the int8 affine mode of qmv_wide, MLX page,
 *           Facts: the int8 M=8 speedup).
 *   scales  IEEE fp16 bit patterns [N][K/gs], row-major.
 *   biases  IEEE fp16 bit patterns [N][K/gs], row-major.
 * Activations x: bfloat16 bit patterns [M][K], row-major (weights are stored
 * [out,in], so the product is x @ W^T; MLX page, Facts: (M,5120)@(17408,5120)^T).
 * Output y: fp32 [M][N], row-major, overwritten (no accumulate).
 *
 * Conventions for every entry point:
 *   - All buffer pointers are DEVICE pointers on the current HIP device.  The
 *     caller owns every buffer; the library allocates no device memory,
 *     keeps no mutable state between calls and never synchronizes the host.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Work is enqueued asynchronously on it.
 *   - Arguments are validated on the host before anything is launched; on
 *     failure a negative status is returned and nothing is enqueued.
 *   - A kernel launch error reported by the HIP runtime returns QGEMV_EHIP.
 *   - Errors inside a running kernel cannot happen for validated arguments
 *     (all accesses are bounded by M, N, K).
 *   - Calls are reentrant and may run concurrently on different streams.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QGEMV_OK 0
#define QGEMV_EINVAL (-1)       /* bad shape / bits / group size / null pointer   */
#define QGEMV_EUNSUPPORTED (-2) /* valid format, but the requested path cannot run it */
#define QGEMV_EALIGN (-3)       /* a buffer pointer is not 16-byte aligned            */
#define QGEMV_EHIP (-4)         /* the HIP runtime rejected a launch                  */

/* Kernel paths. */
#define QGEMV_PATH_AUTO 0 /* let qgemv_select choose                                 */
#define QGEMV_PATH_DOT 1  /* multi-row dot path: one wave per row tile, lanes split K */
#define QGEMV_PATH_MFMA 2 /* split-K bf16 MFMA path: waves split K, LDS reduction    */

/* Limits checked by validation. */
#define QGEMV_MAX_M 16
#define QGEMV_MAX_K 131072
#define QGEMV_MAX_N 4194304
#define QGEMV_MAX_EXPERTS 4096 /* experts per qgemv_gather call */
#define QGEMV_MAX_PAIRS 256    /* (row, expert) pairs per qgemv_gather call */

/*
 * qgemv_small -- y = x . dequant(W)^T for 1 <= M <= 16, path chosen by
 * qgemv_select.
 *
 * Requirements (else QGEMV_EINVAL / QGEMV_EALIGN):
 *   bits in {2, 4, 8}; group_size in {32, 64, 128}; 1 <= M <= 16;
 *   1 <= N <= QGEMV_MAX_N; 64 <= K <= QGEMV_MAX_K; K % 64 == 0;
 *   K % group_size == 0; codes, scales, biases, x, y non-NULL and each
 *   16-byte aligned (every device allocation is).
 * Numerics: products of bf16 activations with exact integer codes are
 * accumulated in fp32 per group; the per-group scale is applied once to the
 * group's partial dot product and the bias once to the group's activation sum
 * (scale hoisted out of the inner loop, MLX page, Facts: the qmv_wide tuning
 * bullet).  Result within 1e-3 * sum_k |x_k w_k| + 1e-6 of the exact value.
 * An output column n whose dequantized weights w[n][*] are all exactly zero
 * gives exactly 0 (exactly r with the residual sum).
 * Results are deterministic (where the MFMA path splits K over two
 * workgroups, y receives exactly two float additions onto zero, which
 * commute bit for bit).  Within one path, row m of an M-row call equals
 * (bitwise) the M=1 call on x[m] whenever both calls run the same kernel
 * configuration, whose per-row accumulation order depends on the shape
 * alone.  One case depends on M: on the MFMA path, with more 16-column
 * tiles than compute units and K too long for the register-resident
 * persistent kernel (K > 4096 for 4-bit codes in groups of 32 or 64, K >
 * 6144 otherwise), the long-K kernel takes its phase count and
 * blocks per wave from an LDS budget that grows with M, and the single-pass
 * kernel runs beyond the largest M that budget holds.  Rows of calls on
 * different sides of such a threshold agree within the tolerance above, not
 * bit for bit (K = 17408, N = 5120, 4-bit, group size 128: M = 1..7, 8..14
 * and 15..16 are three configurations).
 */
int qgemv_small(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                const uint16_t *x, float *y, int M, int N, int K, int bits, int group_size,
                void *stream);

/*
 * qgemv_small_add -- the fused residual sum: y = x . dequant(W)^T + residual,
 * for 1 <= M <= 16, path chosen by qgemv_select (the MUL_MAT + ADD fusion of
 * "metal : few-row MMA mat-mul and batched copies for speculative decoding",
 * Overview: the residual sum is written from the mat-mul's store, saving the
 * separate ADD launch and its read and write of y).
 *
 * residual: fp32 [M][N], row-major, the output's layout; DEVICE pointer,
 * 16-byte aligned, read only.  It may be y itself (in place: y += x W^T);
 * otherwise it must not overlap y (QGEMV_EINVAL).  NULL -> QGEMV_EINVAL.
 * Other arguments, requirements and errors as qgemv_small.
 * Numerics: y[m,n] is the fp32 product that qgemv_small would store for this
 * path, plus residual[m,n] rounded once in fp32 -- bit for bit qgemv_small
 * followed by a separate fp32 add -- except for an in-place call on a shape
 * where the MFMA path splits K across workgroups: that call runs the unsplit
 * kernel (the split needs y prefilled), whose product may differ from the
 * split one in the last bits.  Tolerance against the exact value:
 * 1e-3 * sum_k |x_k w_k| + 1e-6 + 2^-23 * (|r| + sum_k |x_k w_k|).
 * Row m still equals (bitwise) the M=1 call on x[m] and residual[m].
 */
int qgemv_small_add(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                    const uint16_t *x, const float *residual, float *y, int M, int N, int K,
                    int bits, int group_size, void *stream);

/*
 * qgemv_run_path_add -- qgemv_small_add with an explicit path (as
 * qgemv_run_path).
 */
int qgemv_run_path_add(int path, const uint8_t *codes, const uint16_t *scales,
                       const uint16_t *biases, const uint16_t *x, const float *residual, float *y,
                       int M, int N, int K, int bits, int group_size, void *stream);

/*
 * qgemv_select -- the path qgemv_small takes for this shape: QGEMV_PATH_DOT or
 * QGEMV_PATH_MFMA, or a negative status if the shape is invalid.  The choice
 * comes from a crossover table measured on MI355X (which rows of a shape
 * family favour the MFMA path), in the spirit of the per-type start rows of
 * the few-row MMA PR (Overview) and MLX's per-shape qmv batch limit (MLX page,
 * Facts: get_qmv_batch_limit), but calibrated on CDNA4.  Pure host function;
 * touches no device.
 */
int qgemv_select(int M, int N, int K, int bits, int group_size);

/*
 * qgemv_run_path -- qgemv_small with an explicit path (QGEMV_PATH_AUTO,
 * QGEMV_PATH_DOT or QGEMV_PATH_MFMA), for forced-path sweeps and tests (the
 * pages' A/B knobs: the specgate-metal README's GGML_METAL_NO_MV_EXT /
 * GGML_METAL_MM_MIN; MLX page, Facts: forced qmv vs qmm sweeps).
 * Returns QGEMV_EUNSUPPORTED if the path cannot run the shape (the MFMA path
 * needs K to be a multiple of 256 (2-bit) / 128 (4-bit) / 64 (8-bit), and
 * group_size >= 64 for 2-bit codes; K a multiple of 4*group_size, or for 2-
 * and 4-bit codes at least 4 groups, the remainder then running as a partial
 * last block of the single-pass MFMA kernel).  Other arguments as
 * qgemv_small.
 */
int qgemv_run_path(int path, const uint8_t *codes, const uint16_t *scales,
                   const uint16_t *biases, const uint16_t *x, float *y, int M, int N, int K,
                   int bits, int group_size, void *stream);

/*
 * qgemv_path_supported -- 1 if `path` can run this shape, 0 if not, negative
 * status if the shape itself is invalid.  Host only.
 */
int qgemv_path_supported(int path, int M, int N, int K, int bits, int group_size);

/*
 * qgemv_unpack_probe -- writes the integer codes exactly as a path's kernels
 * decode them: q_out[n][k] (uint8, [N][K], row-major) for every n < N, k < K.
 * The kernels turn codes into exact bf16 values q in registers; this probe
 * runs the same device routines (same loads, lane exchanges and conversions;
 * on the MFMA path both of its load forms, which must agree) and writes back
 * q, so the decoded codes can be compared bit-exactly with the format's
 * definition.  path: QGEMV_PATH_DOT or QGEMV_PATH_MFMA (the two
 * paths pair codes differently).  Requirements as qgemv_run_path for that
 * path (group_size only selects the MFMA layout, pass the one you will use);
 * q_out non-NULL.
 */
int qgemv_unpack_probe(int path, const uint8_t *codes, uint8_t *q_out, int N, int K, int bits,
                       int group_size, void *stream);

/*
 * qgemv_stream_probe -- read-only streaming kernel over `nbytes` bytes of
 * `buf` (16-byte aligned, nbytes a multiple of 16): every byte is loaded once
 * with non-temporal 128-bit loads (1 KiB contiguous per wave instruction,
 * `loads_per_thread` loads in flight per thread: 1, 2, 4, 8 or 16), folded with
 * XOR, and one uint32 per 256-thread workgroup is written to
 * out[0 .. qgemv_stream_probe_blocks(nbytes)-1] (enough for every setting;
 * the XOR of all of them is the XOR of the buffer's 32-bit words).
 * layout 0: a thread's loads are one grid-width apart; layout 1: they are
 * 1 KiB apart, so that each wave reads loads_per_thread KiB in one piece.
 * The fastest setting at a byte count is the bandwidth ceiling a pure read of
 * that many bytes reaches, measured the same way as the GEMV kernels.
 * EINVAL for another loads_per_thread or layout.
 */
int qgemv_stream_probe(const uint8_t *buf, size_t nbytes, uint32_t *out, int loads_per_thread,
                       int layout, void *stream);
int qgemv_stream_probe_blocks(size_t nbytes);

/*
 * ---------------------------------------------------------------- FP block formats
 *
 * The block-scaled floating-point modes of qmv_wide (MLX page, Facts: qmv_wide
 * covers affine, nvfp4, mxfp4 and mxfp8, with their M=8 speedups on the
 * Gemma-4-12B gate/up shape).  Element and scale encodings follow the OCP
 * Microscaling Formats (MX) v1.0 specification:
 *   QGEMV_FMT_MXFP4  FP4 E2M1 elements, two per byte (low nibble first);
 *                    one E8M0 scale byte (2^(e-127)) per 32 elements.
 *   QGEMV_FMT_NVFP4  FP4 E2M1 elements as above; one FP8 E4M3 scale byte per
 *                    16 elements (no per-tensor scale: a constant factor the
 *                    caller can apply to y).
 *   QGEMV_FMT_MXFP8  FP8 E4M3 elements (OCP: bias 7, no infinities, S.1111.111
 *                    NaN), one per byte; one E8M0 scale byte per 32 elements.
 * w[n,k] = scale[n, k/block] * element[n,k]; no bias.
 *   codes   uint8 [N][K*bits/8] (bits = 4 or 8), row-major, 16-byte aligned.
 *   scales  uint8 [N][K/block], row-major, 16-byte aligned.
 *   x       bf16 [M][K]; y fp32 [M][N] as for qgemv_small.
 *   residual  NULL for the plain product, else fp32 [M][N] added in the
 *           store exactly as qgemv_small_add (may be y itself, else must not
 *           overlap it).
 * Requirements (else QGEMV_EINVAL / QGEMV_EALIGN): format one of the three;
 * 1 <= M <= 16; 1 <= N <= QGEMV_MAX_N; 64 <= K <= QGEMV_MAX_K, K % 64 == 0.
 * The MFMA path needs K % 128 == 0.  Elements are decoded exactly (every E2M1
 * and E4M3 value is a bf16 value); each block's scale is applied once in fp32
 * to the block's partial dot product, except on the MFMA path for nvfp4, where
 * each element is multiplied by its E4M3 block scale before the product (the
 * product of an E4M3 and an E2M1 value is itself exact in bf16).  Tolerance
 * and row invariance as qgemv_small.
 */
#define QGEMV_FMT_MXFP4 1
#define QGEMV_FMT_NVFP4 2
#define QGEMV_FMT_MXFP8 3

int qgemv_small_fp(const uint8_t *codes, const uint8_t *scales, const uint16_t *x,
                   const float *residual, float *y, int M, int N, int K, int format,
                   void *stream);

/* qgemv_run_path_fp -- qgemv_small_fp with an explicit path (as qgemv_run_path). */
int qgemv_run_path_fp(int path, const uint8_t *codes, const uint8_t *scales, const uint16_t *x,
                      const float *residual, float *y, int M, int N, int K, int format,
                      void *stream);

/* qgemv_select_fp / qgemv_path_supported_fp -- as qgemv_select /
 * qgemv_path_supported, for an FP format.  Host only. */
int qgemv_select_fp(int M, int N, int K, int format);
int qgemv_path_supported_fp(int path, int M, int N, int K, int format);

/*
 * qgemv_unpack_probe_fp -- writes the element values exactly as a path's
 * kernels decode them, as bf16 bit patterns: out[n][k] (uint16, [N][K]), before
 * the block scale is applied, for the bit-exact test of the decoding.
 */
int qgemv_unpack_probe_fp(int path, const uint8_t *codes, uint16_t *out, int N, int K, int format,
                          void *stream);

/*
 * qgemv_gather -- gathered (MoE) verify over (activation row, expert) pairs:
 *
 *   y[p] = x[x_idx[p]] . dequant(W[e_idx[p]])^T,   0 <= p < P
 *
 * the MoE form of the verify product (MLX page, Facts: dense and MoE
 * gather_qmm verify; the expert-union cost per verify row).  Every expert in
 * the union of e_idx is read and dequantized once per call for all the pairs
 * routed to it, instead of once per pair.
 *   codes   uint8 [E][N][K*bits/8]; scales, biases fp16 [E][N][K/group_size]:
 *           E matrices in the affine format of qgemv_small, one after another.
 *   x       bf16 [X][K] activation rows.
 *   x_idx, e_idx  int32 [P], DEVICE arrays (the routing stays on the device):
 *           the activation row and the expert of each pair.
 *   y       fp32 [P][N], row p written for every valid pair.
 * A pair whose x_idx is outside [0, X) or e_idx outside [0, E) is skipped and
 * its row of y is left unchanged (the indices are read on the device; the
 * host cannot check them without a synchronization).
 * Requirements (else QGEMV_EINVAL / QGEMV_EALIGN / QGEMV_EUNSUPPORTED):
 * shape and format as qgemv_run_path with the MFMA path (bits, group_size, N,
 * K, and the MFMA path's K requirements); 1 <= P <= QGEMV_MAX_PAIRS;
 * 1 <= E <= QGEMV_MAX_EXPERTS; X >= 1; pointers non-NULL, codes, scales,
 * biases, x and y 16-byte aligned, x_idx and e_idx 4-byte aligned.
 * Runs on an MFMA kernel (any number of pairs per expert, 16 rows at a
 * time): the single-pass one for X <= 2, the persistent one for X >= 3 where
 * the shape fits it.  Each pair's row has the numerics of the MFMA path
 * (within the tolerance of qgemv_small; its K split over waves is the
 * kernel's own, so it may differ from a dense call, and between the two
 * kernels, in the last bits), is deterministic, and does not depend on the
 * other pairs of the call (bitwise the same as a call with the same x and X
 * and that pair alone).
 */
int qgemv_gather(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                 const uint16_t *x, const int32_t *x_idx, const int32_t *e_idx, float *y, int P,
                 int X, int E, int N, int K, int bits, int group_size, void *stream);

/* qgemv_strerror -- static description of a status code. */
const char *qgemv_strerror(int status);

/* qgemv_version -- library ABI version (major*10000 + minor*100 + patch). */
int qgemv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
