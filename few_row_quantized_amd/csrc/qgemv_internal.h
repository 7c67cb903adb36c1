// Internal interface between the C ABI (qgemv_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qgemv.h"

namespace qgemv {

struct QgemvArgs {
  const uint8_t *codes;
  const uint16_t *scales;
  const uint16_t *biases;
  const uint16_t *x;
  float *y;
  int M, N, K, bits, group_size;
  // Fused residual sum: y = product + res (res [M][N] fp32, may equal y);
  // nullptr for the plain product.
  const float *res = nullptr;
  // Weight format: 0 = affine codes (fp16 scales and biases); otherwise a
  // block-scaled FP format (FpFormat in qgemv_device.h): `scales` then points
  // to one scale byte per block, `biases` is unused, bits is the element width
  // and group_size the block.
  int fmt = 0;
};

// Gathered (MoE) verify limits: experts per matrix set and (row, expert) pairs
// per call.
constexpr int kMaxExperts = QGEMV_MAX_EXPERTS;
constexpr int kMaxPairs = QGEMV_MAX_PAIRS;

// Gathered (MoE) verify: pair p takes activation row x_idx[p] and expert
// e_idx[p]; the experts are E matrices [N][K] stored one after another.
struct GatherArgs {
  const int32_t *x_idx;
  const int32_t *e_idx;
  int P;  // pairs
  int X;  // activation rows
  int E;  // experts
};

// LDS of one workgroup: hardware limit on gfx950, and the dot path's
// preferred x-staging budget (two workgroups per CU).
constexpr size_t kLdsMax = 160 * 1024;
constexpr size_t kDotLdsBudget = 80 * 1024;

// Bit pattern that y holds, before a K-split launch with the residual sum,
// until the first half of K lands.  A NaN payload that no partial sum can
// carry: partials derive from bf16 and fp16 inputs, whose NaNs have zero low
// 13 bits in fp32, and fresh NaNs are the canonical 0x7FC00000.
constexpr uint32_t kSplitSentinel = 0x7FC0DEADu;

// y[0..n) = v (bit pattern) on `stream`: zero before a K-split launch (two
// halves added into y), kSplitSentinel before one with the residual sum.
int launch_fill(float *y, size_t n, uint32_t v, hipStream_t stream);

// Compute units of the current device (cached per device id).
int device_cu_count();

// Allow `func` up to kLdsMax bytes of dynamic LDS on the current device (set
// once per device and function).  Returns false if the runtime refuses.
bool allow_max_dynamic_lds(const void *func);

// Launchers: enqueue on `stream`, return QGEMV_OK / QGEMV_EUNSUPPORTED / QGEMV_EHIP.
int launch_dot(const QgemvArgs &a, hipStream_t stream);
int launch_dot_add(const QgemvArgs &a, hipStream_t stream);  // a.res != nullptr, 2/4-bit
int launch_dot8(const QgemvArgs &a, hipStream_t stream);     // 8-bit codes
int launch_dot_fp(const QgemvArgs &a, hipStream_t stream);   // block-scaled FP formats
int launch_mfma(const QgemvArgs &a, hipStream_t stream);
// Persistent MFMA kernel (QGEMV_EUNSUPPORTED when the activations of a
// wave would not fit its registers).
int launch_persist(const QgemvArgs &a, hipStream_t stream);
// Persistent MFMA kernel with the activations of one half of K staged in LDS
// (long K): QGEMV_EUNSUPPORTED when they would not fit, for an in-place
// residual sum, or with fewer tiles than CUs.
int launch_persist_x(const QgemvArgs &a, hipStream_t stream);

// Shape support of the MFMA path (host check): affine codes, FP formats.
bool mfma_supports(int K, int bits, int group_size);
bool mfma_supports_fp(int K, int fmt);
bool mfma_whole_blocks(int K, int group_size);

// Probes.
int launch_unpack_probe(int path, const uint8_t *codes, uint8_t *q_out, int N, int K, int bits,
                        int group_size, hipStream_t stream);
// Gathered (MoE) verify on the persistent MFMA kernel (QGEMV_EUNSUPPORTED
// for shapes it does not take).
int launch_persist_gather(const QgemvArgs &a, const GatherArgs &ga, hipStream_t stream);
// Gathered (MoE) verify on the MFMA kernel: y[p] = x[x_idx[p]] . W[e_idx[p]]^T.
int launch_gather(const QgemvArgs &a, const int32_t *x_idx, const int32_t *e_idx, int P, int X,
                  int E, hipStream_t stream);
int launch_unpack_probe_fp(int path, const uint8_t *codes, uint16_t *out, int N, int K, int fmt,
                           hipStream_t stream);
int launch_stream_probe(const uint8_t *buf, size_t nbytes, uint32_t *out, int unroll, int layout,
                        hipStream_t stream);
int stream_probe_blocks(size_t nbytes);

}  // namespace qgemv
