// Probe kernels: decoded-code readback (bit-exactness of the unpack stage)
// and a pure streaming read (bandwidth ceiling at a given byte count).

#include "qgemv_device.h"
#include "qgemv_internal.h"

namespace qgemv {

namespace {

// Extract q from a bf16 pair half that should hold the exact value q;
// anything else marks an encoding error (0xFF: outside the 2- and 4-bit
// ranges, and for 8-bit codes an error shows wherever the code is not 255).
__device__ __forceinline__ uint8_t code_of(uint32_t half16) {
  const float f = bf16_bits_to_float(half16);
  return (f >= 0.f && f <= 255.f && f == (float)(int)f) ? (uint8_t)(int)f : (uint8_t)0xFF;
}

// Dot-path decoding: one thread per (row n, 16-byte chunk c), same unpack
// routines and pair-to-column mapping as qgemv_dot_kernel.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_probe_dot(const uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ q, int N, int K) {
  constexpr int CW = 128 / BITS;
  const int NC = K / CW;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)N * NC) return;
  const int n = (int)(idx / NC);
  const int c = (int)(idx % NC);
  const size_t RB = (size_t)K * BITS / 8;
  const uint4 v = *reinterpret_cast<const uint4 *>(codes + (size_t)n * RB + (size_t)c * 16);
  const uint32_t cd[4] = {v.x, v.y, v.z, v.w};
  uint8_t *qr = q + (size_t)n * K + (size_t)c * CW;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (BITS == 8) {
      uint32_t p[2];
      unpack8_pairs(cd[d], p);  // pairs (4d, 4d+1), (4d+2, 4d+3)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        qr[4 * d + 2 * e] = code_of(p[e] & 0xFFFFu);
        qr[4 * d + 2 * e + 1] = code_of(p[e] >> 16);
      }
    } else if constexpr (BITS == 4) {
      uint32_t p[4];
      unpack4_pairs(cd[d], p);  // pair e: codes 8d + 4(e/2) + e%2 and that + 2
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 8 * d + 4 * (e >> 1) + (e & 1);
        qr[k] = code_of(p[e] & 0xFFFFu);
        qr[k + 2] = code_of(p[e] >> 16);
      }
    } else {
      uint32_t p[8];
      unpack2_pairs(cd[d], p);  // pair j: codes 16d + 8(j/4) + j%4 and that + 4
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = 16 * d + 8 * (j >> 2) + (j & 3);
        qr[k] = code_of(p[j] & 0xFFFFu);
        qr[k + 4] = code_of(p[j] >> 16);
      }
    }
  }
}

// The MFMA kernels' code loads for super-chunk sc of 16-row tile `tile`,
// moved to the operand lanes: whole 128-byte lines of two super-chunks
// (LINES: lane L on piece L%8 of row L/8, then rows 8-15; the persistent
// kernel where a bias block holds an even number of super-chunks) or lane
// quads on 64 bytes (lane L: piece L%4 of row L/4; the other kernels).
template <bool LINES>
__device__ __forceinline__ void probe_load_operands(const uint8_t *codes, size_t RB, int tile, int sc, int N,
                                                    uint32_t (&r)[4]) {
  const int lane = threadIdx.x & 63;
  if constexpr (LINES) {
    const size_t off = (size_t)(sc & ~1) * 64 + (lane & 7) * 16;
    const int na = min(tile * 16 + (lane >> 3), N - 1), nb = min(tile * 16 + 8 + (lane >> 3), N - 1);
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(codes + (size_t)na * RB + off);
    const u32x4_t b = *reinterpret_cast<const u32x4_t *>(codes + (size_t)nb * RB + off);
    if (sc & 1)
      pair_to_operand_lanes<1>(a, b, r);
    else
      pair_to_operand_lanes<0>(a, b, r);
  } else {
    const int nq = min(tile * 16 + (lane >> 2), N - 1);
    const u32x4_t v =
        *reinterpret_cast<const u32x4_t *>(codes + (size_t)nq * RB + (size_t)sc * 64 + (lane & 3) * 16);
    to_operand_lanes(v, r);
  }
}

// MFMA-path decoding: one wave per (16-row tile, 64-byte super-chunk), same
// lane-to-address mapping, partial row transpose (level LVL, chosen by the
// group size) and unpack as the MFMA kernels; each B-operand slot is written
// to the column it stands for.  Where both load forms apply (LINES) the
// operands of the two must agree register for register; a lane where they
// do not writes 0xFF (no 2- or 4-bit code) over its first code.
template <int BITS, int LVL, bool LINES>
__global__ __launch_bounds__(64) void unpack_probe_mfma(const uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ q, int N, int K) {
  constexpr int CW = 128 / BITS;
  constexpr int SCW = 4 * CW;
  constexpr int DW = CW / 4;
  const int lane = threadIdx.x;
  const int col = lane & 15, kb = lane >> 4;
  const int nsc = K / SCW;
  const int tile = blockIdx.x / nsc;
  const int sc = blockIdx.x % nsc;
  const int n = min(tile * 16 + col, N - 1);
  const size_t RB = (size_t)K * BITS / 8;
  uint32_t r[4];
  probe_load_operands<false>(codes, RB, tile, sc, N, r);
  bool differ = false;
  if constexpr (LINES) {
    // no line-load check for 8-bit codes: every byte is a code, so no value
    // is left to flag a mismatch (their line loads in the persistent kernel
    // are covered by the parity tests)
    static_assert(BITS != 8, "8-bit codes take the single-pass kernel only");
    uint32_t r2[4];
    probe_load_operands<true>(codes, RB, tile, sc, N, r2);
#pragma unroll
    for (int d = 0; d < 4; ++d) differ |= r2[d] != r[d];
  }
  transpose_rows_lvl<LVL>(r);  // all lanes take part, also those past row N
  if (tile * 16 + col >= N) return;
  uint8_t *qr = q + (size_t)n * K + (size_t)sc * SCW;
  if constexpr (BITS == 8) {
    // MFMA step e: registers 2e, 2e+1 = 8 consecutive codes from k0(2e)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k0 = lvl_chunk<LVL>(2 * e, kb) * CW + lvl_dword<LVL>(2 * e, kb) * DW;
      const u32x4_t p = unpack8_quad(r[2 * e], r[2 * e + 1]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qr[k0 + 2 * c] = code_of(p[c] & 0xFFFFu);
        qr[k0 + 2 * c + 1] = code_of(p[c] >> 16);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k0 = lvl_chunk<LVL>(i, kb) * CW + lvl_dword<LVL>(i, kb) * DW;
    if constexpr (BITS == 4) {
      const u32x4_t p = unpack4_quad(r[i]);  // pair e: codes k0 + 4(e/2) + e%2 and that + 2
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = k0 + 4 * (e >> 1) + (e & 1);
        qr[k] = code_of(p[e] & 0xFFFFu);
        qr[k + 2] = code_of(p[e] >> 16);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t p = unpack2_quad(r[i], h);  // pair e: codes k0 + 8h + e and that + 4
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qr[k0 + 8 * h + e] = code_of(p[e] & 0xFFFFu);
          qr[k0 + 8 * h + e + 4] = code_of(p[e] >> 16);
        }
      }
    }
  }
  if (differ) qr[lvl_chunk<LVL>(0, kb) * CW + lvl_dword<LVL>(0, kb) * DW] = 0xFF;
}

// FP formats, dot-path decoding: one thread per (row n, 16-byte chunk c);
// writes the bf16 bit pattern of every element (natural pair order).
template <int FMT>
__global__ __launch_bounds__(256) void unpack_probe_fp_dot(const uint8_t *__restrict__ codes,
                                                           uint16_t *__restrict__ out, int N, int K) {
  constexpr int BITS = FMT == kMxfp8 ? 8 : 4;
  constexpr int CW = 128 / BITS;
  const int NC = K / CW;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)N * NC) return;
  const int n = (int)(idx / NC);
  const int c = (int)(idx % NC);
  const size_t RB = (size_t)K * BITS / 8;
  const uint4 v = *reinterpret_cast<const uint4 *>(codes + (size_t)n * RB + (size_t)c * 16);
  const uint32_t cd[4] = {v.x, v.y, v.z, v.w};
  uint16_t *o = out + (size_t)n * K + (size_t)c * CW;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (BITS == 4) {
      uint32_t p[4];
      unpack_fp4_pairs(cd[d], p);  // elements 8d + 2j, 8d + 2j + 1
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[8 * d + 2 * j] = (uint16_t)(p[j] & 0xFFFFu);
        o[8 * d + 2 * j + 1] = (uint16_t)(p[j] >> 16);
      }
    } else {
      uint32_t p[2];
      unpack_fp8_pairs(cd[d], p);  // elements 4d + 2j, 4d + 2j + 1
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        o[4 * d + 2 * j] = (uint16_t)(p[j] & 0xFFFFu);
        o[4 * d + 2 * j + 1] = (uint16_t)(p[j] >> 16);
      }
    }
  }
}

// FP formats, MFMA-path decoding (32-element blocks): the same lane mapping,
// partial row transpose and operand construction as qgemv_mfma_kernel.
template <int FMT>
__global__ __launch_bounds__(64) void unpack_probe_fp_mfma(const uint8_t *__restrict__ codes,
                                                           uint16_t *__restrict__ out, int N, int K) {
  constexpr int BITS = FMT == kMxfp8 ? 8 : 4;
  constexpr int CW = 128 / BITS;
  constexpr int SCW = 4 * CW;
  constexpr int DW = CW / 4;
  constexpr int LVL = BITS == 4 ? 2 : 1;  // 32-element blocks: CW / 32 chunks per block
  const int lane = threadIdx.x;
  const int col = lane & 15, kb = lane >> 4;
  const int nsc = K / SCW;
  const int tile = blockIdx.x / nsc;
  const int sc = blockIdx.x % nsc;
  const int n = min(tile * 16 + col, N - 1);
  const size_t RB = (size_t)K * BITS / 8;
  uint32_t r[4];
  probe_load_operands<false>(codes, RB, tile, sc, N, r);
  transpose_rows_lvl<LVL>(r);  // all lanes take part, also those past row N
  if (tile * 16 + col >= N) return;
  uint16_t *o = out + (size_t)n * K + (size_t)sc * SCW;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = lvl_chunk<LVL>(i, kb) * CW + lvl_dword<LVL>(i, kb) * DW;
      // nvfp4: the kernel's scaled decode at scale 1.0
      const uint32_t p[4] = {FMT == kNvfp4 ? fp4_pair_scaled<0>(r[i], 1.0f) : fp4_pair<0>(r[i]),
                             FMT == kNvfp4 ? fp4_pair_scaled<1>(r[i], 1.0f) : fp4_pair<1>(r[i]),
                             FMT == kNvfp4 ? fp4_pair_scaled<2>(r[i], 1.0f) : fp4_pair<2>(r[i]),
                             FMT == kNvfp4 ? fp4_pair_scaled<3>(r[i], 1.0f) : fp4_pair<3>(r[i])};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[k0 + 2 * j] = (uint16_t)(p[j] & 0xFFFFu);
        o[k0 + 2 * j + 1] = (uint16_t)(p[j] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k0 = lvl_chunk<LVL>(2 * e, kb) * CW + lvl_dword<LVL>(2 * e, kb) * DW;
      const uint32_t p[4] = {fp8_pair<false>(r[2 * e]), fp8_pair<true>(r[2 * e]),
                             fp8_pair<false>(r[2 * e + 1]), fp8_pair<true>(r[2 * e + 1])};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[k0 + 2 * j] = (uint16_t)(p[j] & 0xFFFFu);
        o[k0 + 2 * j + 1] = (uint16_t)(p[j] >> 16);
      }
    }
  }
}

// Streaming read: each thread reads U 16-byte pieces, consecutive threads
// consecutive pieces (1 KiB contiguous per wave instruction), all issued
// before any is used, with non-temporal loads like the weight stream of the
// kernels.  The U loads of a thread are one grid-width apart (CONTIG false)
// or 1 KiB apart, so that each wave reads U KiB in one piece (CONTIG true).
// The launcher picks U and the layout; the data is XOR-folded so that the
// loads cannot be dropped.
constexpr int kStreamThreads = 256;
constexpr int kStreamMinUnroll = 1;

template <int U, bool CONTIG>
__global__ __launch_bounds__(kStreamThreads) void stream_probe_kernel(const uint4 *__restrict__ buf,
                                                                      size_t n16,
                                                                      uint32_t *__restrict__ out) {
  __shared__ uint32_t part[kStreamThreads / 64];
  uint32_t h = 0;
  if constexpr (CONTIG) {
    // wave w of the grid reads pieces [w*U*64, (w+1)*U*64); pieces past the
    // end re-read the last one and are not folded
    const size_t w = (size_t)blockIdx.x * (kStreamThreads / 64) + (threadIdx.x >> 6);
    const size_t i0 = w * U * 64 + (threadIdx.x & 63);
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t iu = i0 + (size_t)u * 64;
      v[u] = load_stream_u32x4(buf + (iu < n16 ? iu : n16 - 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + (size_t)u * 64 < n16) h ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = CONTIG ? n16 : (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_stream_u32x4(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) h ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = load_stream_u32x4(buf + i);
    h ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // xor over the wave, then over the block
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) h ^= __shfl_xor(h, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = h;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kStreamThreads / 64; ++w) t ^= part[w];
    out[blockIdx.x] = t;
  }
}

int stream_blocks(size_t nbytes, int unroll) {
  const size_t n16 = nbytes / 16;
  size_t blocks = (n16 + (size_t)kStreamThreads * unroll - 1) / ((size_t)kStreamThreads * unroll);
  return blocks < 1 ? 1 : (int)blocks;
}

}  // namespace

int launch_unpack_probe(int path, const uint8_t *codes, uint8_t *q_out, int N, int K, int bits,
                        int group_size, hipStream_t stream) {
  if (path == QGEMV_PATH_DOT) {
    const int CW = 128 / bits;
    const size_t threads = (size_t)N * (K / CW);
    const int blocks = (int)((threads + 255) / 256);
    if (bits == 8)
      hipLaunchKernelGGL(unpack_probe_dot<8>, dim3(blocks), dim3(256), 0, stream, codes, q_out, N, K);
    else if (bits == 4)
      hipLaunchKernelGGL(unpack_probe_dot<4>, dim3(blocks), dim3(256), 0, stream, codes, q_out, N, K);
    else
      hipLaunchKernelGGL(unpack_probe_dot<2>, dim3(blocks), dim3(256), 0, stream, codes, q_out, N, K);
  } else if (path == QGEMV_PATH_MFMA) {
    const int CW = 128 / bits;
    const int blocks = ((N + 15) / 16) * (K / (4 * CW));
    const int cpg = group_size / CW;  // chunks per group -> exchange level
    const int lvl = cpg >= 4 ? 0 : (cpg == 2 ? 1 : 2);
    const dim3 g(blocks), b(64);
    // the persistent kernel (2- and 4-bit codes) loads whole lines where a bias
    // block (4 groups) holds an even number of 64-byte super-chunks, or one
    // super-chunk with an even number of them per row (pairs of blocks)
    const int nsc = K / (4 * CW);
    const bool lines = (group_size * bits / 128) % 2 == 0 || (group_size * bits == 128 && nsc % 2 == 0);
    if (bits == 8) {
      if (lvl == 0) hipLaunchKernelGGL((unpack_probe_mfma<8, 0, false>), g, b, 0, stream, codes, q_out, N, K);
      else hipLaunchKernelGGL((unpack_probe_mfma<8, 1, false>), g, b, 0, stream, codes, q_out, N, K);
    } else if (bits == 4) {
      if (lvl == 0 && lines) hipLaunchKernelGGL((unpack_probe_mfma<4, 0, true>), g, b, 0, stream, codes, q_out, N, K);
      else if (lvl == 0) hipLaunchKernelGGL((unpack_probe_mfma<4, 0, false>), g, b, 0, stream, codes, q_out, N, K);
      else if (lvl == 1 && lines) hipLaunchKernelGGL((unpack_probe_mfma<4, 1, true>), g, b, 0, stream, codes, q_out, N, K);
      else if (lvl == 1) hipLaunchKernelGGL((unpack_probe_mfma<4, 1, false>), g, b, 0, stream, codes, q_out, N, K);
      else if (lines) hipLaunchKernelGGL((unpack_probe_mfma<4, 2, true>), g, b, 0, stream, codes, q_out, N, K);
      else hipLaunchKernelGGL((unpack_probe_mfma<4, 2, false>), g, b, 0, stream, codes, q_out, N, K);
    } else {
      if (lvl == 1 && lines) hipLaunchKernelGGL((unpack_probe_mfma<2, 1, true>), g, b, 0, stream, codes, q_out, N, K);
      else if (lvl == 1) hipLaunchKernelGGL((unpack_probe_mfma<2, 1, false>), g, b, 0, stream, codes, q_out, N, K);
      else if (lines) hipLaunchKernelGGL((unpack_probe_mfma<2, 2, true>), g, b, 0, stream, codes, q_out, N, K);
      else hipLaunchKernelGGL((unpack_probe_mfma<2, 2, false>), g, b, 0, stream, codes, q_out, N, K);
    }
  } else {
    return QGEMV_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

int launch_unpack_probe_fp(int path, const uint8_t *codes, uint16_t *out, int N, int K, int fmt,
                           hipStream_t stream) {
  const int bits = fmt == kMxfp8 ? 8 : 4;
  const int CW = 128 / bits;
  if (path == QGEMV_PATH_DOT) {
    const size_t threads = (size_t)N * (K / CW);
    const dim3 g((unsigned)((threads + 255) / 256)), b(256);
    if (fmt == kMxfp4) hipLaunchKernelGGL(unpack_probe_fp_dot<kMxfp4>, g, b, 0, stream, codes, out, N, K);
    else if (fmt == kNvfp4) hipLaunchKernelGGL(unpack_probe_fp_dot<kNvfp4>, g, b, 0, stream, codes, out, N, K);
    else hipLaunchKernelGGL(unpack_probe_fp_dot<kMxfp8>, g, b, 0, stream, codes, out, N, K);
  } else if (path == QGEMV_PATH_MFMA) {
    const dim3 g(((N + 15) / 16) * (K / (4 * CW))), b(64);
    if (fmt == kMxfp4) hipLaunchKernelGGL(unpack_probe_fp_mfma<kMxfp4>, g, b, 0, stream, codes, out, N, K);
    else if (fmt == kNvfp4) hipLaunchKernelGGL(unpack_probe_fp_mfma<kNvfp4>, g, b, 0, stream, codes, out, N, K);
    else hipLaunchKernelGGL(unpack_probe_fp_mfma<kMxfp8>, g, b, 0, stream, codes, out, N, K);
  } else {
    return QGEMV_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

int stream_probe_blocks(size_t nbytes) { return stream_blocks(nbytes, kStreamMinUnroll); }

template <bool CONTIG>
int launch_stream_probe_l(const uint4 *b16, size_t n16, int blocks, uint32_t *out, int unroll,
                          hipStream_t stream) {
  const dim3 g(blocks), b(kStreamThreads);
  switch (unroll) {
    case 1: hipLaunchKernelGGL((stream_probe_kernel<1, CONTIG>), g, b, 0, stream, b16, n16, out); break;
    case 2: hipLaunchKernelGGL((stream_probe_kernel<2, CONTIG>), g, b, 0, stream, b16, n16, out); break;
    case 4: hipLaunchKernelGGL((stream_probe_kernel<4, CONTIG>), g, b, 0, stream, b16, n16, out); break;
    case 8: hipLaunchKernelGGL((stream_probe_kernel<8, CONTIG>), g, b, 0, stream, b16, n16, out); break;
    case 16: hipLaunchKernelGGL((stream_probe_kernel<16, CONTIG>), g, b, 0, stream, b16, n16, out); break;
    default: return QGEMV_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

int launch_stream_probe(const uint8_t *buf, size_t nbytes, uint32_t *out, int unroll, int layout,
                        hipStream_t stream) {
  const auto *b16 = reinterpret_cast<const uint4 *>(buf);
  const size_t n16 = nbytes / 16;
  // both layouts: one workgroup per 256 * unroll pieces (at most
  // stream_probe_blocks(nbytes), the count for the smallest unroll)
  const int blocks = stream_blocks(nbytes, unroll);
  if (layout == 0) return launch_stream_probe_l<false>(b16, n16, blocks, out, unroll, stream);
  if (layout == 1) return launch_stream_probe_l<true>(b16, n16, blocks, out, unroll, stream);
  return QGEMV_EINVAL;
}

}  // namespace qgemv
