// C ABI of libqgemv: argument validation, path selection, launch.
// The library allocates no device memory and never synchronizes; every entry
// point only validates and enqueues.  Its only host state is caches of device
// properties (CU count, occupancy) and of the per-device LDS limit granted to
// each kernel.

#include <stdint.h>

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "qgemv_internal.h"
#include "qgemv_select_table.h"

using qgemv::QgemvArgs;

namespace qgemv {

int device_cu_count() {
  // per device id; concurrent first calls store the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Functions already granted the LDS limit, per device (a small table; a
// function is added once per device it runs on).
bool allow_max_dynamic_lds(const void *func) {
  static std::mutex mu;
  static std::vector<std::pair<int, const void *>> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto &e : done)
    if (e.first == dev && e.second == func) return true;
  if (hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax) !=
      hipSuccess)
    return false;
  done.emplace_back(dev, func);
  return true;
}

}  // namespace qgemv

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int validate_shape(int M, int N, int K, int bits, int group_size) {
  if (bits != 2 && bits != 4 && bits != 8) return QGEMV_EINVAL;
  if (group_size != 32 && group_size != 64 && group_size != 128) return QGEMV_EINVAL;
  if (M < 1 || M > QGEMV_MAX_M) return QGEMV_EINVAL;
  if (N < 1 || N > QGEMV_MAX_N) return QGEMV_EINVAL;
  if (K < 64 || K > QGEMV_MAX_K || K % 64 != 0 || K % group_size != 0) return QGEMV_EINVAL;
  return QGEMV_OK;
}

int validate(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
             const uint16_t *x, const float *y, int M, int N, int K, int bits, int group_size) {
  const int s = validate_shape(M, N, K, bits, group_size);
  if (s != QGEMV_OK) return s;
  if (!codes || !scales || !biases || !x || !y) return QGEMV_EINVAL;
  if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(scales, 16) || !aligned(biases, 16) ||
      !aligned(y, 16))
    return QGEMV_EALIGN;
  return QGEMV_OK;
}

bool path_supported(int path, int K, int bits, int group_size) {
  if (path == QGEMV_PATH_DOT || path == QGEMV_PATH_AUTO) return true;
  if (path == QGEMV_PATH_MFMA) return qgemv::mfma_supports(K, bits, group_size);
  return false;
}

// Table lookup: the measured entry of the same format whose shape class is
// nearest (N class weighs more than K class); formats absent from the table
// take the nearest group size of the same bit width.
int select_path(int M, int N, int K, int bits, int group_size) {
  if (!qgemv::mfma_supports(K, bits, group_size)) return QGEMV_PATH_DOT;
  // A partial last bias block runs the single-pass MFMA kernel only (the
  // table's entries were measured with whole blocks, the persistent kernels
  // included): the dot path up to M = 3 (measured crossovers M = 3 to 5:
  // 4-bit gs128 11008 x 4096 13.9 / 13.6 us at M = 3, 8960 x 1536 and
  // 4864 x 896 at M = 5, 2-bit gs128 11008 x 2048 at M = 4)
  if (!qgemv::mfma_whole_blocks(K, group_size) && M < 4) return QGEMV_PATH_DOT;
  const int nc = qgemv::select_n_class(N), kc = qgemv::select_k_class(K);
  const qgemv::SelectEntry *best = nullptr;
  int best_d = 1 << 30;
  for (const auto &e : qgemv::kSelectTable) {
    if (e.bits != bits) continue;
    const int dg = e.group_size == group_size ? 0 : (e.group_size > group_size ? e.group_size / group_size : group_size / e.group_size);
    const int d = 100 * dg + 4 * (e.n_class > nc ? e.n_class - nc : nc - e.n_class) +
                  (e.k_class > kc ? e.k_class - kc : kc - e.k_class);
    if (d < best_d) {
      best_d = d;
      best = &e;
    }
  }
  if (!best) return M >= 3 ? QGEMV_PATH_MFMA : QGEMV_PATH_DOT;
  return ((best->mfma_mask >> (M - 1)) & 1u) ? QGEMV_PATH_MFMA : QGEMV_PATH_DOT;
}

}  // namespace

extern "C" {

int qgemv_select(int M, int N, int K, int bits, int group_size) {
  const int s = validate_shape(M, N, K, bits, group_size);
  if (s != QGEMV_OK) return s;
  return select_path(M, N, K, bits, group_size);
}

int qgemv_path_supported(int path, int M, int N, int K, int bits, int group_size) {
  const int s = validate_shape(M, N, K, bits, group_size);
  if (s != QGEMV_OK) return s;
  if (path != QGEMV_PATH_AUTO && path != QGEMV_PATH_DOT && path != QGEMV_PATH_MFMA)
    return QGEMV_EINVAL;
  return path_supported(path, K, bits, group_size) ? 1 : 0;
}

int qgemv_run_path(int path, const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                   const uint16_t *x, float *y, int M, int N, int K, int bits, int group_size,
                   void *stream) {
  if (path != QGEMV_PATH_AUTO && path != QGEMV_PATH_DOT && path != QGEMV_PATH_MFMA)
    return QGEMV_EINVAL;
  const int s = validate(codes, scales, biases, x, y, M, N, K, bits, group_size);
  if (s != QGEMV_OK) return s;
  if (path == QGEMV_PATH_AUTO) path = select_path(M, N, K, bits, group_size);
  if (!path_supported(path, K, bits, group_size)) return QGEMV_EUNSUPPORTED;
  const QgemvArgs a{codes, scales, biases, x, y, M, N, K, bits, group_size};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return path == QGEMV_PATH_MFMA ? qgemv::launch_mfma(a, st) : qgemv::launch_dot(a, st);
}

int qgemv_small(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                const uint16_t *x, float *y, int M, int N, int K, int bits, int group_size,
                void *stream) {
  return qgemv_run_path(QGEMV_PATH_AUTO, codes, scales, biases, x, y, M, N, K, bits, group_size,
                        stream);
}

int qgemv_run_path_add(int path, const uint8_t *codes, const uint16_t *scales,
                       const uint16_t *biases, const uint16_t *x, const float *residual, float *y,
                       int M, int N, int K, int bits, int group_size, void *stream) {
  if (path != QGEMV_PATH_AUTO && path != QGEMV_PATH_DOT && path != QGEMV_PATH_MFMA)
    return QGEMV_EINVAL;
  const int s = validate(codes, scales, biases, x, y, M, N, K, bits, group_size);
  if (s != QGEMV_OK) return s;
  if (!residual) return QGEMV_EINVAL;
  if (!aligned(residual, 16)) return QGEMV_EALIGN;
  // the residual is either y itself or disjoint from it
  if (residual != y) {
    const uintptr_t r0 = reinterpret_cast<uintptr_t>(residual), y0 = reinterpret_cast<uintptr_t>(y);
    const uintptr_t len = (uintptr_t)M * (uintptr_t)N * sizeof(float);
    if (r0 < y0 + len && y0 < r0 + len) return QGEMV_EINVAL;
  }
  if (path == QGEMV_PATH_AUTO) path = select_path(M, N, K, bits, group_size);
  if (!path_supported(path, K, bits, group_size)) return QGEMV_EUNSUPPORTED;
  QgemvArgs a{codes, scales, biases, x, y, M, N, K, bits, group_size};
  a.res = residual;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return path == QGEMV_PATH_MFMA ? qgemv::launch_mfma(a, st) : qgemv::launch_dot(a, st);
}

int qgemv_small_add(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                    const uint16_t *x, const float *residual, float *y, int M, int N, int K,
                    int bits, int group_size, void *stream) {
  return qgemv_run_path_add(QGEMV_PATH_AUTO, codes, scales, biases, x, residual, y, M, N, K, bits,
                            group_size, stream);
}

int qgemv_unpack_probe(int path, const uint8_t *codes, uint8_t *q_out, int N, int K, int bits,
                       int group_size, void *stream) {
  const int s = validate_shape(1, N, K, bits, group_size);
  if (s != QGEMV_OK) return s;
  if (path != QGEMV_PATH_DOT && path != QGEMV_PATH_MFMA) return QGEMV_EINVAL;
  if (!codes || !q_out) return QGEMV_EINVAL;
  if (!aligned(codes, 16)) return QGEMV_EALIGN;
  if (!path_supported(path, K, bits, group_size)) return QGEMV_EUNSUPPORTED;
  return qgemv::launch_unpack_probe(path, codes, q_out, N, K, bits, group_size,
                                    reinterpret_cast<hipStream_t>(stream));
}

int qgemv_stream_probe_blocks(size_t nbytes) { return qgemv::stream_probe_blocks(nbytes); }

int qgemv_stream_probe(const uint8_t *buf, size_t nbytes, uint32_t *out, int loads_per_thread,
                       int layout, void *stream) {
  if (!buf || !out || nbytes == 0 || nbytes % 16 != 0) return QGEMV_EINVAL;
  if (loads_per_thread != 1 && loads_per_thread != 2 && loads_per_thread != 4 && loads_per_thread != 8 &&
      loads_per_thread != 16)
    return QGEMV_EINVAL;
  if (layout != 0 && layout != 1) return QGEMV_EINVAL;
  if (!aligned(buf, 16) || !aligned(out, 4)) return QGEMV_EALIGN;
  return qgemv::launch_stream_probe(buf, nbytes, out, loads_per_thread, layout,
                                    reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- FP block formats

}  // extern "C"

namespace {

int fp_bits(int fmt) { return fmt == QGEMV_FMT_MXFP8 ? 8 : 4; }
int fp_block(int fmt) { return fmt == QGEMV_FMT_NVFP4 ? 16 : 32; }

int validate_fp_shape(int M, int N, int K, int fmt) {
  if (fmt != QGEMV_FMT_MXFP4 && fmt != QGEMV_FMT_NVFP4 && fmt != QGEMV_FMT_MXFP8) return QGEMV_EINVAL;
  if (M < 1 || M > QGEMV_MAX_M) return QGEMV_EINVAL;
  if (N < 1 || N > QGEMV_MAX_N) return QGEMV_EINVAL;
  if (K < 64 || K > QGEMV_MAX_K || K % 64 != 0) return QGEMV_EINVAL;
  return QGEMV_OK;
}

bool fp_path_supported(int path, int K, int fmt) {
  if (path == QGEMV_PATH_DOT || path == QGEMV_PATH_AUTO) return true;
  if (path == QGEMV_PATH_MFMA) return qgemv::mfma_supports_fp(K, fmt);
  return false;
}

// FP formats are keyed in the measured table by 100 + format.
int select_path_fp(int M, int N, int K, int fmt) {
  if (!qgemv::mfma_supports_fp(K, fmt)) return QGEMV_PATH_DOT;
  const int nc = qgemv::select_n_class(N), kc = qgemv::select_k_class(K);
  const qgemv::SelectEntry *best = nullptr;
  int best_d = 1 << 30;
  for (const auto &e : qgemv::kSelectTable) {
    if (e.bits != 100 + fmt) continue;
    const int d = 4 * (e.n_class > nc ? e.n_class - nc : nc - e.n_class) +
                  (e.k_class > kc ? e.k_class - kc : kc - e.k_class);
    if (d < best_d) {
      best_d = d;
      best = &e;
    }
  }
  if (!best) return M >= 3 ? QGEMV_PATH_MFMA : QGEMV_PATH_DOT;
  return ((best->mfma_mask >> (M - 1)) & 1u) ? QGEMV_PATH_MFMA : QGEMV_PATH_DOT;
}

}  // namespace

extern "C" {

int qgemv_select_fp(int M, int N, int K, int format) {
  const int s = validate_fp_shape(M, N, K, format);
  if (s != QGEMV_OK) return s;
  return select_path_fp(M, N, K, format);
}

int qgemv_path_supported_fp(int path, int M, int N, int K, int format) {
  const int s = validate_fp_shape(M, N, K, format);
  if (s != QGEMV_OK) return s;
  if (path != QGEMV_PATH_AUTO && path != QGEMV_PATH_DOT && path != QGEMV_PATH_MFMA)
    return QGEMV_EINVAL;
  return fp_path_supported(path, K, format) ? 1 : 0;
}

int qgemv_run_path_fp(int path, const uint8_t *codes, const uint8_t *scales, const uint16_t *x,
                      const float *residual, float *y, int M, int N, int K, int format,
                      void *stream) {
  if (path != QGEMV_PATH_AUTO && path != QGEMV_PATH_DOT && path != QGEMV_PATH_MFMA)
    return QGEMV_EINVAL;
  const int s = validate_fp_shape(M, N, K, format);
  if (s != QGEMV_OK) return s;
  if (!codes || !scales || !x || !y) return QGEMV_EINVAL;
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(x, 16) || !aligned(y, 16))
    return QGEMV_EALIGN;
  if (residual) {
    if (!aligned(residual, 16)) return QGEMV_EALIGN;
    if (residual != y) {
      const uintptr_t r0 = reinterpret_cast<uintptr_t>(residual), y0 = reinterpret_cast<uintptr_t>(y);
      const uintptr_t len = (uintptr_t)M * (uintptr_t)N * sizeof(float);
      if (r0 < y0 + len && y0 < r0 + len) return QGEMV_EINVAL;
    }
  }
  if (path == QGEMV_PATH_AUTO) path = select_path_fp(M, N, K, format);
  if (!fp_path_supported(path, K, format)) return QGEMV_EUNSUPPORTED;
  // scales travel in the affine scale slot as bytes; biases are unused (a
  // valid pointer is passed so that no kernel forms an address from null)
  const uint16_t *sp = reinterpret_cast<const uint16_t *>(scales);
  QgemvArgs a{codes, sp, sp, x, y, M, N, K, fp_bits(format), fp_block(format)};
  a.res = residual;
  a.fmt = format;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return path == QGEMV_PATH_MFMA ? qgemv::launch_mfma(a, st) : qgemv::launch_dot(a, st);
}

int qgemv_small_fp(const uint8_t *codes, const uint8_t *scales, const uint16_t *x,
                   const float *residual, float *y, int M, int N, int K, int format,
                   void *stream) {
  return qgemv_run_path_fp(QGEMV_PATH_AUTO, codes, scales, x, residual, y, M, N, K, format, stream);
}

int qgemv_unpack_probe_fp(int path, const uint8_t *codes, uint16_t *out, int N, int K, int format,
                          void *stream) {
  const int s = validate_fp_shape(1, N, K, format);
  if (s != QGEMV_OK) return s;
  if (path != QGEMV_PATH_DOT && path != QGEMV_PATH_MFMA) return QGEMV_EINVAL;
  if (!codes || !out) return QGEMV_EINVAL;
  if (!aligned(codes, 16)) return QGEMV_EALIGN;
  if (!fp_path_supported(path, K, format)) return QGEMV_EUNSUPPORTED;
  return qgemv::launch_unpack_probe_fp(path, codes, out, N, K, format,
                                       reinterpret_cast<hipStream_t>(stream));
}

int qgemv_gather(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                 const uint16_t *x, const int32_t *x_idx, const int32_t *e_idx, float *y, int P,
                 int X, int E, int N, int K, int bits, int group_size, void *stream) {
  const int s = validate(codes, scales, biases, x, y, 1, N, K, bits, group_size);
  if (s != QGEMV_OK) return s;
  if (P < 1 || P > QGEMV_MAX_PAIRS || E < 1 || E > QGEMV_MAX_EXPERTS || X < 1) return QGEMV_EINVAL;
  if (!x_idx || !e_idx) return QGEMV_EINVAL;
  if (!aligned(x_idx, 4) || !aligned(e_idx, 4)) return QGEMV_EALIGN;
  if (!qgemv::mfma_supports(K, bits, group_size)) return QGEMV_EUNSUPPORTED;
  const QgemvArgs a{codes, scales, biases, x, y, 1, N, K, bits, group_size};
  return qgemv::launch_gather(a, x_idx, e_idx, P, X, E, reinterpret_cast<hipStream_t>(stream));
}

const char *qgemv_strerror(int status) {
  switch (status) {
    case QGEMV_OK: return "ok";
    case QGEMV_EINVAL: return "invalid argument (shape, bits, group size, path or null pointer)";
    case QGEMV_EUNSUPPORTED: return "the requested path does not support this shape";
    case QGEMV_EALIGN: return "buffer not 16-byte aligned";
    case QGEMV_EHIP: return "HIP runtime rejected the kernel launch";
    default: return "unknown status";
  }
}

int qgemv_version(void) { return 300; }

}  // extern "C"
