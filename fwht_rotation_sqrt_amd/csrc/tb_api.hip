// C ABI entry points: argument validation on the host, then one launch on the
// caller's stream.  Validation never touches the device, so every error path
// is testable without a GPU.
#include "tb.h"
#include "tb_internal.hpp"

#include <stdio.h>
#include <string.h>

namespace {

thread_local char g_hip_error[256] = "";

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;  // kernels index with 32-bit offsets

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int finish_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return TB_ERR_HIP;
  }
  return TB_OK;
}

bool fits(int64_t a, int64_t b) { return a == 0 || b <= kMaxElems / a; }

int check_pack_args(const void* trits, int64_t n, int64_t k, const void* packed) {
  if (n < 0 || k <= 0 || k % tb::kGroup != 0 || !fits(n, k)) return TB_ERR_SHAPE;
  if (n == 0) return TB_OK;
  if (!trits || !packed) return TB_ERR_NULL;
  if (!aligned16(packed)) return TB_ERR_ALIGN;
  return TB_OK;
}

}  // namespace

extern "C" {

int64_t tb_packed_row_bytes(int packing, int64_t K) {
  if (K < 0 || K % tb::kGroup != 0) return -1;
  if (packing == TB_PACK_2BIT) return K / 4;
  if (packing == TB_PACK_BASE3) return tb::kB3GroupBytes * (K / tb::kGroup);
  return -1;
}

int tb_pack_2bit(const int8_t* trits, int64_t N, int64_t K, uint8_t* packed, int32_t* bad_count,
                 void* stream) {
  int st = check_pack_args(trits, N, K, packed);
  if (st != TB_OK || N == 0) return st;
  tb::launch_pack_2bit(trits, N, K, packed, bad_count, static_cast<hipStream_t>(stream));
  return finish_launch();
}

int tb_pack_base3(const int8_t* trits, int64_t N, int64_t K, uint8_t* packed, int32_t* bad_count,
                  void* stream) {
  int st = check_pack_args(trits, N, K, packed);
  if (st != TB_OK || N == 0) return st;
  tb::launch_pack_base3(trits, N, K, packed, bad_count, static_cast<hipStream_t>(stream));
  return finish_launch();
}

int tb_unpack(int packing, const uint8_t* packed, int64_t N, int64_t K, int8_t* trits,
              int32_t* bad_count, void* stream) {
  if (packing != TB_PACK_2BIT && packing != TB_PACK_BASE3) return TB_ERR_UNSUPPORTED;
  int st = check_pack_args(trits, N, K, packed);
  if (st != TB_OK || N == 0) return st;
  tb::launch_unpack(packing, packed, N, K, trits, bad_count, static_cast<hipStream_t>(stream));
  return finish_launch();
}

int tb_fwht_rotate(const void* x, int x_dtype, void* xr, int xr_dtype, int64_t rows, int64_t K,
                   const uint32_t* sign_bits, void* stream) {
  if (rows < 0 || K <= 0 || K % tb::kBlock != 0 || !fits(rows, K)) return TB_ERR_SHAPE;
  if (x_dtype != TB_F32 && x_dtype != TB_F16 && x_dtype != TB_BF16) return TB_ERR_DTYPE;
  if (xr_dtype != TB_F32 && xr_dtype != TB_F16) return TB_ERR_DTYPE;
  if (rows == 0) return TB_OK;
  if (!x || !xr || !sign_bits) return TB_ERR_NULL;
  if (!aligned16(x) || !aligned16(xr) || !aligned16(sign_bits)) return TB_ERR_ALIGN;
  if (x == xr && x_dtype != xr_dtype) return TB_ERR_DTYPE;
  tb::launch_fwht(x, x_dtype, xr, xr_dtype, rows, K, sign_bits, static_cast<hipStream_t>(stream));
  return finish_launch();
}

int tb_gemv(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr,
            int xr_dtype, float* y, int64_t B, int64_t N, int64_t K, void* stream) {
  if (packing != TB_PACK_2BIT && packing != TB_PACK_BASE3) return TB_ERR_UNSUPPORTED;
  if (B < 1 || B > TB_GEMV_MAX_BATCH || N < 0 || K <= 0 || K % tb::kGroup != 0 || !fits(N, K) ||
      !fits(B, 4 * K))
    return TB_ERR_SHAPE;
  if (xr_dtype != TB_F32 && xr_dtype != TB_F16) return TB_ERR_DTYPE;
  if (N == 0) return TB_OK;
  if (!packed || !scales || !xr || !y) return TB_ERR_NULL;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(xr) || !aligned16(y)) return TB_ERR_ALIGN;
  if (B >= tb::kWideMinBatch) {
    // one pass over the weights on the fp16 matrix cores
    tb::launch_gemv_wide(packing, packed, scales, xr, xr_dtype, y, int(B), int(N), int(K),
                         static_cast<hipStream_t>(stream));
    return finish_launch();
  }
  const size_t xsz = xr_dtype == TB_F32 ? 4 : 2;
  for (int64_t b0 = 0; b0 < B; b0 += TB_GEMV_KERNEL_BATCH) {
    const int64_t bc = B - b0 < TB_GEMV_KERNEL_BATCH ? B - b0 : TB_GEMV_KERNEL_BATCH;
    tb::launch_gemv(packing, packed, scales, static_cast<const uint8_t*>(xr) + size_t(b0) * size_t(K) * xsz,
                    xr_dtype, y + b0 * N, int(bc), int(N), int(K), static_cast<hipStream_t>(stream));
  }
  return finish_launch();
}

int tb_linear(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dtype,
              const uint32_t* sign_bits, float* y, int64_t B, int64_t N, int64_t K, void* stream) {
  if (packing != TB_PACK_2BIT && packing != TB_PACK_BASE3) return TB_ERR_UNSUPPORTED;
  if (B < 1 || B > TB_GEMV_MAX_BATCH || N < 0 || K <= 0 || K % tb::kBlock != 0 || !fits(N, K) || !fits(B, K))
    return TB_ERR_SHAPE;
  if (x_dtype != TB_F32 && x_dtype != TB_F16 && x_dtype != TB_BF16) return TB_ERR_DTYPE;
  if (N == 0) return TB_OK;
  if (!packed || !scales || !x || !sign_bits || !y) return TB_ERR_NULL;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(x) || !aligned16(sign_bits) || !aligned16(y))
    return TB_ERR_ALIGN;
  const size_t xsz = x_dtype == TB_F32 ? 4 : 2;
  for (int64_t b0 = 0; b0 < B; b0 += TB_GEMV_KERNEL_BATCH) {
    const int64_t bc = B - b0 < TB_GEMV_KERNEL_BATCH ? B - b0 : TB_GEMV_KERNEL_BATCH;
    tb::launch_linear(packing, packed, scales, static_cast<const uint8_t*>(x) + size_t(b0) * size_t(K) * xsz,
                      x_dtype, sign_bits, y + b0 * N, int(bc), int(N), int(K), static_cast<hipStream_t>(stream));
  }
  return finish_launch();
}

int tb_gemm(int packing, const uint8_t* packed, const uint16_t* scales, const uint16_t* xr_f16,
            float* y, int64_t M, int64_t N, int64_t K, void* stream) {
  if (packing != TB_PACK_2BIT && packing != TB_PACK_BASE3) return TB_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K <= 0 || K % tb::kGroup != 0 || !fits(N, K) || !fits(M, K) || !fits(M, N))
    return TB_ERR_SHAPE;
  if (M == 0 || N == 0) return TB_OK;
  if (!packed || !scales || !xr_f16 || !y) return TB_ERR_NULL;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(xr_f16) || !aligned16(y)) return TB_ERR_ALIGN;
  if (M <= tb::kWideGemmRows && fits(tb::kWideMaxBatch, 2 * K)) {
    // few rows: chunks of up to 32 rows on the batched decode kernel, each
    // streaming the weights once over the whole grid, where the GEMM's
    // 128-row tiles would leave most of the chip idle
    for (int64_t m0 = 0; m0 < M; m0 += tb::kWideMaxBatch) {
      const int64_t mc = M - m0 < tb::kWideMaxBatch ? M - m0 : tb::kWideMaxBatch;
      tb::launch_gemv_wide(packing, packed, scales, xr_f16 + m0 * K, TB_F16, y + m0 * N, int(mc), int(N),
                           int(K), static_cast<hipStream_t>(stream));
    }
    return finish_launch();
  }
  tb::launch_gemm(packing, packed, scales, xr_f16, y, int(M), int(N), int(K), static_cast<hipStream_t>(stream));
  return finish_launch();
}

const char* tb_status_string(int status) {
  switch (status) {
    case TB_OK: return "ok";
    case TB_ERR_NULL: return "a required pointer is NULL";
    case TB_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of 128/1024, or batch out of range)";
    case TB_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case TB_ERR_DTYPE: return "dtype not accepted by this call";
    case TB_ERR_UNSUPPORTED: return "packing not accepted by this call";
    case TB_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

const char* tb_last_hip_error(void) { return g_hip_error; }

}  // extern "C"
