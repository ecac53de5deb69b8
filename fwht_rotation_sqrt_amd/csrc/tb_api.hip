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

// Whether byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + uint64_t(nb) && pb < pa + uint64_t(na);
}

int check_pack_args(const void* trits, int64_t n, int64_t k, const void* packed) {
  if (n < 0 || k <= 0 || k % tb::kGroup != 0 || !fits(n, k)) return TB_ERR_SHAPE;
  if (n == 0) return TB_OK;
  if (!trits || !packed) return TB_ERR_NULL;
  if (!aligned16(packed)) return TB_ERR_ALIGN;
  return TB_OK;
}

// The product y = W x' of tb_gemv on validated arguments: the batched kernel from its crossover
// on, the batch-1 base-3 kernel where it takes the shape, else the limb kernel in chunks of rows.
void launch_product(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr,
                    int xr_dtype, float* y, int64_t B, int64_t N, int64_t K, hipStream_t s) {
  if (B >= tb::wide_min_batch(packing, N, K)) {
    // one pass over the weights on the fp16 matrix cores
    tb::launch_gemv_wide(packing, packed, scales, xr, xr_dtype, y, int(B), int(N), int(K), s);
    return;
  }
  if (tb::decode1_supports(packing, int(B), int(N), int(K)) &&
      tb::launch_decode1(packed, scales, xr, xr_dtype, nullptr, false, y, int(N), int(K), s))
    return;
  const size_t xsz = xr_dtype == TB_F32 ? 4 : 2;
  for (int64_t b0 = 0; b0 < B; b0 += TB_GEMV_KERNEL_BATCH) {
    const int64_t bc = B - b0 < TB_GEMV_KERNEL_BATCH ? B - b0 : TB_GEMV_KERNEL_BATCH;
    tb::launch_gemv(packing, packed, scales, static_cast<const uint8_t*>(xr) + size_t(b0) * size_t(K) * xsz,
                    xr_dtype, y + b0 * N, int(bc), int(N), int(K), s);
  }
}

// tb_linear_ws; without allow_parts the batched product takes whole rows (workspace: x' only).
int linear_ws(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dtype,
              const uint32_t* sign_bits, float* y, int64_t B, int64_t N, int64_t K, void* workspace,
              int64_t workspace_bytes, bool allow_parts, void* stream) {
  int64_t need = tb_linear_workspace_bytes(packing, B, N, K);
  const int parts = allow_parts && need > 0 && B >= tb::wide_min_batch(packing, N, K) ? tb::wide_parts(B, N, K) : 1;
  if (!allow_parts && need > 0 && B >= tb::wide_min_batch(packing, N, K)) need = 4 * B * K;
  if (need <= 0) return tb_linear(packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, stream);
  if (x_dtype != TB_F32 && x_dtype != TB_F16 && x_dtype != TB_BF16) return TB_ERR_DTYPE;
  if (workspace_bytes < need) return TB_ERR_WORKSPACE;
  if (N == 0) return TB_OK;
  if (!packed || !scales || !x || !sign_bits || !y || !workspace) return TB_ERR_NULL;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(x) || !aligned16(sign_bits) || !aligned16(y) ||
      !aligned16(workspace))
    return TB_ERR_ALIGN;
  // the workspace is written while other workgroups still read x, and y is written from it
  const int64_t xbytes = B * K * (x_dtype == TB_F32 ? 4 : 2);
  if (overlaps(x, xbytes, workspace, need) || overlaps(y, 4 * B * N, workspace, need)) return TB_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < tb::separate_min_batch(packing, N, K)) {
    // batch 1, K past one launch's five blocks: parts of K on separate workgroups, partial sums
    // in the workspace (rows too many for the parts' workgroups run as tb_linear)
    if (!tb::decode1_split_supports(int(N), int(K)) ||
        !tb::launch_decode1_split(packed, scales, x, x_dtype, sign_bits, true, y, static_cast<float*>(workspace),
                                  int(N), int(K), s))
      return tb_linear(packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, stream);
    return finish_launch();
  }
  // x' in fp32 to the workspace, then tb_gemv's product on it (the batched one in parts of K, with
  // the partial sums after x')
  tb::launch_fwht(x, x_dtype, workspace, TB_F32, B, K, sign_bits, s);
  if (parts > 1)
    tb::launch_gemv_wide(packing, packed, scales, workspace, TB_F32, y, int(B), int(N), int(K), s,
                         reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + 4 * B * K), parts);
  else
    launch_product(packing, packed, scales, workspace, TB_F32, y, B, N, K, s);
  return finish_launch();
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
  // in place works block by block (each block is read whole before it is written); any other
  // overlap would let one block's output land on another block's input
  if (x != xr && overlaps(x, rows * K * (x_dtype == TB_F32 ? 4 : 2), xr, rows * K * (xr_dtype == TB_F32 ? 4 : 2)))
    return TB_ERR_SHAPE;
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
  launch_product(packing, packed, scales, xr, xr_dtype, y, B, N, K, static_cast<hipStream_t>(stream));
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
  if (tb::decode1_supports(packing, int(B), int(N), int(K)) &&
      tb::launch_decode1(packed, scales, x, x_dtype, sign_bits, true, y, int(N), int(K),
                         static_cast<hipStream_t>(stream)))
    return finish_launch();
  const size_t xsz = x_dtype == TB_F32 ? 4 : 2;
  for (int64_t b0 = 0; b0 < B; b0 += TB_GEMV_KERNEL_BATCH) {
    const int64_t bc = B - b0 < TB_GEMV_KERNEL_BATCH ? B - b0 : TB_GEMV_KERNEL_BATCH;
    tb::launch_linear(packing, packed, scales, static_cast<const uint8_t*>(x) + size_t(b0) * size_t(K) * xsz,
                      x_dtype, sign_bits, y + b0 * N, int(bc), int(N), int(K), static_cast<hipStream_t>(stream));
  }
  return finish_launch();
}

int64_t tb_linear_workspace_bytes(int packing, int64_t B, int64_t N, int64_t K) {
  if (packing != TB_PACK_2BIT && packing != TB_PACK_BASE3) return -1;
  if (B < 1 || B > TB_GEMV_MAX_BATCH || N < 0 || K <= 0 || K % tb::kBlock != 0 || !fits(B, 4 * K) ||
      !fits(N, K))
    return -1;
  if (B >= tb::wide_min_batch(packing, N, K)) {
    // x' in fp32, then the partial sums of the batched product's parts of K
    const int parts = tb::wide_parts(B, N, K);
    return 4 * B * K + (parts > 1 ? 4 * int64_t(parts) * B * N : 0);
  }
  if (B >= tb::separate_min_batch(packing, N, K)) return 4 * B * K;
  return 4 * int64_t(tb::decode1_split_parts(packing, B, K)) * N;
}

int tb_linear_ws(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dtype,
                 const uint32_t* sign_bits, float* y, int64_t B, int64_t N, int64_t K, void* workspace,
                 int64_t workspace_bytes, void* stream) {
  return linear_ws(packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, workspace, workspace_bytes, true,
                   stream);
}

int tb_linear_noalloc(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dtype,
                      const uint32_t* sign_bits, float* y, int64_t B, int64_t N, int64_t K, void* stream) {
  int64_t need = tb_linear_workspace_bytes(packing, B, N, K);
  if (need <= 0) return tb_linear(packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, stream);
  bool allow_parts = true;
  if (need > 4 * tb::kStaticScratchFloats) {
    // below the batched product's batch the array serves only speed; without room it runs as
    // tb_linear.  The batched product's partial sums, too; without room for them it takes whole
    // rows, which need x' only.
    if (B < tb::wide_min_batch(packing, N, K))
      return tb_linear(packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, stream);
    if (4 * B * K > 4 * tb::kStaticScratchFloats) return TB_ERR_SCRATCH;
    allow_parts = false;
    need = 4 * B * K;
  }
  void* scratch = nullptr;
  const hipError_t e = tb::static_scratch(&scratch);
  if (e != hipSuccess) {
    snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s (static scratch lookup)", hipGetErrorName(e),
             hipGetErrorString(e));
    return TB_ERR_HIP;
  }
  return linear_ws(packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, scratch, need, allow_parts, stream);
}

int tb_decode_chain(int packing, const tb_chain_linear* linears, int count, const void* x0, int x_dtype,
                    const uint32_t* sign_bits, int64_t K, int32_t* sync, int64_t sync_words, int spin_limit,
                    void* stream) {
  if (packing != TB_PACK_2BIT && packing != TB_PACK_BASE3) return TB_ERR_UNSUPPORTED;
  if (count < 1 || count > TB_CHAIN_MAX || K <= 0 || K % tb::kBlock != 0) return TB_ERR_SHAPE;
  if (!linears) return TB_ERR_NULL;
  for (int i = 0; i < count; ++i) {
    const int64_t n = linears[i].N;
    if (n < 1 || !fits(n, K) || (i + 1 < count && n < K)) return TB_ERR_SHAPE;
    if (!linears[i].packed || !linears[i].scales || !linears[i].y) return TB_ERR_NULL;
    if (!aligned16(linears[i].packed) || !aligned16(linears[i].scales) || !aligned16(linears[i].y))
      return TB_ERR_ALIGN;
  }
  if (x_dtype != TB_F32 && x_dtype != TB_F16 && x_dtype != TB_BF16) return TB_ERR_DTYPE;
  if (!x0 || !sign_bits || !sync) return TB_ERR_NULL;
  if (!aligned16(x0) || !aligned16(sign_bits) || !aligned16(sync)) return TB_ERR_ALIGN;
  if (sync_words < count + 2) return TB_ERR_WORKSPACE;
  if (packing != TB_PACK_BASE3 || K > 5120) return TB_ERR_UNSUPPORTED;
  if (!tb::launch_chain(linears, count, x0, x_dtype, sign_bits, int(K), sync, spin_limit > 0 ? spin_limit : 1 << 22,
                        static_cast<hipStream_t>(stream)))
    return TB_ERR_UNSUPPORTED;
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

int tb_ternarize(const float* w, int64_t N, int64_t K, const uint32_t* sign_bits, int8_t* trits,
                 uint16_t* scales, int32_t* bad_count, void* stream) {
  if (N < 0 || K <= 0 || K % tb::kBlock != 0 || !fits(N, K)) return TB_ERR_SHAPE;
  if (N == 0) return TB_OK;
  if (!w || !trits || !scales) return TB_ERR_NULL;
  if (!aligned16(w) || !aligned16(scales) || (sign_bits && !aligned16(sign_bits))) return TB_ERR_ALIGN;
  tb::launch_ternarize(w, N, K, sign_bits, trits, scales, bad_count, static_cast<hipStream_t>(stream));
  return finish_launch();
}

int tb_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words, void* stream) {
  if (bytes < 0 || bytes > kMaxElems || bytes % 16 != 0) return TB_ERR_SHAPE;
  if (bytes == 0) return TB_OK;
  if (!src || !sink) return TB_ERR_NULL;
  if (!aligned16(src) || !aligned16(sink)) return TB_ERR_ALIGN;
  if (sink_words < tb::stream_read_grid(bytes)) return TB_ERR_WORKSPACE;
  tb::launch_stream_read(static_cast<const uint8_t*>(src), bytes, sink, static_cast<hipStream_t>(stream));
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
    case TB_ERR_WORKSPACE: return "workspace smaller than tb_linear_workspace_bytes() asks for";
    case TB_ERR_SCRATCH: return "the call needs more than the library's static scratch (4 MiB: B K <= 2^20)";
    default: return "unknown status";
  }
}

const char* tb_last_hip_error(void) { return g_hip_error; }

}  // extern "C"
