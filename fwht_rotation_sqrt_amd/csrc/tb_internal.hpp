// Internal launch interface between the C ABI layer (tb_api.hip) and the
// kernel translation units.  Shapes and pointers are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tb {

constexpr int kGroup = 128;          // weights per fp16 scale
constexpr int kBlock = 1024;         // rotation block size
constexpr int kB3GroupBytes = 26;    // base-3 bytes per 128-group (25 full bytes + 3 trits and 2 pads)
constexpr int kMaxBatch = 8;         // largest batch of the limb decode product (gemv.hip)
constexpr int kWideMinBatch = 9;     // from this batch on, tb_gemv runs gemv_wide.hip
constexpr int kWideMaxBatch = 32;    // largest batch of gemv_wide.hip
constexpr int kWideGemmRows = 96;    // tb_gemm up to this M runs gemv_wide.hip in chunks of 32 rows

void launch_pack_2bit(const int8_t* trits, int64_t n, int64_t k, uint8_t* packed, int32_t* bad,
                      hipStream_t s);
void launch_pack_base3(const int8_t* trits, int64_t n, int64_t k, uint8_t* packed, int32_t* bad,
                       hipStream_t s);
void launch_unpack(int packing, const uint8_t* packed, int64_t n, int64_t k, int8_t* trits,
                   int32_t* bad, hipStream_t s);
void launch_fwht(const void* x, int x_dt, void* y, int y_dt, int64_t rows, int64_t k,
                 const uint32_t* sign_bits, hipStream_t s);
void launch_gemv(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr,
                 int xr_dt, float* y, int b, int n, int k, hipStream_t s);
void launch_gemv_wide(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr, int xr_dt,
                      float* y, int b, int n, int k, hipStream_t s);
void launch_gemm(int packing, const uint8_t* packed, const uint16_t* scales, const uint16_t* xr, float* y,
                 int m, int n, int k, hipStream_t s);
void launch_linear(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                   const uint32_t* sign_bits, float* y, int b, int n, int k, hipStream_t s);

// Walsh-Hadamard butterflies across lane bits 4 and 5 of a wave (partner
// lane l ^ 16, then l ^ 32), for 16 values per lane: the lane whose bit is 0
// keeps own + partner, the other partner - own.  The permlane swaps are
// VALU operations (no LDS round trip).  With both operands the same value, a
// swap returns (own, partner) in lanes whose bit is 0 and (partner, own) in
// the others, so one fused multiply-add by +-1 (exact: a single rounding of
// the sum or difference) finishes each butterfly.
__device__ __forceinline__ void butterfly_lane_bits_4_5(float (&v)[16], int lane) {
  const float s16 = (lane & 16) ? -1.f : 1.f, s32 = (lane & 32) ? -1.f : 1.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t u = __float_as_uint(v[j]);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v[j] = fmaf(s16, __uint_as_float(p[1]), __uint_as_float(p[0]));
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t u = __float_as_uint(v[j]);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v[j] = fmaf(s32, __uint_as_float(p[1]), __uint_as_float(p[0]));
  }
}

}  // namespace tb
