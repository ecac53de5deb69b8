// Internal launch interface between the C ABI layer (tb_api.hip) and the
// kernel translation units.  Shapes and pointers are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tb {

constexpr int kGroup = 128;          // weights per fp16 scale
constexpr int kBlock = 1024;         // rotation block size
constexpr int kB3GroupBytes = 26;    // base-3 bytes per 128-group (25 full bytes + 3 trits and 2 pads)
constexpr int kMaxBatch = 8;         // largest decode batch

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
void launch_gemm(int packing, const uint8_t* packed, const uint16_t* scales, const uint16_t* xr, float* y,
                 int m, int n, int k, hipStream_t s);
void launch_linear(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                   const uint32_t* sign_bits, float* y, int b, int n, int k, hipStream_t s);

}  // namespace tb
