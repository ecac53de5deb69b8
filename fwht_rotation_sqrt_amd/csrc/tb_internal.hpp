// Internal launch interface between the C ABI layer (tb_api.hip) and the
// kernel translation units.  Shapes and pointers are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>

#include "tb.h"
#include <stdint.h>

namespace tb {

constexpr int kGroup = 128;          // weights per fp16 scale
constexpr int kBlock = 1024;         // rotation block size
constexpr int kB3GroupBytes = 26;    // base-3 bytes per 128-group (25 full bytes + 3 trits and 2 pads)
constexpr int kMaxBatch = 8;         // largest batch of the limb decode product (gemv.hip)
// From this batch on, tb_gemv (and tb_linear_ws) run gemv_wide.hip instead of the limb kernel:
// the measured crossover (fp32 x', weights streamed from HBM).  The limb kernel's cost grows with
// B K (its limbs of x' live in LDS), the batched kernel's hardly with B, so long rows cross first.
inline int wide_min_batch(int packing, int64_t n, int64_t k) {
  if (k >= 8192) return 5;
  if (n < 8192) return 7;
  return packing == 0 ? 9 : 8;
}
// From this batch on (never past wide_min_batch), tb_linear_ws and tb_linear_noalloc rotate x into
// the workspace in fp32 and run tb_gemv's product on it (two launches) instead of the one-launch
// fused kernel, whose activation prologue grows with B K: the measured crossover on the block
// linears (K = 5120: batch 5 base-3, 6 2-bit; K = 17408: batch 2).
inline int separate_min_batch(int packing, int64_t n, int64_t k) {
  const int s = k >= 8192 ? 2 : packing == 0 ? 6 : 5;
  const int w = wide_min_batch(packing, n, k);
  return s < w ? s : w;
}
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
// The batched product; with part_y (fp32 [parts][b][n], device) and parts > 1 it takes K in parts on
// separate workgroups and then adds the parts' partial sums into y in part order (second launch).
void launch_gemv_wide(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr, int xr_dt,
                      float* y, int b, int n, int k, hipStream_t s, float* part_y = nullptr, int parts = 1);
// Parts of K for the batched product where the caller has room for partial sums (tb_linear_ws):
// each workgroup reads the activations of its whole K range, so rows too few to fill the 256
// compute units with five-tile workgroups are taken in parts of K instead of in smaller
// workgroups (each part's workgroups read only that part of the activations).  At most 8 parts
// and at least 8 groups per part; 1 where whole rows fill the units, and two parts only from
// batch 16 (below it the second launch that adds the parts cost more than two parts saved).
// Pure function of the shape.
inline int wide_parts(int64_t b, int64_t n, int64_t k) {
  constexpr int64_t kUnits = 256, kTilesPerWg = 5;
  const int64_t rb = ((n + 15) / 16 + kTilesPerWg - 1) / kTilesPerWg;
  int64_t p = rb > 0 ? kUnits / rb : 1;
  p = p < (k / kGroup) / 8 ? p : (k / kGroup) / 8;
  p = p < 8 ? p : 8;
  if (p == 2 && b < 16) p = 1;
  return p >= 2 ? int(p) : 1;
}
// y[i] = sum over parts p in order of part_y[p count + i] (fp32, device), i < count.
void launch_sum_parts(const float* part_y, float* y, int count, int parts, hipStream_t s);
void launch_gemm(int packing, const uint8_t* packed, const uint16_t* scales, const uint16_t* xr, float* y,
                 int m, int n, int k, hipStream_t s);
void launch_linear(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                   const uint32_t* sign_bits, float* y, int b, int n, int k, hipStream_t s);
void launch_ternarize(const float* w, int64_t n, int64_t k, const uint32_t* sign_bits, int8_t* trits,
                      uint16_t* scales, int32_t* bad_count, hipStream_t s);
// The static device buffer of tb_linear_noalloc (noalloc.hip): 4 MiB, x' of up to 32 rows of
// K = 32768 in fp32.  static_scratch gives the current device's address of it (looked up once
// per device).
constexpr int64_t kStaticScratchFloats = int64_t(1) << 20;
hipError_t static_scratch(void** ptr);
int stream_read_grid(int64_t bytes);
void launch_stream_read(const uint8_t* src, int64_t bytes, uint32_t* sink, hipStream_t s);
// Batch-1 base-3 decode product on independent matrix-core lane groups (decode1.hip): whether it
// takes the shape, and the launch (x is x' when rotate is false, else the unrotated x).
bool decode1_supports(int packing, int b, int n, int k);
bool launch_decode1(const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                    const uint32_t* sign_bits, bool rotate, float* y, int n, int k, hipStream_t s);
// The same product for K > 5120, the rows split into parts of at most five 1024-blocks that
// separate workgroups take: the number of parts by K alone (0 where no split applies), whether
// the launch takes the shape (the row tiles of a part fit its workgroups), and the launch, which
// writes the parts' partial sums to part_y [parts][n] (fp32, device) and then sums them into y in
// part order (a second launch).
inline int decode1_split_parts(int packing, int64_t b, int64_t k) {
  if (packing != 1 || b != 1 || k % kBlock != 0 || k <= 5 * kBlock) return 0;
  return int((k / kBlock + 4) / 5);
}
bool decode1_split_supports(int n, int k);
bool launch_decode1_split(const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                          const uint32_t* sign_bits, bool rotate, float* y, float* part_y, int n, int k,
                          hipStream_t s);
// Chained batch-1 base-3 linears in one launch (decode1.hip): false when the chain is not supported
// (count, K, or too many tiles per workgroup for a linear).
bool launch_chain(const tb_chain_linear* lin, int count, const void* x0, int x_dt, const uint32_t* sign_bits, int k,
                  int32_t* sync, int spin_limit, hipStream_t s);

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
