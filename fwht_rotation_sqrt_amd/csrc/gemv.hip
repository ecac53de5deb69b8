// Decode product y[b][n] = sum_g s[n][g] sum_{k in g} t[n][k] xr[b][k].
//
// First version: one wave per output row, lanes stride over the row's packed
// bytes, trits are decoded in registers and multiplied in fp32.
#include "tb_internal.hpp"

namespace tb {
namespace {

constexpr int kWaves = 4;

template <int XDT>
__device__ __forceinline__ float ldx(const void* xr, int64_t i) {
  if constexpr (XDT == 0) return static_cast<const float*>(xr)[i];
  else return float(__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(xr)[i]));
}

template <int PACK, int XDT>
__global__ __launch_bounds__(64 * kWaves) void gemv_rowwave_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const void* __restrict__ xr, float* __restrict__ y, int nb, int n, int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + wave;
  if (row >= n) return;
  const int groups = k / kGroup;
  const int row_bytes = PACK == 0 ? k / 4 : kB3GroupBytes * groups;
  const uint8_t* p = packed + int64_t(row) * row_bytes;
  const uint16_t* s = scales + int64_t(row) * groups;
  float acc[kMaxBatch];
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) acc[b] = 0.f;

  for (int j = lane; j < row_bytes; j += 64) {
    const unsigned byte = p[j];
    int t[5], k0, cnt, g;
    if constexpr (PACK == 0) {
      k0 = 4 * j;
      cnt = 4;
      g = k0 / kGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = int((byte >> (2 * i)) & 3u) - 1;
      t[4] = 0;
    } else {
      g = j / kB3GroupBytes;
      const int q = j - g * kB3GroupBytes;
      k0 = g * kGroup + 5 * q;
      cnt = q < kB3GroupBytes - 1 ? 5 : 3;
      unsigned rest = byte;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        t[i] = int(rest % 3u) - 1;
        rest /= 3u;
      }
    }
    const float sc = float(__builtin_bit_cast(_Float16, s[g]));
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b >= nb) break;
      float d = 0.f;
      for (int i = 0; i < cnt; ++i) d += float(t[i]) * ldx<XDT>(xr, int64_t(b) * k + k0 + i);
      acc[b] += sc * d;
    }
  }
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) {
    float v = acc[b];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0 && b < nb) y[int64_t(b) * n + row] = v;
  }
}

}  // namespace

void launch_gemv(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr,
                 int xr_dt, float* y, int b, int n, int k, hipStream_t s) {
  const unsigned grid = unsigned((n + kWaves - 1) / kWaves);
  const dim3 block(64 * kWaves);
  if (packing == 0) {
    if (xr_dt == 0) gemv_rowwave_kernel<0, 0><<<grid, block, 0, s>>>(packed, scales, xr, y, b, n, k);
    else gemv_rowwave_kernel<0, 1><<<grid, block, 0, s>>>(packed, scales, xr, y, b, n, k);
  } else {
    if (xr_dt == 0) gemv_rowwave_kernel<1, 0><<<grid, block, 0, s>>>(packed, scales, xr, y, b, n, k);
    else gemv_rowwave_kernel<1, 1><<<grid, block, 0, s>>>(packed, scales, xr, y, b, n, k);
  }
}

}  // namespace tb
