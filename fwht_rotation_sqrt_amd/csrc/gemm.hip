// Prefill product Y[m][n] = sum_k X'[m][k] s[n][k/128] t[n][k] on the matrix cores.
//
// First version: 64x64 output tile per 256-thread workgroup, K step 32.  The
// X' tile is copied to LDS as is; the weight tile is unpacked from 2-bit codes
// to fp16 t*s (exact) into LDS; four waves each run 2x2 v_mfma_f32_16x16x32_f16.
#include "tb_internal.hpp"

namespace tb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTM = 64, kTN = 64, kTK = 32;
constexpr int kRowChunks = kTK / 8 + 1;  // 16-byte chunks per LDS row, one of padding

__global__ __launch_bounds__(256) void gemm_tile64_kernel(const uint8_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ xr,
                                                          float* __restrict__ y, int m, int n, int k) {
  __shared__ uint4 As[kTM][kRowChunks];
  __shared__ uint4 Bs[kTN][kRowChunks];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * kTM, n0 = blockIdx.x * kTN;
  const int wm = wave >> 1, wn = wave & 1;
  const int groups = k / kGroup;
  const int row_bytes = k / 4;
  const int lr = tid >> 2, lq = tid & 3;  // loader: tile row, 8-element chunk

  floatx4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < k; k0 += kTK) {
    // X' tile: 64 rows x 32 fp16
    uint4 av = make_uint4(0, 0, 0, 0);
    if (m0 + lr < m)
      av = *reinterpret_cast<const uint4*>(xr + int64_t(m0 + lr) * k + k0 + 8 * lq);
    // weight tile: 8 codes -> 8 fp16 values t*s
    uint4 bv = make_uint4(0, 0, 0, 0);
    if (n0 + lr < n) {
      const int64_t row = n0 + lr;
      const unsigned codes = *reinterpret_cast<const uint16_t*>(packed + row * row_bytes + (k0 + 8 * lq) / 4);
      const _Float16 sc = __builtin_bit_cast(_Float16, scales[row * groups + k0 / kGroup]);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c0 = int((codes >> (4 * e)) & 3u) - 1, c1 = int((codes >> (4 * e + 2)) & 3u) - 1;
        const uint32_t lo = __builtin_bit_cast(uint16_t, _Float16(c0) * sc);
        const uint32_t hi = __builtin_bit_cast(uint16_t, _Float16(c1) * sc);
        w[e] = lo | (hi << 16);
      }
      bv = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __syncthreads();
    As[lr][lq] = av;
    Bs[lr][lq] = bv;
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const half8 af = __builtin_bit_cast(half8, As[32 * wm + 16 * a + (lane & 15)][lane >> 4]);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const half8 bf = __builtin_bit_cast(half8, Bs[32 * wn + 16 * b + (lane & 15)][lane >> 4]);
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[a][b], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = n0 + 32 * wn + 16 * b + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + 32 * wm + 16 * a + 4 * (lane >> 4) + i;
        if (r < m && col < n) y[int64_t(r) * n + col] = acc[a][b][i];
      }
    }
}

}  // namespace

void launch_gemm(const uint8_t* packed, const uint16_t* scales, const uint16_t* xr, float* y, int m,
                 int n, int k, hipStream_t s) {
  const dim3 grid(unsigned((n + kTN - 1) / kTN), unsigned((m + kTM - 1) / kTM));
  gemm_tile64_kernel<<<grid, 256, 0, s>>>(packed, scales, xr, y, m, n, k);
}

}  // namespace tb
