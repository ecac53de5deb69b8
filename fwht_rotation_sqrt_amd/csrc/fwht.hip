// Blockwise rotation x' = H_1024 (S x) / 32 (the fixed rotated basis of the
// "Ternary Bonsai 2 27B release" page, section "How the ternary weights reach
// 1.76 bit"), evaluated as a Sylvester-ordered fast Walsh-Hadamard transform
// ("TensorSharp view of Ternary Bonsai 2 27B", sections 3.2 and 5.2).
//
// One 64-lane wave owns one 1024-element block; each lane keeps 16 values in
// registers.  The ten butterfly stages run as
//   * index bits 0..3  in registers (lane holds 16 consecutive elements),
//   * index bits 4..7  in registers after one LDS transpose,
//   * index bits 8..9  across lanes with two xor-shuffles,
// and a second LDS transpose returns the block to the contiguous layout, so
// both the load and the store are 16-byte vector accesses.  The sign flip is
// applied on the loaded values and the exact 1/32 on the stored ones.
#include "tb_internal.hpp"

namespace tb {
namespace {

constexpr int kWaves = 4;
constexpr int kLdsStride = 1088;  // 1024 values + one pad per 16 (bank spread)

template <int DT>
__device__ __forceinline__ void load16(const void* base, int64_t off, float v[16]) {
  if constexpr (DT == 0) {  // fp32
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 f = p[q];
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 u = p[q];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo = w[e] & 0xFFFFu, hi = w[e] >> 16;
        if constexpr (DT == 2) {  // bf16: the upper half of an fp32
          v[8 * q + 2 * e] = __uint_as_float(lo << 16);
          v[8 * q + 2 * e + 1] = __uint_as_float(hi << 16);
        } else {                  // fp16
          v[8 * q + 2 * e] = float(__builtin_bit_cast(_Float16, uint16_t(lo)));
          v[8 * q + 2 * e + 1] = float(__builtin_bit_cast(_Float16, uint16_t(hi)));
        }
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void store16(void* base, int64_t off, const float v[16]) {
  if constexpr (DT == 0) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else {  // fp16, round to nearest even
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo = __builtin_bit_cast(uint16_t, _Float16(v[8 * q + 2 * e]));
        uint32_t hi = __builtin_bit_cast(uint16_t, _Float16(v[8 * q + 2 * e + 1]));
        w[e] = lo | (hi << 16);
      }
      p[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Each wave transposes through its own LDS region, so a wave-level LDS fence orders the
// transposes (a workgroup barrier would also wait for the other waves and for this wave's
// outstanding global memory operations).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Butterflies over register index bits: pairs (j, j + h) for h = 1, 2, 4, 8.
__device__ __forceinline__ void butterfly16(float v[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      float a = v[j], c = v[j + h];
      v[j] = a + c;
      v[j + h] = a - c;
    }
  }
}

template <int XDT, int YDT>
__global__ __launch_bounds__(64 * kWaves) void fwht1024_kernel(const void* x, void* y,
                                                               const uint32_t* __restrict__ sign_bits,
                                                               int64_t nblocks, int blocks_per_row) {
  __shared__ float lds[kWaves][kLdsStride];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t blk = int64_t(blockIdx.x) * kWaves + wave;
  const bool active = blk < nblocks;
  const int64_t b = active ? blk : 0;  // idle waves compute on block 0 and store nothing
  const int beta = int(b % blocks_per_row);
  const int64_t off = b * kBlock + 16 * lane;
  float* L = lds[wave];

  float v[16];
  load16<XDT>(x, off, v);
  const uint32_t sw = sign_bits[beta * 32 + (lane >> 1)] >> ((lane & 1) * 16);
#pragma unroll
  for (int j = 0; j < 16; ++j)
    v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((sw >> j) & 1u) << 31));

  butterfly16(v);  // index bits 0..3

  // element i lives at L[i + i/16]; layout A: i = 16*lane + j
#pragma unroll
  for (int j = 0; j < 16; ++j) L[17 * lane + j] = v[j];
  wave_lds_sync();
  // layout B: i = (lane & 15) + 16*j + 256*(lane >> 4)
  const int bidx = (lane & 15) + 272 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = L[bidx + 17 * j];

  butterfly16(v);  // index bits 4..7

  butterfly_lane_bits_4_5(v, lane);  // index bits 8, 9 are lane bits 4, 5

  wave_lds_sync();
#pragma unroll
  for (int j = 0; j < 16; ++j) L[bidx + 17 * j] = v[j];
  wave_lds_sync();
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = L[17 * lane + j] * 0.03125f;

  if (active) store16<YDT>(y, off, v);
}

template <int XDT>
void launch_fwht_x(const void* x, void* y, int y_dt, int64_t nblocks, int bpr, const uint32_t* sb,
                   hipStream_t s) {
  const unsigned grid = unsigned((nblocks + kWaves - 1) / kWaves);
  if (y_dt == 0)
    fwht1024_kernel<XDT, 0><<<grid, 64 * kWaves, 0, s>>>(x, y, sb, nblocks, bpr);
  else
    fwht1024_kernel<XDT, 1><<<grid, 64 * kWaves, 0, s>>>(x, y, sb, nblocks, bpr);
}

}  // namespace

void launch_fwht(const void* x, int x_dt, void* y, int y_dt, int64_t rows, int64_t k,
                 const uint32_t* sign_bits, hipStream_t s) {
  const int bpr = int(k / kBlock);
  const int64_t nblocks = rows * bpr;
  if (x_dt == 0) launch_fwht_x<0>(x, y, y_dt, nblocks, bpr, sign_bits, s);
  else if (x_dt == 1) launch_fwht_x<1>(x, y, y_dt, nblocks, bpr, sign_bits, s);
  else launch_fwht_x<2>(x, y, y_dt, nblocks, bpr, sign_bits, s);
}

}  // namespace tb
