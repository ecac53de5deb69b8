// Packing and unpacking of ternary weights (offline path).
//
// 2-bit: code c = t + 1 in bits 2(k%4).. of byte k/4 (00 = -1, 01 = 0, 10 = +1).
// base-3: "Bonsai low-bit learning path", section "Understand 1.6 bit with five
// numbers": byte = sum_i (t_i + 1) 3^i over five consecutive trits, first trit
// least significant; decoded by (byte / 3^i) % 3 - 1.  Every 128-weight group
// takes 26 bytes, the last one holding three trits and two pad trits of value 0.
//
// One thread per packed byte; rows are contiguous, so a flat byte index maps
// to (row, byte-in-row) without gaps.
#include "tb_internal.hpp"

namespace tb {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int valid_trit(int t) { return t >= -1 && t <= 1; }

__global__ __launch_bounds__(kThreads) void pack2_kernel(const int8_t* __restrict__ trits,
                                                         uint8_t* __restrict__ packed,
                                                         int64_t nbytes, int32_t* bad) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nbytes) return;
  const int8_t* t = trits + 4 * i;
  unsigned byte = 0;
  int nbad = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int v = t[j];
    int ok = valid_trit(v);
    nbad += !ok;
    byte |= unsigned(ok ? v + 1 : 1) << (2 * j);
  }
  packed[i] = uint8_t(byte);
  if (nbad && bad) atomicAdd(bad, nbad);
}

__global__ __launch_bounds__(kThreads) void pack3_kernel(const int8_t* __restrict__ trits,
                                                         uint8_t* __restrict__ packed,
                                                         int64_t nbytes, int k, int32_t* bad) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nbytes) return;
  const int row_bytes = kB3GroupBytes * (k / kGroup);
  const int64_t row = i / row_bytes;
  const int in_row = int(i - row * row_bytes);
  const int g = in_row / kB3GroupBytes;
  const int p = in_row - g * kB3GroupBytes;
  const int8_t* t = trits + row * k + g * kGroup + 5 * p;
  const int real = p < kB3GroupBytes - 1 ? 5 : 3;
  unsigned byte = 0, pow3 = 1;
  int nbad = 0;
  for (int j = 0; j < 5; ++j) {
    int d = 1;  // pad trit 0
    if (j < real) {
      int v = t[j];
      int ok = valid_trit(v);
      nbad += !ok;
      d = ok ? v + 1 : 1;
    }
    byte += unsigned(d) * pow3;
    pow3 *= 3;
  }
  packed[i] = uint8_t(byte);
  if (nbad && bad) atomicAdd(bad, nbad);
}

__global__ __launch_bounds__(kThreads) void unpack2_kernel(const uint8_t* __restrict__ packed,
                                                           int8_t* __restrict__ trits,
                                                           int64_t nbytes, int32_t* bad) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nbytes) return;
  const unsigned byte = packed[i];
  int nbad = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int c = (byte >> (2 * j)) & 3;
    nbad += c == 3;
    trits[4 * i + j] = int8_t(c == 3 ? 0 : c - 1);
  }
  if (nbad && bad) atomicAdd(bad, nbad);
}

__global__ __launch_bounds__(kThreads) void unpack3_kernel(const uint8_t* __restrict__ packed,
                                                           int8_t* __restrict__ trits,
                                                           int64_t nbytes, int k, int32_t* bad) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nbytes) return;
  const int row_bytes = kB3GroupBytes * (k / kGroup);
  const int64_t row = i / row_bytes;
  const int in_row = int(i - row * row_bytes);
  const int g = in_row / kB3GroupBytes;
  const int p = in_row - g * kB3GroupBytes;
  int8_t* t = trits + row * k + g * kGroup + 5 * p;
  const unsigned byte = packed[i];
  const bool over = byte >= 243;
  int digits[5];
  unsigned rest = byte;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    digits[j] = int(rest % 3u);
    rest /= 3u;
  }
  const int real = p < kB3GroupBytes - 1 ? 5 : 3;
  for (int j = 0; j < real; ++j) t[j] = int8_t(over ? 0 : digits[j] - 1);
  int nbad = over;
  if (!over && real == 3 && (digits[3] != 1 || digits[4] != 1)) nbad = 1;
  if (nbad && bad) atomicAdd(bad, nbad);
}

unsigned blocks_for(int64_t n) { return unsigned((n + kThreads - 1) / kThreads); }

}  // namespace

void launch_pack_2bit(const int8_t* trits, int64_t n, int64_t k, uint8_t* packed, int32_t* bad,
                      hipStream_t s) {
  const int64_t nbytes = n * (k / 4);
  pack2_kernel<<<blocks_for(nbytes), kThreads, 0, s>>>(trits, packed, nbytes, bad);
}

void launch_pack_base3(const int8_t* trits, int64_t n, int64_t k, uint8_t* packed, int32_t* bad,
                       hipStream_t s) {
  const int64_t nbytes = n * kB3GroupBytes * (k / kGroup);
  pack3_kernel<<<blocks_for(nbytes), kThreads, 0, s>>>(trits, packed, nbytes, int(k), bad);
}

void launch_unpack(int packing, const uint8_t* packed, int64_t n, int64_t k, int8_t* trits,
                   int32_t* bad, hipStream_t s) {
  if (packing == 0) {
    const int64_t nbytes = n * (k / 4);
    unpack2_kernel<<<blocks_for(nbytes), kThreads, 0, s>>>(packed, trits, nbytes, bad);
  } else {
    const int64_t nbytes = n * kB3GroupBytes * (k / kGroup);
    unpack3_kernel<<<blocks_for(nbytes), kThreads, 0, s>>>(packed, trits, nbytes, int(k), bad);
  }
}

}  // namespace tb
