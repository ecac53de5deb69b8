// Read-only HBM stream: the measured ceiling that the weight-streaming products
// are compared with.  Every byte of the buffer is read once with 16-byte buffer
// loads, four in flight per lane (one launch over 19.5 MB: 5.2 us with four, 5.4
// with eight, 5.2 with two, 5.5 with one; over 2 GB four is also the fastest); a workgroup folds what it read into one XOR
// word and writes it, so the reads cannot be dropped and the writes are
// negligible (4 bytes per 16 KB read).
#include "tb_internal.hpp"

namespace tb {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                                   // 16-byte loads in flight per lane
constexpr uint32_t kChunk = uint32_t(kThreads) * kUnroll * 16;  // bytes per workgroup pass: 16 KB
constexpr int kMaxGrid = 8192;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint8_t* __restrict__ src, uint32_t bytes,
                                                               uint32_t* __restrict__ sink, uint32_t chunks,
                                                               uint32_t grid) {
  // offsets past `bytes` read zero (raw buffer bounds), so the tail needs no branch
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), short(0), int(bytes), 0x00020000);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t c = blockIdx.x; c < chunks; c += grid) {
    const uint32_t base = c * kChunk + 16u * threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + uint32_t(i) * kThreads * 16u, 0, 0);
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) acc ^= v[i];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= uint32_t(__shfl_xor(int(x), o));
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

int stream_read_grid(int64_t bytes) {
  const int64_t chunks = (bytes + kChunk - 1) / kChunk;
  return int(chunks < kMaxGrid ? chunks : kMaxGrid);
}

void launch_stream_read(const uint8_t* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const uint32_t chunks = uint32_t((bytes + kChunk - 1) / kChunk);
  const uint32_t grid = uint32_t(stream_read_grid(bytes));
  stream_read_kernel<<<grid, kThreads, 0, s>>>(src, uint32_t(bytes), sink, chunks, grid);
}

}  // namespace tb
