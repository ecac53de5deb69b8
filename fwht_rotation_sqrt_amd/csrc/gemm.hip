// Prefill product Y[m][n] = sum_k X'[m][k] s[n][k/128] t[n][k] on the matrix cores
// (2-bit codes; v_mfma_f32_16x16x32_f16, fp32 accumulation).
//
// Pages: "Ternary Bonsai 2 27B release", sections "How the ternary weights
// reach 1.76 bit" (g128 fp16 scales; the unpack is part of the product) and
// "Throughput" (pp512 prompt processing).
//
// Work split.  A workgroup of 8 waves (two per SIMD, so one wave's matrix
// work covers the other's LDS and memory waits) computes a 128 (M) x 272 (N)
// tile: 8 M-blocks x 17 N-blocks of 16 x 16 (272 = 17 x 16 makes 512 x 17408
// exactly 256 tiles, one per CU).  Wave (wm, wn) owns M-blocks 4wm..4wm+3 x
// N-blocks 4wn..4wn+3 and M-block 4wm + wn of N-block 16: 17 blocks each.
//
// Operands, per K-step of one 128-group:
//   * X' (A): the 128 x 128 fp16 tile is staged through registers into one of
//     two LDS buffers (rows padded to 272 bytes) while the previous K-step
//     computes.
//   * W (B): never stored as fp16.  Each lane loads the 8 code bytes it needs
//     (one row, 32 codes) straight from global memory; per 8 codes it makes
//     two LDS table lookups (byte -> four fp16 trits {-1, 0, +1}) and two
//     packed fp16 multiplies by the group's scale, which are exact.
//   * K order: inside a group, instruction chunk kc (32 K-slots) takes, from
//     lane group q, the eight codes 32q + 8kc .. 32q + 8kc + 7.  Slot order is
//     free as long as both operands agree, and this one gives every lane a
//     contiguous 8-byte code load and a contiguous 16-byte A read.
// The workgroup-to-tile map keeps the M-tiles that share a weight slab on one
// XCD (workgroups are handed to the 8 XCDs round robin), so the slab is read
// from HBM once per XCD L2.
#include "tb_internal.hpp"

namespace tb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kTileM = 128;                   // 8 M-blocks
constexpr int kNBlocks = 17;                  // N-blocks of 16 per tile
constexpr int kTileN = 16 * kNBlocks;         // 272
constexpr int kARowLds = 2 * kGroup + 16;     // 272 bytes: 128 fp16 + pad (16 lanes of a read in distinct banks)
constexpr int kABuf = kTileM * kARowLds;      // 34816 bytes per A buffer
constexpr int kTableBytes = 256 * 256;        // entry e at 256 e, copy c (lane & 31) at + 8 c
constexpr int kLds = kTableBytes + 2 * kABuf; // 135168
constexpr uint32_t kNoLoad = 0x80000000u;     // buffer offset past any buffer: reads zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
template <typename T, int OFF = 0>
__device__ __forceinline__ T lds_read(uint32_t addr) {
  const lds_u8* p = reinterpret_cast<const lds_u8*>(static_cast<uintptr_t>(addr)) + OFF;
  return *reinterpret_cast<__attribute__((address_space(3))) const T*>(p);
}
template <typename T, int OFF = 0>
__device__ __forceinline__ void lds_write(uint32_t addr, T v) {
  lds_u8* p = reinterpret_cast<lds_u8*>(static_cast<uintptr_t>(addr)) + OFF;
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}

// Four fp16 trits of one code byte (code i in bits 2i..2i+1, c = t + 1;
// the invalid code 3 reads as 0).
__device__ __forceinline__ u32x2 trit_halves(uint32_t byte) {
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = (byte >> (2 * i)) & 3u;
    h[i] = c == 0u ? 0xBC00u : c == 2u ? 0x3C00u : 0u;
  }
  return u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// Per-lane state of one of the wave's five decoded column blocks.
struct ColBlock {
  u32x2 codes;     // this lane's 32 codes (8 bytes) of the current group
  uint32_t s2;     // the group's fp16 scale, twice
};

// Operands of one chunk (32 K-slots) in flight: the wave's four A rows and
// the raw table entries of its five column blocks.
struct ChunkRaw {
  u32x4 a[4];
  u32x2 t[5][2];
};

// Issue the LDS reads of chunk KC: A rows (rotated order: local i = M-block
// 4wm + ((i + wn) mod 4), so the one also used with N-block 16 is local 0)
// and, per column block, the table entries of code bytes 2KC and 2KC+1 of
// the lane's 8-byte code run (address (byte << 8) | 8 * copy, by one byte
// permute).
template <int KC>
__device__ __forceinline__ void fetch(const uint32_t (&a_addr)[4], uint32_t buf, const ColBlock (&cb)[5],
                                      uint32_t tab, ChunkRaw& r) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) r.a[mb] = lds_read<u32x4, 16 * KC>(a_addr[mb] + buf);
  constexpr uint32_t sel0 = 0x0C0C0004u | (uint32_t(2 * (KC & 1)) << 8);
  constexpr uint32_t sel1 = 0x0C0C0004u | (uint32_t(2 * (KC & 1) + 1) << 8);
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    const uint32_t w = KC < 2 ? uint32_t(cb[c].codes[0]) : uint32_t(cb[c].codes[1]);
    r.t[c][0] = lds_read<u32x2>(__builtin_amdgcn_perm(tab, w, sel0));
    r.t[c][1] = lds_read<u32x2>(__builtin_amdgcn_perm(tab, w, sel1));
  }
}

// B operand of one column block: the four fp16 trit pairs times the scale
// (exact).  Vector elements go through plain integers first: a bit cast
// applied to an element expression of a vector compiles to the first element.
__device__ __forceinline__ half8 b_operand(const u32x2 (&t)[2], uint32_t s2) {
  const uint32_t d0 = t[0][0], d1 = t[0][1], d2 = t[1][0], d3 = t[1][1];
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 s = __builtin_bit_cast(h2, s2);
  const h2 p0 = __builtin_bit_cast(h2, d0) * s, p1 = __builtin_bit_cast(h2, d1) * s;
  const h2 p2 = __builtin_bit_cast(h2, d2) * s, p3 = __builtin_bit_cast(h2, d3) * s;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The 17 matrix instructions of one fetched chunk.
__device__ __forceinline__ void chunk_mma(const ChunkRaw& r, const ColBlock (&cb)[5], floatx4 (&acc)[4][4],
                                          floatx4& acc16) {
  half8 a[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) a[mb] = __builtin_bit_cast(half8, r.a[mb]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half8 b = b_operand(r.t[j], cb[j].s2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], b, acc[mb][j], 0, 0, 0);
  }
  acc16 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b_operand(r.t[4], cb[4].s2), acc16, 0, 0, 0);
}

// One K-step (one 128-group): chunk kc+1's LDS reads are issued before chunk
// kc's matrix instructions, so their latency hides behind them.
__device__ __forceinline__ void k_step(const uint32_t (&a_addr)[4], uint32_t buf, const ColBlock (&cb)[5],
                                       uint32_t tab, floatx4 (&acc)[4][4], floatx4& acc16) {
  ChunkRaw r0, r1;
  fetch<0>(a_addr, buf, cb, tab, r0);
  fetch<1>(a_addr, buf, cb, tab, r1);
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r0, cb, acc, acc16);
  __builtin_amdgcn_sched_barrier(0);
  fetch<2>(a_addr, buf, cb, tab, r0);
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r1, cb, acc, acc16);
  __builtin_amdgcn_sched_barrier(0);
  fetch<3>(a_addr, buf, cb, tab, r1);
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r0, cb, acc, acc16);
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r1, cb, acc, acc16);
}

__global__ __launch_bounds__(64 * kWaves) void gemm_t2_kernel(const uint8_t* __restrict__ packed,
                                                              const uint16_t* __restrict__ scales,
                                                              const uint16_t* __restrict__ xr,
                                                              float* __restrict__ y, int m, int n, int k,
                                                              int tiles_m, int tiles) {
  extern __shared__ __align__(16) uint8_t smem[];
  (void)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 2, wn = w & 3;
  const int nl = lane & 15, q = lane >> 4;

  // tile of this workgroup: the blocks an XCD receives (every 8th) take a
  // contiguous run of tiles, M fastest
  const int b = blockIdx.x, x = b & 7, j = b >> 3;
  const int per = tiles >> 3, extra = tiles & 7;
  const int t = x * per + min(x, extra) + j;
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int m0 = tm * kTileM, n0 = tn * kTileN;
  const int groups = k / kGroup;

  // ---- resources and per-lane addresses
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xr, uint32_t(m) * uint32_t(k) * 2u);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, uint32_t(n) * uint32_t(k / 4));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(scales, uint32_t(n) * uint32_t(groups) * 2u);
  // A staging: thread -> (row tid / 4, quarter tid % 4 of the 256-byte group row)
  const int arow = tid >> 2, aq = tid & 3;
  const uint32_t a_src = m0 + arow < m ? uint32_t((m0 + arow) * k * 2 + aq * 64) : kNoLoad;
  const uint32_t a_dst = uint32_t(kTableBytes + arow * kARowLds + aq * 64);
  // B: the lane's row in each of its five column blocks
  uint32_t w_src[5], s_src[5];
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    const int row = n0 + 16 * (c < 4 ? 4 * wn + c : 16) + nl;
    w_src[c] = row < n ? uint32_t(row * (k / 4) + 8 * q) : kNoLoad;
    s_src[c] = row < n ? uint32_t(row * groups * 2) : kNoLoad;
  }
  const uint32_t tab = uint32_t(8 * (lane & 31));
  // A operand read: row nl of each M-block (rotated order), K-slots 32q + 8kc .. of the group
  uint32_t a_addr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a_addr[i] = uint32_t(kTableBytes + (16 * (4 * wm + ((i + wn) & 3)) + nl) * kARowLds + 64 * q);

  auto load_a = [&](int g, u32x4 (&ra)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, a_src == kNoLoad ? kNoLoad : a_src + g * 256 + 16 * i, 0, 0);
  };
  auto load_b = [&](int g, ColBlock (&cb)[5]) {
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      cb[c].codes = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(wrs, w_src[c] == kNoLoad ? kNoLoad : w_src[c] + 32 * g, 0, 0));
      const uint32_t s = __builtin_amdgcn_raw_buffer_load_b16(srs, s_src[c] == kNoLoad ? kNoLoad : s_src[c] + 2 * g, 0, 0);
      cb[c].s2 = s | (s << 16);
    }
  };
  auto store_a = [&](int buf, const u32x4 (&ra)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_write<u32x4>(a_dst + buf * kABuf + 16 * i, ra[i]);
  };

  // ---- prologue: first loads, then the table while they fly
  u32x4 ra[4];
  ColBlock cur[5], nxt[5];
  load_a(0, ra);
  load_b(0, cur);
  {
    // table: thread -> entry tid / 2, half of its 32 copies
    const u32x2 v = trit_halves(uint32_t(tid >> 1));
    const uint32_t v0 = v[0], v1 = v[1];
    const u32x4 v2 = u32x4{v0, v1, v0, v1};
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_write<u32x4>(uint32_t(256 * (tid >> 1) + 128 * (tid & 1) + 16 * i), v2);
  }
  store_a(0, ra);
  if (groups > 1) {
    load_a(1, ra);
    load_b(1, nxt);
  }
  __syncthreads();

  floatx4 acc[4][4], acc16;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[mb][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  acc16 = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < groups; ++g) {
    k_step(a_addr, uint32_t((g & 1) * kABuf), cur, tab, acc, acc16);
    if (g + 1 < groups) {
      // stage K-step g+1 (its buffer was last read in iteration g-1, before
      // the previous barrier), then start the loads of K-step g+2
      store_a((g + 1) & 1, ra);
#pragma unroll
      for (int c = 0; c < 5; ++c) cur[c] = nxt[c];
      if (g + 2 < groups) {
        load_a(g + 2, ra);
        load_b(g + 2, nxt);
      }
    }
    __syncthreads();
  }

  // ---- store: lane holds rows 4q..4q+3 of column nl of each block
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = n0 + 16 * (4 * wn + c) + nl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * (4 * wm + ((mb + wn) & 3)) + 4 * q + i;
        if (row < m && col < n) y[int64_t(row) * n + col] = acc[mb][c][i];
      }
    }
  {
    const int col = n0 + 16 * 16 + nl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 16 * (4 * wm + wn) + 4 * q + i;
      if (row < m && col < n) y[int64_t(row) * n + col] = acc16[i];
    }
  }
}

}  // namespace

void launch_gemm(const uint8_t* packed, const uint16_t* scales, const uint16_t* xr, float* y, int m,
                 int n, int k, hipStream_t s) {
  static bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_t2_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    return true;
  }();
  (void)attr;
  const int tiles_m = (m + kTileM - 1) / kTileM, tiles_n = (n + kTileN - 1) / kTileN;
  const int tiles = tiles_m * tiles_n;
  gemm_t2_kernel<<<dim3(unsigned(tiles)), dim3(64 * kWaves), kLds, s>>>(packed, scales, xr, y, m, n, k, tiles_m,
                                                                       tiles);
}

}  // namespace tb
