// Prefill product Y[m][n] = sum_k X'[m][k] s[n][k/128] t[n][k] on the matrix cores
// (2-bit codes or base-3 bytes; v_mfma_f32_16x16x32_f16, fp32 accumulation).
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
//   * W (B): never stored as fp16.  The tile's 272 rows x 32 code bytes of a
//     group are loaded once per workgroup (two threads per row, coalesced)
//     and staged in LDS, as are the scales, 8 groups at a time; a load
//     instruction that served one wave's 16 rows instead would touch 16
//     cache lines for 32 bytes each, and the other waves would repeat it.
//     Each lane reads its 8 code bytes and its scale one K-step ahead; per 8
//     codes it makes two LDS table lookups (byte -> four fp16 trits
//     {-1, 0, +1}) and two packed fp16 multiplies by the scale, which are
//     exact.
//   * K order: inside a group, instruction chunk kc (32 K-slots) takes, from
//     lane group q, the eight codes 32q + 8kc .. 32q + 8kc + 7.  Slot order is
//     free as long as both operands agree, and this one gives every lane a
//     contiguous 8-byte code read and a contiguous 16-byte A read.
// Base-3 weights (26 bytes per row and group, five trits per byte, least
// significant digit first, digit = t + 1) are turned into the same 2-bit codes
// on their way into LDS: the digits of a byte are exactly the codes of its
// five weights, so one lookup per byte (byte -> the five codes as a 10-bit
// field) and shifts assemble a row's 32 code bytes (the last byte's two pad
// trits are dropped).  Everything after the code buffers is shared.
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
// decode table: entry e at 256 e.  2-bit codes: 32 copies of the fp16 trits,
// copy c (lane & 31) at + 8 c.  Base-3: 16 copies of the fp16 trits at + 8 c
// (c = lane & 15), then 32 copies of the byte's five codes at + 128 + 4 c.
constexpr int kTableBytes = 256 * 256;
constexpr int kCodeRow = kGroup / 4;          // 32 code bytes per row and group
constexpr int kCBuf = kTileN * kCodeRow;      // 8704 bytes per code buffer
constexpr int kSChunk = 8;                    // groups per staged scale chunk
constexpr int kSBuf = kTileN * kSChunk * 2;   // 4352 bytes per scale buffer
constexpr int kAOff = kTableBytes;            // two A buffers
constexpr int kCOff = kAOff + 2 * kABuf;      // two code buffers
constexpr int kSOff = kCOff + 2 * kCBuf;      // two scale buffers
constexpr int kLds = kSOff + 2 * kSBuf;       // 161280 of the 163840 a workgroup may hold
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

// The five base-3 digits of a byte (value sum d_i 3^i, d_i = t_i + 1) as a
// 10-bit field of 2-bit codes, digit i at bits 2i..2i+1.  Bytes >= 243 are
// invalid; they map to code 01 (zero) throughout.
__device__ __forceinline__ uint32_t base3_codes(uint32_t byte) {
  if (byte >= 243u) return 0x155u;
  uint32_t f = 0, v = byte;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    f |= (v % 3u) << (2 * i);
    v /= 3u;
  }
  return f;
}

// Per-lane B inputs of one K-step in one of the wave's five column blocks.
struct ColBlock {
  u32x2 codes;     // this lane's 32 codes (8 bytes) of the group
  uint32_t s;      // the group's fp16 scale (low half)
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
__device__ __forceinline__ void chunk_mma(const ChunkRaw& r, const uint32_t (&s2)[5], floatx4 (&acc)[4][4],
                                          floatx4& acc16) {
  half8 a[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) a[mb] = __builtin_bit_cast(half8, r.a[mb]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half8 b = b_operand(r.t[j], s2[j]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], b, acc[mb][j], 0, 0, 0);
  }
  acc16 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b_operand(r.t[4], s2[4]), acc16, 0, 0, 0);
}

// One K-step (one 128-group): chunk kc+1's LDS reads are issued before chunk
// kc's matrix instructions, so their latency hides behind them.  `mid` (the
// staging of later steps' operands) runs after the second chunk's matrix
// instructions are issued, so it overlaps them; `ahead` issues the reads of
// the next K-step's codes and scales, after this step's own reads.
template <typename Mid, typename Ahead>
__device__ __forceinline__ void k_step(const uint32_t (&a_addr)[4], uint32_t buf, const ColBlock (&cb)[5],
                                       uint32_t tab, floatx4 (&acc)[4][4], floatx4& acc16, Mid&& mid, Ahead&& ahead) {
  uint32_t s2[5];
#pragma unroll
  for (int c = 0; c < 5; ++c) s2[c] = cb[c].s * 0x10001u;
  ChunkRaw r0, r1;
  fetch<0>(a_addr, buf, cb, tab, r0);
  fetch<1>(a_addr, buf, cb, tab, r1);
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r0, s2, acc, acc16);
  __builtin_amdgcn_sched_barrier(0);
  fetch<2>(a_addr, buf, cb, tab, r0);
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r1, s2, acc, acc16);
  __builtin_amdgcn_sched_barrier(0);
  mid();
  __builtin_amdgcn_sched_barrier(0);
  fetch<3>(a_addr, buf, cb, tab, r1);
  ahead();
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r0, s2, acc, acc16);
  __builtin_amdgcn_sched_barrier(0);
  chunk_mma(r1, s2, acc, acc16);
}

template <int PACK>
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
  const uint32_t row_bytes = PACK == 0 ? uint32_t(k / 4) : uint32_t(kB3GroupBytes * groups);
  const uint32_t group_bytes = PACK == 0 ? uint32_t(kCodeRow) : uint32_t(kB3GroupBytes);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, uint32_t(n) * row_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(scales, uint32_t(n) * uint32_t(groups) * 2u);
  // A staging: load i takes rows 32 i .. 32 i + 31, sixteen threads per
  // 256-byte group row (a wave reads 4 whole rows, 8 full cache lines)
  // (load i reads 32 i rows past load 0: one register holds the source of all four)
  const int arow = tid >> 4, apiece = tid & 15;
  const uint32_t a_src = uint32_t((m0 + arow) * k * 2 + apiece * 16);
  const uint32_t a_dst = uint32_t(kAOff + arow * kARowLds + apiece * 16);
  // code staging, 544 16-byte pieces per group; thread tid takes piece tid,
  // and the first 32 threads also piece 512 + tid.
  //   2-bit: piece p = row p / 2, bytes 16 (p % 2) .. of the row's 32.
  //   base-3: piece p < 272 = bytes 0..15 of row p (-> codes 0..79, code
  //   bytes 0..19); piece p >= 272 = bytes 10..25 of row p - 272, of which
  //   bytes 16..25 give codes 80..127 (code bytes 20..31).
  constexpr int kPieces2 = 2 * kTileN - 64 * kWaves;   // 32
  const bool two_pieces = tid < kPieces2;
  uint32_t c_src[2], c_dst[2];
  bool c_hi[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pc = tid + 64 * kWaves * i;
    const bool hi = PACK == 0 ? (pc & 1) != 0 : pc >= kTileN;
    const int lrow = PACK == 0 ? pc >> 1 : (hi ? pc - kTileN : pc), row = n0 + lrow;
    const uint32_t off = PACK == 0 ? 16u * hi : 10u * hi;
    c_src[i] = (i == 0 || two_pieces) && row < n ? uint32_t(row) * row_bytes + off : kNoLoad;
    c_dst[i] = uint32_t(kCOff + lrow * kCodeRow + (PACK == 0 ? 16 : 20) * hi);
    c_hi[i] = hi;
  }
  const uint32_t tabc = uint32_t(128 + 4 * (lane & 31));   // base-3 code-field copy of this lane
  // scale staging: element e = tid + 512 i of a 272 x 8 chunk: row e / 8,
  // group 8 chunk + e % 8 (eight threads read a row's 16 contiguous bytes)
  constexpr int kSElems = kTileN * kSChunk;             // 2176
  const int sj = tid & 7;
  const uint32_t s_dst = uint32_t(kSOff + tid * 2);     // element e sits at 2 e
  // per-lane reads: row nl of each column block, code bytes 8q .. 8q + 7
  const uint32_t code_rd = uint32_t(kCOff + (64 * wn + nl) * kCodeRow + 8 * q);
  const uint32_t code_rd16 = uint32_t(kCOff + (256 + nl) * kCodeRow + 8 * q);
  const uint32_t scale_rd = uint32_t(kSOff + (64 * wn + nl) * kSChunk * 2);
  const uint32_t scale_rd16 = uint32_t(kSOff + (256 + nl) * kSChunk * 2);
  const uint32_t tab = uint32_t(8 * (lane & (PACK == 0 ? 31 : 15)));
  // A operand read: row nl of each M-block (rotated order), K-slots 32q + 8kc .. of the group
  uint32_t a_addr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a_addr[i] = uint32_t(kAOff + (16 * (4 * wm + ((i + wn) & 3)) + nl) * kARowLds + 64 * q);

  // Loads of a group past the end read zeros (offset outside the buffer).
  auto load_a = [&](int g, u32x4 (&ra)[4]) {
    const bool live = g < groups;
    uint32_t src = a_src;
    asm volatile("" : "+v"(src));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(
          xrs, live && m0 + arow + 32 * i < m ? src + uint32_t(64 * i * k + g * 256) : kNoLoad, 0, 0);
  };
  auto store_a = [&](int buf, const u32x4 (&ra)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_write<u32x4>(a_dst + buf * kABuf + 32 * kARowLds * i, ra[i]);
  };
  auto load_codes = [&](int g, u32x4 (&rc)[2]) {
    const bool live = g < groups;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rc[i] = __builtin_amdgcn_raw_buffer_load_b128(
          wrs, c_src[i] == kNoLoad || !live ? kNoLoad : c_src[i] + g * group_bytes, 0, 0);
  };
  // base-3 piece -> code dwords: the 10-bit code field of byte j lands at bit
  // 10 (j - J0) of the piece's code run
  auto b3_field = [&](const u32x4& v, int j) -> uint32_t {
    const uint32_t w = v[j >> 2];
    return lds_read<uint32_t>(__builtin_amdgcn_perm(tabc, w, 0x0C0C0004u | (uint32_t(j & 3) << 8)));
  };
  auto store_piece = [&](uint32_t dst, const u32x4& v, bool hi) {
    if constexpr (PACK == 0) {
      lds_write<u32x4>(dst, v);
    } else if (!hi) {
      uint32_t o[5] = {0, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t f = b3_field(v, j);
        const int bit = 10 * j;
        o[bit >> 5] |= f << (bit & 31);
        if ((bit & 31) > 22) o[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
      }
      lds_write<u32x4>(dst, u32x4{o[0], o[1], o[2], o[3]});
      lds_write<uint32_t>(dst + 16, o[4]);
    } else {
      uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 6; j < 16; ++j) {
        const uint32_t f = b3_field(v, j);
        const int bit = 10 * (j - 6);
        o[bit >> 5] |= f << (bit & 31);
        if ((bit & 31) > 22) o[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
      }
      // bits 96..99 are the group's two pad trits
      lds_write<uint32_t>(dst, o[0]);
      lds_write<u32x2>(dst + 4, u32x2{o[1], o[2]});
    }
  };
  auto store_codes = [&](int buf, const u32x4 (&rc)[2]) {
    store_piece(c_dst[0] + buf * kCBuf, rc[0], c_hi[0]);
    if (two_pieces) store_piece(c_dst[1] + buf * kCBuf, rc[1], c_hi[1]);
  };
  // element tid + 512 i sits at row n0 + tid / 8 + 64 i: its source is the first element's plus i
  // strides of 64 scale rows, so one register serves all five (made opaque at each use: otherwise
  // the compiler keeps five loop-invariant offsets live across the K loop and spills)
  const uint32_t s_src = uint32_t(((n0 + (tid >> 3)) * groups + sj) * 2);
  auto load_scales = [&](int chunk, uint32_t (&rs)[5]) {
    const bool live = kSChunk * chunk + sj < groups;
    uint32_t src = s_src;
    asm volatile("" : "+v"(src));
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int e = tid + 64 * kWaves * i, row = n0 + (e >> 3);
      rs[i] = __builtin_amdgcn_raw_buffer_load_b16(
          srs, live && e < kSElems && row < n ? src + uint32_t((64 * i * groups + kSChunk * chunk) * 2) : kNoLoad, 0, 0);
    }
  };
  auto store_scales = [&](int buf, const uint32_t (&rs)[5]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_write<uint16_t>(s_dst + buf * kSBuf + 64 * kWaves * 2 * i, uint16_t(rs[i]));
    if (tid + 64 * kWaves * 4 < kSElems) lds_write<uint16_t>(s_dst + buf * kSBuf + 64 * kWaves * 2 * 4, uint16_t(rs[4]));
  };
  // this lane's codes and scales of K-step g (code buffer g % 2, scale
  // buffer (g / 8) % 2)
  auto read_b = [&](int g, ColBlock (&cb)[5]) {
    const uint32_t cbuf = uint32_t(g & 1) * kCBuf;
    const uint32_t sbuf = uint32_t((g / kSChunk) & 1) * kSBuf + uint32_t(g % kSChunk) * 2;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      cb[c].codes = lds_read<u32x2>(code_rd + cbuf + c * 16 * kCodeRow);
      cb[c].s = lds_read<uint16_t>(scale_rd + sbuf + c * 16 * kSChunk * 2);
    }
    cb[4].codes = lds_read<u32x2>(code_rd16 + cbuf);
    cb[4].s = lds_read<uint16_t>(scale_rd16 + sbuf);
  };

  // ---- prologue: first loads, then the table while they fly.  K-step g
  // takes A from buffer g % 2 (staged at the end of step g - 1), its codes
  // and scales from registers read at the top of step g - 1; even steps keep
  // them in bA, odd ones in bB.
  u32x4 ra[4], rc[2];
  uint32_t rs[5];
  load_scales(0, rs);
  load_a(0, ra);
  load_codes(0, rc);
  {
    // table: thread -> entry tid / 2, one 128-byte half of it (2-bit: 16 of
    // the 32 fp16 copies; base-3: the 16 fp16 copies, or the 32 code fields)
    const u32x2 v = trit_halves(uint32_t(tid >> 1));
    const uint32_t v0 = v[0], v1 = v[1];
    u32x4 v2 = u32x4{v0, v1, v0, v1};
    if (PACK == 1 && (tid & 1)) {
      const uint32_t f = base3_codes(uint32_t(tid >> 1));
      v2 = u32x4{f, f, f, f};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_write<u32x4>(uint32_t(256 * (tid >> 1) + 128 * (tid & 1) + 16 * i), v2);
  }
  store_scales(0, rs);
  store_a(0, ra);
  if constexpr (PACK == 1) __syncthreads();   // the code-field table is read by the conversion
  store_codes(0, rc);
  load_a(1, ra);
  load_codes(1, rc);
  store_codes(1, rc);
  load_codes(2, rc);
  __syncthreads();
  ColBlock bA[5], bB[5];
  read_b(0, bA);
  // step 0 rewrites code buffer 0: every wave's reads of it come first
  __syncthreads();

  floatx4 acc[4][4], acc16;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[mb][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  acc16 = floatx4{0.f, 0.f, 0.f, 0.f};

  // Step g, p = g % 2.  After its matrix work it stages A of step g + 1
  // (buffer p ^ 1, last read in step g - 1), codes of step g + 2 (code
  // buffer p, last read at the top of step g - 1) and, every 8 steps, the
  // next scale chunk, then starts the loads for later steps.  The barrier
  // orders LDS traffic only: the loads in flight target registers, so it
  // waits for the LDS counter, not the memory one.
  // The staging goes in the middle of the step: A buffer p ^ 1 was last read in step g - 1, code
  // buffer p at the top of step g - 1, and the scale buffer it may write is not the one that
  // read_b(g + 1) reads, so every wave is done with what it overwrites once barrier g - 1 passed.
  auto step = [&](int g, uint32_t p, const ColBlock (&cb)[5], ColBlock (&nb)[5]) {
    k_step(a_addr, p * uint32_t(kABuf), cb, tab, acc, acc16,
           [&] {
             store_a(int(p ^ 1u), ra);
             store_codes(int(p), rc);
             if (((g + 2) % kSChunk) == 0) store_scales(((g + 2) / kSChunk) & 1, rs);
             load_a(g + 2, ra);
             load_codes(g + 3, rc);
             if (((g + 3) % kSChunk) == 0) load_scales((g + 3) / kSChunk, rs);
           },
           [&] { read_b(g + 1, nb); });
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  int g = 0;
  for (; g + 1 < groups; g += 2) {
    step(g, 0u, bA, bB);
    step(g + 1, 1u, bB, bA);
  }
  if (g < groups) step(g, 0u, bA, bB);

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

template <int PACK>
void launch_pack(const uint8_t* packed, const uint16_t* scales, const uint16_t* xr, float* y, int m, int n, int k,
                 hipStream_t s) {
  static bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_t2_kernel<PACK>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    return true;
  }();
  (void)attr;
  const int tiles_m = (m + kTileM - 1) / kTileM, tiles_n = (n + kTileN - 1) / kTileN;
  const int tiles = tiles_m * tiles_n;
  gemm_t2_kernel<PACK><<<dim3(unsigned(tiles)), dim3(64 * kWaves), kLds, s>>>(packed, scales, xr, y, m, n, k,
                                                                             tiles_m, tiles);
}

void launch_gemm(int packing, const uint8_t* packed, const uint16_t* scales, const uint16_t* xr, float* y, int m,
                 int n, int k, hipStream_t s) {
  if (packing == 0) launch_pack<0>(packed, scales, xr, y, m, n, k, s);
  else launch_pack<1>(packed, scales, xr, y, m, n, k, s);
}

}  // namespace tb
