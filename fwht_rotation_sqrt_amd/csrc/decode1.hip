// Decode product at batch 1 for base-3 weights, y[n] = sum_g s[n][g] sum_{k in g} t[n][k] x'[k],
// optionally with the rotation x' = R_K x done in the prologue (the decode linear of tb_linear).
//
// Pages: "Ternary Bonsai 2 27B release" (linlog.top/article/1481), section "How the ternary
// weights reach 1.76 bit" (g128 fp16 scales, unpack and scale inside the product, f(x) = W(Rx)
// with R = H_1024 S / 32 blockwise) and section "Throughput" (decode streams the packed weights
// once per token); "Bonsai low-bit learning path", section "Understand 1.6 bit with five numbers"
// (byte = sum_i (t_i + 1) 3^i, five trits per byte).
//
// Design (gfx950, one workgroup per compute unit):
//  * Streaming.  A wave owns one tile of 16 weight rows and the whole of K.  Each lane loads its
//    share of the tile (its codes and scales, about 280 bytes at K = 5120) into registers: the
//    scales and the first 64-byte chunk when the kernel starts, then the next chunk each time the
//    matrix loop reaches a chunk, so the weight stream starts at launch and the activation
//    prologue runs while the first loads are outstanding.
//  * Matrix cores.  v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 (e2m1) weights and fp6 (e2m3)
//    activations.  Its four lane groups (16 lanes each, one per 32 K-slots) are made independent:
//    A row 4q + j (j = 0..3) carries data only in the K-slots of lane group q (the other lanes of
//    that row read a zero record), so result rows 4q .. 4q + 3, which lane group q holds, see only
//    lane group q's weights.  Lane group q of a wave walks its own quarter of K (G4 = K/512
//    groups), so one instruction advances four groups of one tile at once.
//  * Sparse slots.  A code byte takes 8 K-slots: its five trits, then three empty slots.  One LDS
//    lookup (243 entries, 32 bank-spread copies, 256-byte stride so one byte permute forms the
//    address) turns a byte into the nibble dword of its trits, with no shifting or merging, and a
//    lane's 4-byte code dword is one B operand.  A 26-byte group takes seven 4-byte steps; an odd
//    group of a lane starts 2 bytes into a dword, so the dword holding the end of one group and
//    the start of the next is used by both groups, each with its own A data.
//  * Activations.  x' is split per (group, step) into four fp6 limbs, x' ~ sum_j v_j 2^(E - 4j),
//    each the round-to-nearest of what the previous limbs left (exact residuals through the
//    hardware conversions), so the absolute error is at most about 2^-16 of the largest |x'| of
//    the step's 20 activations.  The limb exponent rides in the instruction's E8M0 A scale, so
//    the four result rows of a lane add up to the group's partial sum with no multiply.
//  * Records.  A record (group, step) holds the four limbs (24 bytes each); each limb carries its
//    own E8M0 scale code in K-slots 5 and 6 (bits 30..37), which face the empty nibbles of every
//    weight operand and so add nothing, so a lane reads its limb as 16 + 8 bytes and takes the
//    scale with one funnel shift.  Records live in the upper half of a table entry slot (table
//    entry i at 256 i, record i at 256 i + 128), so table and records share one 256-byte-stride
//    region.
//    256 i + 128), so table and records share one 256-byte-stride region.
#include "tb.h"
#include "tb_internal.hpp"

#include <mutex>
#include <type_traits>
#include <utility>

namespace tb {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef uint32_t v6u __attribute__((ext_vector_type(6)));
typedef uint32_t v16u __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSteps = 7;            // 4-byte matrix steps per 26-byte group
constexpr int kSlot = 256;           // LDS bytes per table entry / record slot
constexpr int kRecOff = 128;         // record i at kSlot * i + kRecOff
constexpr int kLimbBytes = 32;       // one limb of a record: 6 dwords of fp6 (scale code in slots 5-6) + pad
constexpr int kTableEntries = 243;   // base-3 bytes 0..242
constexpr int kCopies = 32;          // table copies, one per lane of a half wave
constexpr int kMaxWaves = 16;
constexpr int kRotScratch = 1088 * 4;  // a rotating wave's transpose scratch (bytes)
constexpr int kXGroup = 136;           // floats between 128-groups of x' in LDS: 8 groups fill one scratch
constexpr int kAhead = 1;              // weight chunks a tile wave has in flight ahead of its matrix loop

typedef __attribute__((address_space(3))) uint8_t lds_u8;

template <typename T, int OFF = 0>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
  const lds_u8* p = reinterpret_cast<const lds_u8*>(static_cast<uintptr_t>(addr)) + OFF;
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_st(uint32_t addr, const T& v) {
  lds_u8* p = reinterpret_cast<lds_u8*>(static_cast<uintptr_t>(addr));
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads (the weight stream stays in flight across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  // raw buffer; offsets outside [0, bytes) read zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}

// fp32 -> fp6 (e2m3), round to nearest even, value / scale; element 2i from even[i], 2i + 1 from
// odd[i], element e at bits 6e .. 6e + 5 (the matrix instruction's operand layout).  The result
// registers must not overlap the sources (the instruction writes them while it still reads), so
// the output is an early-clobber operand.
__device__ __forceinline__ v6u cvt_fp6(const v16f& even, const v16f& odd, float scale) {
  v6u d;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(d) : "v"(even), "v"(odd), "v"(scale));
  return d;
}
// fp6 (e2m3) -> fp16, unscaled (every e2m3 value is exact in fp16), element e of p to half e.
__device__ __forceinline__ v16u fp6_f16(const v6u& p) {
  v16u d;
  asm("v_cvt_scalef32_pk32_f16_fp6 %0, %1, %2" : "=&v"(d) : "v"(p), "v"(1.0f));
  return d;
}

// e2m1 nibbles of the five trits of base-3 byte e (digit d -> trit d - 1: -1.0 = 0xA, 0 = 0,
// +1.0 = 0x2), trit i in nibble i; nibbles 5..7 stay 0 (the empty K-slots).  Bytes above 242 are
// not codes and read as zero trits.
__device__ __forceinline__ uint32_t trit_nibbles(uint32_t e) {
  if (e >= 243u) return 0u;
  uint32_t v = 0;
#pragma unroll
  for (int d = 0; d < 5; ++d) {
    const uint32_t digit = e % 3u;
    v |= (digit == 0u ? 0xAu : digit == 2u ? 0x2u : 0x0u) << (4 * d);
    e /= 3u;
  }
  return v;
}

template <int DT>
__device__ __forceinline__ void load16(const void* base, int64_t off, float (&v)[16]) {
  if constexpr (DT == TB_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = p[q];
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 u = p[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = w[e] & 0xFFFFu, hi = w[e] >> 16;
        if constexpr (DT == TB_BF16) {
          v[8 * q + 2 * e] = __uint_as_float(lo << 16);
          v[8 * q + 2 * e + 1] = __uint_as_float(hi << 16);
        } else {
          v[8 * q + 2 * e] = float(__builtin_bit_cast(_Float16, uint16_t(lo)));
          v[8 * q + 2 * e + 1] = float(__builtin_bit_cast(_Float16, uint16_t(hi)));
        }
      }
    }
  }
}

__device__ __forceinline__ void butterfly16(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      const float a = v[j], c = v[j + h];
      v[j] = a + c;
      v[j + h] = a - c;
    }
}

// x' of one 1024-block, H_1024 (S x) / 32 as a Sylvester-ordered fast Walsh-Hadamard transform
// ("TensorSharp view of Ternary Bonsai 2 27B", sections 3.2 and 5.2): lane l holds elements
// 16 l .. 16 l + 15 (signs applied); index bits 0..3 in registers, bits 4..7 in registers after a
// transpose through LDS (padded, 17 floats per 16, against bank conflicts), bits 8..9 across lanes.
// The result goes to xb in the x' layout (each 128-group contiguous, groups kXGroup floats apart),
// which may reuse the transpose's own scratch.
__device__ __forceinline__ void rotate_block(float (&v)[16], uint32_t scratch, uint32_t xb, int lane) {
  butterfly16(v);
#pragma unroll
  for (int j = 0; j < 16; ++j) lds_st<float>(scratch + 4u * (17 * lane + j), v[j]);
  wave_lds_fence();
  const int bidx = (lane & 15) + 272 * (lane >> 4);  // element (lane & 15) + 16 j + 256 (lane >> 4)
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = lds_ld<float>(scratch + 4u * (bidx + 17 * j));
  butterfly16(v);
  butterfly_lane_bits_4_5(v, lane);
  wave_lds_fence();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = (lane & 15) + 16 * j + 256 * (lane >> 4);
    lds_st<float>(xb + 4u * uint32_t(kXGroup * (e >> 7) + (e & 127)), v[j] * 0.03125f);
  }
}

// One record (group g, step s): the 32 K-slots of the step (4 code bytes x (5 trits + 3 empty
// slots)) as four fp6 limbs with their E8M0 scales.  Byte j of the step is byte 4s + j of the
// group (even g) or 4s - 2 + j (odd g: the group starts 2 bytes into its first dword); bytes
// outside 0..25 and trits past 127 (the pads) are 0.
__device__ __forceinline__ void build_record(uint32_t xb, int g, int s, uint32_t rec) {
  // The step's 20 trits are 20 consecutive elements of the group: 20 s .. (even g) or
  // 20 s - 10 .. (odd g), read as ten 8-byte pairs; elements outside 0..127 (the neighbouring
  // groups and the pad trits) count as 0.  ev[i] / od[i] hold K-slot 2i / 2i + 1, where slot
  // 8 j + i (i < 5) holds element 5 j + i of the run.
  const int first = (g & 1) ? 20 * s - 10 : 20 * s;
  const uint32_t base = xb + 4u * uint32_t(kXGroup * g + first);
  float run[20];
#pragma unroll
  for (int p = 0; p < 10; ++p) {
    const v2f v2 = lds_ld<v2f>(base + 8u * p);
    run[2 * p] = v2[0];
    run[2 * p + 1] = v2[1];
  }
  v16f ev, od;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int j = e >> 3, i = e & 7;
    float v = 0.f;
    if (i < 5) {
      const int t = first + 5 * j + i;
      v = (t >= 0 && t < kGroup) ? run[5 * j + i] : 0.f;
    }
    if (e & 1) od[e >> 1] = v;
    else ev[e >> 1] = v;
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fmaxf(fabsf(ev[i]), fabsf(od[i])));
  // limb 0 exponent E: m / 2^E in [2, 4); kept so every limb scale 2^(E - 4j) is a normal float
  // and its E8M0 code 127 + E - 4j lies in 1..254
  int E = m > 0.f ? ilogbf(m) - 1 : 0;
  E = min(max(E, -114), 127);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sc = __builtin_ldexpf(1.0f, E - 4 * j);
    const v6u l = cvt_fp6(ev, od, sc);
    if (j < 3) {
      // subtract the limb's value: h * sc is exact (a power-of-two scale) and so is the difference
      // (the rounding error of this limb); the empty slots stay 0
      const v16u h = fp6_f16(l);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t pair = h[i];  // halves: element 2i (low), 2i + 1 (high)
        if (((2 * i) & 7) < 5)
          ev[i] = fmaf(-float(__builtin_bit_cast(_Float16, uint16_t(pair & 0xFFFFu))), sc, ev[i]);
        if (((2 * i + 1) & 7) < 5)
          od[i] = fmaf(-float(__builtin_bit_cast(_Float16, uint16_t(pair >> 16))), sc, od[i]);
      }
    }
    // the limb's E8M0 code 127 + E - 4j goes into its K-slots 5 and 6 (bits 30..37, zero so far):
    // every weight operand has empty nibbles there, so the matrix instruction adds nothing for them
    const uint32_t a = rec + uint32_t(kLimbBytes * j);
    const uint32_t code = uint32_t(127 + E - 4 * j);
    lds_st<u32x4>(a, u32x4{l[0] | (code << 30), l[1] | (code >> 2), l[2], l[3]});
    lds_st<u32x2>(a + 16, u32x2{l[4], l[5]});
  }
}

// 4x4 transpose of 16-byte pieces across the four lane groups: on entry lane group a holds in
// r[b] (b = 0..3) piece a of quarter b's 64-byte chunk; on exit it holds in r[b] piece b of its own
// quarter a.  Two rounds of lane swaps: across lane bit 5 (lane group bit 1), then lane bit 4.
__device__ __forceinline__ void transpose_pieces(u32x4 (&r)[4]) {
#pragma unroll
  for (int lo = 0; lo < 2; ++lo)      // pieces (b, b + 2): lanes 0..31 keep b, send b + 2
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto p = __builtin_amdgcn_permlane32_swap(r[lo][d], r[lo + 2][d], false, false);
      r[lo][d] = p[0];
      r[lo + 2][d] = p[1];
    }
#pragma unroll
  for (int lo = 0; lo < 4; lo += 2)   // pieces (b, b + 1): even lane groups keep b, send b + 1
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto p = __builtin_amdgcn_permlane16_swap(r[lo][d], r[lo + 1][d], false, false);
      r[lo][d] = p[0];
      r[lo + 1][d] = p[1];
    }
}

// The activation part of one linear, for activation wave `wave`: block `blk` of x (one of K/1024),
// rotated (or copied) into x' slot `wave`, then the records of the slot's groups 8 wave ..
// 8 wave + 7 (they read only this block of x').  blk < 0: a block past the end of the rows (the
// padding of a K-part), whose x' and records are zero.  COHERENT: x is fp32 written by other
// workgroups of the same launch, read at the device coherence point (no stale cache lines).
template <int XDT, bool ROT, bool COHERENT = false>
__device__ __forceinline__ void prep_linear(const void* __restrict__ x, const uint32_t* __restrict__ sign_bits,
                                            int wave, int blk, int lane, uint32_t xb) {
  float xv[16];
  uint32_t sw = 0;
  if constexpr (COHERENT) {
    float* xp = const_cast<float*>(static_cast<const float*>(x)) + int64_t(blk) * kBlock + 16 * lane;
#pragma unroll
    for (int j = 0; j < 16; ++j) xv[j] = __hip_atomic_load(xp + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (ROT) sw = sign_bits[blk * 32 + (lane >> 1)] >> ((lane & 1) * 16);
  } else if (blk >= 0) {
    load16<XDT>(x, int64_t(blk) * kBlock + 16 * lane, xv);
    if constexpr (ROT) sw = sign_bits[blk * 32 + (lane >> 1)] >> ((lane & 1) * 16);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) xv[j] = 0.f;
  }
  const uint32_t xblock = xb + uint32_t(kRotScratch * wave);
  if constexpr (ROT) {
#pragma unroll
    for (int j = 0; j < 16; ++j) xv[j] = __uint_as_float(__float_as_uint(xv[j]) ^ (((sw >> j) & 1u) << 31));
    rotate_block(xv, xblock, xblock, lane);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = 16 * lane + j;
      lds_st<float>(xblock + 4u * uint32_t(kXGroup * (e >> 7) + (e & 127)), xv[j]);
    }
  }
  wave_lds_fence();
  if (lane < 8 * kSteps) {
    const int task = 8 * kSteps * wave + lane;
    const int g = task / kSteps, st = task - kSteps * g;
    build_record(xb, g, st, uint32_t(kSlot * task + kRecOff));
  }
}

// f(integral_constant<H>) for the H equal to h, so that H is a compile-time constant inside f.
template <typename F, int... H>
__device__ __forceinline__ void dispatch_part(int h, F& f, std::integer_sequence<int, H...>) {
  ((h == H ? f(std::integral_constant<int, H>{}) : void()), ...);
}

// Where a workgroup's part of K lies in the packed rows: code bytes and scale bytes per row, the
// part's first code byte and first scale byte within a row, and how many of the part's 4 G4
// groups exist (fewer only in the last part of a split row: its padding groups have zero
// activations, and their loads and scales are not read).
struct RowPart {
  uint32_t row_bytes, part_off, srow_bytes, spart_off;
  int real_groups;
};
template <int G4>
__device__ __forceinline__ RowPart whole_rows() {
  return RowPart{uint32_t(kB3GroupBytes * 4 * G4), 0u, uint32_t(2 * 4 * G4), 0u, 4 * G4};
}

// The tile part of one linear, for tile wave cw of the workgroup: the decode table (with_table),
// the weight loads, barrier C (the records are ready), the matrix loop, barrier D, y.  The
// workgroup takes tiles [t0, t1) (HALVES waves each); lane group kb of the wave of half h walks
// groups h G4 / HALVES .. of quarter kb of its tile's 16 rows (within the part rp of each row),
// and the halves' sums meet in LDS.
template <int G4, int HALVES, int PD = 0, bool COHERENT = false, bool PARTS = false>
__device__ __forceinline__ void tile_linear(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                                            float* __restrict__ y, int n, const RowPart& rp, int t0, int t1, int cw,
                                            int lane, uint32_t part_lds, bool with_table, int ctid, int cthreads) {
  constexpr int kGroups = 4 * G4;
  constexpr int kLaneBytes = kB3GroupBytes * G4;             // a quarter of a row
  constexpr int kHG = G4 / HALVES;                            // groups of a quarter per wave
  constexpr int kDw = (13 * kHG + 1) / 2;                     // code dwords a wave's lane reads
  constexpr int kChunks = kDw / 16;                           // whole 64-byte chunks of them
  constexpr int kTailLoads = (kDw - 16 * kChunks + 3) / 4;    // 16-byte loads for the rest
  constexpr int kTotal = kSteps * kHG;                        // matrix steps of a wave
  // operands fetched this many steps ahead of their matrix instruction (fewer when the lane holds
  // the codes of a whole quarter, to stay within the registers of 16 waves; PD > 0 overrides)
  constexpr int kPD = PD > 0 ? PD : HALVES > 1 ? 3 : kDw > 40 ? 1 : 2;
  const int kb = lane >> 4, col = lane & 15;
  const int h = cw % HALVES;
  const int tile_in_wg = cw / HALVES;
  const bool has_tile = tile_in_wg < t1 - t0;
  const int row = 16 * (t0 + tile_in_wg) + col;
  const int d0w = (13 * h * kHG - ((h * kHG) & 1)) / 2;       // first code dword of this wave's groups
  // ---- decode table first (once per launch): the activation waves (launched first) get their
  // loads of x out ahead of the weight stream; then the decode table (entry e at 256 e, copies at
  // 4 c) and the zero records
  if (with_table) {
    for (int e = ctid; e < kTableEntries; e += cthreads) {
      const uint32_t v = trit_nibbles(uint32_t(e));
#pragma unroll
      for (int part = 0; part < kCopies / 4; ++part) lds_st<u32x4>(uint32_t(e) * kSlot + 16u * part, u32x4{v, v, v, v});
    }
    for (int k = ctid; k < kSteps * 8; k += cthreads) {  // records 7 kGroups .. 7 kGroups + 6: zeros
      const uint32_t a = uint32_t(kSlot * (kSteps * kGroups + (k >> 3)) + kRecOff + 16 * (k & 7));
      lds_st<u32x4>(a, u32x4{0u, 0u, 0u, 0u});
    }
  }
  u32x4 R[kChunks > 0 ? kChunks : 1][4];
  u32x4 Tl[kTailLoads > 0 ? kTailLoads : 1];
  uint32_t S[(G4 + 1) / 2];
  // Each 16-byte load covers 64 contiguous bytes of 16 rows (the four lane groups of a row read
  // consecutive pieces of one quarter); the pieces move to their lane group later.  A lane without
  // a tile, and a load that starts past the part's last group, reads past the buffers (zeros):
  // every load is issued on every path.
  // (whole rows: the row geometry as compile-time constants, and no padding groups)
  const uint32_t row_bytes = PARTS ? rp.row_bytes : uint32_t(kB3GroupBytes * kGroups);
  const uint32_t srow_bytes = PARTS ? rp.srow_bytes : uint32_t(2 * kGroups);
  const uint32_t wbytes = uint32_t(n) * row_bytes, sbytes = uint32_t(n) * srow_bytes;
  const auto wr = rsrc(packed, wbytes);
  const auto sr = rsrc(scales, sbytes);
  const uint32_t rrow = has_tile ? uint32_t(row) * row_bytes + (PARTS ? rp.part_off : 0u) : wbytes;
  const uint32_t lim = uint32_t(kB3GroupBytes * rp.real_groups);
  auto woff = [&](int o) {
    if constexpr (!PARTS) return rrow + uint32_t(4 * d0w + o);
    return uint32_t(4 * d0w + o) < lim ? rrow + uint32_t(4 * d0w + o) : wbytes;
  };
  // the loads of chunk m (m == kChunks: the tail loads, if any)
  auto issue = [&](int m) {
    if (m < kChunks) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, woff(kLaneBytes * q + 64 * m + 16 * kb), 0, 0);
        R[m][q] = u32x4{v[0], v[1], v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTailLoads; ++i) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, woff(kLaneBytes * kb + 64 * kChunks + 16 * i), 0, 0);
        Tl[i] = u32x4{v[0], v[1], v[2], v[3]};
      }
    }
    // chunk by chunk in issue order, so that waiting for chunk m leaves the later ones in flight
    __builtin_amdgcn_sched_barrier(0);
  };
  {
    // the quarter's G4 scales first (the halves take theirs from them; a padding group's scale
    // reads 0): loads complete in issue order, so a scale issued after the codes could only be
    // used once every code load of the wave had arrived
    const uint32_t srow = has_tile ? uint32_t(row) * srow_bytes + (PARTS ? rp.spart_off : 0u) : sbytes;
#pragma unroll
    for (int i = 0; i < (G4 + 1) / 2; ++i) {
      const uint32_t soff =
          !PARTS || G4 * kb + 2 * i < rp.real_groups ? srow + uint32_t(2 * G4 * kb + 4 * i) : sbytes;
      S[i] = __builtin_amdgcn_raw_buffer_load_b32(sr, soff, 0, 0);
    }
    // The first kAhead chunks now; chunk c + kAhead when chunk c is moved to its lane groups in the
    // matrix loop.  With every chunk issued at once, all compute units' requests queue together
    // and a wave's first chunk lands about as late as its last; with one chunk ahead per wave
    // (about 20 KB per compute unit at 17408 x 5120, still enough to keep HBM busy) the early
    // chunks land early (34816 x 5120: 17.5 -> 15.2 us; two chunks ahead: 16.2, three: 17.6).
#pragma unroll
    for (int m = 0; m < kAhead && m <= kChunks; ++m)
      if (m < kChunks || kTailLoads > 0) issue(m);
  }
  lds_barrier();  // C

  float acc = 0.f;
  // the wave's half as a compile-time constant, so every register index below is one
  auto run_half = [&](auto hc) {
    constexpr int H = decltype(hc)::value;
    constexpr int i0 = H * kHG;                               // first group (of the quarter) of this wave
    constexpr int d0 = (13 * i0 - (i0 & 1)) / 2;              // its first code dword
    uint32_t W[16 * kChunks + 4 * kTailLoads + 1];            // dword d0 + d of the lane's quarter in W[d]
    // A 64-byte chunk's pieces are moved to their lane groups just before the first step that
    // needs one of its dwords, so the matrix loop starts on the first chunks while the later ones
    // are still arriving (waiting for a chunk waits only for the loads issued before it).
    auto fill = [&](int c) {
      if (c + kAhead <= kChunks && (c + kAhead < kChunks || kTailLoads > 0)) issue(c + kAhead);
      if (c < kChunks) {
        transpose_pieces(R[c]);
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int d = 0; d < 4; ++d) W[16 * c + 4 * p + d] = R[c][p][d];
      } else {
#pragma unroll
        for (int i = 0; i < kTailLoads; ++i)
#pragma unroll
          for (int d = 0; d < 4; ++d) W[16 * kChunks + 4 * i + d] = Tl[i][d];
      }
    };

    const uint32_t copy = uint32_t(4 * (lane & 31));
    // A row col of this lane: limb (col & 3) of lane group (col >> 2)'s record; zero records off
    // the block diagonal
    const bool diag = (col >> 2) == kb;
    const uint32_t a_base = diag ? uint32_t(kSlot * kSteps * (col >> 2) * G4 + kRecOff + kLimbBytes * (col & 3))
                                 : uint32_t(kSlot * kSteps * kGroups + kRecOff + kLimbBytes * (col & 3));
    const uint32_t a_step = diag ? uint32_t(kSlot * kSteps) : 0u;

    auto bop = [&](uint32_t w) -> v8i {
      const uint32_t e0 = lds_ld<uint32_t>(__builtin_amdgcn_perm(copy, w, 0x0C0C0004u));
      const uint32_t e1 = lds_ld<uint32_t>(__builtin_amdgcn_perm(copy, w, 0x0C0C0104u));
      const uint32_t e2 = lds_ld<uint32_t>(__builtin_amdgcn_perm(copy, w, 0x0C0C0204u));
      const uint32_t e3 = lds_ld<uint32_t>(__builtin_amdgcn_perm(copy, w, 0x0C0C0304u));
      return v8i{int(e0), int(e1), int(e2), int(e3), 0, 0, 0, 0};
    };
    // step k of the wave: group i = i0 + k / 7 of the quarter, step s = k % 7; its code dword
    // (an odd group starts 2 bytes into the dword that ends the even group before it, and the
    // two share that dword's lookups when both are this wave's)
    auto group_of = [&](int k) { return i0 + k / kSteps; };
    auto step_dword = [&](int k) { const int i = group_of(k); return (13 * i - (i & 1)) / 2 + k % kSteps - d0; };
    auto step_reuses_b = [&](int k) { return k > 0 && (group_of(k) & 1) && k % kSteps == 0; };

    // the chunk holding step k's code dword (the tail loads count as the last one)
    auto chunk_of = [&](int k) { return min(step_dword(k) / 16, kChunks); };
    v8i Bq[kPD + 1];
    u32x4 Alo[kPD + 1];
    u32x2 Ahi[kPD + 1];
    auto fetch = [&](int k) {
      const int slot = k % (kPD + 1);
      if (k == 0 || chunk_of(k) != chunk_of(k - 1)) fill(chunk_of(k));
      if (step_reuses_b(k)) Bq[slot] = Bq[(k - 1) % (kPD + 1)];
      else Bq[slot] = bop(W[step_dword(k)]);
      const uint32_t ab = a_base + uint32_t(group_of(k)) * a_step + uint32_t(kSlot * (k % kSteps));
      Alo[slot] = lds_ld<u32x4>(ab);
      Ahi[slot] = lds_ld<u32x2>(ab + 16);
    };
#pragma unroll
    for (int k = 0; k < kPD; ++k) fetch(k);
    v4f d = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kTotal; ++k) {
      if (k + kPD < kTotal) fetch(k + kPD);
      // keep the fetch ahead of this step's matrix instruction (the scheduler would otherwise
      // sink each fetch to its use and expose every LDS round trip)
      __builtin_amdgcn_sched_barrier(0);
      const int slot = k % (kPD + 1), s = k % kSteps;
      const v8i a = v8i{int(Alo[slot][0]), int(Alo[slot][1]), int(Alo[slot][2]), int(Alo[slot][3]),
                        int(Ahi[slot][0]), int(Ahi[slot][1]), 0, 0};
      d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, Bq[slot], s == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : d, 2, 4, 0,
                                                           int(__builtin_amdgcn_alignbit(Alo[slot][1], Alo[slot][0], 30)), 0, 127);  // A scale: bits 30..37
      if (s == kSteps - 1) {
        const int i = group_of(k);
        const uint32_t sw = S[i >> 1];
        const float sc = float(__builtin_bit_cast(_Float16, uint16_t((i & 1) ? sw >> 16 : sw & 0xFFFFu)));
        acc = fmaf(sc, (d[0] + d[1]) + (d[2] + d[3]), acc);
      }
    }
    // the four lane groups' partial sums of a row: lanes col, col + 16, col + 32, col + 48
    const uint32_t u = __float_as_uint(acc);
    const auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    acc = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    const uint32_t u2 = __float_as_uint(acc);
    const auto p16 = __builtin_amdgcn_permlane16_swap(u2, u2, false, false);
    acc = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    if (HALVES > 1 && H > 0 && lane < 16) lds_st<float>(part_lds + 4u * uint32_t(16 * (HALVES * tile_in_wg + H) + col), acc);
  };
  if (has_tile) dispatch_part(h, run_half, std::make_integer_sequence<int, HALVES>{});
  lds_barrier();  // D: the halves' partial sums are in LDS
  if (has_tile && h == 0 && lane < 16) {
#pragma unroll
    for (int hh = 1; hh < HALVES; ++hh) acc += lds_ld<float>(part_lds + 4u * uint32_t(16 * (HALVES * tile_in_wg + hh) + col));
    if (row < n) {
      if constexpr (COHERENT)  // written through to the device coherence point (read by other XCDs next)
        __hip_atomic_store(y + row, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        y[row] = acc;
    }
  }
}

// Kernel.  Waves 0 .. kPrep - 1 prepare the activations (kPrep = 4 G4 / 8, one 1024-block each:
// rotation, then the records of the block's 8 groups); the tile waves follow, HALVES per tile.
// A row of row_groups groups (nblocks 1024-blocks) is split into parts of 4 G4 groups, the last
// one padded with zero blocks; `grid` workgroups take each part (workgroup w: part w / grid), and
// part p writes its partial sums to y + p n (one part: y itself).
template <int G4, int HALVES, int XDT, bool ROT, bool PARTS>
__global__ __launch_bounds__(64 * kMaxWaves) void decode1_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales, const void* __restrict__ x,
    const uint32_t* __restrict__ sign_bits, float* __restrict__ y, int n, int tiles, int nslots, int grid, int nthreads,
    int row_groups, int nblocks) {
  constexpr int kPrep = G4 / 2;                               // activation waves (1024-blocks of a part)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = PARTS ? int(blockIdx.x) / grid : 0, w = int(blockIdx.x) - part * grid;
  const uint32_t xb = uint32_t(nslots * kSlot);              // x' (fp32, 136 floats per 128-group)
  const uint32_t part_lds = xb + uint32_t(kPrep * kRotScratch);  // halves' partial sums
  if (wave < kPrep) {
    const int blk = kPrep * part + wave;
    prep_linear<XDT, ROT>(x, sign_bits, wave, !PARTS || blk < nblocks ? blk : -1, lane, xb);
    lds_barrier();  // C: records complete
    lds_barrier();  // D
    return;
  }
  const int g0 = 4 * G4 * part;
  const RowPart rp{uint32_t(kB3GroupBytes * row_groups), uint32_t(kB3GroupBytes * g0), uint32_t(2 * row_groups),
                   uint32_t(2 * g0), min(4 * G4, row_groups - g0)};
  // workgroup w of the part takes tiles [w T / G, (w + 1) T / G)
  const int t0 = int((int64_t(w) * tiles) / grid);
  const int t1 = int((int64_t(w + 1) * tiles) / grid);
  tile_linear<G4, HALVES, 0, false, PARTS>(packed, scales, y + int64_t(part) * n, n, rp, t0, t1, wave - kPrep, lane,
                                            part_lds, true, int(threadIdx.x) - 64 * kPrep, nthreads - 64 * kPrep);
}

// y[i] = sum over parts p in order of part_y[p n + i]: the partial sums of a split row.  Every
// part's load is issued before the first add (a loop over a runtime count of parts would wait for
// each load in turn).
constexpr int kMaxParts = 8;
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part_y, float* __restrict__ y, int n,
                                                        int parts) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i >= n) return;
  float v[kMaxParts];
#pragma unroll
  for (int p = 0; p < kMaxParts; ++p) v[p] = p < parts ? part_y[int64_t(p) * n + i] : 0.f;
  float acc = v[0];
#pragma unroll
  for (int p = 1; p < kMaxParts; ++p)
    if (p < parts) acc += v[p];
  y[i] = acc;
}

// ---------------------------------------------------------------- chained linears
// One launch runs linears 0 .. count - 1 in order; linear i + 1 takes the first K outputs of
// linear i as its activations.  Every workgroup is resident at once (one per compute unit), and
// between linears each one waits on a device-wide count of the workgroups that have stored their
// rows of the previous output.  The tile waves issue the next linear's weight loads before that
// wait (they do not depend on x), so a linear's weight stream overlaps the previous linear's tail
// and the hand-over, and no launch separates the linears.  (Measured: the hand-over through the
// count costs more than a kernel boundary in a HIP graph, so separate launches are faster.)
struct ChainArgs {
  const uint8_t* packed[TB_CHAIN_MAX];
  const uint16_t* scales[TB_CHAIN_MAX];
  float* y[TB_CHAIN_MAX];
  int n[TB_CHAIN_MAX];
  const void* x0;
  const uint32_t* sign_bits;
  int32_t* sync;  // [0, count): arrivals per linear; [count]: finished workgroups; [count + 1]: status
  int count, spin_limit, nslots, grid, nthreads;
};

// Wait until *ctr reaches target, polling at most `limit` times; on time-out set bit 0 of *status
// and return anyway (the results of the call are then invalid, and the caller sees the status).
//
// Hand-over without cache maintenance: the producers write y with device-coherent stores (written
// through to the coherence point, complete once the store barrier has waited for them) before
// they bump the count, and the consumers poll the count and then read x with device-coherent loads.
// So no level of cache holds a stale copy on either side, and the count is only bumped after the
// data it announces is in place.  (Release/acquire fences at device scope would write back and
// invalidate each XCD's whole L2 every time: measured at about 50 us per hand-over.)
__device__ __forceinline__ void wait_count(int32_t* ctr, int target, int limit, int32_t* status, int lane) {
  for (int it = 0;; ++it) {
    const int v = __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v >= target) return;
    if (it >= limit) {
      if (lane == 0) __hip_atomic_fetch_or(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

template <int G4, int XDT0>
__global__ __launch_bounds__(64 * kMaxWaves) void chain_kernel(ChainArgs a) {
  constexpr int kPrep = G4 / 2;
  constexpr int kTilesPerRound = (kMaxWaves - kPrep) / 2;  // two waves (halves of K) per tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t xb = uint32_t(a.nslots * kSlot);
  const uint32_t part_lds = xb + uint32_t(kPrep * kRotScratch);
  // This workgroup's tiles [t0, t1) of linear i, taken kTilesPerRound at a time.
  auto tile_range = [&](int n, int& t0, int& t1) {
    const int tiles = (n + 15) / 16;
    t0 = int((int64_t(blockIdx.x) * tiles) / a.grid);
    t1 = int((int64_t(blockIdx.x + 1) * tiles) / a.grid);
  };
  auto rounds_of = [&](int t0, int t1) { return max(1, (t1 - t0 + kTilesPerRound - 1) / kTilesPerRound); };
  // Each role runs its own loop over the linears with the same workgroup barriers (C and D per
  // round, then the store barrier), so neither role's state is live in the other's code.
  if (wave < kPrep) {
    int32_t* status = a.sync + a.count + 1;
    for (int i = 0; i < a.count; ++i) {
      // linear i's row count and the previous output, by selects over the unrolled index
      // (indexing the argument arrays with i would copy them to scratch memory)
      int n = a.n[0];
      const float* xprev = a.y[0];
#pragma unroll
      for (int j = 1; j < TB_CHAIN_MAX; ++j)
        if (i == j) {
          n = a.n[j];
          xprev = a.y[j - 1];
        }
      if (i == 0) {
        prep_linear<XDT0, true>(a.x0, a.sign_bits, wave, wave, lane, xb);
      } else {
        wait_count(a.sync + i - 1, a.grid, a.spin_limit, status, lane);
        prep_linear<TB_F32, true, true>(xprev, a.sign_bits, wave, wave, lane, xb);
      }
      int t0, t1;
      tile_range(n, t0, t1);
      for (int r = rounds_of(t0, t1); r > 0; --r) {
        lds_barrier();  // C
        lds_barrier();  // D
      }
      // every wave's device-coherent stores of y_i are complete (the barrier waits for them): count
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_fetch_add(a.sync + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the last workgroup to finish (no workgroup waits any more) clears the counts for the next call
    if (threadIdx.x == 0) {
      const int prev = __hip_atomic_fetch_add(a.sync + a.count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == a.grid - 1)
        for (int i = 0; i <= a.count; ++i) __hip_atomic_store(a.sync + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  for (int i = 0; i < a.count; ++i) {
    const uint8_t* packed = a.packed[0];
    const uint16_t* scales = a.scales[0];
    float* y = a.y[0];
    int n = a.n[0];
#pragma unroll
    for (int j = 1; j < TB_CHAIN_MAX; ++j)
      if (i == j) {
        packed = a.packed[j];
        scales = a.scales[j];
        y = a.y[j];
        n = a.n[j];
      }
    int t0, t1;
    tile_range(n, t0, t1);
    const int rounds = rounds_of(t0, t1);
    for (int r = 0; r < rounds; ++r) {
      // the lane index made opaque per round, so the lane-dependent set-up is not hoisted out of
      // the loops (it would stay live across them and spill)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int u0 = t0 + r * kTilesPerRound, u1 = min(t1, u0 + kTilesPerRound);
      tile_linear<G4, 2, 2, true>(packed, scales, y, n, whole_rows<G4>(), u0, u1, wave - kPrep, ln, part_lds, i == 0 && r == 0,
                                  64 * (wave - kPrep) + ln, a.nthreads - 64 * kPrep);
    }
    __syncthreads();  // this wave's rows of y_i are stored
  }
}

int cu_count() {
  static int count = 0;
  static std::once_flag once;
  std::call_once(once, [] {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      count = c;
    else
      count = 256;
  });
  return count;
}

template <int G4, int HALVES, int XDT, bool ROT, bool PARTS>
void run_h(const uint8_t* packed, const uint16_t* scales, const void* x, const uint32_t* sign_bits, float* y, int n,
           int k, int parts, int grid, int per_wg, hipStream_t s) {
  constexpr int kGroups = 4 * G4;
  const int nw = kGroups / 8 + HALVES * per_wg;  // activation waves (one per 1024-block of x), then tile waves
  const int nslots = max(kTableEntries, kSteps * kGroups + kSteps);
  const size_t lds = size_t(nslots) * kSlot + size_t(kGroups / 8) * kRotScratch + size_t(64) * kMaxWaves;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&decode1_kernel<G4, HALVES, XDT, ROT, PARTS>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  const int tiles = (n + 15) / 16;
  decode1_kernel<G4, HALVES, XDT, ROT, PARTS><<<parts * grid, 64 * nw, lds, s>>>(
      packed, scales, x, sign_bits, y, n, tiles, nslots, grid, 64 * nw, k / kGroup, k / kBlock);
}

// Workgroups per part and tiles per workgroup for N rows in `parts` parts of K: at most one
// workgroup per compute unit in all.
void plan(int n, int parts, int& grid, int& per_wg) {
  const int tiles = (n + 15) / 16;
  grid = max(1, min(tiles, cu_count() / parts));
  per_wg = (tiles + grid - 1) / grid;
}

template <int G4, int XDT, bool ROT>
void run(const uint8_t* packed, const uint16_t* scales, const void* x, const uint32_t* sign_bits, float* y, int n,
         int k, int parts, hipStream_t s) {
  int grid, per_wg;
  plan(n, parts, grid, per_wg);
  // two waves per tile (each half of K) while they fit in a workgroup, else one (17408 x 5120 with
  // the rotation: two 9.5-9.7 us, one 9.9 us)
  const bool two = G4 % 2 == 0 && G4 / 2 >= 1 && (4 * G4) / 8 + 2 * per_wg <= kMaxWaves;
  // five waves per tile (two groups of each quarter each) where K = 5120 leaves room for them:
  // a workgroup with one or two tiles then runs 14 matrix steps per wave instead of 35 (x' given:
  // 5120 x 5120 7.05 -> 6.4 us; with the rotation in the prologue the extra waves slow the
  // prologue as much as they shorten the loop, so that keeps two)
  const bool five = !ROT && G4 % 5 == 0 && (4 * G4) / 8 + 5 * per_wg <= kMaxWaves;
  if (parts == 1) {
    if constexpr (G4 % 5 == 0 && !ROT) {
      if (five) return run_h<G4, 5, XDT, ROT, false>(packed, scales, x, sign_bits, y, n, k, parts, grid, per_wg, s);
    }
    if (two) run_h<G4, 2, XDT, ROT, false>(packed, scales, x, sign_bits, y, n, k, parts, grid, per_wg, s);
    else run_h<G4, 1, XDT, ROT, false>(packed, scales, x, sign_bits, y, n, k, parts, grid, per_wg, s);
  } else if constexpr (G4 >= 6) {  // parts of three to five blocks
    if (two) run_h<G4, 2, XDT, ROT, true>(packed, scales, x, sign_bits, y, n, k, parts, grid, per_wg, s);
    else run_h<G4, 1, XDT, ROT, true>(packed, scales, x, sign_bits, y, n, k, parts, grid, per_wg, s);
  }
}

// One part of `part_blocks` 1024-blocks (all of K when parts is 1).
template <int XDT, bool ROT>
bool dispatch_k(int part_blocks, int k, int parts, const uint8_t* packed, const uint16_t* scales, const void* x,
                const uint32_t* sb, float* y, int n, hipStream_t s) {
  switch (part_blocks) {
    case 1: run<2, XDT, ROT>(packed, scales, x, sb, y, n, k, parts, s); return true;
    case 2: run<4, XDT, ROT>(packed, scales, x, sb, y, n, k, parts, s); return true;
    case 3: run<6, XDT, ROT>(packed, scales, x, sb, y, n, k, parts, s); return true;
    case 4: run<8, XDT, ROT>(packed, scales, x, sb, y, n, k, parts, s); return true;
    case 5: run<10, XDT, ROT>(packed, scales, x, sb, y, n, k, parts, s); return true;
    default: return false;
  }
}

// Parts of a row of K (a multiple of 1024): as few as hold at most five blocks each, of equal
// block counts (the last one padded).
void split_of(int k, int& parts, int& part_blocks) {
  const int nb = k / kBlock;
  parts = decode1_split_parts(1, 1, k);
  part_blocks = (nb + parts - 1) / parts;
}

}  // namespace

// Largest tiles-per-workgroup the kernel takes (waves per workgroup).
bool decode1_supports(int packing, int b, int n, int k) {
  if (packing != 1 || b != 1 || k % kBlock != 0 || k > 5120 || n < 1) return false;
  int grid, per_wg;
  plan(n, 1, grid, per_wg);
  return k / kBlock + per_wg <= kMaxWaves;
}

bool decode1_split_supports(int n, int k) {
  if (k % kBlock != 0 || k <= 5 * kBlock || n < 1) return false;
  int parts, part_blocks, grid, per_wg;
  split_of(k, parts, part_blocks);
  if (parts > kMaxParts || parts > cu_count()) return false;
  plan(n, parts, grid, per_wg);
  return part_blocks + per_wg <= kMaxWaves;
}

namespace {

template <int G4, int XDT0>
void run_chain(ChainArgs& a, int nw, hipStream_t s) {
  constexpr int kGroups = 4 * G4;
  a.nslots = max(kTableEntries, kSteps * kGroups + kSteps);
  const size_t lds = size_t(a.nslots) * kSlot + size_t(G4 / 2) * kRotScratch + size_t(64) * kMaxWaves;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<G4, XDT0>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  a.nthreads = 64 * nw;
  chain_kernel<G4, XDT0><<<a.grid, 64 * nw, lds, s>>>(a);
}

template <int XDT0>
void chain_k(int k, ChainArgs& a, int nw, hipStream_t s) {
  switch (k) {
    case 1024: run_chain<2, XDT0>(a, nw, s); break;
    case 2048: run_chain<4, XDT0>(a, nw, s); break;
    case 3072: run_chain<6, XDT0>(a, nw, s); break;
    case 4096: run_chain<8, XDT0>(a, nw, s); break;
    default: run_chain<10, XDT0>(a, nw, s); break;
  }
}

}  // namespace

// The chained launch's plan: one workgroup per compute unit, two waves per tile (halves of K),
// at most (16 - K/1024) / 2 tiles at a time (more run in rounds).  Returns the waves per workgroup.
int chain_plan(const int64_t* n, int count, int k) {
  const int grid = cu_count(), prep = k / kBlock, per_round = (kMaxWaves - prep) / 2;
  int tiles_wg = 1;
  for (int i = 0; i < count; ++i) tiles_wg = max(tiles_wg, int(((n[i] + 15) / 16 + grid - 1) / grid));
  return prep + 2 * min(tiles_wg, per_round);
}

bool launch_chain(const tb_chain_linear* lin, int count, const void* x0, int x_dt, const uint32_t* sign_bits, int k,
                  int32_t* sync, int spin_limit, hipStream_t s) {
  if (count < 1 || count > TB_CHAIN_MAX || k % kBlock != 0 || k < kBlock || k > 5120) return false;
  int64_t n[TB_CHAIN_MAX];
  for (int i = 0; i < count; ++i) n[i] = lin[i].N;
  const int nw = chain_plan(n, count, k);
  ChainArgs a{};
  for (int i = 0; i < count; ++i) {
    a.packed[i] = lin[i].packed;
    a.scales[i] = lin[i].scales;
    a.y[i] = lin[i].y;
    a.n[i] = int(lin[i].N);
  }
  a.x0 = x0;
  a.sign_bits = sign_bits;
  a.sync = sync;
  a.count = count;
  a.spin_limit = spin_limit;
  a.grid = cu_count();
  if (x_dt == TB_F32) chain_k<TB_F32>(k, a, nw, s);
  else if (x_dt == TB_F16) chain_k<TB_F16>(k, a, nw, s);
  else chain_k<TB_BF16>(k, a, nw, s);
  return true;
}

namespace {

bool launch_parts(const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt, const uint32_t* sign_bits,
                  bool rotate, float* y, int n, int k, int parts, int part_blocks, hipStream_t s) {
  if (rotate) {
    if (x_dt == TB_F32) return dispatch_k<TB_F32, true>(part_blocks, k, parts, packed, scales, x, sign_bits, y, n, s);
    if (x_dt == TB_F16) return dispatch_k<TB_F16, true>(part_blocks, k, parts, packed, scales, x, sign_bits, y, n, s);
    return dispatch_k<TB_BF16, true>(part_blocks, k, parts, packed, scales, x, sign_bits, y, n, s);
  }
  if (x_dt == TB_F32) return dispatch_k<TB_F32, false>(part_blocks, k, parts, packed, scales, x, nullptr, y, n, s);
  return dispatch_k<TB_F16, false>(part_blocks, k, parts, packed, scales, x, nullptr, y, n, s);
}

}  // namespace

bool launch_decode1(const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                    const uint32_t* sign_bits, bool rotate, float* y, int n, int k, hipStream_t s) {
  return launch_parts(packed, scales, x, x_dt, sign_bits, rotate, y, n, k, 1, k / kBlock, s);
}

bool launch_decode1_split(const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                          const uint32_t* sign_bits, bool rotate, float* y, float* part_y, int n, int k,
                          hipStream_t s) {
  int parts, part_blocks;
  split_of(k, parts, part_blocks);
  if (!launch_parts(packed, scales, x, x_dt, sign_bits, rotate, part_y, n, k, parts, part_blocks, s)) return false;
  launch_sum_parts(part_y, y, n, parts, s);
  return true;
}

void launch_sum_parts(const float* part_y, float* y, int count, int parts, hipStream_t s) {
  sum_parts_kernel<<<(count + 255) / 256, 256, 0, s>>>(part_y, y, count, parts);
}

}  // namespace tb
