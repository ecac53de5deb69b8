// Decode product y[b][n] = sum_g s[n][g] sum_{k in g} t[n][k] xr[b][k]  (batch 1..8).
//
// Pages: "Ternary Bonsai 2 27B release", section "How the ternary weights
// reach 1.76 bit" (g128 fp16 scales, unpack and scale fused in the product)
// and section "Throughput" (decode streams the packed weights once per token).
//
// The weights never become fp16: they enter the matrix cores as fp4 (e2m1).
//   * 2-bit codes c = t + 1 in {0, 1, 2}: the 2-bit field already is the
//     nibble of c / 2, so a dword of 16 codes splits into two operand dwords
//     with one AND (and one shift), and sum_k t_k x_k = 2 sum_k (c_k / 2) x_k
//     - sum_k x_k (the activation sum is kept per group).
//   * base-3 bytes: one LDS table lookup turns a byte into a dword holding the
//     nibbles of its five trits themselves (-1.0, 0, +1.0); the table has 32
//     bank-spread copies so a wave's lookups do not conflict.  Per-row E8M0
//     scales of the matrix instruction carry each A row's power of two.  The 128 trits
//     of a group fill the 128 K-slots of one matrix instruction densely (the
//     group's two pad trits are left out), so a group costs one instruction,
//     as for 2-bit codes.
// The activations become three fp8 (e4m3) limbs per element, per 128-group
// scaled by a power of two so the largest magnitude lies in [128, 256):
//   x * 2^sig = l0 + l1/16 + l2/256, each limb the e4m3 rounding of what is
//   left, so the reconstruction error is about 2^-12 of the element.
// One v_mfma_scale_f32_16x16x128_f8f6f4 multiplies 16 weight rows by 128
// K-slots; its A rows are (batch, limb) pairs (row 4b + limb), so one matrix
// instruction serves up to four batch rows.  Per group the limbs are combined
// in fp32 and the fp16 scale and 2^-sig applied, in fp32.
//
// Work split: a workgroup of up to 16 waves holds rt tiles of 16 weight rows;
// the 8-group stages (1024 weights per row) of a tile are split over ks waves.
// A wave's packed bytes stream through registers with coalesced 16-byte
// buffer loads (a stage's loads go out before the matrix work of the stage
// before it), go to a per-wave LDS buffer and are read back in the operand
// layout.  A few "prep" waves turn the activations into
// limbs in LDS (for as many groups as fit; larger K takes several launches)
// while the other waves already stream weights; a launch may add waves that
// only build limbs.  The host picks the plan per call (tiles per workgroup,
// K-part waves, groups per launch, limb-only waves, rotation waves, and for
// base-3 a 64 KB or a 32 KB decode table) from a rough cost per launch,
// stage and prep pass.
#include "tb_internal.hpp"

#include <mutex>

namespace tb {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 16;       // waves per workgroup

constexpr int kStageGroups = 8;     // groups per stage (1024 weights per row)
constexpr int kCopies = 32;         // bank-spread copies of the base-3 table (one per half-wave lane)
constexpr int kLdsBytes = 160 * 1024;
constexpr int kTeam = 16;           // threads preparing one (batch, group) of activations
constexpr uint32_t kNoLoad = 0x80000000u;  // buffer offset past any buffer: reads zero

// LDS layouts below keep the rows that 16 consecutive lanes read in distinct
// 4-byte banks (or on the same dword); the base-3 table is spread over 32
// lanes, as bank-conflict counters show lanes 16 apart colliding.
template <int PACK>
struct Fmt {
  static constexpr int kGroupBytes = PACK == 0 ? 32 : kB3GroupBytes;
  static constexpr int kMfmas = 1;                             // matrix instructions per group
  // register slots of staged stages per wave: 2-bit stages load while the
  // stage before them computes (one slot); base-3 stages two ahead (two
  // slots, refilled after the compute)
  static constexpr int kDepth = PACK == 0 ? 1 : 2;
  static constexpr int kRowStage = kGroupBytes * kStageGroups;  // 256 or 208 bytes of a row per stage
  // LDS row stride: 66 or 54 dwords, so the 16 rows a quarter-wave reads
  // (two dwords each) fall in distinct banks
  static constexpr int kRowLds = kRowStage + 8;
  static constexpr int kChunksPerRow = kRowStage / 16;          // 16 or 13
  static constexpr int kStageChunks = 16 * kChunksPerRow;       // 256 or 208
  static constexpr int kLoads = (kStageChunks + 63) / 64;       // 4
  static constexpr int kStageLds = 16 * kRowLds + 32;           // + pad for operand over-reads
  // base-3 table: entry e at byte 256 e (PACK 1, 64 KB) or 128 e (PACK 2,
  // 32 KB, for launches that need the LDS), copy c (lane & 31) at + 4c.  One
  // byte permute forms (e << 8) | 4c from the staged bytes, or (e << 8) | 8c
  // and a shift halves it.
  static constexpr int kTable = PACK == 1 ? 256 * 256 : PACK == 2 ? 128 * 256 : 0;
  static constexpr int kEntry = PACK == 2 ? 128 : 256;  // base-3 table entry stride
};

// Activation limb rows in LDS: 128 K-slot bytes padded to 36 dwords so the
// three limb rows of a batch start in different banks.
constexpr int kARow = 144;
constexpr int kAGroup = 3 * kARow;   // one batch's three limb rows

// Limb block of batch b: [ng groups][instructions per group][kAGroup], so the
// offset of a group inside it is a compile-time constant.  The stride between
// batches is padded to 48 mod 128 bytes (as kAGroup is) so the rows of the
// four batches one instruction reads start in different banks.
__host__ __device__ constexpr int a_batch_stride(int ng, int mfmas) {
  const int base = ng * mfmas * kAGroup;
  return base + (48 - base % 128 + 128) % 128;
}
// Bytes of the per-(batch, group) factor region: the factors, then one
// exponent byte per (batch, group), each rounded to 16, plus 16 for the
// workgroup's ready counter.
__host__ __device__ constexpr int f_bytes(int nb, int ng) { return (nb * ng * 8 + 15) & ~15; }
__host__ __device__ constexpr int e0_stride(int ng) { return (ng + 7) & ~7; }  // 8-byte aligned rows
__host__ __device__ constexpr int f_region_bytes(int nb, int ng) {
  return f_bytes(nb, ng) + ((nb * e0_stride(ng) + 15) & ~15) + 16;
}

// Trit (0..127) of a group that sits in K-slot s of the base-3 layout.  B
// operand lane group q supplies slots 32q .. 32q + 31: the trits of bytes
// 6q .. 6q + 5 (trits 30q .. 30q + 29) in slots 0..29, and trits 120 + 2q,
// 121 + 2q (from bytes 24 and 25) in slots 30, 31; the pad trits have none.
// (2-bit codes need no map: dword w of lane group q holds the even (w even)
// or odd codes of bytes 8q + 4 (w / 2) .., and the activations are stored in
// that order by their own team layout.)
__host__ __device__ constexpr int b3_tau_of_slot(int s) {
  return (s & 31) < 30 ? 30 * (s >> 5) + (s & 31) : 120 + 2 * (s >> 5) + ((s & 31) - 30);
}

// LDS of a workgroup, in this order: the base-3 table (at address 0, so a
// table address needs no base), the activation limbs, the per-(batch, group)
// factors, then the waves' staging buffers.
// A operand slot s of lane group q' reads K-slot 16q'+s (s < 16) or 64+16q'+s-16.
struct Smem {
  uint8_t* lds;     // LDS address 0: the base-3 table, 256 entries x 256 (or 128) bytes
  uint8_t* a;       // [B][ng][mfmas][3][144] activation limbs in K-slot order
  int a_bstride;    // bytes between batches in a
  float2* f;        // [B][ng] = {2^-sig, sum of reconstructed activations}
  uint8_t* e0;      // [B][e0_stride(ng)] = 127 - sig, the E8M0 exponent of limb 0 (after f)
  int ng;           // groups of this launch
  int* ready;       // count of prep waves done (after f)
  uint8_t* stage;   // waves x kStageLds (reused for the K-part reduction at the end)
};

// LDS reads at a plain byte address.  The kernel declares no static LDS, so
// its dynamic LDS starts at address 0; building addresses as integers lets
// constant offsets fold into the instructions' offset field.
// (The constant offset is added to the pointer, not the integer, so the
// compiler knows the sum does not wrap and may fold it.)
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
template <typename T, int OFF = 0>
__device__ __forceinline__ T lds_read(uint32_t addr) {
  lds_u8* p = reinterpret_cast<lds_u8*>(static_cast<uintptr_t>(addr)) + OFF;
  return *reinterpret_cast<__attribute__((address_space(3))) const T*>(p);
}

// Table entry of a base-3 byte: its five digits d, low digit first, as e2m1
// nibbles of the trit t = d - 1 (-1.0 = 0xA, 0 = 0x0, +1.0 = 0x2); bytes
// above 242 are not codes and read as five zero trits.
__device__ __forceinline__ uint32_t base3_t_nibbles(uint32_t e) {
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

// Table entry e at LDS byte kEntry e: kCopies copies of its trit nibbles, one
// per lane of a half-wave, so the lanes' lookups fall in distinct banks.
template <int PACK>
__device__ __forceinline__ void write_b3_entry(uint8_t* lds, uint32_t e) {
  const uint32_t v = base3_t_nibbles(e);
  uint4* dst = reinterpret_cast<uint4*>(lds + Fmt<PACK>::kEntry * e);
#pragma unroll
  for (int i = 0; i < kCopies / 4; ++i) dst[i] = make_uint4(v, v, v, v);

}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer, 32-bit data format; offsets outside [0, bytes) read zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}

// Elements of a (batch, group) that thread l16 of its team of 16 converts, as
// four pairs of consecutive elements:
//   2-bit: 8 consecutive elements 8 l16 ..; they land in two limb dwords.
//   base-3: the trits of K-slots 8 l16 .. 8 l16 + 7, which land in one limb
//   qword; pair e starts at trit b3_tau_of_slot(8 l16 + 2 e).
template <int PACK>
struct XMap {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ int pair(int l16, int e) {
    return PACK == 0 ? 8 * l16 + 2 * e : b3_tau_of_slot(8 * l16 + 2 * e);
  }
};

template <int XDT, int PACK>
__device__ __forceinline__ void load_x(const void* __restrict__ xr, int k, int b, int g, int l16, float (&x)[10]) {
  const int64_t row = int64_t(b) * k + int64_t(g) * kGroup;
  x[8] = x[9] = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = XMap<PACK>::pair(l16, e);
    const int ic = min(idx, kGroup - 2);  // in-bounds address; the value is dropped below
    float2 v;
    if constexpr (XDT == 0) {
      v = *reinterpret_cast<const float2*>(static_cast<const float*>(xr) + row + ic);
    } else {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(xr) + row + ic);
      v.x = float(__builtin_bit_cast(_Float16, uint16_t(u & 0xFFFFu)));
      v.y = float(__builtin_bit_cast(_Float16, uint16_t(u >> 16)));
    }
    const bool ok = idx < kGroup;
    x[2 * e] = ok ? v.x : 0.f;
    x[2 * e + 1] = ok ? v.y : 0.f;
  }
}

// ---------------------------------------------------------------- fused rotation
//
// With the rotation fused (tb_linear), a prep wave rotates whole (batch,
// 1024-block) units: x' = H_1024 (S x) / 32 ("Ternary Bonsai 2 27B release",
// section "How the ternary weights reach 1.76 bit"), as a Sylvester-ordered
// fast Walsh-Hadamard transform ("TensorSharp view of Ternary Bonsai 2 27B",
// sections 3.2 and 5.2): index bits 0..3 in registers (16 consecutive
// values per lane), bits 4..7 in registers after a transpose through the
// wave's LDS scratch, bits 8..9 across lanes.  The result stays in the
// scratch (element i at i + i/16, padded against bank conflicts) for the
// limb teams.
constexpr int kRotScratch = 1088 * 4;  // bytes of one wave's scratch
constexpr int kMaxRotWaves = 16;  // rotation waves per workgroup, when LDS holds their scratch

template <int DT>
__device__ __forceinline__ void load16_x(const void* base, int64_t off, float (&v)[16]) {
  if constexpr (DT == 0) {  // fp32
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
        if constexpr (DT == 2) {  // bf16: the upper half of an fp32
          v[8 * q + 2 * e] = __uint_as_float(lo << 16);
          v[8 * q + 2 * e + 1] = __uint_as_float(hi << 16);
        } else {  // fp16
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

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rotate one block held as 16 values per lane (lane l: elements 16l..16l+15,
// sign flip already applied) into the wave's scratch L.
__device__ __forceinline__ void rotate_block(float (&v)[16], float* L, int lane) {
  butterfly16(v);  // index bits 0..3
#pragma unroll
  for (int j = 0; j < 16; ++j) L[17 * lane + j] = v[j];
  wave_fence();
  const int bidx = (lane & 15) + 272 * (lane >> 4);  // element (lane & 15) + 16 j + 256 (lane >> 4)
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = L[bidx + 17 * j];
  butterfly16(v);  // index bits 4..7
  butterfly_lane_bits_4_5(v, lane);  // index bits 8, 9 = lane bits 4, 5
  wave_fence();
#pragma unroll
  for (int j = 0; j < 16; ++j) L[bidx + 17 * j] = v[j] * 0.03125f;
  wave_fence();
}

// A thread's elements of group gi (0..7) of the rotated block in L, in the
// same assignment as load_x.
template <int PACK>
__device__ __forceinline__ void load_x_rot(const float* L, int gi, int l16, float (&x)[10]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = XMap<PACK>::pair(l16, e >> 1) + (e & 1);
    const int i = gi * kGroup + min(t, kGroup - 1);
    const float v = L[i + (i >> 4)];
    x[e] = t < kGroup ? v : 0.f;
  }
  x[8] = x[9] = 0.f;
}

// Butterfly reductions over the 16 lanes of a DPP row (a team), no LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

// The four e4m3 bytes of d as floats, to a[first + stride * i].
template <int FIRST, int STRIDE>
__device__ __forceinline__ void fp8x4_to_f32(int d, float (&a)[10]) {
  a[FIRST] = __builtin_amdgcn_cvt_f32_fp8(d, 0);
  a[FIRST + STRIDE] = __builtin_amdgcn_cvt_f32_fp8(d, 1);
  a[FIRST + 2 * STRIDE] = __builtin_amdgcn_cvt_f32_fp8(d, 2);
  a[FIRST + 3 * STRIDE] = __builtin_amdgcn_cvt_f32_fp8(d, 3);
}

// Split a thread's elements of one (batch, group) into three e4m3 limbs at
// the group's power-of-two scale and store them in their K-slots; lane 0 of
// the team records {2^-sig, sum of the reconstructed values}.  The limb
// values are decoded back from the stored bytes, so the residuals are exact
// whatever the conversion's rounding.
template <int PACK>
__device__ __forceinline__ void limbs_for_group(const Smem& sm, int b, int g, int l16, const float (&x)[10]) {
  constexpr int E = XMap<PACK>::kElems;
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) mx = fmaxf(mx, fabsf(x[e]));
  mx = row16_max(mx);
  int sig = 0;
  if (mx > 0.f) {
    int ex;
    frexpf(mx, &ex);  // mx = f * 2^ex, f in [0.5, 1)
    // mx * 2^sig in [128, 256), kept within [-127, 119] so that every limb
    // exponent 127 - sig - 4 limb is a valid E8M0 value.  Only a group whose
    // maximum is below 2^-111 is scaled less; its elements keep full limb
    // precision down to about 2^-125, so only fp32 subnormals are affected.
    sig = min(max(8 - ex, -127), 119);
  }
  float cur[10];
#pragma unroll
  for (int e = 0; e < 10; ++e) cur[e] = ldexpf(x[e], sig);
  float sum = 0.f;
  uint8_t* rowbase;
  int off;
  if constexpr (PACK == 0) {
    rowbase = sm.a + b * sm.a_bstride + g * kAGroup;
    off = 32 * (l16 >> 2) + 16 * ((l16 & 3) >> 1) + 4 * (l16 & 1);
  } else {
    rowbase = sm.a + b * sm.a_bstride + g * kAGroup;
    off = 8 * l16;
  }
  constexpr float kW[3] = {1.f, 0.0625f, 0.00390625f};
#pragma unroll
  for (int limb = 0; limb < 3; ++limb) {
    float a[10];
    uint8_t* dst = rowbase + limb * kARow + off;
    if constexpr (PACK == 0) {
      // even elements -> slots off..off+3, odd elements -> off+8..off+11
      int de = __builtin_amdgcn_cvt_pk_fp8_f32(cur[0], cur[2], 0, false);
      de = __builtin_amdgcn_cvt_pk_fp8_f32(cur[4], cur[6], de, true);
      int dd = __builtin_amdgcn_cvt_pk_fp8_f32(cur[1], cur[3], 0, false);
      dd = __builtin_amdgcn_cvt_pk_fp8_f32(cur[5], cur[7], dd, true);
      fp8x4_to_f32<0, 2>(de, a);
      fp8x4_to_f32<1, 2>(dd, a);
      a[8] = a[9] = 0.f;
      *reinterpret_cast<uint32_t*>(dst) = uint32_t(de);
      *reinterpret_cast<uint32_t*>(dst + 8) = uint32_t(dd);
    } else {
      // the thread's 8 K-slots in order: one qword
      int d0 = __builtin_amdgcn_cvt_pk_fp8_f32(cur[0], cur[1], 0, false);
      d0 = __builtin_amdgcn_cvt_pk_fp8_f32(cur[2], cur[3], d0, true);
      int d1 = __builtin_amdgcn_cvt_pk_fp8_f32(cur[4], cur[5], 0, false);
      d1 = __builtin_amdgcn_cvt_pk_fp8_f32(cur[6], cur[7], d1, true);
      fp8x4_to_f32<0, 1>(d0, a);
      fp8x4_to_f32<4, 1>(d1, a);
      a[8] = a[9] = 0.f;
      *reinterpret_cast<uint2*>(dst) = make_uint2(uint32_t(d0), uint32_t(d1));
    }
#pragma unroll
    for (int e = 0; e < 10; ++e) {
      if constexpr (PACK == 0) sum = fmaf(a[e], kW[limb], sum);
      cur[e] = (cur[e] - a[e]) * 16.f;
    }
  }
  if constexpr (PACK == 0) sum = row16_sum(sum);  // only the 2-bit path needs it
  // every lane of the team holds the same sig and sum (the butterfly
  // reductions leave the result in all 16 lanes), so all store: the same
  // bytes to the same address, and no branch splits the caller's code, which
  // lets the limbs of two groups interleave
  sm.f[b * sm.ng + g] = make_float2(ldexpf(1.f, -sig), sum);
  sm.e0[b * e0_stride(sm.ng) + g] = uint8_t(127 - sig);
}

// ---------------------------------------------------------------- matrix work

// Per-lane constants of the matrix work.
struct LaneCtx {
  int b_row;      // byte offset of this lane's staged row (2-bit: plus its 8q code bytes)
  int a_lane[2];  // per row set: LDS address of this lane's A-operand row in group 0
  int f_lane[2];  // per row set: index of this lane's batch row in f
  uint32_t tab;   // base-3 table: this lane's copy offset 4 * (lane & 31) in byte 0
  // base-3, by group parity P: offset of the dword pair holding bytes
  // 6q .. 6q + 5 from the group pair's start, and their shift in bytes
  // within it (0 or 2)
  uint32_t b3_off[2], b3_sh[2];
  uint32_t q8;    // 8 * lane group: which two of the ten extra trits are this lane's
  // base-3, per row set: LDS address of the e0 row of this lane's A-row
  // batch, and 4 * its limb in every byte (the limb's exponent offset)
  uint32_t e_lane[2], e_limb;
};

// A float2 from LDS (vector types have no address-space-qualified copy).
template <int OFF>
__device__ __forceinline__ float2 lds_f2(uint32_t addr) {
  const u32x2 w = lds_read<u32x2, OFF>(addr);
  return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
}

// ---- 2-bit, unrolled group sequence: every offset is an immediate.

// Per-stage base addresses: the lane's staged codes, its A row of the
// stage's first group, and its factor entry of that group.
struct StageBase {
  uint32_t row, a[2], f[2];
};

// The lane's two code dwords of group G (G may be the stage's group count:
// the row padding is then read, in bounds, and never used).
template <int G>
__device__ __forceinline__ void read_group_codes(const StageBase& sb, uint32_t (&raw)[2]) {
  const u32x2 w = lds_read<u32x2, 32 * G>(sb.row);
  raw[0] = w.x;
  raw[1] = w.y;
}

// B operand of a group: the 2-bit codes already are e2m1 nibbles for c/2;
// even and odd codes of each dword go to separate dwords.
__device__ __forceinline__ v8i make_bop2(const uint32_t (&raw)[2]) {
  const uint32_t m = 0x33333333u;
  return v8i{int(raw[0] & m), int((raw[0] >> 2) & m), int(raw[1] & m), int((raw[1] >> 2) & m), 0, 0, 0, 0};
}

// A operands of group G of the stage (lane rows of unused (batch, limb) pairs
// read a valid limb row: row i of A only feeds row i of the result, never
// stored).
template <int NR, int G>
__device__ __forceinline__ void load_aop(const StageBase& sb, v8i (&aops)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const u32x4 lo = lds_read<u32x4, G * kAGroup>(sb.a[r]), hi = lds_read<u32x4, G * kAGroup + 64>(sb.a[r]);
    aops[r] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
  }
}

template <int NR>
__device__ __forceinline__ void group_mma(const v8i (&aops)[NR], const v8i& bop, v4f (&out)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r)
    out[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aops[r], bop, v4f{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0,
                                                              127);
}

// y += s 2^-sig (2 (d0 + d1/16 + d2/256) - S) for group G, with d the limb
// rows of this lane's result (batch 4r + q), the nibbles holding c/2 (hence
// the doubling), S the activation sum and s the group's fp16 scale, half
// G & 1 of sq[G / 2] (the stage's scales of the lane's row, two per dword).
// Lanes of batches >= nb accumulate values that are never stored.  No branch
// here on purpose: a matrix instruction must run with the whole wave active,
// so its result may not feed a lane-divergent block.
template <int NR, int G>
__device__ __forceinline__ void group_epilogue(const v4f (&acc)[NR], const float2 (&fs)[NR], const uint32_t (&sq)[4],
                                               float (&yacc)[NR]) {
  const float sc = float(__builtin_bit_cast(_Float16, uint16_t((G & 1) ? sq[G >> 1] >> 16 : sq[G >> 1] & 0xFFFFu)));
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float p = fmaf(fmaf(acc[r][2], 0.00390625f, fmaf(acc[r][1], 0.0625f, acc[r][0])), 2.f, -fs[r].y);
    yacc[r] = fmaf(sc, p * fs[r].x, yacc[r]);
  }
}

// Pipeline state of one stage's group sequence.
template <int NR>
struct GroupPipe {
  uint32_t raw[2][2];  // code dwords of the next group, by parity
  v4f prev[NR];        // matrix results of the previous group
};

// Group G of a stage: B operand from codes read one step earlier, A
// operands, the next group's codes and the previous group's factors, the
// matrix instruction, then the previous group's epilogue (its matrix
// results have had a whole step to arrive).
template <int NR, int G>
__device__ __forceinline__ void group_step(const StageBase& sb, const uint32_t (&sq)[4], GroupPipe<NR>& st,
                                           float (&yacc)[NR]) {
  constexpr int P = G & 1;
  // the LDS reads stay in their step (not sunk to their use in the next)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  const v8i bop = make_bop2(st.raw[P]);
  v8i aops[NR];
  load_aop<NR, G>(sb, aops);
  read_group_codes<G + 1>(sb, st.raw[P ^ 1]);
  float2 fs[NR];
  if constexpr (G > 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) fs[r] = lds_f2<8 * (G - 1)>(sb.f[r]);
  }
  v4f cur[NR];
  group_mma<NR>(aops, bop, cur);
  if constexpr (G > 0) group_epilogue<NR, G - 1>(st.prev, fs, sq, yacc);
#pragma unroll
  for (int r = 0; r < NR; ++r) st.prev[r] = cur[r];
  asm volatile("" ::: "memory");
}

// Groups G .. sg - 1 of a stage, unrolled (sg = 8 for full stages, where
// every guard folds away; the launch's last stage may have fewer).
template <int NR, int G>
__device__ __forceinline__ void stage_groups(const StageBase& sb, int sg, const uint32_t (&sq)[4], GroupPipe<NR>& st,
                                             float (&yacc)[NR]) {
  if constexpr (G < kStageGroups) {
    if (G < sg) {
      group_step<NR, G>(sb, sq, st, yacc);
      stage_groups<NR, G + 1>(sb, sg, sq, st, yacc);
    } else if constexpr (G > 0) {
      // the last group's epilogue
      float2 fs[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) fs[r] = lds_f2<8 * (G - 1)>(sb.f[r]);
      group_epilogue<NR, G - 1>(st.prev, fs, sq, yacc);
    }
  } else {
    float2 fs[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) fs[r] = lds_f2<8 * (kStageGroups - 1)>(sb.f[r]);
    group_epilogue<NR, kStageGroups - 1>(st.prev, fs, sq, yacc);
  }
}

// ---- base-3, rolled group loop: two groups per iteration, each group's
// table lookups made in its own step (the compute of a base-3 group is bound
// by its LDS instructions, which unrolling does not reduce; rolled, two
// stages of loads fit in registers).

// Raw staged bytes of a group of parity P from bo (the group pair's start in
// the lane's staged row): the dword pair holding bytes 6q .. 6q + 5 (a group
// starts 2-byte aligned) and the dword holding bytes 24 and 25.
template <int P>
__device__ __forceinline__ void b3r_read_bytes(const LaneCtx& lc, uint32_t bo, uint32_t (&raw)[4]) {
  const uint32_t a = bo + lc.b3_off[P];
  raw[0] = lds_read<uint32_t>(a);
  raw[1] = lds_read<uint32_t, 4>(a);
  raw[2] = lds_read<uint32_t, P ? 48 : 24>(bo);
  raw[3] = 0;
}

// B operand of a base-3 group of parity P: one lookup per byte in the plain
// table (its five trits as nibbles 0..4 of a dword), shifted and ORed into
// 32 dense nibbles: bytes 6q .. 6q + 5 in slots 0..29 and two of the ten
// trits of bytes 24, 25 in slots 30, 31.
template <int PACK, int P>
__device__ __forceinline__ v8i b3r_make_bop(const LaneCtx& lc, const uint32_t (&raw)[4]) {
  const uint32_t sh = lc.b3_sh[P];
  const uint32_t w0 = __builtin_amdgcn_alignbyte(raw[1], raw[0], sh);
  const uint32_t w1 = raw[1] >> (8 * sh);
  auto look = [&](uint32_t w, int byte) -> uint32_t {
    // permuted bytes: [0] = lane copy offset (times 2 for PACK 2), [1] = the
    // code byte, [2..3] = 0; PACK 2 halves it to 128 x byte + 4 x copy
    const uint32_t a = __builtin_amdgcn_perm(lc.tab, w, 0x0C0C0004u | (uint32_t(byte) << 8));
    return lds_read<uint32_t>(PACK == 2 ? a >> 1 : a);
  };
  const uint32_t e0 = look(w0, 0), e1 = look(w0, 1), e2 = look(w0, 2), e3 = look(w0, 3);
  const uint32_t e4 = look(w1, 0), e5 = look(w1, 1);
  // bytes 24 and 25: byte 0 and 1 (even group) or 2 and 3 (odd group) of raw[2]
  const uint32_t e24 = look(raw[2], P ? 2 : 0), e25 = look(raw[2], P ? 3 : 1);
  const uint32_t extra = ((e24 | (e25 << 20)) >> lc.q8) & 0xFFu;
  return v8i{int(e0 | (e1 << 20)), int((e1 >> 12) | (e2 << 8) | (e3 << 28)), int((e3 >> 4) | (e4 << 16)),
             int((e4 >> 16) | (e5 << 4) | (extra << 24)), 0, 0, 0, 0};
}

// A operands of group gc of the launch.
template <int NR>
__device__ __forceinline__ void b3r_load_aop(const LaneCtx& lc, int gc, v8i (&aops)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint32_t ag = uint32_t(lc.a_lane[r] + gc * kAGroup);
    const u32x4 lo = lds_read<u32x4, 0>(ag), hi = lds_read<u32x4, 64>(ag);
    aops[r] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
  }
}

// Pipeline state of a stage's rolled group loop.
template <int NR>
struct B3Pipe {
  uint32_t raw[2][4];  // staged bytes of the next groups, by parity
  v4f prev[NR];        // matrix results of the previous group
  float sprev;         // its fp16 weight scale
  uint32_t ex[NR][2];  // E8M0 exponents of this lane's A row for the stage's next groups, one a byte
};

// One group gc of parity P: B operand from bytes read one group earlier, the
// A operands, the next group's bytes, the matrix instruction, then the
// previous group's epilogue.  So every dependent LDS round trip except the
// table lookup is a group ahead of its use.  The matrix instruction scales
// A row (batch, limb) by 2^-sig 16^-limb through its E8M0 scale (byte P of
// ex[r][0]), so a result is just s (d0 + d1 + d2); the group's fp16 scale s
// is half P of sq0.
template <int PACK, int NR, int P>
__device__ __forceinline__ void b3r_group_step(const LaneCtx& lc, uint32_t bo, int gc, uint32_t sq0, B3Pipe<NR>& st,
                                               float (&yacc)[NR]) {
  __builtin_amdgcn_sched_barrier(0);
  const v8i bop = b3r_make_bop<PACK, P>(lc, st.raw[P]);
  v8i aops[NR];
  b3r_load_aop<NR>(lc, gc, aops);
  // the next group's bytes (past the stage's last group: the row padding, ignored)
  if constexpr (P == 0) b3r_read_bytes<1>(lc, bo, st.raw[1]);
  else b3r_read_bytes<0>(lc, bo + 2 * kB3GroupBytes, st.raw[0]);
  const float sc = float(__builtin_bit_cast(_Float16, uint16_t(P ? sq0 >> 16 : sq0 & 0xFFFFu)));
  v4f cur[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r)
    cur[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aops[r], bop, v4f{0.f, 0.f, 0.f, 0.f}, 0, 4, P,
                                                              int(st.ex[r][0]), 0, 127);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    yacc[r] = fmaf(st.sprev, st.prev[r][0] + st.prev[r][1] + st.prev[r][2], yacc[r]);
    st.prev[r] = cur[r];
  }
  st.sprev = sc;
}

// All groups of one staged block of sg (1..8) base-3 groups starting at group
// gc0 of the launch, two per iteration of a rolled loop.
template <int PACK, int NR>
__device__ __forceinline__ void b3r_stage_compute(uint32_t stage, const LaneCtx& lc, int sg, int gc0,
                                                  const uint32_t (&sreg)[4], float (&yacc)[NR]) {
  B3Pipe<NR> st;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    st.prev[r] = v4f{0.f, 0.f, 0.f, 0.f};
    // the stage's eight limb-0 exponents of this lane's batch, less 4 limb
    // (no byte borrows: 127 - sig >= 8)
    const uint32_t e = lc.e_lane[r] + uint32_t(gc0);
    st.ex[r][0] = lds_read<uint32_t>(e) - lc.e_limb;
    st.ex[r][1] = lds_read<uint32_t, 4>(e) - lc.e_limb;
  }
  st.sprev = 0.f;
  uint32_t sq[4] = {sreg[0], sreg[1], sreg[2], sreg[3]};
  uint32_t bo = stage + lc.b_row;
  b3r_read_bytes<0>(lc, bo, st.raw[0]);
  int g = 0;
#pragma unroll 1
  for (; g + 1 < sg; g += 2) {
    b3r_group_step<PACK, NR, 0>(lc, bo, gc0 + g, sq[0], st, yacc);
    b3r_group_step<PACK, NR, 1>(lc, bo, gc0 + g + 1, sq[0], st, yacc);
    bo += 2 * kB3GroupBytes;
    sq[0] = sq[1];
    sq[1] = sq[2];
    sq[2] = sq[3];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      st.ex[r][0] = __builtin_amdgcn_alignbyte(st.ex[r][1], st.ex[r][0], 2);
      st.ex[r][1] >>= 16;
    }
  }
  if (g < sg) b3r_group_step<PACK, NR, 0>(lc, bo, gc0 + g, sq[0], st, yacc);
#pragma unroll
  for (int r = 0; r < NR; ++r) yacc[r] = fmaf(st.sprev, st.prev[r][0] + st.prev[r][1] + st.prev[r][2], yacc[r]);
}

// All groups of one staged block of sg (1..8) groups starting at group gc0
// of the launch.
template <int PACK, int NR>
__device__ __forceinline__ void stage_compute(const Smem& sm, uint32_t stage, const LaneCtx& lc, int sg,
                                              int gc0, const uint32_t (&sreg)[4], float (&yacc)[NR]) {
  if constexpr (PACK != 0) {
    b3r_stage_compute<PACK, NR>(stage, lc, sg, gc0, sreg, yacc);
    return;
  }
  StageBase sb;
  sb.row = stage + lc.b_row;
  const uint32_t f0 = uint32_t(reinterpret_cast<uintptr_t>(sm.f) - reinterpret_cast<uintptr_t>(sm.lds));
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    sb.a[r] = uint32_t(lc.a_lane[r] + gc0 * kAGroup);
    sb.f[r] = f0 + 8u * uint32_t(lc.f_lane[r] + gc0);
  }
  GroupPipe<NR> st;
  read_group_codes<0>(sb, st.raw[0]);
  // the group count stays opaque, so every group is its own basic block:
  // within one block the compiler would gather the matrix instructions at
  // the end and keep every group's operands alive until then
  asm volatile("" : "+s"(sg));
  stage_groups<NR, 0>(sb, sg, sreg, st, yacc);
}

// ---------------------------------------------------------------- streaming

// Issue the loads of full stage s into registers.  Every lane issues every
// load (a lane with nothing to load, or a stage past this wave's range, uses
// an offset past the end of the buffer and reads zero), so the compiler
// counts outstanding loads exactly and keeps every register slot's stage in
// flight.
template <int PACK, bool ALIGNED>
__device__ __forceinline__ void issue_stage(__amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t srs,
                                            const uint32_t (&src)[Fmt<PACK>::kLoads], uint32_t srow_scale,
                                            int s, int s_end, uint4 (&regs)[Fmt<PACK>::kLoads],
                                            uint32_t (&sreg)[4]) {
  using F = Fmt<PACK>;
  const bool live = s < s_end;
#pragma unroll
  for (int j = 0; j < F::kLoads; ++j) {
    const uint32_t off = (live && src[j] != kNoLoad) ? src[j] + uint32_t(s * F::kRowStage) : kNoLoad;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0);
    regs[j] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  // scales of row (lane & 15) for the stage's 8 groups, byte offset
  const uint32_t soff =
      (live && srow_scale != kNoLoad) ? 2u * (srow_scale + uint32_t(s * kStageGroups)) : kNoLoad;
  if constexpr (ALIGNED) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(srs, soff, 0, 0);
    sreg[0] = v[0]; sreg[1] = v[1]; sreg[2] = v[2]; sreg[3] = v[3];
  } else {
    // 2-byte aligned: five dwords from the dword boundary below, then realign
    const uint32_t base = soff == kNoLoad ? kNoLoad : (soff & ~3u);
    uint32_t wd[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) wd[i] = __builtin_amdgcn_raw_buffer_load_b32(srs, base + 4u * i, 0, 0);
    const uint32_t sh = soff & 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) sreg[i] = __builtin_amdgcn_alignbyte(wd[i + 1], wd[i], sh);
  }
  // keep each stage's loads together and in stage order: the waits before a
  // stage's use count outstanding loads, so a later stage's load scheduled
  // ahead of this one would be waited for as well
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One full stage: registers -> this wave's LDS buffer, the matrix work, and
// the refill of the register slot with stage s + kDepth (with one slot the
// refill goes out before the matrix work, so a stage's loads are in flight
// while the stage before it computes).
template <int PACK, int NR, bool ALIGNED>
__device__ __forceinline__ void run_stage(const Smem& sm, uint8_t* my_stage, uint32_t stage_addr, const LaneCtx& lc,
                                          __amdgpu_buffer_rsrc_t wrs,
                                          __amdgpu_buffer_rsrc_t srs, const uint32_t (&src)[Fmt<PACK>::kLoads],
                                          uint32_t srow_scale, int s, int s_end, int nb,
                                          uint4 (&regs)[Fmt<PACK>::kLoads], uint32_t (&sreg)[4],
                                          float (&yacc)[NR]) {
  using F = Fmt<PACK>;
  const int lane = threadIdx.x & 63;
  wave_lds_fence();  // the previous stage's operand reads of this buffer come first
#pragma unroll
  for (int j = 0; j < F::kLoads; ++j) {
    const int c = 64 * j + lane;
    if (c < F::kStageChunks) {
      // chunk c = row c / chunks-per-row, 16-byte column c % chunks-per-row; rows are
      // 8-byte aligned at the padded stride, so two 8-byte writes
      const int r = c / F::kChunksPerRow;
      uint2* dst = reinterpret_cast<uint2*>(my_stage + r * F::kRowLds + 16 * (c - r * F::kChunksPerRow));
      dst[0] = make_uint2(regs[j].x, regs[j].y);
      dst[1] = make_uint2(regs[j].z, regs[j].w);
    }
  }
  wave_lds_fence();
  if constexpr (F::kDepth == 1) {
    const uint32_t sq[4] = {sreg[0], sreg[1], sreg[2], sreg[3]};
    issue_stage<PACK, ALIGNED>(wrs, srs, src, srow_scale, s + 1, s_end, regs, sreg);
    stage_compute<PACK, NR>(sm, stage_addr, lc, kStageGroups, s * kStageGroups, sq, yacc);
  } else {
    stage_compute<PACK, NR>(sm, stage_addr, lc, kStageGroups, s * kStageGroups, sreg, yacc);
    issue_stage<PACK, ALIGNED>(wrs, srs, src, srow_scale, s + F::kDepth, s_end, regs, sreg);
  }
}

// ---------------------------------------------------------------- kernel

// One launch covers groups [g_begin, g_begin + ng) of every row (the host
// issues several launches, each adding into y, when the activation limbs of
// all of K do not fit in LDS; a wave owns the same rows in every launch and
// launches on one stream run in order).  A workgroup holds rt row tiles of
// 16 rows; the stages of a tile are split over ks waves, and the ks partial
// sums are added through LDS at the end.
// ROT: xr is the unrotated x (dtype XDT: fp32, fp16, bf16) and the prep waves
// rotate it (g_begin and ng are then multiples of 8 groups = whole blocks);
// otherwise xr is x' (XDT: fp32, fp16).
template <int PACK, int NR, int XDT, bool ALIGNED, bool ROT>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_mfma_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales, const void* __restrict__ xr,
    const uint32_t* __restrict__ sign_bits, float* __restrict__ y, int nb, int n, int k, int g_begin, int ng,
    int accumulate, int rt, int ks, int rot_waves) {
  using F = Fmt<PACK>;
  extern __shared__ __align__(16) uint8_t smem[];
  // the wave index through readfirstlane: per-wave quantities below become
  // scalar (SALU) work instead of vector work
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int groups = k / kGroup;
  const int row_bytes = F::kGroupBytes * groups;
  const int tile = wave / ks, kp = wave - tile * ks;
  const int row0 = (blockIdx.x * rt + tile) * 16;
  const int nl = lane & 15, q = lane >> 4;

  Smem sm;
  sm.lds = smem;
  sm.a = smem + F::kTable;
  sm.a_bstride = a_batch_stride(ng, F::kMfmas);
  const int a_bytes = nb * sm.a_bstride;
  sm.f = reinterpret_cast<float2*>(sm.a + a_bytes);
  sm.e0 = sm.a + a_bytes + f_bytes(nb, ng);
  sm.ng = ng;
  sm.ready = reinterpret_cast<int*>(sm.a + a_bytes + f_region_bytes(nb, ng) - 16);
  sm.stage = sm.a + a_bytes + f_region_bytes(nb, ng);
  uint8_t* my_stage = sm.stage + wave * F::kStageLds;
  const uint32_t my_stage_addr = uint32_t(F::kTable + a_bytes + f_region_bytes(nb, ng) + wave * F::kStageLds);
  LaneCtx lc;
  lc.b_row = nl * F::kRowLds + (PACK == 0 ? 8 * q : 0);
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int o = kB3GroupBytes * par + 6 * q;  // even: 0, 6, 12, 18; odd: 26, 32, 38, 44
    lc.b3_off[par] = uint32_t(o & ~3);
    lc.b3_sh[par] = uint32_t(o & 3);
  }
  lc.q8 = uint32_t(8 * q);
  lc.e_limb = uint32_t(4 * min(nl & 3, 2)) * 0x01010101u;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    // A rows are 4b + limb; unused rows (limb 3, or batch >= nb) read a valid
    // limb row instead (they only feed result rows that are never read)
    const int limb = min(nl & 3, 2), b = min(4 * r + (nl >> 2), nb - 1);
    lc.a_lane[r] = F::kTable + b * sm.a_bstride + limb * kARow + 16 * q;
    lc.e_lane[r] = uint32_t(F::kTable + a_bytes + f_bytes(nb, ng) + b * e0_stride(ng));
    lc.f_lane[r] = min(4 * r + q, nb - 1) * ng;
  }
  lc.tab = uint32_t((PACK == 2 ? 8 : 4) * (lane & (kCopies - 1)));  // < 256: fits the permute's byte 0

  // ---- roles.  Waves 0 .. rt*ks - 1 own row tiles and stages (compute
  // waves); a launch may add waves beyond them that only build limbs (more
  // (batch, group) pairs than the compute waves' teams would cover in a few
  // passes, as at batch 8).  Prep waves are taken in prep-rank order: the
  // extra waves first, then compute waves 0, 1, ...  A compute wave that
  // preps loads its weights only afterwards; the others (after the base-3
  // table, when they write it) start the weight stream at once.  A wave
  // starts its matrix work when the LDS counter shows every prep wave done,
  // not at a workgroup barrier, so it never waits for another wave's weight
  // loads to be issued.
  const int pairs = ng * nb;
  const int ncomp = rt * ks;
  const int nw = int(blockDim.x) >> 6;
  const bool comp = wave < ncomp;
  const int prank = comp ? wave + (nw - ncomp) : wave - ncomp;
  // rotation units: (batch, block) pairs, one wave each at a time
  const int nblk = ng / 8, units = nb * nblk;
  const int prep_waves = ROT ? min(min(nw, units), rot_waves)
                             : max(nw - ncomp, min(nw, (pairs + 11) / 12));  // ~3 (batch, group) pairs per team
  const bool prep = prank < prep_waves;
  const int team = prank * (64 / kTeam) + (lane >> 4), l16 = lane & (kTeam - 1), nteams = prep_waves * (64 / kTeam);
  // The base-3 decode table is written by the waves that build no limbs
  // (they would otherwise sit idle until the limbs are ready), or by the prep
  // waves when every wave is one.  Each table wave adds 1 to the ready count.
  const bool tab_by_rest = PACK != 0 && nw > prep_waves;
  const int ready_target = prep_waves + (tab_by_rest ? nw - prep_waves : 0);
  float xa[10], xb[10], xc[10];
  float va[16];
  uint32_t sw_next = 0;  // sign words of the rotation unit about to be rotated
  if constexpr (ROT) {
    if (prep) {
      // the first unit's activations and sign words go out before any weight load
      const int b = prank % nb, blk = prank / nb;
      load16_x<XDT>(xr, int64_t(b) * k + int64_t(g_begin + 8 * blk) * kGroup + 16 * lane, va);
      sw_next = sign_bits[((g_begin >> 3) + blk) * 32 + (lane >> 1)];
    }
  } else if (prep) {
    // the activation loads go out before any weight load of the workgroup
    // (loads return in order, so whatever is issued behind the weight stream
    // arrives after it)
    const int p0 = team, p1 = team + nteams, p2 = team + 2 * nteams;
    if (p0 < pairs) load_x<XDT, PACK>(xr, k, p0 % nb, g_begin + p0 / nb, l16, xa);
    if (p1 < pairs) load_x<XDT, PACK>(xr, k, p1 % nb, g_begin + p1 / nb, l16, xb);
    if (p2 < pairs) load_x<XDT, PACK>(xr, k, p2 % nb, g_begin + p2 / nb, l16, xc);
  }
  if (tid == 0) *sm.ready = 0;
  __syncthreads();

  // ---- this wave's stages: [s_lo, s_hi); only the launch's last stage may be partial
  const int nst = (ng + kStageGroups - 1) / kStageGroups;
  const int s_lo = kp * nst / ks, s_hi = (kp + 1) * nst / ks;
  const bool has_tail = (ng % kStageGroups) != 0 && s_hi == nst;
  const int s_full = has_tail ? s_hi - 1 : s_hi;

  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, uint32_t(n) * uint32_t(row_bytes));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(scales, uint32_t(n) * uint32_t(groups) * 2u);
  uint32_t src[F::kLoads];
#pragma unroll
  for (int j = 0; j < F::kLoads; ++j) {
    const int c = 64 * j + lane;
    const int r = c / F::kChunksPerRow, cc = c - r * F::kChunksPerRow;
    const bool ok = c < F::kStageChunks && row0 + r < n;
    src[j] = ok ? uint32_t((row0 + r) * row_bytes + g_begin * F::kGroupBytes + 16 * cc) : kNoLoad;
  }
  const uint32_t srow_scale = row0 + nl < n ? uint32_t((row0 + nl) * groups + g_begin) : kNoLoad;

  uint4 stg[F::kDepth][F::kLoads];
  uint32_t scl[F::kDepth][4];
  if (prep) {
    if (PACK != 0 && !tab_by_rest) {
      for (int e = prank * 64 + lane; e < 256; e += 64 * prep_waves) {
        write_b3_entry<PACK>(sm.lds, uint32_t(e));
      }
    }
    if constexpr (ROT) {
      // units prank, prank + prep_waves, ...: sign flip, rotate into this
      // wave's scratch (inside the staging region, unused until matrix work
      // starts, plus any LDS the launch adds for it), then four teams make the
      // limbs of the block's 8 groups
      float* L = reinterpret_cast<float*>(sm.stage + prank * kRotScratch);
      const int tw = lane >> 4;
      for (int u = prank; u < units; u += prep_waves) {
        const int b = u % nb, blk = u / nb;
        if (u != prank) {
          load16_x<XDT>(xr, int64_t(b) * k + int64_t(g_begin + 8 * blk) * kGroup + 16 * lane, va);
          sw_next = sign_bits[((g_begin >> 3) + blk) * 32 + (lane >> 1)];  // this block's sign words
        }
        const uint32_t sw = sw_next >> ((lane & 1) * 16);
#pragma unroll
        for (int j = 0; j < 16; ++j) va[j] = __uint_as_float(__float_as_uint(va[j]) ^ (((sw >> j) & 1u) << 31));
        rotate_block(va, L, lane);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gi = tw + 4 * h;
          float xg[10];
          load_x_rot<PACK>(L, gi, l16, xg);
          limbs_for_group<PACK>(sm, b, 8 * blk + gi, l16, xg);
        }
        wave_fence();  // the scratch is rewritten by the next unit
      }
    } else {
      const int p0 = team, p1 = team + nteams, p2 = team + 2 * nteams;
      if (p0 < pairs) limbs_for_group<PACK>(sm, p0 % nb, p0 / nb, l16, xa);
      if (p1 < pairs) limbs_for_group<PACK>(sm, p1 % nb, p1 / nb, l16, xb);
      if (p2 < pairs) limbs_for_group<PACK>(sm, p2 % nb, p2 / nb, l16, xc);
      for (int pr = team + 3 * nteams; pr < pairs; pr += nteams) {
        load_x<XDT, PACK>(xr, k, pr % nb, g_begin + pr / nb, l16, xa);
        limbs_for_group<PACK>(sm, pr % nb, pr / nb, l16, xa);
      }
    }
    // this wave's LDS writes complete before its count is seen
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(sm.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (PACK != 0 && tab_by_rest && !prep) {
    // the table comes before this wave's weight loads: the loads would delay
    // it (it gates every wave's matrix work) more than it delays them
    for (int e = (prank - prep_waves) * 64 + lane; e < 256; e += 64 * (nw - prep_waves)) {
      write_b3_entry<PACK>(sm.lds, uint32_t(e));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the table writes come before the count
    if (lane == 0) __hip_atomic_fetch_add(sm.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (comp) {
#pragma unroll
    for (int d = 0; d < F::kDepth; ++d)
      issue_stage<PACK, ALIGNED>(wrs, srs, src, srow_scale, s_lo + d, s_full, stg[d], scl[d]);
  }
  // every prep wave (and table wave) has finished (each adds 1 exactly once,
  // and none waits on anything, so this ends)
  while (__hip_atomic_load(sm.ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < ready_target)
    __builtin_amdgcn_s_sleep(1);


  float yacc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) yacc[r] = 0.f;

  // ---- full stages, kDepth at a time so every register slot index is static
  // (waves beyond the compute waves have none)
  int s = comp ? s_lo : s_full;
  for (; s + F::kDepth <= s_full; s += F::kDepth) {
#pragma unroll
    for (int d = 0; d < F::kDepth; ++d)
      run_stage<PACK, NR, ALIGNED>(sm, my_stage, my_stage_addr, lc, wrs, srs, src, srow_scale, s + d, s_full, nb, stg[d],
                                   scl[d], yacc);
  }
#pragma unroll
  for (int d = 0; d < F::kDepth - 1; ++d)
    if (s + d < s_full)
      run_stage<PACK, NR, ALIGNED>(sm, my_stage, my_stage_addr, lc, wrs, srs, src, srow_scale, s + d, s_full, nb, stg[d],
                                   scl[d], yacc);

  if (comp && has_tail) {
    // partial last stage: fewer groups, 2-byte granular loads straight to LDS
    const int sg = ng - s_full * kStageGroups;
    const int rb = sg * F::kGroupBytes;
    wave_lds_fence();
    const int halves = 16 * rb / 2;
    for (int c = lane; c < halves; c += 64) {
      const int r = c / (rb / 2), cc = c - r * (rb / 2);
      uint16_t v = 0;
      if (row0 + r < n)
        v = *reinterpret_cast<const uint16_t*>(packed + (row0 + r) * row_bytes +
                                               (g_begin + s_full * kStageGroups) * F::kGroupBytes + 2 * cc);
      *reinterpret_cast<uint16_t*>(my_stage + r * F::kRowLds + 2 * cc) = v;
    }
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      h[i] = (i < sg && srow_scale != kNoLoad) ? scales[srow_scale + s_full * kStageGroups + i] : 0u;
    const uint32_t hw[4] = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    wave_lds_fence();
    stage_compute<PACK, NR>(sm, my_stage_addr, lc, sg, s_full * kStageGroups, hw, yacc);
  }

  // ---- add the ks partial sums of each tile (through the staging buffers)
  __syncthreads();
  float* red = reinterpret_cast<float*>(my_stage);
  if (comp) {
#pragma unroll
    for (int r = 0; r < NR; ++r) red[r * 64 + lane] = yacc[r];
  }
  __syncthreads();
  if (comp && kp == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float v = 0.f;
      for (int p = 0; p < ks; ++p)
        v += reinterpret_cast<const float*>(sm.stage + (wave + p) * F::kStageLds)[r * 64 + lane];
      const int b = 4 * r + q;
      if (b < nb && row0 + nl < n) {
        float* dst = y + int64_t(b) * n + row0 + nl;
        *dst = accumulate ? *dst + v : v;
      }
    }
  }
}

// ---------------------------------------------------------------- host side

struct Plan {
  int rt, ks, ng;
  bool extra_waves;  // launch 16 waves, the ones beyond rt * ks only building limbs
  int rot_waves;     // fused rotation: most waves that rotate at once (their scratch is in LDS)
  int kind;          // kernel packing kind: 0 2-bit, 1 base-3, 2 base-3 with the 32 KB table
};

// LDS beyond the staging region (ncomp compute waves' buffers) that the fused
// rotation's scratch needs: the nw waves' prep waves borrow the staging
// buffers, which are free until the matrix work starts.
inline int rot_extra(int stage_lds, int nw, int ncomp, int units, int rot_waves) {
  const int p = nw < units ? nw : units;
  const int need = (p < rot_waves ? p : rot_waves) * kRotScratch - ncomp * stage_lds;
  return need > 0 ? (need + 15) / 16 * 16 : 0;
}

template <int PACK>
struct KindInfo {
  static constexpr int kTable = Fmt<PACK>::kTable, kStageLds = Fmt<PACK>::kStageLds;
};

// Groups per launch whose limbs fit in the LDS the other regions leave, for
// ks K-part waves per tile (a multiple of 8 when at least 8).
inline int plan_groups(int table, int stage_lds, bool rot, int b, int groups, int rt, int ks, bool extra,
                       int rot_waves) {
  const int nw = extra ? kMaxWaves : rt * ks;
  const int ex = rot ? rot_extra(stage_lds, nw, rt * ks, 1 << 20, rot_waves) : 0;
  const int room = kLdsBytes - table - rt * ks * stage_lds - b * 134 - 46 - ex;
  const int per_group = kAGroup * b + b * 9;  // + b * 127 bytes of batch padding, b * 7 of e0 rows
  int ng = room > 0 ? room / per_group : 0;
  if (ng >= kStageGroups) ng = ng / kStageGroups * kStageGroups;
  return ng < groups ? ng : groups;
}

// Estimated time of a plan, in rough microseconds, from what measurements
// show dominates: a fixed cost per launch (launch, activation fetch, table),
// the longest wave's stages (about 2 us each; 8 % more with the 32 KB table,
// whose lookups take a shift), the limb passes (about 0.6 us each) or, when
// the rotation is fused, the rotation-and-limb passes (about 1.3 us each; a
// launch whose every wave rotates issues no weight load meanwhile: +1.5 us).
inline double plan_cost(bool rot, int b, int groups, int rt, int ks, int ng, bool extra, int rot_waves,
                        bool compact) {
  double c = 0.0;
  for (int g0 = 0; g0 < groups; g0 += ng) {
    const int ngi = groups - g0 < ng ? groups - g0 : ng;
    const int nst = (ngi + kStageGroups - 1) / kStageGroups;
    const int ksi = ks < nst ? ks : nst;
    const int ncomp = rt * ksi, nw = extra ? kMaxWaves : ncomp;
    const int crit = (nst + ksi - 1) / ksi;
    c += 4.0 + crit * 2.0 * (compact ? 1.08 : 1.0);
    if (rot) {
      const int units = b * (ngi / kStageGroups);
      int rw = nw < units ? nw : units;
      rw = rw < rot_waves ? rw : rot_waves;
      c += ((units + rw - 1) / rw) * 1.3;
      if (rw >= nw && nw < 15) c += 1.5;
    } else {
      const int pairs = b * ngi;
      const int by_need = (pairs + 11) / 12;
      int pw = nw < by_need ? nw : by_need;
      if (nw - ncomp > pw) pw = nw - ncomp;
      c += ((pairs + 4 * pw - 1) / (4 * pw)) * 0.6;
    }
  }
  return c;
}

// The cheapest base-3 plan over: the table size (64 KB, or 32 KB when the
// room buys fewer launches or more K-part waves), limb-only waves or not
// (batches of 2 and more), 8 or 16 rotation waves, and the K-part waves per
// tile.  rt, the tiles per workgroup, is the smallest that keeps the grid
// within one workgroup per CU.
template <bool ROT>
Plan make_plan(int packing, int b, int n, int k) {
  const int tiles = (n + 15) / 16;
  const int groups = k / kGroup;
  int rt = 1;
  while (rt < kMaxWaves && (tiles + rt - 1) / rt > 256) ++rt;
  Plan best{rt, 1, 0, false, 8, packing == 0 ? 0 : 1};
  double best_cost = 1e30;
  for (int kind = packing == 0 ? 0 : 1; kind <= (packing == 0 ? 0 : 2); ++kind) {
    const int table = kind == 0 ? KindInfo<0>::kTable : kind == 1 ? KindInfo<1>::kTable : KindInfo<2>::kTable;
    const int stage_lds = kind == 0 ? KindInfo<0>::kStageLds : KindInfo<1>::kStageLds;
    for (int extra = 0; extra <= (b > 1 ? 1 : 0); ++extra)
      for (int rw = 8; rw <= (ROT ? kMaxRotWaves : 8); rw += 8)
        for (int ks = kMaxWaves / rt; ks >= 1; --ks) {
          const int ng = plan_groups(table, stage_lds, ROT, b, groups, rt, ks, extra != 0, rw);
          if (ng < 1 || (ROT && ng % kStageGroups != 0)) continue;
          if (ng < kStageGroups && ng < groups && ks > 1) continue;
          if (ks > (ng + kStageGroups - 1) / kStageGroups) continue;
          const double c = plan_cost(ROT, b, groups, rt, ks, ng, extra != 0, rw, kind == 2);
          if (c < best_cost - 1e-9) {
            best_cost = c;
            best = Plan{rt, ks, ng, extra != 0, rw, kind};
          }
        }
  }
  return best;
}

template <int PACK, int NR, int XDT, bool ALIGNED, bool ROT>
void run_plan(const Plan& pl, const uint8_t* packed, const uint16_t* scales, const void* xr,
              const uint32_t* sign_bits, float* y, int b, int n, int k, hipStream_t s) {
  using F = Fmt<PACK>;
  const int groups = k / kGroup;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_mfma_kernel<PACK, NR, XDT, ALIGNED, ROT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  });
  const int tiles = (n + 15) / 16;
  const unsigned grid = unsigned((tiles + pl.rt - 1) / pl.rt);
  for (int g0 = 0; g0 < groups; g0 += pl.ng) {
    const int ng = groups - g0 < pl.ng ? groups - g0 : pl.ng;
    const int nst = (ng + kStageGroups - 1) / kStageGroups;
    const int ks = pl.ks < nst ? pl.ks : nst;
    const int nw = pl.extra_waves ? kMaxWaves : pl.rt * ks;
    const int extra = ROT ? rot_extra(F::kStageLds, nw, pl.rt * ks, b * (ng / 8), pl.rot_waves) : 0;
    const int lds = F::kTable + b * a_batch_stride(ng, F::kMfmas) + f_region_bytes(b, ng) +
                    pl.rt * ks * F::kStageLds + extra;
    gemv_mfma_kernel<PACK, NR, XDT, ALIGNED, ROT><<<grid, 64 * nw, lds, s>>>(
        packed, scales, xr, sign_bits, y, b, n, k, g0, ng, g0 > 0 ? 1 : 0, pl.rt, ks, pl.rot_waves);
  }
}

// The 2-bit plan (its loop is faster, so the cost weights above, set on
// base-3, misjudge it): the most K-part waves whose limbs still leave room for
// a stage each; 16 waves with limb-only ones when that saves a launch or the
// plain plan has at most 8 waves; 16 rotation waves when the launch has 15 or
// more waves (or limb-only ones) and they fit without more launches.
template <bool ROT>
Plan make_plan_2bit(int b, int n, int k) {
  const int tiles = (n + 15) / 16;
  const int groups = k / kGroup;
  const int table = KindInfo<0>::kTable, stage_lds = KindInfo<0>::kStageLds;
  int rt = 1;
  while (rt < kMaxWaves && (tiles + rt - 1) / rt > 256) ++rt;
  auto plan = [&](bool extra, int rw) {
    int ks = 1, ng = plan_groups(table, stage_lds, ROT, b, groups, rt, 1, extra, rw);
    if (extra) {
      // fewest launches first, then the most K-part waves that still get a stage each
      for (int c = 2; c <= kMaxWaves / rt; ++c) {
        const int g = plan_groups(table, stage_lds, ROT, b, groups, rt, c, extra, rw);
        if (g < kStageGroups || c > (g + kStageGroups - 1) / kStageGroups) break;
        if ((groups + g - 1) / g > (groups + ng - 1) / ng) break;
        ks = c;
        ng = g;
      }
    } else {
      for (ks = kMaxWaves / rt; ks >= 1; --ks) {
        ng = plan_groups(table, stage_lds, ROT, b, groups, rt, ks, extra, rw);
        if (ng >= kStageGroups || ks == 1) break;
      }
    }
    const int nst = (ng + kStageGroups - 1) / kStageGroups;
    if (ks > nst) ks = nst;
    if (ks < 1) ks = 1;
    return Plan{rt, ks, ng, extra, rw, 0};
  };
  auto launches = [&](const Plan& p) { return p.ng >= 1 ? (groups + p.ng - 1) / p.ng : 1 << 30; };
  Plan pl = plan(false, 8);
  if (b > 1) {
    const Plan px = plan(true, 8);
    if (launches(px) < launches(pl) || (launches(px) == launches(pl) && pl.rt * pl.ks <= 8)) pl = px;
  }
  if (ROT && (pl.extra_waves || pl.rt * pl.ks >= 15)) {
    const Plan p16 = plan(pl.extra_waves, kMaxRotWaves);
    if (launches(p16) <= launches(pl) && p16.ks >= pl.ks) pl = p16;
  }
  return pl;
}

template <int PACKING, int NR, int XDT, bool ALIGNED, bool ROT>
void launch_one(const uint8_t* packed, const uint16_t* scales, const void* xr, const uint32_t* sign_bits, float* y,
                int b, int n, int k, hipStream_t s) {
  const Plan pl = PACKING == 0 ? make_plan_2bit<ROT>(b, n, k) : make_plan<ROT>(PACKING, b, n, k);
  if (pl.ng < 1) return;  // unreachable for batch <= 8 (room for >= 8 groups); never loop without progress
  if constexpr (PACKING == 0) {
    run_plan<0, NR, XDT, ALIGNED, ROT>(pl, packed, scales, xr, sign_bits, y, b, n, k, s);
  } else {
    if (pl.kind == 2) run_plan<2, NR, XDT, ALIGNED, ROT>(pl, packed, scales, xr, sign_bits, y, b, n, k, s);
    else run_plan<1, NR, XDT, ALIGNED, ROT>(pl, packed, scales, xr, sign_bits, y, b, n, k, s);
  }
}

template <int PACK, int NR, int XDT>
void launch_a(const uint8_t* p, const uint16_t* sc, const void* xr, float* y, int b, int n, int k, hipStream_t s) {
  // 16-byte scale loads need every row's scales 16-byte aligned: K % 1024 == 0
  if ((k / kGroup) % 8 == 0) launch_one<PACK, NR, XDT, true, false>(p, sc, xr, nullptr, y, b, n, k, s);
  else launch_one<PACK, NR, XDT, false, false>(p, sc, xr, nullptr, y, b, n, k, s);
}

template <int PACK, int NR>
void launch_x(const uint8_t* p, const uint16_t* sc, const void* xr, int xdt, float* y, int b, int n, int k,
              hipStream_t s) {
  if (xdt == 0) launch_a<PACK, NR, 0>(p, sc, xr, y, b, n, k, s);
  else launch_a<PACK, NR, 1>(p, sc, xr, y, b, n, k, s);
}

template <int PACK, int NR>
void launch_rot(const uint8_t* p, const uint16_t* sc, const void* x, int xdt, const uint32_t* sb, float* y, int b,
                int n, int k, hipStream_t s) {
  // K % 1024 == 0 here, so the scales are always 16-byte aligned per row
  if (xdt == 0) launch_one<PACK, NR, 0, true, true>(p, sc, x, sb, y, b, n, k, s);
  else if (xdt == 1) launch_one<PACK, NR, 1, true, true>(p, sc, x, sb, y, b, n, k, s);
  else launch_one<PACK, NR, 2, true, true>(p, sc, x, sb, y, b, n, k, s);
}

}  // namespace

void launch_gemv(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr, int xr_dt, float* y,
                 int b, int n, int k, hipStream_t s) {
  if (packing == 0) {
    if (b <= 4) launch_x<0, 1>(packed, scales, xr, xr_dt, y, b, n, k, s);
    else launch_x<0, 2>(packed, scales, xr, xr_dt, y, b, n, k, s);
  } else {
    if (b <= 4) launch_x<1, 1>(packed, scales, xr, xr_dt, y, b, n, k, s);
    else launch_x<1, 2>(packed, scales, xr, xr_dt, y, b, n, k, s);
  }
}

void launch_linear(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dt,
                   const uint32_t* sign_bits, float* y, int b, int n, int k, hipStream_t s) {
  if (packing == 0) {
    if (b <= 4) launch_rot<0, 1>(packed, scales, x, x_dt, sign_bits, y, b, n, k, s);
    else launch_rot<0, 2>(packed, scales, x, x_dt, sign_bits, y, b, n, k, s);
  } else {
    if (b <= 4) launch_rot<1, 1>(packed, scales, x, x_dt, sign_bits, y, b, n, k, s);
    else launch_rot<1, 2>(packed, scales, x, x_dt, sign_bits, y, b, n, k, s);
  }
}

}  // namespace tb
