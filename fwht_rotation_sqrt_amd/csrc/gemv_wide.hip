// Batched decode product y[b][n] = sum_g s[n][g] sum_{k in g} t[n][k] x'[b][k]
// for up to 32 activation rows in ONE pass over the packed weights, on the
// fp16 matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulation).
// Pages: "Ternary Bonsai 2 27B release", sections "How the ternary weights
// reach 1.76 bit" (g128 fp16 scales; unpacking and the group scale fused into
// the product) and "Throughput" (decode streams every weight byte once per
// step, so a batch should share that stream).
//
// Layout of the work:
//   * Matrix rows are activation rows (one or two blocks of 16), matrix
//     columns are 16 weight rows (a "tile").  A workgroup owns T consecutive
//     tiles; its 8 waves split K by 128-groups.  A wave loads the activations
//     of one group once and uses them for all T tiles, so the activations are
//     read once per workgroup and the weights once per call.  At the end the
//     waves' partial sums meet in LDS and are added in wave order.
//   * Where the caller has room for partial sums, the workgroups of a call
//     can take K in parts (five tiles each, workgroup w: part w / rb): a part's
//     workgroups read only that part's activations and write its partial sums,
//     which a second launch adds in part order.  So rows too few to fill the
//     compute units with five-tile workgroups do not make every workgroup read
//     all of the activations for fewer tiles.
//   * Weight codes become fp16 B operands without a table: a 2-bit code c
//     moved to bits 10-11 of a half is the fp16 number c * 2^-14 (exponent
//     field c, mantissa 0: 0, 2^-14, 2^-13), and one AND with 0x0C000C00 takes
//     two codes that sit 16 bits apart into the two halves of a dword.  So the
//     lane's 32 codes (64 bits) become its 16 operand dwords with one shift
//     and one AND each.  Base-3 bytes are first turned into the same 64-bit
//     code word by LDS lookups (byte -> its five digits as a 10-bit field of
//     2-bit codes; digit d of a byte is the code c = t + 1 of its weight).
//   * t = c - 1: the product of a (tile, group) starts from the accumulator
//     -2^-14 sum_{k in g} x'[b][k], which one chain of matrix instructions
//     with the constant B operand -2^-14 gives once per group for all tiles.
//     Then acc += (2^14 s) * partial (2^14 s is exact in fp32).
//   * fp32 activations first get a power-of-two scale per (activation row,
//     group): 2^-e with e chosen so that the group's largest |x'| of the row
//     lands in [2^14, 2^15).  The scaled values are split into hi (mantissa cut
//     to fp16 precision) and lo = fp16(x - hi); both go through the matrix
//     cores into the same accumulator, and the group's partial sum is scaled
//     back by 2^e in fp32.  So any finite fp32 x' is carried to about 2^-21 of
//     its size, with an absolute floor near 2^-38 of the group's largest value.
//     fp16 activations are used as they are.
//
// K order inside a group (any order works when both operands use it): lane
// group q = lane / 16 of an instruction supplies the group's codes
// 32q .. 32q + 31 (its "word", code i at bits 2i).  In K-step j (0..3), dword
// p (0..3) of the operand holds word codes (a, a + 8) with
// a = 16 (j / 2) + 4 (j % 2) + p, and the activation operand holds
// x'[128 g + 32 q + a] and x'[... + a + 8] in the same halves.
#include "tb_internal.hpp"

#include <algorithm>

namespace tb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;                    // waves per workgroup, splitting K
constexpr uint32_t kCodeMask = 0x0C000C00u;  // bits 10-11 of both halves
constexpr uint32_t kNegUnitPair = 0x84008400u;  // two fp16 -2^-14
constexpr uint32_t kFar = 0x80000000u;       // buffer offset past any valid range: loads read 0
// a group index whose weight and scale offsets (< 2^31) are past any valid
// range: the buffers hold fewer than 2^29 bytes (N K < 2^31)
constexpr uint32_t kPastGroups = 1u << 26;
constexpr int kTableBytes = 256 * 256;       // base-3 table: entry e at 256 e, copy c at + 4c
constexpr int kRedSlot = 64 * 16;            // one float4 per lane

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  // raw buffer, 32-bit data format; offsets outside [0, bytes) read zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) uint8_t lds_byte;
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
  return *reinterpret_cast<__attribute__((address_space(3))) const T*>(
      reinterpret_cast<lds_byte*>(static_cast<uintptr_t>(addr)));
}
template <typename T>
__device__ __forceinline__ void lds_st(uint32_t addr, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(reinterpret_cast<lds_byte*>(static_cast<uintptr_t>(addr))) = v;
}

// The five base-3 digits of byte e (low digit first) as 2-bit codes, digit i
// at bits 2i.  Bytes above 242 are not codes; they read as five zero weights.
__device__ __forceinline__ uint32_t base3_code_field(uint32_t e) {
  if (e >= 243u) return 0x155u;
  uint32_t v = 0;
#pragma unroll
  for (int d = 0; d < 5; ++d) {
    v |= (e % 3u) << (2 * d);
    e /= 3u;
  }
  return v;
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const h2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Activation operands of one group for one block of 16 rows: hi (and lo) per
// K-step, from the lane's 32 consecutive values X[0..31].
template <int XF32>
struct ARaw {
  u32x4 v[XF32 ? 8 : 4];
};

template <int XF32>
__device__ __forceinline__ void a_issue(ARaw<XF32>& r, __amdgpu_buffer_rsrc_t xrs, uint32_t off) {
#pragma unroll
  for (int i = 0; i < (XF32 ? 8 : 4); ++i) r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off + 16u * i, 0, 0);
}

// The exponent e of the (activation row, group) scale: the largest |x'| of the row's 128 values
// (this lane's 32 and those of the lanes l ^ 16, l ^ 32, l ^ 48, which hold the row's other
// quarters) times 2^-e lies in [2^14, 2^15).  All four lanes get the same e.  e = 0 (no scale)
// for an all-zero group and for a largest value in [2^-6, 2^15): there the unscaled split already
// carries every value to 2^-18 of the largest (the fp16 subnormal floor is 2^-24), so typical
// activations skip the scaling work.
__device__ __forceinline__ int a_exponent(const ARaw<1>& r) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) m = max(m, r.v[i][c] & 0x7FFFFFFFu);
  auto p = __builtin_amdgcn_permlane16_swap(m, m, false, false);
  m = max(uint32_t(p[0]), uint32_t(p[1]));
  p = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  m = max(uint32_t(p[0]), uint32_t(p[1]));
  if (m == 0 || (m >= 0x3C800000u && m < 0x47000000u)) return 0;   // 0, or 2^-6 <= max < 2^15
  const int ef = int(m >> 23);                 // an fp32 subnormal maximum counts as exponent -126
  return (ef > 0 ? ef : 1) - 127 - 14;
}

template <int XF32, bool SCALED>
__device__ __forceinline__ void a_operands(const ARaw<XF32>& r, int e, u32x4 (&hi)[4], u32x4 (&lo)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int a = 16 * (j >> 1) + 4 * (j & 1) + p;
      if constexpr (XF32) {
        // scaled by 2^-e (exact unless far below the group's largest value); hi: cut to fp16
        // precision (exact in fp16 for 2^-14 <= |x| < 65520); lo: the exact rest, rounded to fp16
        uint32_t u0 = r.v[a >> 2][a & 3], u1 = r.v[(a + 8) >> 2][(a + 8) & 3];
        if constexpr (SCALED) {
          u0 = __float_as_uint(__builtin_amdgcn_ldexpf(__uint_as_float(u0), -e));
          u1 = __float_as_uint(__builtin_amdgcn_ldexpf(__uint_as_float(u1), -e));
        }
        const float h0 = __uint_as_float(u0 & 0xFFFFE000u), h1 = __uint_as_float(u1 & 0xFFFFE000u);
        hi[j][p] = pack_f16(h0, h1);
        lo[j][p] = pack_f16(__uint_as_float(u0) - h0, __uint_as_float(u1) - h1);
      } else {
        const uint32_t d0 = r.v[(a >> 1) >> 2][(a >> 1) & 3];
        const uint32_t d1 = r.v[((a >> 1) + 4) >> 2][((a >> 1) + 4) & 3];
        hi[j][p] = __builtin_amdgcn_perm(d1, d0, (a & 1) ? 0x07060302u : 0x05040100u);
        lo[j][p] = 0u;
      }
    }
  }
}

// The 16 B-operand dwords of a lane's 64-bit code word.
__device__ __forceinline__ void b_operands(u32x2 w, u32x4 (&b)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = 4 * (j & 1) + p, sh = 10 - 2 * i;
      const uint32_t v = w[j >> 1];
      b[j][p] = (sh >= 0 ? v << sh : v >> -sh) & kCodeMask;
    }
  }
}

// Base-3: the lane's 8 loaded bytes (group bytes 6q .. 6q + 7, trits
// 30q .. 30q + 39) -> code word of trits 32q .. 32q + 31.
__device__ __forceinline__ u32x2 base3_word(u32x2 raw, uint32_t tab, uint32_t shift) {
  uint32_t f[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
    f[m] = lds_ld<uint32_t>(__builtin_amdgcn_perm(tab, raw[m >> 2], 0x0C0C0004u | (uint32_t(m & 3) << 8)));
  const uint32_t lo = f[0] | (f[1] << 10) | (f[2] << 20) | (f[3] << 30);
  const uint32_t mid = (f[3] >> 2) | (f[4] << 8) | (f[5] << 18) | (f[6] << 28);
  const uint32_t hi = (f[6] >> 4) | (f[7] << 6);
  return u32x2{__builtin_amdgcn_alignbit(mid, lo, shift), __builtin_amdgcn_alignbit(hi, mid, shift)};
}

__device__ __forceinline__ floatx4 mfma(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// PACK: 0 = 2-bit codes, 1 = base-3 bytes.  MB: blocks of 16 activation rows.
// T: tiles of 16 weight rows per workgroup.  NW: waves per workgroup.  The
// weights and activations of the next group are loaded while this one
// computes (one register slot per tile).
template <int PACK, int XF32, int MB, int T, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_wide_kernel(const uint8_t* __restrict__ packed,
                                                            const uint16_t* __restrict__ scales,
                                                            const void* __restrict__ xr, float* __restrict__ y,
                                                            int nb, int n, int k, int rb, int gpp) {
  constexpr int kGroupBytes = PACK == 0 ? 32 : kB3GroupBytes;
  constexpr int kXsz = XF32 ? 4 : 2;
  constexpr uint32_t kTab = 0;  // the reduction area reuses the table's LDS once every wave has left the loop
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 15, q = lane >> 4;
  const int groups = k / kGroup;
  const uint32_t row_bytes = uint32_t(groups) * kGroupBytes;
  const __amdgpu_buffer_rsrc_t wrs = rsrc(packed, uint32_t(n) * row_bytes);
  const __amdgpu_buffer_rsrc_t srs = rsrc(scales, uint32_t(n) * uint32_t(groups) * 2u);
  const __amdgpu_buffer_rsrc_t xrs = rsrc(xr, uint32_t(nb) * uint32_t(k) * kXsz);

  // This workgroup's part of K: groups [gp0, gp1) (part blockIdx / rb; one part: all of K), with its
  // partial sums at y + part B N; then this wave's groups of the part.
  const int part = int(blockIdx.x) / rb, blk = int(blockIdx.x) - part * rb;
  const int gp0 = min(groups, part * gpp), gp1 = min(groups, gp0 + gpp);
  y += size_t(part) * size_t(nb) * size_t(n);
  const int per_wave = (gp1 - gp0 + NW - 1) / NW;
  const int g0 = min(gp1, gp0 + wave * per_wave), g1 = min(gp1, g0 + per_wave);

  // Per-lane offsets of group 0.  Rows past n and activation rows past nb
  // fall outside their buffers and read zero, and so does every group at or
  // past g1 (group kPastGroups, activation offset kFar).  Tile t lies t
  // wave-uniform strides further; with up to 3 tiles the T offsets are kept
  // in registers, with more they are recomputed at each load (registers).
  constexpr bool kEarly = T <= 3;  // also: all next-group weight loads at the group start
  const int tile0 = blk * T;
  const uint32_t row0 = uint32_t(16 * tile0 + r);
  const uint32_t wbase = row0 * row_bytes + uint32_t(PACK == 0 ? 8 * q : 6 * q), wstride = 16u * row_bytes;
  const uint32_t sbase = row0 * uint32_t(groups) * 2u, sstride = 32u * uint32_t(groups);
  uint32_t xbase[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xbase[mb] = (uint32_t(16 * mb + r) * uint32_t(k) + uint32_t(32 * q)) * kXsz;

  u32x2 wr[T];
  uint32_t sr[T];
  ARaw<XF32> an[MB];
  // group kPastGroups lies past the end of both buffers for every row
  auto group_or_past = [&](int g) { return g < g1 ? uint32_t(g) : kPastGroups; };
  uint32_t wb[T], sb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    wb[t] = wbase + uint32_t(t) * wstride;
    sb[t] = sbase + uint32_t(t) * sstride;
  }
  auto issue_w = [&](int t, uint32_t gg) {
    const uint32_t wo = kEarly ? wb[t] : wbase + uint32_t(t) * wstride;
    const uint32_t so = kEarly ? sb[t] : sbase + uint32_t(t) * sstride;
    wr[t] = __builtin_amdgcn_raw_buffer_load_b64(wrs, wo + gg * kGroupBytes, 0, 0);
    sr[t] = __builtin_amdgcn_raw_buffer_load_b16(srs, so + 2u * gg, 0, 0);
  };
  auto issue_a = [&](int g) {
    const bool ok = g < g1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a_issue<XF32>(an[mb], xrs, ok ? xbase[mb] + uint32_t(kGroup * kXsz) * g : kFar);
  };
  // the first groups' loads go out before the table is built
#pragma unroll
  for (int t = 0; t < T; ++t) issue_w(t, group_or_past(g0));
  issue_a(g0);

  const uint32_t tab = 4u * uint32_t(lane & 31);
  if constexpr (PACK == 1) {
    for (int i = threadIdx.x; i < kTableBytes / 16; i += 64 * NW) {
      const uint32_t e = uint32_t(i) >> 4;  // 16 chunks of 16 bytes per 256-byte entry
      const uint32_t v = (i & 15) < 8 ? base3_code_field(e) : 0u;
      lds_st<u32x4>(16u * uint32_t(i), u32x4{v, v, v, v});
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  floatx4 acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const u32x4 neg_unit = u32x4{kNegUnitPair, kNegUnitPair, kNegUnitPair, kNegUnitPair};
  for (int g = g0; g < g1; ++g) {
    ARaw<XF32> ac[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ac[mb] = an[mb];
    const uint32_t gn = group_or_past(g + 1);
    // With few tiles a group's work is short, so the next group's weights go
    // out now; with many, each tile's go out after its decode (registers).
    u32x2 wc[T];
    uint32_t sc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      wc[t] = wr[t];
      sc[t] = sr[t];
      if constexpr (kEarly) issue_w(t, gn);
    }
    // the next group's activations go out now (past g1 they read zero); with two fp32 row blocks
    // and 4-5 tiles, only once this group's have been turned into operands (registers)
    constexpr bool kLateA = XF32 && MB == 2 && T >= 4;
    if constexpr (!kLateA) issue_a(g + 1);

    // activation operands and the group's -2^-14 sum_k x'; with fp32 activations, eo[mb][i] is
    // the scale exponent of activation row 16 mb + 4 q + i, the row of accumulator element i
    u32x4 ahi[MB][4], alo[MB][4];
    floatx4 neg_sum[MB];
    int eo[MB][4];
    bool scaled = false;  // wave-uniform: some row of the group needs its scale
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int e = 0;
      if constexpr (XF32) {
        e = a_exponent(ac[mb]);
        const bool sc_mb = __builtin_amdgcn_ballot_w64(e != 0) != 0;
        scaled = scaled || sc_mb;
#pragma unroll
        for (int i = 0; i < 4; ++i) eo[mb][i] = sc_mb ? __shfl(e, 4 * q + i) : 0;
        if (sc_mb) a_operands<XF32, true>(ac[mb], e, ahi[mb], alo[mb]);
        else a_operands<XF32, false>(ac[mb], 0, ahi[mb], alo[mb]);
      } else {
        a_operands<XF32, false>(ac[mb], 0, ahi[mb], alo[mb]);
      }
      neg_sum[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        neg_sum[mb] = mfma(ahi[mb][j], neg_unit, neg_sum[mb]);
        if constexpr (XF32) neg_sum[mb] = mfma(alo[mb][j], neg_unit, neg_sum[mb]);
      }
    }
    if constexpr (kLateA) issue_a(g + 1);

#pragma unroll
    for (int t = 0; t < T; ++t) {
      u32x2 w = wc[t];
      const uint32_t sbits = sc[t];
      if constexpr (PACK == 1) w = base3_word(w, tab, 4u * uint32_t(q));
      u32x4 b[4];
      b_operands(w, b);
      if constexpr (!kEarly) issue_w(t, gn);  // this tile's next group
      floatx4 part[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) part[mb] = neg_sum[mb];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          part[mb] = mfma(ahi[mb][j], b[j], part[mb]);
          if constexpr (XF32) part[mb] = mfma(alo[mb][j], b[j], part[mb]);
        }
      const float s = 16384.f * static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sbits)));
      if (XF32 && scaled) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][mb][i] = fmaf(s, __builtin_amdgcn_ldexpf(part[mb][i], eo[mb][i]), acc[t][mb][i]);
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][mb][i] = fmaf(s, part[mb][i], acc[t][mb][i]);
      }
    }
  }

  // partial sums of the waves -> LDS -> added in wave order -> y
  if constexpr (PACK == 1) {  // the table is overwritten: every wave must be past its last lookup
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      lds_st<floatx4>(kTab + uint32_t((wave * T + t) * MB + mb) * kRedSlot + 16u * uint32_t(lane), acc[t][mb]);
  __syncthreads();
  constexpr int kCols = 16 * T;
  for (int f = threadIdx.x; f < kCols * 16 * MB; f += 64 * NW) {
    const int bl = f / kCols, nl = f % kCols;
    const int t = nl >> 4, rr = nl & 15, mb = bl >> 4, qq = (bl >> 2) & 3, i = bl & 3;
    const uint32_t a0 = kTab + uint32_t(t * MB + mb) * kRedSlot + 16u * uint32_t(16 * qq + rr) + 4u * uint32_t(i);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += lds_ld<float>(a0 + uint32_t(w * T * MB) * kRedSlot);
    const int col = 16 * tile0 + nl;
    if (bl < nb && col < n) y[size_t(bl) * size_t(n) + size_t(col)] = sum;
  }
}

template <int PACK, int XF32, int MB, int T>
void run(const uint8_t* p, const uint16_t* sc, const void* x, float* y, int b, int n, int k, int parts,
         hipStream_t s) {
  constexpr int NW = kWaves;
  constexpr int kRed = NW * T * MB * kRedSlot;
  constexpr int lds = PACK == 1 && kTableBytes > kRed ? kTableBytes : kRed;
  static const bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_wide_kernel<PACK, XF32, MB, T, NW>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    return true;
  }();
  (void)attr;
  const int tiles = (n + 15) / 16, rb = (tiles + T - 1) / T, groups = k / kGroup;
  gemv_wide_kernel<PACK, XF32, MB, T, NW><<<rb * parts, 64 * NW, lds, s>>>(p, sc, x, y, b, n, k, rb,
                                                                          (groups + parts - 1) / parts);
}

template <int PACK, int XF32, int MB>
void run_t(int t, const uint8_t* p, const uint16_t* sc, const void* x, float* y, int b, int n, int k, int parts,
           hipStream_t s) {
  switch (t) {
    case 1: run<PACK, XF32, MB, 1>(p, sc, x, y, b, n, k, parts, s); break;
    case 2: run<PACK, XF32, MB, 2>(p, sc, x, y, b, n, k, parts, s); break;
    case 3: run<PACK, XF32, MB, 3>(p, sc, x, y, b, n, k, parts, s); break;
    case 4: run<PACK, XF32, MB, 4>(p, sc, x, y, b, n, k, parts, s); break;
    default: run<PACK, XF32, MB, 5>(p, sc, x, y, b, n, k, parts, s); break;
  }
}

template <int PACK>
void run_pack(int xr_dt, const uint8_t* p, const uint16_t* sc, const void* x, float* y, int b, int n, int k,
              int parts, hipStream_t s) {
  // tiles per workgroup: the fewest that keep the grid within one workgroup per compute unit
  // (at most 5); two workgroups per unit with fewer tiles each ran 20-80 % slower at every shape
  // and batch (each workgroup fetches the whole activation block, and the operands built from it
  // serve fewer tiles).  In parts of K, five tiles per workgroup (wide_parts fills the units).
  const int tiles = (n + 15) / 16;
  const int t = parts > 1 ? 5 : std::min(5, std::max(1, (tiles + 255) / 256));
  const bool f32 = xr_dt == 0;
  if (b <= 16) {
    if (f32) run_t<PACK, 1, 1>(t, p, sc, x, y, b, n, k, parts, s);
    else run_t<PACK, 0, 1>(t, p, sc, x, y, b, n, k, parts, s);
  } else {
    if (f32) run_t<PACK, 1, 2>(t, p, sc, x, y, b, n, k, parts, s);
    else run_t<PACK, 0, 2>(t, p, sc, x, y, b, n, k, parts, s);
  }
}

}  // namespace

void launch_gemv_wide(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr, int xr_dt,
                      float* y, int b, int n, int k, hipStream_t s, float* part_y, int parts) {
  if (parts > 1 && part_y) {
    // parts of K on separate workgroups, partial sums to part_y [parts][b][n], then added in order
    if (packing == 0) run_pack<0>(xr_dt, packed, scales, xr, part_y, b, n, k, parts, s);
    else run_pack<1>(xr_dt, packed, scales, xr, part_y, b, n, k, parts, s);
    launch_sum_parts(part_y, y, b * n, parts, s);
    return;
  }
  if (packing == 0) run_pack<0>(xr_dt, packed, scales, xr, y, b, n, k, 1, s);
  else run_pack<1>(xr_dt, packed, scales, xr, y, b, n, k, 1, s);
}

}  // namespace tb
