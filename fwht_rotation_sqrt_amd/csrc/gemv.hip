// Decode product y[b][n] = sum_g s[n][g] sum_{k in g} t[n][k] xr[b][k]  (batch 1..8).
//
// Pages: "Ternary Bonsai 2 27B release", section "How the ternary weights
// reach 1.76 bit" (g128 fp16 scales, unpack and scale fused in the product)
// and section "Throughput" (decode streams the packed weights once per token).
//
// The weights never become fp16.  Each ternary code c = t + 1 in {0, 1, 2} is
// used directly as an fp4 (e2m1) matrix-core operand: the nibble c encodes
// c / 2, so sum_k t_k x_k = 2 sum_k (c_k / 2) x_k - sum_k x_k.
//   * 2-bit codes: a dword of 16 codes splits into two dwords of 8 nibbles with
//     one AND (and one shift): the 2-bit fields already are the nibble values.
//   * base-3 bytes: one LDS table lookup turns a byte into a dword holding its
//     five base-3 digits as nibbles (the table has 32 bank-spread copies so a
//     wave's lookups do not conflict).
// The activations become three fp8 (e4m3) limbs per element, per 128-group
// scaled by a power of two so the largest magnitude lies in [128, 256):
//   x * 2^sig = l0 + l1/16 + l2/256, each limb the e4m3 rounding of what is
//   left, so the reconstruction error is about 2^-12 of the element.
// One v_mfma_scale_f32_16x16x128_f8f6f4 multiplies 16 weight rows by 128
// K-slots; its A rows are (batch, limb) pairs (row 4b + limb), so one matrix
// instruction serves up to four batch rows.  Per group the limbs are combined
// in fp32, the sum of the group's activations is subtracted, and the fp16
// scale and 2^-sig are applied, all in fp32.
//
// Work split: a workgroup of kWaves waves; each wave owns a tile of 16 weight
// rows over all of K.  The packed tile streams through registers kDepth
// stages ahead (a stage is 8 groups = 1024 weights per row), is written to a
// per-wave LDS buffer with coalesced 16-byte loads, and is read back in the
// matrix-core operand layout.  The workgroup prepares the activation limbs
// for as many groups as fit in LDS, with two barriers per such chunk (one
// chunk covers all of K at batch 1 for K up to 5120 x 2).
#include "tb_internal.hpp"

#include <mutex>

namespace tb {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 16;       // waves per workgroup
constexpr int kDepth = 2;           // staged stages in flight per wave (registers)
constexpr int kStageGroups = 8;     // groups per stage (1024 weights per row)
constexpr int kCopies = 32;         // bank-spread copies of the base-3 table
constexpr int kLdsBytes = 160 * 1024;
constexpr int kTeam = 16;           // threads preparing one (batch, group) of activations
constexpr uint32_t kNoLoad = 0x80000000u;  // buffer offset past any buffer: reads zero

template <int PACK>
struct Fmt {
  static constexpr int kGroupBytes = PACK == 0 ? 32 : kB3GroupBytes;
  static constexpr int kMfmas = PACK == 0 ? 1 : 2;             // matrix instructions per group
  static constexpr int kRowStage = kGroupBytes * kStageGroups;  // 256 or 208 bytes
  static constexpr int kChunksPerRow = kRowStage / 16;          // 16 or 13
  static constexpr int kStageChunks = 16 * kChunksPerRow;       // 256 or 208
  static constexpr int kLoads = (kStageChunks + 63) / 64;       // 4
  static constexpr int kScaleOff = 16 * kRowStage + 32;         // + pad for operand over-reads
  static constexpr int kStageLds = kScaleOff + 16 * 16;         // + the stage's scales [16 rows][8]
  static constexpr int kTable = PACK == 1 ? 256 * kCopies * 4 : 0;
};

// K-slot of trit tau (0..127) of a group, and which matrix instruction of the
// group it belongs to.  B operand: lane group q supplies slots 32q..32q+31.
template <int PACK>
__device__ __forceinline__ int slot_of(int tau, int* mi) {
  if constexpr (PACK == 0) {
    // dword w of lane group q: w=0 even / w=1 odd codes of bytes 8q..8q+3,
    // w=2 / w=3 the same for bytes 8q+4..8q+7; nibble j = code 2j (+1).
    const int q = tau >> 5, r = tau & 31;
    const int w = ((r >> 4) << 1) | (r & 1);
    *mi = 0;
    return 32 * q + 8 * w + ((r & 15) >> 1);
  } else {
    // byte p = tau / 5 goes to instruction p / 16, lane group (p % 16) / 4,
    // dword p % 4; digit d = tau % 5 is nibble d of that dword.
    const int p = tau / 5, d = tau - 5 * p;
    *mi = p >> 4;
    const int pp = p & 15;
    return 32 * (pp >> 2) + 8 * (pp & 3) + d;
  }
}

// A operand slot s of lane group q' reads K-slot 16q'+s (s < 16) or 64+16q'+s-16.
struct Smem {
  uint8_t* stage;   // waves x kStageLds (reused for the K-part reduction at the end)
  uint32_t* table;  // 256 x kCopies (base-3)
  uint8_t* a;       // [ng][mfmas][B][3][128] activation limbs in K-slot order
  float2* f;        // [ng][B] = {2^-sig, sum of reconstructed activations}
};

__device__ __forceinline__ uint32_t base3_nibbles(uint32_t e) {
  if (e >= 243u) return 0u;
  uint32_t v = 0;
#pragma unroll
  for (int d = 0; d < 5; ++d) {
    v |= (e % 3u) << (4 * d);
    e /= 3u;
  }
  return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer, 32-bit data format; offsets outside [0, bytes) read zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}

// Eight consecutive activations of batch row b, group g (absolute), from lane
// (tid % 16) of a team.
template <int XDT>
__device__ __forceinline__ void load_x8(const void* __restrict__ xr, int k, int b, int g, int l16, float x[8]) {
  const int64_t base = int64_t(b) * k + int64_t(g) * kGroup + 8 * l16;
  if constexpr (XDT == 0) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(xr) + base);
    const float4 u = p[0], v = p[1];
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xr) + base);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = float(__builtin_bit_cast(_Float16, uint16_t(w[i] & 0xFFFFu)));
      x[2 * i + 1] = float(__builtin_bit_cast(_Float16, uint16_t(w[i] >> 16)));
    }
  }
}

// Split eight activations of one (batch, group) into three e4m3 limbs at the
// group's power-of-two scale and write them to their K-slots; lane 0 of the
// team records {2^-sig, sum of the reconstructed values}.  The limb values
// are decoded back from the stored bytes, so the residuals are exact whatever
// the conversion's rounding.
template <int PACK>
__device__ __forceinline__ void limbs_for_group(const Smem& sm, int nb, int b, int g, int l16, const float x[8]) {
  constexpr int M = Fmt<PACK>::kMfmas;
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(x[i]));
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kTeam));
  int sig = 0;
  if (mx > 0.f) {
    int e;
    frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
    sig = 8 - e;     // mx * 2^sig in [128, 256)
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float xa = ldexpf(x[i], sig), xb = ldexpf(x[i + 1], sig);
    const int p0 = __builtin_amdgcn_cvt_pk_fp8_f32(xa, xb, 0, false);
    const float a0 = __builtin_amdgcn_cvt_f32_fp8(p0, 0), b0 = __builtin_amdgcn_cvt_f32_fp8(p0, 1);
    const float ra = (xa - a0) * 16.f, rb = (xb - b0) * 16.f;
    const int p1 = __builtin_amdgcn_cvt_pk_fp8_f32(ra, rb, 0, false);
    const float a1 = __builtin_amdgcn_cvt_f32_fp8(p1, 0), b1 = __builtin_amdgcn_cvt_f32_fp8(p1, 1);
    const float sa = (ra - a1) * 16.f, sb = (rb - b1) * 16.f;
    const int p2 = __builtin_amdgcn_cvt_pk_fp8_f32(sa, sb, 0, false);
    const float a2 = __builtin_amdgcn_cvt_f32_fp8(p2, 0), b2 = __builtin_amdgcn_cvt_f32_fp8(p2, 1);
    sum += (a0 + a1 * 0.0625f + a2 * 0.00390625f) + (b0 + b1 * 0.0625f + b2 * 0.00390625f);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int mi;
      const int slot = slot_of<PACK>(8 * l16 + i + h, &mi);
      uint8_t* row = sm.a + ((((g * M + mi) * nb + b) * 3) << 7) + slot;
      row[0] = uint8_t(p0 >> (8 * h));
      row[128] = uint8_t(p1 >> (8 * h));
      row[256] = uint8_t(p2 >> (8 * h));
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, kTeam);
  if (l16 == 0) sm.f[g * nb + b] = make_float2(ldexpf(1.f, -sig), sum);
}

// ---------------------------------------------------------------- matrix work

// B operand(s) of group g for row (lane & 15) from the staged bytes, then one
// (2-bit) or two (base-3) instructions per row set.
template <int PACK, int NR>
__device__ __forceinline__ void group_mfma(const Smem& sm, const uint8_t* stage, int rb, int g, int gc, int nb,
                                           v4f out[NR]) {
  using F = Fmt<PACK>;
  const int lane = threadIdx.x & 63, nl = lane & 15, q = lane >> 4;
  const int a_limb = nl & 3, a_bq = nl >> 2;
  v8i bop[F::kMfmas];
  if constexpr (PACK == 0) {
    const uint2 w = *reinterpret_cast<const uint2*>(stage + nl * rb + 32 * g + 8 * q);
    const uint32_t m = 0x33333333u;
    bop[0] = v8i{int(w.x & m), int((w.x >> 2) & m), int(w.y & m), int((w.y >> 2) & m), 0, 0, 0, 0};
  } else {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int o = nl * rb + kB3GroupBytes * g + 16 * mi + 4 * q;
      const uint32_t* p32 = reinterpret_cast<const uint32_t*>(stage + (o & ~3));
      const uint32_t bytes = __builtin_amdgcn_alignbyte(p32[1], p32[0], uint32_t(o & 3));
      int dw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t e = (bytes >> (8 * w)) & 0xFFu;
        uint32_t v = sm.table[e * kCopies + (lane & (kCopies - 1))];
        if (mi == 1 && 4 * q + w >= kB3GroupBytes - 16) v = 0;
        dw[w] = int(v);
      }
      bop[mi] = v8i{dw[0], dw[1], dw[2], dw[3], 0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    v4f a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mi = 0; mi < F::kMfmas; ++mi) {
      v8i aop = {0, 0, 0, 0, 0, 0, 0, 0};
      const int b = 4 * r + a_bq;
      if (a_limb < 3 && b < nb) {
        const uint8_t* ap = sm.a + ((((gc * F::kMfmas + mi) * nb + b) * 3 + a_limb) << 7) + 16 * q;
        const uint4 lo = *reinterpret_cast<const uint4*>(ap);
        const uint4 hi = *reinterpret_cast<const uint4*>(ap + 64);
        aop = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
      a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[mi], a4, 0, 4, 0, 127, 0, 127);
    }
    out[r] = a4;
  }
  // keep the next group's operand loads from being hoisted above this point
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of one group.  D rows 4*(lane/16)+i: this lane holds batch 4r + q,
// limbs i = 0..2.  Branch-free on purpose: a matrix instruction must run with
// the whole wave active, so its result may not feed a lane-divergent block.
template <int NR>
__device__ __forceinline__ void group_epilogue(const Smem& sm, const v4f acc[NR], float sc, int gc, int nb,
                                               float yacc[NR]) {
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int b = 4 * r + q;
    const float2 fs = sm.f[gc * nb + min(b, nb - 1)];
    const float p = acc[r][0] + acc[r][1] * 0.0625f + acc[r][2] * 0.00390625f;
    const float contrib = (sc * fs.x) * fmaf(2.f, p, -fs.y);
    yacc[r] += b < nb ? contrib : 0.f;
  }
}

// fp16 scale of group g of row (lane & 15) from the stage's LDS copy
template <int PACK>
__device__ __forceinline__ float scale_of(const uint8_t* stage, int g) {
  const int nl = threadIdx.x & 15;
  return float(*reinterpret_cast<const _Float16*>(stage + Fmt<PACK>::kScaleOff + 16 * nl + 2 * g));
}

// All groups of one staged block (sg <= 8 groups).  A rolled loop on purpose:
// unrolling lets the compiler hoist every group's operand loads at once and
// run out of registers.  The epilogue of group g-1 runs after the
// instructions of group g are issued, hiding the matrix-core latency.
template <int PACK, int NR>
__device__ __forceinline__ void stage_compute(const Smem& sm, const uint8_t* stage, int rb, int sg, int gc0,
                                              int nb, float yacc[NR]) {
  v4f prev[NR], cur[NR];
  group_mfma<PACK, NR>(sm, stage, rb, 0, gc0, nb, prev);
#pragma unroll 1
  for (int g = 1; g < sg; ++g) {
    group_mfma<PACK, NR>(sm, stage, rb, g, gc0 + g, nb, cur);
    group_epilogue<NR>(sm, prev, scale_of<PACK>(stage, g - 1), gc0 + g - 1, nb, yacc);
#pragma unroll
    for (int r = 0; r < NR; ++r) prev[r] = cur[r];
  }
  group_epilogue<NR>(sm, prev, scale_of<PACK>(stage, sg - 1), gc0 + sg - 1, nb, yacc);
}

// ---------------------------------------------------------------- streaming

// Issue the loads of full stage s into registers.  Every lane issues every
// load (a lane with nothing to load, or a stage past this wave's range, uses
// an offset past the end of the buffer and reads zero), so the compiler
// counts outstanding loads exactly and keeps kDepth stages in flight.
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
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One full stage: registers -> this wave's LDS buffer, matrix work, then
// refill the same register slot with stage s + kDepth.
template <int PACK, int NR, bool ALIGNED>
__device__ __forceinline__ void run_stage(const Smem& sm, uint8_t* my_stage, __amdgpu_buffer_rsrc_t wrs,
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
    if (c < F::kStageChunks) reinterpret_cast<uint4*>(my_stage)[c] = regs[j];
  }
  if (lane < 16)
    *reinterpret_cast<uint4*>(my_stage + F::kScaleOff + 16 * lane) = make_uint4(sreg[0], sreg[1], sreg[2], sreg[3]);
  wave_lds_fence();
  stage_compute<PACK, NR>(sm, my_stage, F::kRowStage, kStageGroups, s * kStageGroups, nb, yacc);
  issue_stage<PACK, ALIGNED>(wrs, srs, src, srow_scale, s + kDepth, s_end, regs, sreg);
}

// ---------------------------------------------------------------- kernel

// One launch covers groups [g_begin, g_begin + ng) of every row (the host
// issues several launches, each adding into y, when the activation limbs of
// all of K do not fit in LDS; a wave owns the same rows in every launch and
// launches on one stream run in order).  A workgroup holds rt row tiles of
// 16 rows; the stages of a tile are split over ks waves, and the ks partial
// sums are added through LDS at the end.
template <int PACK, int NR, int XDT, bool ALIGNED>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_mfma_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales, const void* __restrict__ xr,
    float* __restrict__ y, int nb, int n, int k, int g_begin, int ng, int accumulate, int rt, int ks) {
  using F = Fmt<PACK>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nthreads = 64 * rt * ks;
  const int groups = k / kGroup;
  const int row_bytes = F::kGroupBytes * groups;
  const int tile = wave / ks, kp = wave - tile * ks;
  const int row0 = (blockIdx.x * rt + tile) * 16;
  const int nl = lane & 15, q = lane >> 4;

  Smem sm;
  sm.stage = smem;
  sm.table = reinterpret_cast<uint32_t*>(smem + rt * ks * F::kStageLds);
  sm.a = reinterpret_cast<uint8_t*>(sm.table) + F::kTable;
  const int a_bytes = ng * F::kMfmas * nb * 3 * 128;
  sm.f = reinterpret_cast<float2*>(sm.a + a_bytes);
  uint8_t* my_stage = sm.stage + wave * F::kStageLds;

  // ---- activations of this thread's first (batch, group): loads go out first
  const int team = tid / kTeam, l16 = tid % kTeam, nteams = nthreads / kTeam;
  const int pairs = ng * nb;
  float xv[8];
  {
    const int pr = team < pairs ? team : 0;
    const int g = pr / nb, b = pr - g * nb;
    load_x8<XDT>(xr, k, b, g_begin + g, l16, xv);
  }

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

  uint4 stg[kDepth][F::kLoads];
  uint32_t scl[kDepth][4];
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    issue_stage<PACK, ALIGNED>(wrs, srs, src, srow_scale, s_lo + d, s_full, stg[d], scl[d]);

  // ---- workgroup set-up while the weights stream in
  if constexpr (PACK == 1) {
    for (int e = tid; e < 256; e += nthreads) {
      const uint32_t v = base3_nibbles(uint32_t(e));
      uint4* dst = reinterpret_cast<uint4*>(sm.table + e * kCopies);
#pragma unroll
      for (int i = 0; i < kCopies / 4; ++i) dst[i] = make_uint4(v, v, v, v);
    }
  }
  for (int i = tid; i < a_bytes / 16; i += nthreads) reinterpret_cast<uint4*>(sm.a)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  if (team < pairs) {
    const int g = team / nb, b = team - g * nb;
    limbs_for_group<PACK>(sm, nb, b, g, l16, xv);
  }
  for (int pr = team + nteams; pr < pairs; pr += nteams) {
    const int g = pr / nb, b = pr - g * nb;
    load_x8<XDT>(xr, k, b, g_begin + g, l16, xv);
    limbs_for_group<PACK>(sm, nb, b, g, l16, xv);
  }
  __syncthreads();

  float yacc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) yacc[r] = 0.f;

  // ---- full stages, kDepth at a time so every register slot index is static
  int s = s_lo;
  for (; s + kDepth <= s_full; s += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      run_stage<PACK, NR, ALIGNED>(sm, my_stage, wrs, srs, src, srow_scale, s + d, s_full, nb, stg[d], scl[d],
                                   yacc);
  }
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (s + d < s_full)
      run_stage<PACK, NR, ALIGNED>(sm, my_stage, wrs, srs, src, srow_scale, s + d, s_full, nb, stg[d], scl[d],
                                   yacc);

  if (has_tail) {
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
      reinterpret_cast<uint16_t*>(my_stage)[c] = v;
    }
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      h[i] = (i < sg && srow_scale != kNoLoad) ? scales[srow_scale + s_full * kStageGroups + i] : 0u;
    if (lane < 16)
      *reinterpret_cast<uint4*>(my_stage + F::kScaleOff + 16 * lane) =
          make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    wave_lds_fence();
    stage_compute<PACK, NR>(sm, my_stage, rb, sg, s_full * kStageGroups, nb, yacc);
  }

  // ---- add the ks partial sums of each tile (through the staging buffers)
  __syncthreads();
  float* red = reinterpret_cast<float*>(my_stage);
#pragma unroll
  for (int r = 0; r < NR; ++r) red[r * 64 + lane] = yacc[r];
  __syncthreads();
  if (kp == 0) {
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
};

template <int PACK>
Plan make_plan(int b, int n, int k) {
  using F = Fmt<PACK>;
  const int tiles = (n + 15) / 16;
  const int groups = k / kGroup;
  // smallest tiles-per-workgroup that keeps the grid within one workgroup per CU
  int rt = 1;
  while (rt < kMaxWaves && (tiles + rt - 1) / rt > 256) ++rt;
  // groups per launch: activation limbs of all launches' groups must fit in LDS
  const int fixed = kMaxWaves * F::kStageLds + F::kTable;
  const int per_group = F::kMfmas * b * 3 * 128 + b * 8;
  int ng = (kLdsBytes - fixed) / per_group;
  ng = ng / kStageGroups * kStageGroups;  // >= 8 for every batch <= 8
  if (ng > groups) ng = groups;
  const int nst = (ng + kStageGroups - 1) / kStageGroups;
  int ks = kMaxWaves / rt;
  if (ks > nst) ks = nst;
  return Plan{rt, ks, ng};
}

template <int PACK, int NR, int XDT, bool ALIGNED>
void launch_one(const uint8_t* packed, const uint16_t* scales, const void* xr, float* y, int b, int n, int k,
                hipStream_t s) {
  using F = Fmt<PACK>;
  const int groups = k / kGroup;
  const Plan pl = make_plan<PACK>(b, n, k);
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_mfma_kernel<PACK, NR, XDT, ALIGNED>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  });
  const int tiles = (n + 15) / 16;
  const unsigned grid = unsigned((tiles + pl.rt - 1) / pl.rt);
  const int per_group = F::kMfmas * b * 3 * 128 + b * 8;
  for (int g0 = 0; g0 < groups; g0 += pl.ng) {
    const int ng = groups - g0 < pl.ng ? groups - g0 : pl.ng;
    const int nst = (ng + kStageGroups - 1) / kStageGroups;
    const int ks = pl.ks < nst ? pl.ks : nst;
    const int lds = pl.rt * ks * F::kStageLds + F::kTable + ng * per_group;
    gemv_mfma_kernel<PACK, NR, XDT, ALIGNED><<<grid, 64 * pl.rt * ks, lds, s>>>(
        packed, scales, xr, y, b, n, k, g0, ng, g0 > 0 ? 1 : 0, pl.rt, ks);
  }
}

template <int PACK, int NR, int XDT>
void launch_a(const uint8_t* p, const uint16_t* sc, const void* xr, float* y, int b, int n, int k, hipStream_t s) {
  // 16-byte scale loads need every row's scales 16-byte aligned: K % 1024 == 0
  if ((k / kGroup) % 8 == 0) launch_one<PACK, NR, XDT, true>(p, sc, xr, y, b, n, k, s);
  else launch_one<PACK, NR, XDT, false>(p, sc, xr, y, b, n, k, s);
}

template <int PACK, int NR>
void launch_x(const uint8_t* p, const uint16_t* sc, const void* xr, int xdt, float* y, int b, int n, int k,
              hipStream_t s) {
  if (xdt == 0) launch_a<PACK, NR, 0>(p, sc, xr, y, b, n, k, s);
  else launch_a<PACK, NR, 1>(p, sc, xr, y, b, n, k, s);
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

}  // namespace tb
