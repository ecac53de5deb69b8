// Offline weight quantiser: full-precision weights into the rotated basis, then
// onto the g128 ternary grid.
//
// "Ternary Bonsai 2 27B release", section "How the ternary weights reach 1.76
// bit": the weights are moved into the fixed basis R = H_1024 S / 32 before they
// are ternarised, and inference computes W(Rx); so W' = W R_K^T, whose row n is
// R_K applied to row n of W.  "TensorSharp view of Ternary Bonsai 2 27B",
// section 2.1: each block has its own scale from its mean absolute weight times
// a correction, weights with |w / scale| under a threshold become 0 and the rest
// their sign, and the finer form tries candidate thresholds and keeps the one
// with the least reconstruction error.  Here, per 128-group with a = mean |w|:
// candidate j = 0..63 keeps |w| >= (j + 1) / 32 * a; its scale is the mean kept
// magnitude (the least-squares scale of its trits) rounded once to fp16; its
// error is the squared reconstruction error with that rounded scale; the least
// error wins, the lowest j on ties.  Every step runs in fp64, so the integer
// outcome (trits, fp16 scale) does not depend on summation order except at
// exact fp64 ties.
//
// One workgroup of 256 lanes per 1024-block of a row.  The block is rotated in
// fp64 in LDS (two butterfly stages in registers, eight through LDS); then each
// wave searches two groups with one candidate threshold per lane (64 lanes = 64
// candidates), reading the group's weights as LDS broadcasts, and the wave's
// minimum picks the winner.
#include "tb_internal.hpp"

namespace tb {
namespace {

constexpr int kThreads = 256;

// float64 -> fp16 bits, one rounding to nearest even.  v >= 0 (a mean of
// magnitudes); +inf and values from 65520 up give the fp16 infinity.
__device__ __forceinline__ uint32_t f64_to_f16_rne(double v) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const int ef = int(b >> 52);                 // biased exponent (sign is 0)
  if (ef >= 2047) return 0x7C00u;
  if (ef == 0) return 0u;                      // zero or an fp64 subnormal: far below fp16's least value
  const int e = ef - 1023;
  if (e >= 16) return 0x7C00u;
  const uint64_t m = (b & ((uint64_t(1) << 52) - 1)) | (uint64_t(1) << 52);
  int shift;
  uint32_t base;
  if (e >= -14) {                              // normal: 11 significant bits kept
    shift = 42;
    base = uint32_t(e + 14) << 10;             // (e + 15) << 10 minus the implicit 1024 of q
  } else {                                     // subnormal: units of 2^-24
    shift = 42 - 14 - e;
    base = 0;
    if (shift > 63) return 0u;
  }
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((uint64_t(1) << shift) - 1);
  const uint64_t half = uint64_t(1) << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;   // a carry moves into the exponent field
  return base + uint32_t(q);
}

__device__ __forceinline__ double f16_to_f64(uint32_t h) {
  const uint32_t ef = (h >> 10) & 31u, m = h & 1023u;
  if (ef == 31) return __longlong_as_double(0x7FF0000000000000ll);  // +inf (NaN never produced)
  if (ef == 0) return double(m) * 0x1p-24;
  return __longlong_as_double(int64_t(uint64_t(ef + 1008) << 52 | uint64_t(m) << 42));
}

template <bool ROT>
__global__ __launch_bounds__(kThreads) void ternarize_kernel(const float* __restrict__ w,
                                                             const uint32_t* __restrict__ sign_bits,
                                                             int8_t* __restrict__ trits,
                                                             uint16_t* __restrict__ scales,
                                                             int32_t* __restrict__ bad_count, int k) {
#pragma clang fp contract(off)
  __shared__ double v[kBlock];
  __shared__ int nbad;
  const int blocks = k / kBlock;
  const int row = int(blockIdx.x) / blocks;
  const int blk = int(blockIdx.x) - row * blocks;
  const int t = threadIdx.x;
  const int64_t base = int64_t(row) * k + int64_t(kBlock) * blk;
  if (t == 0) nbad = 0;

  const float4 f = *reinterpret_cast<const float4*>(w + base + 4 * t);
  double a0 = f.x, a1 = f.y, a2 = f.z, a3 = f.w;
  if constexpr (ROT) {
    const uint32_t s = sign_bits[(kBlock * blk + 4 * t) >> 5] >> ((4 * t) & 31);
    if (s & 1u) a0 = -a0;
    if (s & 2u) a1 = -a1;
    if (s & 4u) a2 = -a2;
    if (s & 8u) a3 = -a3;
    // stages of span 1 and 2 inside the lane's four consecutive elements
    const double b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
    a0 = b0 + b2;
    a1 = b1 + b3;
    a2 = b0 - b2;
    a3 = b1 - b3;
  }
  v[4 * t] = a0;
  v[4 * t + 1] = a1;
  v[4 * t + 2] = a2;
  v[4 * t + 3] = a3;
  __syncthreads();
  if constexpr (ROT) {
    for (int h = 4; h < kBlock; h <<= 1) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int p = t + kThreads * r;
        const int i = (p / h) * 2 * h + (p % h);
        const double x = v[i], y = v[i + h];
        v[i] = x + y;
        v[i + h] = x - y;
      }
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) v[t + kThreads * r] *= 0.03125;  // 1/32, exact
    __syncthreads();
  }

  const int lane = t & 63, wave = t >> 6;
  for (int r = 0; r < 2; ++r) {
    const int g = 2 * wave + r;
    const double* vg = v + kGroup * g;
    const double e0 = vg[lane], e1 = vg[lane + 64];
    const bool finite = __all(isfinite(e0) && isfinite(e1));
    // mean |w|: the xor butterfly leaves the same sum, bit for bit, in every lane
    double sum = finite ? fabs(e0) + fabs(e1) : 0.0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    const double a = sum / kGroup;
    uint32_t h_best = 0;
    int j_best = -1;
    if (finite && a > 0.0) {
      const double theta = double(lane + 1) * 0.03125 * a;
      double kept = 0.0;
      int cnt = 0;
      for (int i = 0; i < kGroup; ++i) {
        const double m = fabs(vg[i]);
        if (m >= theta) {
          kept += m;
          ++cnt;
        }
      }
      const uint32_t h = f64_to_f16_rne(cnt ? kept / cnt : 0.0);
      const double s = f16_to_f64(h);
      double err = 0.0;
      for (int i = 0; i < kGroup; ++i) {
        const double m = fabs(vg[i]);
        const double d = m >= theta ? m - s : m;
        err += d * d;
      }
      double e_best = err;
      j_best = lane;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const double oe = __shfl_xor(e_best, o);
        const int oj = __shfl_xor(j_best, o);
        if (oe < e_best || (oe == e_best && oj < j_best)) {
          e_best = oe;
          j_best = oj;
        }
      }
      h_best = uint32_t(__shfl(int(h), j_best));
    }
    const bool bad = !finite || h_best == 0x7C00u;
    int8_t t0 = 0, t1 = 0;
    if (!bad && j_best >= 0) {
      const double theta = double(j_best + 1) * 0.03125 * a;
      t0 = fabs(e0) >= theta ? (e0 > 0.0 ? 1 : -1) : 0;
      t1 = fabs(e1) >= theta ? (e1 > 0.0 ? 1 : -1) : 0;
    }
    trits[base + kGroup * g + lane] = t0;
    trits[base + kGroup * g + 64 + lane] = t1;
    if (lane == 0) {
      scales[int64_t(row) * (k / kGroup) + (kBlock / kGroup) * blk + g] = bad ? 0 : uint16_t(h_best);
      if (bad) atomicAdd(&nbad, 1);
    }
  }
  __syncthreads();
  if (t == 0 && nbad && bad_count) atomicAdd(bad_count, nbad);
}

}  // namespace

void launch_ternarize(const float* w, int64_t n, int64_t k, const uint32_t* sign_bits, int8_t* trits,
                      uint16_t* scales, int32_t* bad_count, hipStream_t stream) {
  const unsigned grid = unsigned(n * (k / kBlock));
  if (sign_bits)
    ternarize_kernel<true><<<grid, kThreads, 0, stream>>>(w, sign_bits, trits, scales, bad_count, int(k));
  else
    ternarize_kernel<false><<<grid, kThreads, 0, stream>>>(w, nullptr, trits, scales, bad_count, int(k));
}

}  // namespace tb
