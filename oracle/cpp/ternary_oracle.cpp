// Plain C++ reference for y = W(Rx) on packed ternary weights, and for the two packings
// (test infrastructure only).
//
// Only the tests and the benchmark's CPU-baseline leg load this library.  It is
// a slow, literal transcription of the same definitions as the numpy oracle
// (oracle/ternary.py), in float64, shares nothing with the HIP path, and is
// cross-checked against the numpy oracle and a closed form by the CPU tests.
//
// Pages (title and section):
//   "Bonsai low-bit learning path", section "Understand 1.6 bit with five
//   numbers": trit i of a base-3 byte b is (b / 3^i) mod 3 - 1.
//   "Ternary Bonsai 2 27B release", section "How the ternary weights reach
//   1.76 bit": one fp16 scale per 128 weights; R = H_1024 S / sqrt(1024)
//   applied blockwise; f(x) = W(Rx).
//   "TensorSharp view of Ternary Bonsai 2 27B", section 3.2: Sylvester-ordered
//   Hadamard matrix, here through its closed form H[i][j] = (-1)^popcount(i & j).
// Layout readings (as in the numpy oracle): 2-bit code c = t + 1 at bits
// 2 (k mod 4) of byte k / 4; base-3 groups of 128 weights in 26 bytes, five
// trits per byte, first trit least significant, the last byte holding three
// trits and two pads; scales fp16 [N][K/128]; the sign mask bit set = -1.
#include <stdint.h>

#include <thread>
#include <vector>

namespace {

double half_to_double(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  const double sign = (h & 0x8000) ? -1.0 : 1.0;
  if (e == 0) return sign * m * (1.0 / 16777216.0);  // m * 2^-24
  if (e == 31) return m ? 0.0 / 0.0 : sign / 0.0;
  double v = 1.0 + m / 1024.0;
  int p = e - 15;
  while (p > 0) { v *= 2.0; --p; }
  while (p < 0) { v *= 0.5; ++p; }
  return sign * v;
}

int trit_2bit(const uint8_t* row, int64_t k) {
  const int c = (row[k / 4] >> (2 * (k % 4))) & 3;
  return c == 3 ? 0 : c - 1;  // code 11 is invalid; read as 0
}

int trit_base3(const uint8_t* row, int64_t k) {
  const int64_t g = k / 128, i = k % 128;
  int b = row[26 * g + i / 5];
  if (b >= 243) return 0;  // not a code
  for (int d = 0; d < i % 5; ++d) b /= 3;
  return b % 3 - 1;
}

int popcount(unsigned v) {
  int c = 0;
  while (v) { c += v & 1u; v >>= 1; }
  return c;
}

// x' = R_K x for one row: each 1024-block becomes H (S x) / 32.
void rotate_row(const double* x, const uint32_t* sign_bits, int64_t k, double* xr) {
  for (int64_t blk = 0; blk < k; blk += 1024) {
    for (int i = 0; i < 1024; ++i) {
      double acc = 0.0;
      for (int j = 0; j < 1024; ++j) {
        const int64_t ch = blk + j;
        const double s = (sign_bits[ch / 32] >> (ch % 32)) & 1u ? -1.0 : 1.0;
        const double h = popcount(unsigned(i) & unsigned(j)) & 1 ? -1.0 : 1.0;
        acc += h * s * x[ch];
      }
      xr[blk + i] = acc / 32.0;
    }
  }
}

void product_rows(int packing, const uint8_t* packed, const uint16_t* scales, const double* xr, int64_t b,
                  int64_t n0, int64_t n1, int64_t k, double* y, int64_t n) {
  const int64_t row_bytes = packing == 0 ? k / 4 : 26 * (k / 128);
  for (int64_t r = 0; r < b; ++r) {
    for (int64_t row = n0; row < n1; ++row) {
      const uint8_t* w = packed + row * row_bytes;
      double acc = 0.0;
      for (int64_t g = 0; g < k / 128; ++g) {
        double part = 0.0;
        for (int64_t kk = 128 * g; kk < 128 * g + 128; ++kk) {
          const int t = packing == 0 ? trit_2bit(w, kk) : trit_base3(w, kk);
          part += t * xr[r * k + kk];
        }
        acc += half_to_double(scales[row * (k / 128) + g]) * part;
      }
      y[r * n + row] = acc;
    }
  }
}

}  // namespace

extern "C" {

// Trits int8 [n][k] -> packed bytes.  2-bit: byte j = sum_{i<4} (t_{4j+i} + 1) << 2i.  Base-3,
// per 128-group: 26 bytes, byte j = sum_{i<5} (t_{5j+i} + 1) 3^i over the group extended by two
// trits of 0.  A trit outside {-1, 0, 1} counts once and is packed as 0.  Returns the count, or
// -1 on bad sizes.
int64_t oracle_pack(int packing, const int8_t* trits, int64_t n, int64_t k, uint8_t* packed) {
  if ((packing != 0 && packing != 1) || n < 0 || k <= 0 || k % 128 != 0) return -1;
  int64_t bad = 0;
  auto trit = [&](int64_t r, int64_t i) -> int {
    const int t = trits[r * k + i];
    if (t < -1 || t > 1) {
      ++bad;
      return 0;
    }
    return t;
  };
  for (int64_t r = 0; r < n; ++r) {
    if (packing == 0) {
      for (int64_t j = 0; j < k / 4; ++j) {
        int byte = 0;
        for (int i = 0; i < 4; ++i) byte |= (trit(r, 4 * j + i) + 1) << (2 * i);
        packed[r * (k / 4) + j] = uint8_t(byte);
      }
    } else {
      for (int64_t g = 0; g < k / 128; ++g)
        for (int j = 0; j < 26; ++j) {
          int byte = 0, pow3 = 1;
          for (int i = 0; i < 5; ++i, pow3 *= 3) {
            const int e = 5 * j + i;  // element of the extended group
            byte += (e < 128 ? trit(r, 128 * g + e) + 1 : 1) * pow3;
          }
          packed[r * 26 * (k / 128) + 26 * g + j] = uint8_t(byte);
        }
    }
  }
  return bad;
}

// Packed bytes -> trits int8 [n][k].  2-bit: code 11 counts once and decodes as 0.  Base-3:
// trit i of byte b is (b / 3^i) mod 3 - 1; a byte >= 243 counts once and its trits decode as 0; a
// valid last byte of a group whose two pad digits are not 1 counts once.  Returns the count, or
// -1 on bad sizes.
int64_t oracle_unpack(int packing, const uint8_t* packed, int64_t n, int64_t k, int8_t* trits) {
  if ((packing != 0 && packing != 1) || n < 0 || k <= 0 || k % 128 != 0) return -1;
  int64_t bad = 0;
  for (int64_t r = 0; r < n; ++r) {
    if (packing == 0) {
      for (int64_t i = 0; i < k; ++i) {
        const int c = (packed[r * (k / 4) + i / 4] >> (2 * (i % 4))) & 3;
        if (c == 3) ++bad;
        trits[r * k + i] = int8_t(c == 3 ? 0 : c - 1);
      }
    } else {
      for (int64_t g = 0; g < k / 128; ++g)
        for (int j = 0; j < 26; ++j) {
          const int b = packed[r * 26 * (k / 128) + 26 * g + j];
          if (b >= 243) ++bad;
          else if (j == 25 && ((b / 27) % 3 != 1 || (b / 81) % 3 != 1)) ++bad;  // pad digits 3, 4 not 1
          int rest = b;
          for (int i = 0; i < 5; ++i) {
            const int digit = rest % 3;
            rest /= 3;
            const int e = 5 * j + i;
            if (e < 128) trits[r * k + 128 * g + e] = int8_t(b >= 243 ? 0 : digit - 1);
          }
        }
    }
  }
  return bad;
}

// y[b][n] = sum_g s[n][g] sum_{k in g} t[n][k] (R_K x[b])[k], all in float64.
// x: float64 [B][K] unrotated; sign_bits NULL means x is already rotated.
// The output rows are split over `threads` std::threads.  Returns 0, or -1 on
// bad sizes.
int oracle_linear(int packing, const uint8_t* packed, const uint16_t* scales, const double* x,
                  const uint32_t* sign_bits, int64_t b, int64_t n, int64_t k, double* y, int threads) {
  if ((packing != 0 && packing != 1) || b < 0 || n < 0 || k <= 0 || k % 128 != 0) return -1;
  if (sign_bits && k % 1024 != 0) return -1;
  std::vector<double> xr(size_t(b * k));
  for (int64_t r = 0; r < b; ++r) {
    if (sign_bits)
      rotate_row(x + r * k, sign_bits, k, xr.data() + r * k);
    else
      for (int64_t i = 0; i < k; ++i) xr[size_t(r * k + i)] = x[r * k + i];
  }
  if (threads < 1) threads = 1;
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) {
    const int64_t n0 = n * t / threads, n1 = n * (t + 1) / threads;
    pool.emplace_back(product_rows, packing, packed, scales, xr.data(), b, n0, n1, k, y, n);
  }
  for (auto& th : pool) th.join();
  return 0;
}

}  // extern "C"
