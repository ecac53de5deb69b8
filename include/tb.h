/* tb.h -- C ABI of the MI355X (gfx950) ternary rotated-basis linear, y = W(Rx).
 *
 * What is computed (pages: "Ternary Bonsai 2 27B release", linlog.top/article/1481,
 * section "How the ternary weights reach 1.76 bit"): W holds weights in
 * {-1, 0, +1} with one fp16 scale per 128 consecutive weights of a row (g128);
 * activations are rotated by the fixed basis R = (1/sqrt(n)) H_n S, n = 1024,
 * S a fixed +-1 diagonal, applied blockwise; inference computes f(x) = W(Rx)
 * with the unpack and the group scale done inside the product, never writing
 * dequantised weights to memory.
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) unless a
 *    comment says otherwise.  The caller owns all memory; the library never
 *    allocates, frees or synchronises.  Every call only enqueues work on
 *    `stream` (a hipStream_t; NULL = the default stream) and returns.
 *  - Matrices are row-major and dense.  W is N x K (N outputs, K inputs);
 *    packed rows are contiguous with stride tb_packed_row_bytes().
 *  - scales: fp16 bit patterns, [N][K/128] row-major; group g of row n covers
 *    weights 128g .. 128g+127.
 *  - Shapes: K % 128 == 0 for packing and products, K % 1024 == 0 for the
 *    rotation; N, rows, M >= 0 (0 is a valid empty call that does nothing).
 *  - Alignment: packed, scales, activations and outputs must be 16-byte
 *    aligned, else TB_ERR_ALIGN.  int8 trits need only natural alignment.
 *  - Every shape/pointer/alignment/dtype problem is reported by the return
 *    value before anything is launched.  A launch failure returns TB_ERR_HIP;
 *    tb_last_hip_error() then gives the HIP error text (thread-local).
 *  - Calls are thread-safe: the library keeps no global mutable state apart
 *    from the thread-local error text.
 */
#ifndef TB_H
#define TB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TB_OK = 0,
  TB_ERR_NULL = 1,        /* a required pointer is NULL                        */
  TB_ERR_SHAPE = 2,       /* negative size, K not a multiple of 128/1024, B out of range */
  TB_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                  */
  TB_ERR_DTYPE = 4,       /* dtype code not accepted by this call              */
  TB_ERR_UNSUPPORTED = 5, /* packing code not accepted by this call            */
  TB_ERR_HIP = 6          /* the HIP runtime reported an error at launch       */
} tb_status;

typedef enum { TB_PACK_2BIT = 0, TB_PACK_BASE3 = 1 } tb_packing;
typedef enum { TB_F32 = 0, TB_F16 = 1, TB_BF16 = 2 } tb_dtype;

/* Largest batch tb_gemv and tb_linear accept.  tb_gemv runs every batch in
 * one pass over the weights.  tb_linear runs up to TB_GEMV_KERNEL_BATCH rows
 * in one pass; a larger batch runs in chunks of TB_GEMV_KERNEL_BATCH rows,
 * each streaming the weights again. */
#define TB_GEMV_MAX_BATCH 32
#define TB_GEMV_KERNEL_BATCH 8

/* Bytes of one packed row of K weights: K/4 for 2-bit codes, 26*K/128 for
 * base-3 codes; -1 if K is negative or not a multiple of 128 or the packing
 * code is unknown.  Pure host function. */
int64_t tb_packed_row_bytes(int packing, int64_t K);

/* 2-bit packing.  trits: int8 [N][K] with values in {-1,0,1}.  packed: uint8
 * [N][K/4]; weight k of a row goes to bits 2(k%4), 2(k%4)+1 of byte k/4 as the
 * code c = t+1 (00 = -1, 01 = 0, 10 = +1; 11 is never written).
 * Pages: "Ternary Bonsai 2 27B release", section "How the ternary weights reach
 * 1.76 bit" (two bits hold the three states; PQ2_0 is the plain 2-bit format).
 * bad_count: NULLABLE device int32; each input trit outside {-1,0,1} adds 1
 * (the caller zeroes it) and is packed as 0. */
int tb_pack_2bit(const int8_t* trits, int64_t N, int64_t K, uint8_t* packed,
                 int32_t* bad_count, void* stream);

/* Base-3 packing, five trits per byte.  Pages: "Bonsai low-bit learning path"
 * (adenzhou1350.github.io/learn/bonsai-low-bit/), section "Understand 1.6 bit
 * with five numbers": byte = sum_i (t_i + 1) * 3**i, first trit least
 * significant, every byte < 243.  Each 128-weight group takes 26 bytes:
 * bytes 0..24 hold weights 5j..5j+4, byte 25 holds weights 125..127 and two
 * pad trits equal to 0 (digit 1), so 1.75 bits/weight with the fp16 scale.
 * packed: uint8 [N][26*K/128].  bad_count as for tb_pack_2bit. */
int tb_pack_base3(const int8_t* trits, int64_t N, int64_t K, uint8_t* packed,
                  int32_t* bad_count, void* stream);

/* Inverse of the two packings (the validator of packed weights).  trits: int8
 * [N][K] out.  bad_count (NULLABLE): +1 per 2-bit code 11 (decoded 0), per
 * base-3 byte >= 243 (its five trits decoded 0) and per group whose last byte
 * has pad digits other than 1.  The products do not check codes: their result
 * on invalid codes is unspecified (but they never read or write out of bounds). */
int tb_unpack(int packing, const uint8_t* packed, int64_t N, int64_t K, int8_t* trits,
              int32_t* bad_count, void* stream);

/* Blockwise rotation xr = R_K x, R_K = blockdiag(H_1024 S_b / 32).
 * Pages: "Ternary Bonsai 2 27B release", section "How the ternary weights
 * reach 1.76 bit" (R = H_n S / sqrt(n), n = 1024, applied blockwise to the
 * activations) and section "Known shortcomings" (this transform is the largest
 * cost after the product at batch 1); "TensorSharp view of Ternary Bonsai 2
 * 27B" (2kiu.com/news/5337570/), sections 3.2 and 5.2 (Sylvester-ordered H,
 * butterfly evaluation).
 * x: [rows][K] of x_dtype (TB_F32, TB_F16 or TB_BF16).  xr: [rows][K] of
 * xr_dtype (TB_F32 or TB_F16; fp16 is rounded to nearest even once, at the
 * store).  sign_bits: uint32 [K/32]; bit b of word w is channel 32w+b, set
 * means S = -1; the same mask is used for every row.  Blocks are consecutive
 * 1024-slices of each row.  x == xr is allowed when the dtypes match. */
int tb_fwht_rotate(const void* x, int x_dtype, void* xr, int xr_dtype, int64_t rows, int64_t K,
                   const uint32_t* sign_bits, void* stream);

/* Decode product y[b][n] = sum_g s[n][g] * sum_{k in g} t[n][k] * xr[b][k].
 * Pages: "Ternary Bonsai 2 27B release", sections "How the ternary weights
 * reach 1.76 bit" (g128 fp16 scales; unpack and group scale fused inside the
 * product, no fp16 weight copy) and "Throughput" (decode is bound by the
 * weight bytes streamed per token).
 * packed: [N][tb_packed_row_bytes(packing, K)]; scales: fp16 [N][K/128];
 * xr: [B][K] rotated activations of xr_dtype (TB_F32 or TB_F16), read as
 * given; y: fp32 [B][N], overwritten.  1 <= B <= TB_GEMV_MAX_BATCH and
 * B * K * 4 < 2^31.
 * B <= TB_GEMV_KERNEL_BATCH: fp8 limbs of xr against fp4 codes, any
 * magnitude (a power-of-two scale per row and 128-group).
 * B > TB_GEMV_KERNEL_BATCH: fp16 matrix cores; fp32 xr is split into
 * fp16 hi + lo (about 2^-21 of |x| lost), so |xr| must stay below 65504
 * (larger values give inf or NaN), and values below 2^-14 keep an absolute
 * error of at most 2^-24 instead of a relative one.
 * Accumulation is fp32 (not bit-reproducible across kernel versions). */
int tb_gemv(int packing, const uint8_t* packed, const uint16_t* scales, const void* xr,
            int xr_dtype, float* y, int64_t B, int64_t N, int64_t K, void* stream);

/* The whole linear at decode, y[b][n] = sum_k W_hat[n][k] (R_K x[b])[k], in one
 * launch: the rotation of x is done inside the product's prologue instead of
 * by a separate tb_fwht_rotate call.
 * Pages: "Ternary Bonsai 2 27B release", sections "How the ternary weights
 * reach 1.76 bit" (f(x) = W(Rx) with R = H_1024 S / 32 blockwise) and "Known
 * weaknesses" (at batch 1 the activation transform is the largest cost
 * besides the product).
 * x: [B][K] unrotated activations of x_dtype (TB_F32, TB_F16 or TB_BF16);
 * sign_bits, packed, scales and y as for tb_fwht_rotate and tb_gemv.
 * K % 1024 == 0; 1 <= B <= TB_GEMV_MAX_BATCH (chunked as tb_gemv).  x' is kept in fp32 inside the
 * call (never rounded to fp16), so the result matches tb_fwht_rotate to fp32
 * followed by tb_gemv to fp32 accumulation order. */
int tb_linear(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dtype,
              const uint32_t* sign_bits, float* y, int64_t B, int64_t N, int64_t K, void* stream);

/* Prefill product Y = X' W_hat^T for many rows: Y[m][n] = sum_k X'[m][k] s[n][k/128] t[n][k].
 * Pages: "Ternary Bonsai 2 27B release", sections "How the ternary weights
 * reach 1.76 bit" and "Throughput" (pp512 prompt processing).
 * packing: TB_PACK_2BIT or TB_PACK_BASE3; packed [N][tb_packed_row_bytes(packing, K)]
 * as written by tb_pack_2bit / tb_pack_base3 (any address alignment for base-3
 * rows is handled; the buffer itself 16-byte aligned); scales [N][K/128].
 * xr_f16: fp16 [M][K]; y: fp32 [M][N], overwritten.  Products t*s are exact in
 * fp16; accumulation is fp32 on the matrix cores.  K % 128 == 0.
 * M <= 96 runs as chunks of up to 32 rows on the batched decode kernel of
 * tb_gemv (one pass over the weights per chunk); larger M on 128 x 272
 * output tiles. */
int tb_gemm(int packing, const uint8_t* packed, const uint16_t* scales, const uint16_t* xr_f16,
            float* y, int64_t M, int64_t N, int64_t K, void* stream);

/* Static text for a status code. */
const char* tb_status_string(int status);

/* Thread-local text of the last HIP error seen by a tb_ call on this thread
 * ("" if none). */
const char* tb_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
