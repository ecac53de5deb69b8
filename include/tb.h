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
  TB_ERR_HIP = 6,         /* the HIP runtime reported an error at launch       */
  TB_ERR_WORKSPACE = 7,   /* a workspace is smaller than the call needs        */
  TB_ERR_SCRATCH = 8      /* the call needs more than the static scratch holds */
} tb_status;

typedef enum { TB_PACK_2BIT = 0, TB_PACK_BASE3 = 1 } tb_packing;
typedef enum { TB_F32 = 0, TB_F16 = 1, TB_BF16 = 2 } tb_dtype;

/* Largest batch tb_gemv, tb_linear and tb_linear_ws accept.  tb_gemv and
 * tb_linear_ws run every batch in one pass over the weights.  tb_linear (no
 * workspace) runs up to TB_GEMV_KERNEL_BATCH rows in one pass; a larger batch
 * runs in chunks of TB_GEMV_KERNEL_BATCH rows, each streaming the weights
 * again. */
#define TB_GEMV_MAX_BATCH 32
#define TB_GEMV_KERNEL_BATCH 8

/* Bytes of one packed row of K weights: K/4 for 2-bit codes, 26*K/128 for
 * base-3 codes; -1 if K is negative or not a multiple of 128 or the packing
 * code is unknown.  Pure host function.
 * Pages: "TensorSharp view of Ternary Bonsai 2 27B" (2kiu.com/news/5337570/),
 * section 1.2 (bits per weight = stored bytes * 8 / weights): with the fp16
 * scale of each 128-group this gives 2.125 bits/weight for 2-bit codes and
 * 1.75 for base-3 codes; "Bonsai low-bit learning path", section "Understand
 * 1.6 bit with five numbers" (five trits per base-3 byte). */
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

/* Inverse of the two packings (the validator of packed weights).
 * Pages: "Bonsai low-bit learning path", section "Understand 1.6 bit with
 * five numbers": trit i of a base-3 byte b is (b / 3**i) mod 3 - 1 (integer
 * division), i = 0..4; 2-bit codes decode as t = c - 1.  trits: int8
 * [N][K] out.  bad_count (NULLABLE): +1 per 2-bit code 11 (decoded 0), per
 * base-3 byte >= 243 (its five trits decoded 0) and per group whose last byte
 * has pad digits other than 1.  The products do not check codes: their result
 * on invalid codes is unspecified (but they never read or write out of bounds). */
int tb_unpack(int packing, const uint8_t* packed, int64_t N, int64_t K, int8_t* trits,
              int32_t* bad_count, void* stream);

/* Blockwise rotation xr = R_K x, R_K = blockdiag(H_1024 S_b / 32).
 * Pages: "Ternary Bonsai 2 27B release", section "How the ternary weights
 * reach 1.76 bit" (R = H_n S / sqrt(n), n = 1024, applied blockwise to the
 * activations) and section "Known weaknesses" (this transform is the largest
 * cost after the product at batch 1); "TensorSharp view of Ternary Bonsai 2
 * 27B" (2kiu.com/news/5337570/), sections 3.2 and 5.2 (Sylvester-ordered H,
 * butterfly evaluation).
 * x: [rows][K] of x_dtype (TB_F32, TB_F16 or TB_BF16).  xr: [rows][K] of
 * xr_dtype (TB_F32 or TB_F16; fp16 is rounded to nearest even once, at the
 * store).  sign_bits: uint32 [K/32]; bit b of word w is channel 32w+b, set
 * means S = -1; the same mask is used for every row.  Blocks are consecutive
 * 1024-slices of each row.  x == xr is allowed when the dtypes match; any
 * other overlap of x and xr returns TB_ERR_SHAPE. */
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
 * Small batches run fp8 (fp6 for base-3 at B = 1) limbs of xr against fp4
 * codes; from B = 5 (K >= 8192), 7 (N < 8192), 8 (base-3) or 9 (2-bit) on,
 * one pass on the fp16 matrix cores, fp32 xr split into fp16 hi + lo (about
 * 2^-21 of |x| lost).  Both take any finite
 * magnitude: xr gets a power-of-two scale per row and 128-group, undone in
 * fp32 after the group's sum.
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

/* Workspace that tb_linear_ws needs for (packing, B, N, K): 4 B K bytes (x'
 * in fp32) when that call rotates into the workspace and runs tb_gemv's product
 * on it, which is from batch 2 for K >= 8192, else from batch 5 (base-3) or 6
 * (2-bit), and in any case from the batch at which tb_gemv runs the batched
 * matrix-core product; from that batch on, plus 4 P B N bytes where the rows
 * are too few to fill the compute units with five row tiles per workgroup and
 * the product takes K in P parts on separate workgroups (P = 2..8: the fp32
 * partial sums of each part, e.g. 4 parts for 5120 rows; P = 2 only from batch
 * 16); for base-3 weights at batch 1 with K above 5120, 4 P N
 * bytes (the fp32 partial sums of P = ceil(K / 5120) parts of each row, which
 * separate workgroups take); 0 when the one-launch fused kernel of tb_linear
 * serves the call; -1 for an unknown packing, B outside 1..TB_GEMV_MAX_BATCH,
 * N < 0, K not a positive multiple of 1024 or sizes past 32-bit offsets.  Pure
 * host function of its arguments. */
int64_t tb_linear_workspace_bytes(int packing, int64_t B, int64_t N, int64_t K);

/* tb_linear with one pass over the weights at every batch: where
 * tb_linear_workspace_bytes > 0 and B > 1, x' = R_K x is written in fp32 to the
 * caller's workspace and tb_gemv's product reads it, two launches on `stream`
 * (from those batches on the fused kernel's activation prologue costs more than
 * the separate rotation; above 8 rows the product is the batched one, which
 * streams the weights once, and with few rows takes K in parts whose partial
 * sums a third launch adds in part order, so the result does not depend on
 * timing).  At batch 1 with base-3 rows longer than 5120 the
 * fused one-launch kernel takes the rows in parts of K on separate workgroups
 * (all compute units busy where the rows alone are too few), writes each
 * part's partial sums to the workspace and a second launch adds them in part
 * order (deterministic); with more row tiles than the parts' workgroups hold it
 * runs as tb_linear.  Otherwise exactly tb_linear.  Same pages, arguments
 * and result as tb_linear, plus workspace: device memory of at least
 * workspace_bytes >= tb_linear_workspace_bytes(packing, B, N, K) bytes (else
 * TB_ERR_WORKSPACE), 16-byte aligned, owned by the caller, overwritten, and
 * sharing no byte with x or y (else TB_ERR_SHAPE; only the first
 * tb_linear_workspace_bytes bytes are used and checked).  The library still
 * allocates nothing.  Calls that share a workspace must be ordered (one
 * stream). */
int tb_linear_ws(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dtype,
                 const uint32_t* sign_bits, float* y, int64_t B, int64_t N, int64_t K, void* workspace,
                 int64_t workspace_bytes, void* stream);

/* tb_linear_ws without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Where
 * tb_linear_workspace_bytes(packing, B, N, K) > 0, x' goes to a static device
 * array of the library (4 MiB per GPU, held until the process ends) instead of
 * a caller workspace.  The call returns TB_ERR_SCRATCH when x' alone would need
 * more (B K > 2^20 floats), except that a call below the batch of tb_gemv's
 * batched product (partial sums of batch 1, or x' of a few rows) runs as
 * tb_linear when the array cannot hold it, and a batched call whose x' fits
 * but whose parts' partial sums do not takes whole rows (the same result up to
 * rounding: another summation order).  Otherwise it has the same arguments,
 * kernels and result as tb_linear_ws.  Every call on one GPU shares that
 * array: calls that overlap on one GPU (different streams without ordering,
 * or several host threads) race on it; order them on one stream.  x' and the
 * partial sums are fully written before they are read, so no clearing is
 * needed between calls.  The
 * first call on a device looks the array's address up (no allocation). */
int tb_linear_noalloc(int packing, const uint8_t* packed, const uint16_t* scales, const void* x, int x_dtype,
                      const uint32_t* sign_bits, float* y, int64_t B, int64_t N, int64_t K, void* stream);

/* Persistent multi-linear decode: up to TB_CHAIN_MAX dependent batch-1 linears
 * in ONE launch.  Linear 0 computes y_0 = W_0 (R_K x0); linear i > 0 computes
 * y_i = W_i (R_K y_{i-1}[0 .. K)), i.e. it takes the first K outputs of the
 * previous linear as its (unrotated, fp32) activations.  Between linears every
 * workgroup waits on a device-side count of the workgroups that have stored
 * their rows of the previous output; the weight loads of the next linear are
 * issued before that wait (weights do not depend on x), so no launch separates
 * the linears and the next weight stream overlaps the previous one's tail.
 * Pages: "Ternary Bonsai 2 27B release", sections "How the ternary weights
 * reach 1.76 bit" (f(x) = W(Rx), g128 scales) and "Throughput" (decode reads
 * every weight byte once per token; tg128 is a chain of such products).
 * packing: TB_PACK_BASE3 only (else TB_ERR_UNSUPPORTED).  linears: HOST array
 * of count (1..TB_CHAIN_MAX) descriptors {packed [N][26 K/128], scales fp16
 * [N][K/128], y fp32 [N], N}, read during the call; N_i >= K for every linear
 * but the last (else TB_ERR_SHAPE).  x0: [K] of x_dtype; sign_bits: uint32
 * [K/32], the same R_K for every linear.  K a multiple of 1024 up to 5120
 * (else TB_ERR_UNSUPPORTED), and at most 16 - K/1024 row tiles of 16 per
 * compute unit for any linear (about 176 x the compute units rows at K = 5120;
 * else TB_ERR_UNSUPPORTED).
 * sync: device int32 [sync_words >= count + 2], all zero before the first call
 * (the caller clears it once); a call that completes leaves its counts zero for
 * the next call on the same stream.  Word count + 1 is the status: bit 0 is
 * set when a wait polled spin_limit times without the count arriving (spin_limit
 * <= 0: 2^22 polls, about 0.1-1 s); every wait is bounded, the launch always
 * ends, but its outputs are then invalid and the caller must clear sync again.
 * The launch needs every one of its workgroups (one per compute unit) resident
 * at once, so it should not share the GPU with other work.  Calls sharing a
 * sync buffer must be ordered (one stream).
 * Measured on MI355X it is SLOWER than one tb_linear launch per linear in a
 * HIP graph (q/k/v -> o: 33 us against 16 us): a device-wide hand-over costs
 * about 10 us of atomics and polling, a kernel boundary in a graph about 1-2 us,
 * and even with no hand-over at all the chained launch does not beat separate
 * ones.  Prefer tb_linear (or tb_linear_ws) under a HIP graph for decode. */
#define TB_CHAIN_MAX 8
typedef struct tb_chain_linear {
  const uint8_t* packed;
  const uint16_t* scales;
  float* y;
  int64_t N;
} tb_chain_linear;
int tb_decode_chain(int packing, const tb_chain_linear* linears, int count, const void* x0, int x_dtype,
                    const uint32_t* sign_bits, int64_t K, int32_t* sync, int64_t sync_words, int spin_limit,
                    void* stream);

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

/* Offline quantiser: fp32 weights W (y = W x) -> ternary trits and g128 fp16
 * scales of W' = W R_K^T, the weights in the rotated basis, so that
 * W x is approximated by (trits * scales)(R_K x).
 * Pages: "Ternary Bonsai 2 27B release", section "How the ternary weights
 * reach 1.76 bit" (the weights are moved into the fixed rotated basis before
 * they are ternarised; one fp16 scale per 128 weights); "TensorSharp view of
 * Ternary Bonsai 2 27B" (2kiu.com/news/5337570/), section 2.1 (a scale per
 * block from its mean absolute weight times a correction; |w / scale| below
 * the threshold gives 0, otherwise the sign; the finer form tries candidate
 * thresholds and keeps the least reconstruction error).
 * Per 128-group of W' with a = mean |w|: candidate j = 0..63 keeps the
 * weights with |w| >= (j + 1) / 32 * a as sign(w) and zeroes the rest; its
 * scale is the mean kept magnitude rounded once to fp16 (nearest even); the
 * candidate with the least squared reconstruction error under that rounded
 * scale wins (the lowest j on ties; a scale that overflows fp16 counts as
 * infinite error).  Rotation and search run in fp64.
 * w: fp32 [N][K].  sign_bits: uint32 [K/32] as for tb_fwht_rotate, or NULL
 * when w is already in the rotated basis (the search alone).  trits: int8
 * [N][K] out; scales: fp16 [N][K/128] out; pack the trits afterwards with
 * tb_pack_2bit or tb_pack_base3.  bad_count (NULLABLE): +1 per group holding
 * a non-finite value or whose chosen scale overflows fp16; such groups, and
 * all-zero groups, are written as zero trits with scale 0.  K % 1024 == 0;
 * w, scales (and sign_bits when given) 16-byte aligned. */
int tb_ternarize(const float* w, int64_t N, int64_t K, const uint32_t* sign_bits, int8_t* trits,
                 uint16_t* scales, int32_t* bad_count, void* stream);

/* Measurement aid, not part of the product path: read `bytes` bytes of device
 * memory once (16-byte loads) and write one XOR word per workgroup to sink,
 * which must hold TB_STREAM_SINK_WORDS uint32 (else TB_ERR_WORKSPACE).  The
 * time of this call is the measured HBM read ceiling the weight-streaming
 * products are compared with.  Pages: "Ternary Bonsai 2 27B release", section
 * "Throughput" (decode is bound by the weight bytes read per token).
 * 0 <= bytes < 2^31, a multiple of 16; src and sink 16-byte aligned. */
#define TB_STREAM_SINK_WORDS 8192
int tb_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words, void* stream);

/* Static text for a status code. */
const char* tb_status_string(int status);

/* Thread-local text of the last HIP error seen by a tb_ call on this thread
 * ("" if none). */
const char* tb_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
