/*
 * bsgemm.h -- C ABI of libbsgemm, the MI355X (gfx950) hot path of a
 * row-parallel block-scale fp8 linear layer (DeepSeek-V4-Pro's wo_b):
 *
 *   bsgemm_fp8   block-scale fp8 GEMM, fp32 accumulate, bf16 out, written as
 *                destination-major row bands
 *   band_reduce  fp32 sum of P bf16 partial bands into one bf16 band
 *   rowq_e4m3    per-row e4m3 quantize with one fp32 scale per row
 *   band_rowq_e4m3  band_reduce and rowq_e4m3 fused into one pass (the fused
 *                variant the pages measured and found slower; here it is the
 *                faster path and the one the benchmark's step runs)
 *   rowdq_e4m3   per-row e4m3 dequantize back to bf16
 *   blockq_e4m3  fp32 operand -> e4m3 codes + fp32 block scales (the
 *                activation/weight quantizer that produces bsgemm_fp8's input)
 *   actq_e4m3    bf16 activation -> e4m3 codes + fp32 1x128 scales (the
 *                on-GPU step before bsgemm_fp8 when the layer input is bf16)
 *   bprepack_e4m3  one-time rearrangement of the weight B into the GEMM's
 *                operand order (load-time weight preparation)
 *   bsgemm_fp8_pb  the GEMM reading B in that prepacked form
 *   mxgemm_fp8   the mxfp8 variant of the GEMM: e4m3 operands with E8M0 scales
 *                per 1x32 block on both A and B, applied by the MFMA
 *   mxq_e4m3     bf16 -> e4m3 codes + E8M0 1x32 scales (mxgemm_fp8's operands)
 *
 * Pages defining the operations (cited by title and section):
 *   [PR40757] sglang PR 40757 "[AMD][gfx950] DSV4: fuse wo_b's GEMM with its
 *             all-reduce via mori cco": "What" (block-scale fp8 GEMM followed
 *             by an all-reduce of [M, hidden]; each destination's row band
 *             written as its own unit), "Numbers" (fused and unfused agree up
 *             to accumulation order).
 *   [PR43480] sglang PR 43480 (DeepSeek-V4.1-Flash wo_b): "What" (an mxfp8
 *             GEMM followed by the all-reduce), "Not in this PR" (V4.1-Flash
 *             quantises at 32-wide ue8m0), "Numerics, measured where the path
 *             engages" (on the aiter route wo_b is handed a plain bf16
 *             activation and quantises it itself); "Worth a reviewer's
 *             attention" (the native gfx950 route rebinds the weight to a
 *             shuffled [N/16, K/128, 2048] layout, and reading one layout as
 *             the other gives an uncorrelated result instead of an error);
 *             the review reply on the duplicated ue8m0 scale rule (exponent
 *             from the IEEE bits, exact at powers of two) and the one on the
 *             lazy second copy of the weight (weight preparation moved to
 *             load time).
 *   [MORI]    "MORI GEMM + All-Reduce Benchmark": "Running the benchmark"
 *             (--quant blockscale: A per 1x128, B per 128x128, fp32 scales;
 *             shape [M,7168], K=2048), "Where the time goes" (reduce /
 *             quantize / dequantize phases), "The fp8 wire" (e4m3 with one
 *             fp32 scale per row; the reduce accumulates in fp32 and outputs
 *             bf16), "Negative results" (the pages keep reduce and quantize
 *             as separate kernels; band_rowq_e4m3 fuses them).
 *
 * Conventions shared by every call:
 *  - All data pointers are DEVICE memory owned by the caller (the library
 *    never allocates, frees or keeps a pointer after returning).  The only
 *    host memory argument is band_reduce's array of part pointers, read
 *    before the call returns.
 *  - bf16 values are passed as their uint16_t bit patterns; e4m3 values as
 *    uint8_t codes of the OCP FP8 E4M3 ("fn") format (max 448, NaN at
 *    S.1111.111, no infinities).  Every matrix is dense row-major.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    only enqueue work: they return before the device finishes and never
 *    synchronize.
 *  - Arguments are validated on the host before anything is enqueued.  On
 *    BS_ERR_INVALID or BS_ERR_UNSUPPORTED nothing is launched and no output
 *    byte is written.  BS_ERR_LAUNCH means the HIP runtime refused the launch
 *    (hipGetLastError after the enqueue); outputs are then unspecified.
 *  - Results are bitwise deterministic for identical inputs and shapes.
 *  - The library holds no global state that calls depend on, reads no
 *    environment variables and is safe to call from several host threads.
 *    Calls whose output ranges overlap another call's input or output on a
 *    concurrently running stream race, as with any kernel.
 */
#ifndef BSGEMM_H
#define BSGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BS_OK = 0,
    BS_ERR_INVALID = 1,     /* null pointer, negative size, aliasing outputs */
    BS_ERR_UNSUPPORTED = 2, /* well-formed but not expressible by the kernels */
    BS_ERR_LAUNCH = 3       /* the HIP runtime rejected the launch */
} bs_status;

/*
 * Block-scale fp8 GEMM with a destination-major band epilogue.
 * [PR40757] "What"; [MORI] "Running the benchmark" (--quant blockscale).
 *
 *   C[m, n] = bf16_rne( acc[m, n] ),  acc accumulated in fp32 over the K
 *   blocks kb = 0 .. K/128-1 in ascending order:
 *     acc += ( sum_{k in block kb} A[m,k] * B[n,k] ) * (a_scale[m,kb] * b_scale[n/128,kb])
 *   the block dot product being one 16x16x128 fp8 MFMA with fp32 result.
 *
 *   A        [M, K]          e4m3 codes (activations)
 *   a_scale  [M, K/128]      fp32, one scale per 1x128 block of A
 *   B        [N, K]          e4m3 codes (the weight as stored, [out, in])
 *   b_scale  [N/128, K/128]  fp32, one scale per 128x128 block of B
 *   C        bf16 output as `bands` row bands of band_rows = M / bands rows:
 *            row m lives in band d = m / band_rows at row r = m % band_rows,
 *            element (m, n) at C[d * band_stride + r * N + n].
 *            band_stride = 0 means band_rows * N (contiguous: identical to a
 *            row-major [M, N] matrix).  Elements between bands are untouched.
 *
 * Requirements: M >= 0 (M = 0 is a no-op); N > 0 and N % 128 == 0;
 * K > 0 and K % 128 == 0; 1 <= bands <= 64 and M % bands == 0;
 * band_stride == 0 or band_stride >= band_rows * N; A, B and C 16-byte
 * aligned, a_scale and b_scale 4-byte aligned; C must not overlap any input.
 * Violations: null pointers, negative sizes, bands < 1 or overlap ->
 * BS_ERR_INVALID; the rest -> BS_ERR_UNSUPPORTED.  M need not be a multiple
 * of the tile: ragged rows are handled in the kernel.
 */
bs_status bsgemm_fp8(const uint8_t *A, const float *a_scale,
                     const uint8_t *B, const float *b_scale,
                     uint16_t *C,
                     int64_t M, int64_t N, int64_t K,
                     int32_t bands, int64_t band_stride,
                     void *stream);

/*
 * Band reduce: out = bf16_rne( sum_{p=0..P-1} widen(parts[p]) ), the sum in
 * fp32 starting from +0.0 and taken in part-index order.
 * [MORI] "Where the time goes" (reduce), "The fp8 wire" (fp32 accumulate,
 * bf16 output), "Negative results" (one pass streams all P source slices).
 *
 *   parts  HOST array of P device pointers, each a bf16 [rows, N] band
 *   out    bf16 [rows, N]; may not overlap any part
 *
 * Requirements: 1 <= P <= 16; rows >= 0, N > 0, N % 8 == 0; every pointer
 * 16-byte aligned.  Null or out-of-range P -> BS_ERR_INVALID; N % 8 or
 * misalignment -> BS_ERR_UNSUPPORTED.
 */
bs_status band_reduce(const uint16_t *const *parts, int32_t P,
                      uint16_t *out, int64_t rows, int64_t N,
                      void *stream);

/*
 * Per-row e4m3 quantize (the "fp8 wire").  [MORI] "The fp8 wire" (e4m3 with
 * one fp32 scale per row), "What fp8 costs, numerically" (per row chosen).
 *
 *   for each row r:  amax = max_n |x[r,n]|;  scale[r] = amax / 448 (fp32,
 *   round to nearest even);  q[r,n] = e4m3 code nearest to the fp32 quotient
 *   x[r,n] / scale[r] (ties to even, |.| > 448 saturates, sign kept so a
 *   negative value that rounds to zero gives 0x80).  A row whose scale is 0
 *   (all zeros, or amax/448 underflowing) gets scale 0 and codes 0x00.
 *
 *   x      bf16 [rows, N] (finite values; non-finite input is outside the
 *          contract and gives unspecified codes)
 *   q      e4m3 [rows, N]
 *   scale  fp32 [rows]
 *
 * Requirements: rows >= 0, N > 0, N % 8 == 0; x, q 16-byte aligned, scale
 * 4-byte aligned; q and scale must not overlap x or each other.
 */
bs_status rowq_e4m3(const uint16_t *x, uint8_t *q, float *scale,
                    int64_t rows, int64_t N, void *stream);

/*
 * Per-row e4m3 dequantize ("widen" after the gather).  [MORI] "Where the
 * time goes" (dequantize), "Who moves the gather".
 *
 *   y[r,n] = bf16_rne( fp32(decode(q[r,n])) * scale[r] )   (one fp32 multiply)
 *
 *   q      e4m3 [rows, N] (NaN codes 0x7F/0xFF are never produced by
 *          rowq_e4m3 and are outside the contract)
 *   scale  fp32 [rows]
 *   y      bf16 [rows, N]
 *
 * Requirements: rows >= 0, N > 0, N % 8 == 0; q, y 16-byte aligned, scale
 * 4-byte aligned; y must not overlap q or scale.
 */
bs_status rowdq_e4m3(const uint8_t *q, const float *scale, uint16_t *y,
                     int64_t rows, int64_t N, void *stream);

/*
 * Block quantizer for GEMM operands.  [MORI] "Running the benchmark"
 * (--quant blockscale: activations per 1x128 block, weights per 128x128
 * block, fp32 scales).  For each block of block_rows x 128 elements:
 * amax = max |x|; s = amax / 448 (fp32); codes = e4m3 of the fp32 quotient
 * x / s exactly as rowq_e4m3 (zero scale -> codes 0x00).
 *
 *   x      fp32 [rows, cols] (finite)
 *   q      e4m3 [rows, cols]
 *   scale  fp32 [ceil(rows/block_rows), cols/128]
 *
 * Requirements: block_rows is 1 or 128; rows >= 0; cols > 0, cols % 128 ==
 * 0; x, q 16-byte aligned; scale 4-byte aligned; no output overlaps x.
 */
bs_status blockq_e4m3(const float *x, uint8_t *q, float *scale,
                      int64_t rows, int64_t cols, int32_t block_rows,
                      void *stream);

/*
 * Activation quantizer: the bf16 layer input of bsgemm_fp8 quantised on the
 * GPU, as the layer does when it is handed a plain bf16 tensor ([PR43480]
 * "Numerics, measured where the path engages"), at the activation
 * granularity of [MORI] "Running the benchmark" (1x128 blocks, fp32 scales).
 * For each block of 128 consecutive elements of a row: amax = max |x|;
 * s = amax / 448 (fp32); codes = e4m3 of the fp32 quotient x / s exactly as
 * rowq_e4m3 (zero scale -> codes 0x00).  Identical to blockq_e4m3 with
 * block_rows = 1 on the fp32 values of x (every bf16 value is an fp32 value).
 *
 *   x      bf16 [rows, cols] (finite)
 *   q      e4m3 [rows, cols]
 *   scale  fp32 [rows, cols/128]
 *
 * Requirements: rows >= 0; cols > 0, cols % 128 == 0; x, q 16-byte aligned;
 * scale 4-byte aligned; no output overlaps x or the other output.
 */
bs_status actq_e4m3(const uint16_t *x, uint8_t *q, float *scale,
                    int64_t rows, int64_t cols, void *stream);

/*
 * Prepacks the weight B for bsgemm_fp8_pb: a one-time rearrangement done when
 * the weight is loaded ([PR43480], the review reply on the lazy second copy
 * of the weight; [PR40757] "What": the fused path serves only a weight that
 * was preshuffled at load).  Bp holds the same N*K bytes as B in the order
 * the GEMM's MFMA consumes them:
 *
 *   Bp[((nt * (K/128) + kb) * 2 + h) * 1024 + (16 g + r) * 16 + e]
 *       = B[brow(16 nt + r), 128 kb + 16 g + 64 h + e],
 *   brow(64 b + 16 j + r) = 64 b + 32 (j/2) + 8 (r/4) + 4 (j%2) + r%4
 *
 * for 16-row group nt, K block kb, half h in {0,1}, g in [0,4), r in [0,16),
 * e in [0,16): each 2 KiB block is one 16-row x 128 tile of B, laid out as
 * the 64 lanes' operand bytes, its rows taken within each 64-row group in the
 * order the GEMM's epilogue needs (brow).  The layout is a contract between this call and
 * bsgemm_fp8_pb only; nothing infers it from a shape ([PR43480] "Worth a
 * reviewer's attention": one layout read as the other gives garbage, not an
 * error).
 *
 *   B   e4m3 [N, K] row-major (the weight as stored, [out, in])
 *   Bp  e4m3, N*K bytes, prepacked (caller-owned, written here)
 *
 * Requirements: N > 0, N % 128 == 0; K > 0, K % 128 == 0, K <= 2^22; B and Bp
 * 16-byte aligned and not overlapping (no in-place prepack).
 */
bs_status bprepack_e4m3(const uint8_t *B, uint8_t *Bp, int64_t N, int64_t K,
                        void *stream);

/*
 * bsgemm_fp8 with the weight in the prepacked form bprepack_e4m3 writes: the
 * same operation, arguments, requirements, errors and results (bit for bit)
 * as bsgemm_fp8, except that B is replaced by Bp.  The kernel loads each
 * wave's B operands straight from Bp into registers (fully coalesced 1 KiB
 * loads), so B takes no LDS staging; A and the scales are staged as in
 * bsgemm_fp8.  Passing an unpacked B here (or Bp to bsgemm_fp8) is not
 * detected and gives a wrong result.
 */
bs_status bsgemm_fp8_pb(const uint8_t *A, const float *a_scale,
                        const uint8_t *Bp, const float *b_scale,
                        uint16_t *C, int64_t M, int64_t N, int64_t K,
                        int32_t bands, int64_t band_stride, void *stream);

/*
 * mxfp8 GEMM, the variant of [PR43480] "What" / "Not in this PR": C = A * B^T
 * with A [M,K] e4m3 and a_scale [M, K/32] E8M0 bytes (one per 1x32 block of
 * a row; value 2^(byte - 127)), B [N,K] e4m3 and b_scale [N, K/32] E8M0
 * bytes, fp32 accumulation, bf16 output, written in the same destination-major
 * bands as bsgemm_fp8 (bands, band_stride as there).  The block scales are
 * applied by gfx950's scaled MFMA; the sum is accumulated over K in fp32 in
 * the instruction's own order, so results are compared with the exact product
 * at a relL2 tolerance.
 *
 * Requirements: M >= 0; N > 0, N % 128 == 0; K > 0, K % 128 == 0, K <= 2^22;
 * bands in [1, 64] dividing M; band_stride 0 or >= (M/bands)*N and a multiple
 * of 8; A, B, C 16-byte aligned; a_scale, b_scale 4-byte aligned; C must not
 * overlap an input.
 */
bs_status mxgemm_fp8(const uint8_t *A, const uint8_t *a_scale,
                     const uint8_t *B, const uint8_t *b_scale,
                     uint16_t *C, int64_t M, int64_t N, int64_t K,
                     int32_t bands, int64_t band_stride, void *stream);

/*
 * mxfp8 operand quantizer ([PR43480] "Not in this PR": 32-wide ue8m0; the
 * review reply on the ue8m0 scale rule: exponent from the IEEE bits, exact at
 * powers of two).  For each block of 32 consecutive elements of a row:
 * amax = max |x|; the scale is 2^k with k the smallest integer such that
 * amax <= 448 * 2^k (clamped below at -127); scale byte = k + 127; codes =
 * e4m3 round-to-nearest-even of x * 2^-k (never saturating).  A zero block
 * gets scale byte 0 and codes 0x00.
 *
 *   x      bf16 [rows, cols] (finite)
 *   q      e4m3 [rows, cols]
 *   scale  E8M0 bytes [rows, cols/32]
 *
 * Requirements: rows >= 0; cols > 0, cols % 32 == 0; x, q 16-byte aligned; no
 * output overlaps x or the other output.
 */
bs_status mxq_e4m3(const uint16_t *x, uint8_t *q, uint8_t *scale,
                   int64_t rows, int64_t cols, void *stream);

/*
 * band_reduce followed by rowq_e4m3, fused into one kernel that never writes
 * the bf16 band: q, scale = rowq_e4m3(band_reduce(parts)), bit for bit (the
 * fp32 part-order sum is rounded to bf16 before the row quantizer sees it).
 * [MORI] "Negative results" reports that fusing the reduce with the quantize
 * was slower than the two separate kernels, because a row's amax needs the
 * whole row before any code can be written.  Here one workgroup takes each
 * row with several parts' loads in flight at once, and the fused pass moves
 * fewer bytes than the two kernels (the bf16 band is neither written nor
 * read back), so it is the faster of the two.
 *
 *   parts  host array of P device pointers, each bf16 [rows, N] (1 <= P <= 16)
 *   q      e4m3 [rows, N];  scale  fp32 [rows]
 *
 * Requirements: 0 <= rows < 2^31 (one workgroup per row); N > 0, N % 8 == 0,
 * N <= 8192; parts and q 16-byte aligned, scale 4-byte aligned; no output
 * overlaps a part or the other output.
 */
bs_status band_rowq_e4m3(const uint16_t *const *parts, int32_t P, uint8_t *q,
                         float *scale, int64_t rows, int64_t N, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *bs_status_str(bs_status status);

#ifdef __cplusplus
}
#endif

#endif /* BSGEMM_H */
