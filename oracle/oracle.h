/*
 * CPU oracle for the quantized GEMV / small-N GEMM / LM-head argmax path.
 *
 * TEST INFRASTRUCTURE ONLY. It is plain, slow and written to be checked by eye
 * against the definitions; it shares no code with the GPU library and the GPU
 * library never links it. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.
 *
 * Everything is computed in fp64 with sequential (k = 0, 1, 2, ...) summation.
 *
 * Formats. The pages name the block formats (the dotLLM README, "Key Features /
 * Performance: Quantized inference" lists FP16, Q8_0 and Q4_K_M with fused
 * scale x int dot products on the quantized blocks; its CUDA backend news entry
 * lists decode GEMV for Q8_0 and Q4_K) but print no byte layout. The layout used
 * here is the GGUF reading:
 *   Q4_K (144 B / 256 weights): fp16 d, fp16 dmin, 12 bytes of 6-bit sub-scales
 *     sc[0..7] and mins m[0..7], 128 bytes of nibbles. Weight 32*j + l of the
 *     block is d*sc[j]*q - dmin*m[j], q its 4-bit quant. Quant byte 32*g + l
 *     holds weight 64*g + l in its low nibble and weight 64*g + 32 + l in its
 *     high nibble.
 *   Q8_0 (34 B / 32 weights): fp16 d, 32 int8 q; weight i is d*q[i].
 *   Q6_K (210 B / 256 weights; the third K-quant of the dotLLM README's news
 *     entries, which the pages name without a layout): 128 bytes ql (low four
 *     bits of each quant), 64 bytes qh (high two bits), 16 int8 sub-block
 *     scales, fp16 d. Weight i is d*sc[i/16]*(q_i - 32), q_i its 6-bit quant.
 *     In each 128-weight half h (ql + 64h, qh + 32h), for l < 32 and p < 4,
 *     weight 128h + 32p + l takes its low four bits from byte ql[l + 32(p%2)]
 *     (low nibble for p < 2, high nibble for p >= 2) and its high two bits from
 *     bits 2p, 2p+1 of qh[l].
 * Compatibility of this reading with real GGUF files is parity unpinned (no
 * file, decoder or format document is available); the pins in the tests fix the
 * oracle to the reading itself.
 */
#ifndef QG_ORACLE_H
#define QG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 bit pattern -> double, exactly (subnormals, inf, NaN). */
double or_half_to_double(uint16_t h);

/* Unpack the twelve 6-bit-field bytes of a Q4_K block into sc[8], m[8]. */
void or_q4k_unpack_scales(const uint8_t s[12], int sc[8], int m[8]);

/* Dequantize one block. w receives 256 (Q4_K, Q6_K) or 32 (Q8_0) doubles. */
void or_q4k_dequant_block(const uint8_t blk[144], double w[256]);
void or_q8_0_dequant_block(const uint8_t blk[34], double w[32]);
void or_q6k_dequant_block(const uint8_t blk[210], double w[256]);

/* Dequantize a whole row of K weights (K/256 Q4_K or K/32 Q8_0 blocks). */
void or_q4k_dequant_row(const uint8_t* row, int64_t K, double* w);
void or_q8_0_dequant_row(const uint8_t* row, int64_t K, double* w);
void or_q6k_dequant_row(const uint8_t* row, int64_t K, double* w);

/*
 * y = W x for the rows listed in rows[0..nrows) (rows == NULL: rows 0..nrows-1).
 * W is canonical row-major blocks, M rows of K weights. Outputs are indexed by
 * list position i: y[i] = sum_k w[r][k] * x[k], a[i] = sum_k |w[r][k] * x[k]|
 * (a may be NULL). Dense form: dequantize the row, then one sequential dot.
 */
void or_gemv_q4k(const uint8_t* W, int64_t M, int64_t K, const float* x,
                 const int64_t* rows, int64_t nrows, double* y, double* a);
void or_gemv_q8_0(const uint8_t* W, int64_t M, int64_t K, const float* x,
                  const int64_t* rows, int64_t nrows, double* y, double* a);
void or_gemv_q6k(const uint8_t* W, int64_t M, int64_t K, const float* x,
                 const int64_t* rows, int64_t nrows, double* y, double* a);

/*
 * Factored Q4_K form: per 32-weight sub-block, S = sum q*x and X = sum x, then
 * y += d*sc*S - dmin*m*X. Same result as the dense form up to rounding order.
 */
void or_gemv_q4k_factored(const uint8_t* W, int64_t M, int64_t K, const float* x,
                          const int64_t* rows, int64_t nrows, double* y);

/*
 * Small-N product Y[:, n] = W X[:, n], n < N. X is column-major with leading
 * dimension ldx (column n starts at X + n*ldx). Outputs: Y[n*nrows + i] and
 * A[n*nrows + i] (A may be NULL) for listed row i.
 */
void or_gemm_q4k(const uint8_t* W, int64_t M, int64_t K, const float* X, int64_t ldx,
                 int64_t N, const int64_t* rows, int64_t nrows, double* Y, double* A);

/* Lowest index i with y[i] == max_j y[j] (first maximum); -1 if n <= 0. */
int64_t or_argmax(const double* y, int64_t n);

/* Number of OpenMP threads the row loops use (1 without OpenMP). */
int or_num_threads(void);
void or_set_num_threads(int n); /* threads for later calls (scheduling only) */

/*
 * Integer-activation form (dotLLM README news: Q8_1 / Q8_K input quantization,
 * a float32 scale per block of activations with precomputed block sums, feeding
 * fused K-quant dot products). Reading, with the Q8_1 block of 32 (one block per
 * Q4_K sub-block; a scale per 256 was measured to exceed the product tolerance on
 * some rows at K = 3584): per block of 32 activations, amax = max |x|,
 * d = amax / 127 and q = round-half-even(x / d) clamped to [-127, 127], both in
 * float32 as written (q = 0 when d = 0); s = the sum of the block's q. The
 * quantization takes integer decisions, so it is done in the float32 arithmetic
 * a GPU kernel would use (one correctly rounded division and one rounding per
 * element) rather than in fp64.
 */
void or_quantize_q8_1(const float* x, int64_t K, float* d, int8_t* q, int16_t* s);

/* y = W xq for a Q4_K matrix W and the dequantized activations xq_k = d[k/32] * q[k]
 * (fp64, dense form; rows and a as for or_gemv_q4k). */
void or_gemv_q4k_q8_1(const uint8_t* W, int64_t M, int64_t K, const float* d, const int8_t* q,
                      const int64_t* rows, int64_t nrows, double* y, double* a);

/* y = W xq for a Q8_0 matrix W (the LM head) and the same dequantized activations
 * xq_k = d[k/32] * q[k] (fp64, dense form; rows and a as for or_gemv_q8_0). */
void or_gemv_q8_0_q8_1(const uint8_t* W, int64_t M, int64_t K, const float* d, const int8_t* q,
                       const int64_t* rows, int64_t nrows, double* y, double* a);

/*
 * Sampling-side reductions over a logit vector (dotLLM README: the news entry on
 * log-probabilities, top_logprobs 0..20 from the per-token log-softmax taken
 * before sampling; Key Features, composable sampling: temperature -> top-k ->
 * top-p -> min-p -> categorical draw). NaN logits count as -inf throughout.
 */

/* The k best entries of z[0..n), best first, in the order "larger value first,
 * equal values by lower index": k rounds of a first-maximum search that skips
 * the entries already taken. Requires 1 <= k <= n. */
void or_topk(const double* z, int64_t n, int k, int64_t* out_idx);

/* log(sum_i exp(z_i)) as max + log(sum exp(z_i - max)); -inf if every entry is
 * -inf. */
double or_logsumexp(const double* z, int64_t n);

/*
 * One draw from the sampler chain over the k best logits z[0..k), best first:
 * temperature T (T <= 0: greedy, returns 0), weights q_i = exp((z_i - z_0) / T);
 * top-p keeps the shortest prefix whose weight reaches top_p of the k-total
 * (top_p >= 1 keeps all); min-p keeps, of those, the entries with
 * q_i >= min_p * q_0; the draw returns the first position j whose cumulative
 * weight exceeds u times the kept total (u in [0, 1) is the caller's uniform
 * random number).
 */
int or_sample_topk(const double* z, int k, double temperature, double top_p, double min_p, double u);

#ifdef __cplusplus
}
#endif
#endif
