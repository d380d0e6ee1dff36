/*
 * qgemv.h - C ABI of the MI355X (gfx950) quantized GEMV library.
 *
 * What it computes (sources named by page title and section):
 *   - y = W x with W stored as GGUF-style Q4_K super-blocks or Q8_0 blocks and
 *     the dot products done directly on the packed blocks, dequantizing in
 *     registers ("dotLLM" README, Key Features / Performance: quantized inference
 *     with fused scale x int dot products on the quantized blocks; its news entry
 *     on the CUDA backend's custom quantized GEMV for decode; "Why Local LLMs Don't
 *     Need C++ or Python", section 1: dequantization multipliers and accumulators
 *     live in registers).
 *   - Y = W X for a few columns in one pass over the weights: the batched
 *     verification of K draft tokens (same page, section 4: the weights cross the
 *     memory bus once for the whole candidate batch) and the 32-token prefill tile
 *     (section 3).
 *   - the vocabulary projection fused with an on-device argmax that leaves one
 *     int32 token id (plus its logit) in device memory (same page, section 2).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host". They must be 16-byte
 *     aligned (hipMalloc and torch allocations are); otherwise QG_ERR_ALIGN.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronizes. Results are valid once the caller
 *     synchronizes or orders later work on the same stream.
 *   - The caller allocates and frees every buffer, including workspaces; the
 *     library holds no device memory of its own (the one exception,
 *     lmhead_argmax_noalloc, says so). Outputs must not alias inputs.
 *     Buffer ownership and explicit release follow "Building a Fully Custom C#
 *     LLM Runtime" (lease and dispose rules of its native buffers).
 *   - Arguments are validated on the host before anything is launched; on error
 *     the call returns a status, launches nothing and qg_last_error() (per host
 *     thread) describes the problem. A failed launch returns QG_ERR_DEVICE. A
 *     fault inside a kernel surfaces at the caller's next synchronization. A
 *     length that does not fit the operands is an error, never a silent
 *     truncation (the same page's checked dot product).
 *   - Calls are thread-safe. Two calls that share one workspace must be ordered
 *     on one stream (they would race otherwise).
 *
 * Arithmetic. fp32 activations are rounded to fp16 (round to nearest even) inside
 * the fp32-activation kernels, which multiply them by the integer quants exactly
 * and accumulate in fp32 (the dotLLM README's FP16 activation pipeline of its CUDA
 * decode GEMV). Each product then carries a relative error of at most 2^-11 for
 * |x| in the fp16 normal range [2^-14, 65504]; below it x becomes an fp16
 * subnormal (absolute error at most 2^-25), and |x| > 65504 becomes infinite, so
 * results turn into inf or NaN: keep activations inside +-65504. Every
 * per-block activation sum (the Q4_K mins, the Q6_K offset 32, the Q8_0 byte
 * bias) is taken over the same rounded values, so the result is within
 * 2^-11 * sum|w x| plus fp32 accumulation error of the exact product.
 *
 * Weight layout: the GEMV entry points take the *packed* layout written by
 * qg_pack_q4k / qg_pack_q8_0 / qg_pack_q6k, a byte permutation of the canonical
 * row-major block stream of exactly the same size (the dotLLM README's
 * row-interleaved weight repacking at load time, re-designed for 64-lane
 * wavefronts). Canonical blocks (GGUF reading; the pages name the formats but do
 * not print their bytes):
 *   Q4_K, 144 B per 256 weights: fp16 d, fp16 dmin, 12 bytes of 6-bit sub-scales
 *     and mins, 128 bytes of 4-bit quants; weight = d*sc*q - dmin*m.
 *   Q8_0, 34 B per 32 weights: fp16 d, 32 int8 q; weight = d*q.
 *
 * Workspaces: only the LM-head entry points (lmhead_argmax, lmhead_argmax_verify,
 * lmhead_argmax_verify_q8_1, lmhead_topk) and logits_topk take one; each reports
 * the bytes it needs through its *_workspace_bytes query. A workspace must be
 * all-zero when first used (qg_workspace_clear, or any zero-filled allocation)
 * and every call leaves it all-zero again, so one workspace can serve every entry
 * point in turn. A call that fails on the device may leave it dirty: clear it
 * again.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 2
#define QG_MAX_BATCH 8
#define QG_SMALLN_MAX 32

typedef void* qg_stream_t; /* hipStream_t */

typedef enum {
    QG_OK = 0,
    QG_ERR_NULL = 1,        /* a required pointer is NULL */
    QG_ERR_SHAPE = 2,       /* M, K, N, ld* or batch size out of range */
    QG_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    QG_ERR_WORKSPACE = 4,   /* workspace missing or too small */
    QG_ERR_DEVICE = 5,      /* HIP error at launch or device query */
    QG_ERR_UNSUPPORTED = 6  /* current device is not gfx950 */
} qg_status;

/* Library and status helpers (host only, never fail). */
int qg_abi_version(void);
const char* qg_status_string(int status);   /* static string */
const char* qg_last_error(void);            /* detail of this thread's last failure */

/* Size in bytes of an M x K matrix in Q4_K (K % 256 == 0) or Q8_0 (K % 32 == 0)
 * blocks; 0 for an invalid shape. Canonical and packed sizes are identical. */
size_t qg_q4k_bytes(int64_t M, int64_t K);
size_t qg_q8_0_bytes(int64_t M, int64_t K);

/*
 * Repack canonical row-major blocks (src) into the packed layout (dst), both
 * device buffers of qg_*_bytes(M, K); src and dst must not overlap (QG_ERR_SHAPE).
 * Load-time work, asynchronous on `stream` (dotLLM README, news entry on
 * row-interleaved weight repacking for all quantized GEMV kernels). Q4_K packed
 * layout: tiles of 16 rows (rt in the last tile); a super-block is nine 16-byte
 * segments (0: d, dmin and the scale bytes; 1+p: quant bytes 16p..16p+15), and
 * segment s of super-block b of row i sits at tile_base + ((b*9 + s)*rt + i)*16,
 * tile_base = tile*16*(K/256)*144. Q8_0: eight blocks form a macro-block of 17
 * segments (0: the eight scales; 1+2k+h: quants 16h..16h+15 of block k),
 * interleaved the same way; when K/32 is not a multiple of 8 the remaining blocks
 * of each row follow the tile's macro-blocks in canonical form. Shapes: M >= 1
 * (< 2^31), K as for the products below.
 */
qg_status qg_pack_q4k(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream);
qg_status qg_pack_q8_0(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream);

/* Zero-fill `bytes` of a device buffer with a kernel (no memset node, so it can
 * sit in a captured graph). */
qg_status qg_workspace_clear(void* workspace, size_t bytes, qg_stream_t stream);

/*
 * y[M] = W x[K], W an M x K Q4_K matrix in packed layout, x and y fp32 (dotLLM
 * README, Key Features: fused scale x int dot products on Q4_K blocks; news entry
 * on the CUDA backend's quantized decode GEMV). Per row r and super-block b:
 * y_r += d * sum_j sc_j * S_j - dmin * sum_j m_j * X_j over the eight 32-weight
 * sub-blocks, S_j the quant dot product and X_j the activation sum (the README's
 * precomputed block sums). x is rounded to fp16 (see Arithmetic above).
 * 1 <= M <= 2^31-1, K % 256 == 0, 256 <= K <= 2^24. Needs no workspace.
 */
qg_status qgemv_q4k(const void* w_packed, const float* x, float* y, int64_t M, int64_t K, qg_stream_t stream);

/*
 * Several independent Q4_K GEMVs in one launch (the dotLLM README's fused decode
 * dispatch of Q/K/V and of gate/up, news entry on the CUDA decode path). Problems
 * must not write overlapping outputs. 1 <= count <= QG_MAX_BATCH; each entry
 * follows qgemv_q4k's rules. Needs no workspace.
 */
typedef struct {
    const void* w_packed;
    const float* x;
    float* y;
    int64_t M;
    int64_t K;
} qg_gemv_problem;
qg_status qgemv_q4k_batch(const qg_gemv_problem* problems /* host */, int count, qg_stream_t stream);

/*
 * y[M] = W x[K], W an M x K Q8_0 matrix in packed layout (dotLLM README, Key
 * Features / Performance: Q8_0 blocks with fused scale x int dot products; news
 * entry on the CUDA decode GEMV). Per 32-block: y_r += d * sum q_l x_l. x is
 * rounded to fp16. 1 <= M <= 2^31-1, K % 32 == 0, 32 <= K <= 2^24. Needs no
 * workspace.
 */
qg_status qgemv_q8_0(const void* w_packed, const float* x, float* y, int64_t M, int64_t K, qg_stream_t stream);

/*
 * y[M] = W x[K], W an M x K Q6_K matrix in packed layout (qg_pack_q6k), x and y
 * fp32. Q6_K is the third K-quant format the dotLLM README's CUDA decode GEMV
 * covers (news entry on the CUDA backend; "Q4_K_M dequantization and vec_dot
 * kernels"). Canonical block, 210 B per 256 weights (GGUF reading; the pages name
 * the format but do not spell out its bytes): 128 bytes ql of low nibbles, 64
 * bytes qh of two-bit high parts, 16 int8 sub-scales, fp16 d; weight k of
 * sub-block j = k/16 is d * sc_j * (q_k - 32) with the six-bit q_k. Packed
 * layout, tiles of 16 rows (rt in the last tile): segment s < 13 (16 bytes: the
 * block's bytes 16s..16s+15) of super-block b of row i at
 * tile_base + ((b*13 + s)*rt + i)*16, d at tile_base + nb*13*rt*16 + (b*rt + i)*2,
 * tile_base = tile*16*nb*210. x is rounded to fp16. 1 <= M <= 2^31-17,
 * K % 256 == 0, 256 <= K <= 2^24. Needs no workspace.
 */
size_t qg_q6k_bytes(int64_t M, int64_t K);
qg_status qg_pack_q6k(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream);
qg_status qgemv_q6k(const void* w_packed, const float* x, float* y, int64_t M, int64_t K, qg_stream_t stream);

/*
 * Integer activations (dotLLM README, news entries on Q8_1 / Q8_K input
 * quantization: a float32 scale per block of activations with precomputed block
 * sums, feeding the fused K-quant dot products; the Q8_1 block of 32, one per
 * Q4_K sub-block). qg_quantize_q8_1 writes, for an fp32 x[K] (K % 256 == 0), the
 * buffer xq of qg_q8_1_bytes(K) bytes:
 *   float d[K/32] at 0; int8 q[K] at q_off = align16(4*(K/32));
 *   int16 s[K/32] at align16(q_off + K);
 * with d_c = max|x| / 127 over block c and q = round-half-to-even(x / d_c) in
 * float32 (0 when d_c = 0), s_c = the sum of the block's q. qgemv_q4k_q8_1
 * computes y[M] = W xq for the packed Q4_K matrix W and the quantized activations
 * xq_k = d[k/32] * q[k]: each 32-weight dot product is an exact int32
 * (v_dot4c_i32_i8), scaled by d, dmin and d_c in fp32. The quantization error
 * stays within the library's 1e-3 * sum|w x| bound at the 7B decode shapes
 * (measured below 0.8 of it at K = 3584), with a smaller margin at small K.
 * qg_quantize_q8_1_columns quantizes N columns of a column-major K x N matrix
 * (column n at X + n*ldx, ldx >= K, a multiple of 4) into N consecutive buffers
 * (buffer n at xq + n*qg_q8_1_bytes(K)) in one launch; 1 <= N <= QG_SMALLN_MAX.
 * No workspace; shape rules as for qgemv_q4k.
 */
size_t qg_q8_1_bytes(int64_t K);
qg_status qg_quantize_q8_1(const float* x, int64_t K, void* xq, qg_stream_t stream);
qg_status qg_quantize_q8_1_columns(const float* X, int64_t ldx, int64_t K, int64_t N, void* xq,
                                   qg_stream_t stream);
qg_status qgemv_q4k_q8_1(const void* w_packed, const void* xq, float* y, int64_t M, int64_t K,
                         qg_stream_t stream);

/* Several independent qgemv_q4k_q8_1 products in one launch (as qgemv_q4k_batch:
 * the dotLLM README's fused Q/K/V and gate/up decode dispatch). No workspace. */
typedef struct {
    const void* w_packed;
    const void* xq;
    float* y;
    int64_t M;
    int64_t K;
} qg_gemv_q8_1_problem;
qg_status qgemv_q4k_q8_1_batch(const qg_gemv_q8_1_problem* problems /* host */, int count, qg_stream_t stream);

/*
 * Y = W Xq for N <= 8 int8-quantized activation columns in one pass over the
 * packed Q4_K matrix W (batched verification, "Why Local LLMs Don't Need C++ or
 * Python", section 4, on the integer path of the dotLLM README's Q8_1 input
 * quantization). xq holds N consecutive buffers of qg_q8_1_bytes(K) bytes, column n
 * at xq + n * qg_q8_1_bytes(K), each written by qg_quantize_q8_1 (or all by
 * qg_quantize_q8_1_columns). Y is column-major (column n at Y + n * ldy, ldy >= M,
 * a multiple of 4). Column n equals qgemv_q4k_q8_1 of buffer n (bit for bit when
 * K >= 2304). 1 <= N <= 8; other shape rules as for qgemv_q4k_q8_1. No workspace.
 */
typedef struct {
    const void* w_packed;
    const void* xq;
    float* Y;
    int64_t ldy;
    int64_t M;
    int64_t K;
    int64_t N;
} qg_gemm_q8_1_problem;
qg_status qgemm_q4k_q8_1_smalln(const void* w_packed, const void* xq, float* Y, int64_t ldy, int64_t M, int64_t K,
                                int64_t N, qg_stream_t stream);
qg_status qgemm_q4k_q8_1_smalln_batch(const qg_gemm_q8_1_problem* problems /* host */, int count,
                                      qg_stream_t stream);

/*
 * Small-N verify / prefill product, one pass over the weights ("Why Local LLMs
 * Don't Need C++ or Python", section 4, batched verification; section 3, the
 * 32-token prefill tile):
 *   Y[:, n] = W X[:, n] for 0 <= n < N, 1 <= N <= QG_SMALLN_MAX.
 * W is an M x K Q4_K matrix in packed layout. X is column-major K x N with
 * leading dimension ldx >= K (column n starts at X + n*ldx); Y is column-major
 * M x N with ldy >= M. ldx and ldy must be multiples of 4, and X must span less
 * than 2^31 bytes ((N-1)*ldx + K < 2^29 elements; otherwise QG_ERR_SHAPE). The
 * activations are rounded to fp16 (see Arithmetic above). Up to four columns run
 * on the vector ALUs (four dot2 operations per 8 weights and column); above, each
 * 32-weight sub-block is a 16 x 16 x 32 fp16 matrix-core product of the
 * activations with the quants, scaled in fp32. Only Y[0..M) of each column is
 * written. Results are deterministic. Needs no workspace.
 */
qg_status qgemm_q4k_smalln(const void* w_packed, const float* X, int64_t ldx, float* Y, int64_t ldy,
                           int64_t M, int64_t K, int64_t N, qg_stream_t stream);

/*
 * Several independent small-N products in one launch (the same grouping as
 * qgemv_q4k_batch: the dotLLM README's fused Q/K/V and gate/up dispatch, here for
 * the verification batch of "Why Local LLMs Don't Need C++ or Python", section
 * 4). 1 <= count <= QG_MAX_BATCH; each entry follows
 * qgemm_q4k_smalln's rules; outputs must not overlap. No workspace.
 */
typedef struct {
    const void* w_packed;
    const float* X;
    int64_t ldx;
    float* Y;
    int64_t ldy;
    int64_t M;
    int64_t K;
    int64_t N;
} qg_gemm_problem;
qg_status qgemm_q4k_smalln_batch(const qg_gemm_problem* problems /* host */, int count, qg_stream_t stream);

/*
 * The same batch with a caller-owned workspace ("Why Local LLMs Don't Need C++ or
 * Python", section 4: the batched verification pass, here for batches of few
 * tiles and many columns, where the activations outweigh the weights). With a
 * workspace the library may split each product over groups of tiles that share
 * one staging of the activations and over slices of K; the slices' partial sums go
 * to the workspace, and the last workgroup of each tile group to finish (counted
 * on a per-group counter in the workspace) adds them in slice order, so results
 * stay deterministic and equal, to the bound in Arithmetic above, those of
 * qgemm_q4k_smalln_batch (with another rounding order). _workspace_bytes gives
 * the bytes the batch needs on the current device (0: none; invalid problems:
 * 0). The workspace (16-byte aligned, at least that size) must be zero-filled
 * before its first use (qg_workspace_clear); the counters sit in a fixed block at
 * its start that every call leaves zero, and the rest of it is left with undefined
 * contents, so one workspace serves calls of any shapes, but a buffer shared with
 * the LM-head calls (whose workspaces must stay all-zero) has to be cleared again
 * before they use it. A smaller or NULL workspace where one is needed:
 * QG_ERR_WORKSPACE. Calls that share a workspace must not overlap.
 */
size_t qgemm_q4k_smalln_batch_workspace_bytes(const qg_gemm_problem* problems /* host */, int count);
qg_status qgemm_q4k_smalln_batch_ws(const qg_gemm_problem* problems /* host */, int count, void* workspace,
                                    size_t workspace_bytes, qg_stream_t stream);

/*
 * Fused LM head ("Why Local LLMs Don't Need C++ or Python", section 2: the final
 * projection and the argmax reduction stay on the device and a single int32 token
 * id crosses to the host instead of the logit vector): logits = W x (W an M x K
 * Q8_0 matrix, packed; x fp32 rounded to fp16) reduced on the device to the first
 * maximum: out_index[0] = min{ i : logit_i = max_j logit_j } and, if out_value is
 * not NULL, out_value[0] = logit_{out_index}. The logits never leave the chip.
 * 1 <= M <= 2^31-1 (the index is int32), K as for qgemv_q8_0. NaN logits never
 * win; if every logit is NaN (only possible with |x| > 65504 or NaN inputs),
 * out_index[0] = -1 and out_value[0] = -inf. out_index / out_value are device
 * pointers (4-byte alignment suffices). Workspace: 8 bytes per 16-row tile
 * (lmhead_argmax_workspace_bytes), left all-zero.
 */
size_t lmhead_argmax_workspace_bytes(int64_t M, int64_t K);
qg_status lmhead_argmax(const void* w_packed_q8_0, const float* x, int64_t M, int64_t K,
                        void* workspace, size_t workspace_bytes,
                        int32_t* out_index, float* out_value, qg_stream_t stream);

/*
 * lmhead_argmax for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and the same result as lmhead_argmax, bit for bit, with the per-tile
 * partials in a fixed array inside the library instead of a caller workspace:
 * 256 KiB per GPU, present from library load until the process ends, so
 * M <= 524288 (QG_ERR_SHAPE above). The call allocates nothing. Every call on one
 * GPU uses that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and give wrong results; order them on one stream. The array needs
 * no clearing between calls (every partial is written before it is read).
 */
qg_status lmhead_argmax_noalloc(const void* w_packed_q8_0, const float* x, int64_t M, int64_t K,
                                int32_t* out_index, float* out_value, qg_stream_t stream);

/*
 * Batched greedy verification on the LM head ("Why Local LLMs Don't Need C++ or
 * Python", section 2: projection and argmax fused on the device, one int32 per
 * decision; section 4: the candidate tokens are verified in one batched pass over
 * the weights). For each column n < N of X (column-major K x N, ldx >= K, a
 * multiple of 4): out_index[n] = min{ i : logit_{i,n} = max_j logit_{j,n} } and,
 * if out_value is not NULL, out_value[n] = that logit, with logits = W X[:, n] and
 * W an M x K Q8_0 matrix in packed layout. 1 <= N <= QG_SMALLN_MAX, K % 256 == 0.
 * The weights are read once for all N columns and no logit reaches HBM. Needs
 * lmhead_argmax_verify_workspace_bytes(M, K, N) bytes of workspace (8 bytes per
 * 16-row tile and column, and for N <= 6 another 2.125 K bytes per column for the
 * columns rounded to fp16 and their block sums; left zero). The activations are
 * rounded to fp16 for the products in either case. NaN logits never win; a column
 * whose logits are all NaN gets index -1.
 */
size_t lmhead_argmax_verify_workspace_bytes(int64_t M, int64_t K, int64_t N);
qg_status lmhead_argmax_verify(const void* w_packed_q8_0, const float* X, int64_t ldx, int64_t M, int64_t K,
                               int64_t N, void* workspace, size_t workspace_bytes,
                               int32_t* out_index, float* out_value, qg_stream_t stream);

/*
 * The same batched verification with int8 activations (the dotLLM README's Q8_1
 * input quantization on the integer path): xq holds N consecutive buffers of
 * qg_q8_1_bytes(K) bytes, column n at xq + n * qg_q8_1_bytes(K), each written by
 * qg_quantize_q8_1. logit_{i,n} = sum_k w_ik d_n[k/32] q_n[k]; both quant operands
 * are int8, the integer block products are exact and each block's term is scaled in
 * fp32. 1 <= N <= 8, K % 256 == 0; outputs, workspace
 * (lmhead_argmax_verify_q8_1_workspace_bytes(M, K, N), left zero) and the argmax
 * rule as for lmhead_argmax_verify.
 */
size_t lmhead_argmax_verify_q8_1_workspace_bytes(int64_t M, int64_t K, int64_t N);
qg_status lmhead_argmax_verify_q8_1(const void* w_packed_q8_0, const void* xq, int64_t M, int64_t K, int64_t N,
                                    void* workspace, size_t workspace_bytes,
                                    int32_t* out_index, float* out_value, qg_stream_t stream);

/*
 * Top-k, log-softmax and the top-k sampler over a logit vector, on the device
 * (dotLLM README: the news entry on log-probabilities, top_logprobs 0..20 from
 * the per-token log-softmax taken before sampling; Key Features, composable
 * sampling: temperature -> top-k -> top-p -> min-p -> categorical draw). The k
 * best rows are ranked by logit, equal logits by lower row; NaN logits count as
 * -inf. Results (device pointers in qg_topk_out; NULL skips an optional one):
 *   index[k]   row ids, best first (required)
 *   logit[k]   their logits
 *   logprob[k] logit - lse
 *   lse[1]     log(sum_r exp(logit_r)) over all M rows, fp32
 *   token[1]   with a sampler: one draw from the chain over the k best, at
 *              temperature T (T <= 0: index[0]); top-p keeps the shortest prefix
 *              whose weight exp((z_i - z_0)/T) reaches top_p of the k-total, min-p
 *              the entries whose weight is at least min_p times the largest, and
 *              the draw returns the first kept position whose cumulative weight
 *              exceeds u times the kept total. u is one uniform number in [0, 1)
 *              that the caller draws and passes in device memory.
 * 1 <= k <= QG_TOPK_MAX, k <= M <= QG_TOPK_MAX_ROWS; 0 < top_p <= 1, 0 <= min_p <= 1.
 * Workspace: 16 bytes per 16 rows (per-tile maxima and exponential sums), cleared
 * again by the call.
 */
#define QG_TOPK_MAX 64
#define QG_TOPK_MAX_ROWS 262144

typedef struct {
    int32_t* index;
    float* logit;
    float* logprob;
    float* lse;
    int32_t* token;
} qg_topk_out;

typedef struct {
    float temperature;
    float top_p;
    float min_p;
    const float* u; /* device pointer to one float */
} qg_sampler;

/* Over an fp32 logit vector already in device memory (the dotLLM README's
 * log-probability and sampling chain, as above, on logits another kernel wrote). */
size_t logits_topk_workspace_bytes(int64_t M);
qg_status logits_topk(const float* logits, int64_t M, int k, const qg_sampler* sampler /* host, or NULL */,
                      void* workspace, size_t workspace_bytes, const qg_topk_out* out /* host */,
                      qg_stream_t stream);

/*
 * Fused with the Q8_0 LM head ("Why Local LLMs Don't Need C++ or Python", section
 * 2, with the dotLLM README's top_logprobs): logits = W x (W packed, M x K, K % 32 == 0) are
 * computed tile by tile and left in the caller's device buffer logits[M] (they
 * never cross to the host); the per-tile statistics come out of the same kernel,
 * and one more launch selects, normalizes and samples.
 */
size_t lmhead_topk_workspace_bytes(int64_t M, int64_t K);
qg_status lmhead_topk(const void* w_packed, const float* x, int64_t M, int64_t K, int k, float* logits,
                      const qg_sampler* sampler /* host, or NULL */, void* workspace, size_t workspace_bytes,
                      const qg_topk_out* out /* host */, qg_stream_t stream);

/*
 * Launch override, for tests and measurements only (not needed for correct
 * results): forces a kernel form or launch shape for every later call made from
 * the calling host thread, until reset by a NULL argument. A zero field keeps the
 * automatic choice. Every form computes the same products to the same bound;
 * forcing a form outside the range it supports (a dot form above 8 columns, the
 * single-pass small-N form above K = 4096 or 8 columns) falls back to the
 * automatic choice. Values outside the listed ones give QG_ERR_SHAPE and leave
 * the override unchanged.
 *   gemv_waves    wavefronts per 16-row tile of the single-column kernels
 *                 (qgemv_q4k*, qgemv_q4k_q8_1*, qgemv_q6k, qgemv_q8_0, the LM-head
 *                 tile kernels): 1, 2, 4, 8.
 *   smalln_form   qgemm_q4k_smalln*: register-staged matrix-core, chunked-LDS
 *                 matrix-core, single-pass-LDS matrix-core, vector-ALU dot form,
 *                 the streamed single-pass form (workgroups walk several tiles;
 *                 the single-pass shapes, the weights of each matrix < 2 GiB), or
 *                 the chunked walk form (one workgroup per CU walks several tiles
 *                 chunk by chunk along K; any K, the weights of each matrix < 2 GiB),
 *                 or that form over tile groups and K slices (the _ws entry point
 *                 with a workspace only), or tile groups and K slices whose
 *                 activations are staged whole before the weights are walked (the
 *                 _ws entry point, up to 16 columns and N times the slice's
 *                 super-blocks at most 160; else as the previous value; without
 *                 a workspace, the same form with no K slices over groups of two
 *                 tiles, where N times K / 256 is at most 160).
 *   smalln_waves  wavefronts per workgroup of the register-staged form: 1..8.
 *   smalln_tiles  16-row tiles per workgroup (matrix-core forms): 1, 2, 4.
 *   smalln_depth  weight-queue depth in chunks of the chunked-LDS form: 2..4.
 *   verify_form   lmhead_argmax_verify: matrix-core, vector-ALU dot, or streamed
 *                 matrix-core form (N <= 16, K <= 4096).
 *   verify_waves  wavefronts per workgroup of the verify tile kernels (the dot
 *                 and int8 forms: 1 or 4; the matrix-core form: 4 or 8).
 *   verify_tiles  tiles per workgroup of the matrix-core verify form: 1, 2, 4.
 */
#define QG_FORM_AUTO 0
#define QG_FORM_SMALLN_REGS 1
#define QG_FORM_SMALLN_LDS 2
#define QG_FORM_SMALLN_LDS1 3
#define QG_FORM_SMALLN_DOT 4
#define QG_FORM_SMALLN_STREAM 5
#define QG_FORM_SMALLN_WALK 6
#define QG_FORM_SMALLN_SPLIT 7
#define QG_FORM_SMALLN_SLICE 8
#define QG_FORM_VERIFY_MFMA 1
#define QG_FORM_VERIFY_DOT 2
#define QG_FORM_VERIFY_STREAM 3
typedef struct {
    int gemv_waves;
    int smalln_form;
    int smalln_waves;
    int smalln_tiles;
    int smalln_depth;
    int verify_form;
    int verify_waves;
    int verify_tiles;
} qg_launch_override;
qg_status qg_set_launch_override(const qg_launch_override* o /* host, or NULL */);
qg_status qg_get_launch_override(qg_launch_override* o /* host */);

#ifdef __cplusplus
}
#endif
#endif
