// Host-side helpers of the C ABI: argument checks, the per-thread error text, the
// workspace plan and the device check.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstddef>

#include "../../include/qgemv.h"

namespace qg {

qg_status fail(int status, const char* fmt, ...);   // records the message, returns status
void clear_error();

bool aligned16(const void* p);

// Returns QG_OK if the current device is gfx950, else an error status.
qg_status check_device();

// Compute units of the current device (after a successful check_device()).
int device_cus();

// Translate a launch error into QG_ERR_DEVICE (records the HIP message).
qg_status launch_status(const char* what);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Launch override of the calling host thread (qg_set_launch_override); all fields
// zero (automatic choice) unless a test or a measurement set them.
const qg_launch_override& launch_override();

// Top-k selection stage shared by logits_topk and lmhead_topk (topk_logprobs.hip).
// validate_topk checks k, M, the sampler and the outputs. The workspace starts
// with `tiles` per-tile partials (float4: max, row bits, exponential sum);
// launch_topk_select reduces them and the logits to the outputs and leaves the
// workspace all-zero.
qg_status validate_topk(int64_t M, int k, const qg_sampler* sampler, const qg_topk_out* out);
size_t topk_ws_bytes(int64_t M);
qg_status launch_topk_select(void* ws, int tiles, const float* logits, int64_t M, int k, const qg_sampler* sampler,
                       const qg_topk_out& out, hipStream_t s);

// Byte offsets of the int8 quants and of the block sums in a Q8_1 activation
// buffer of qg_q8_1_bytes(K) bytes (the block scales start at 0).
void q8_1_offsets(int64_t K, size_t* q_off, size_t* s_off);

// Vector-ALU dot-product form of the small-N product (q4k_smalln_dot.hip), for
// problems the small-N entry points have validated, each with N <= 8.
qg_status smalln_dot_launch(const qg_gemm_problem* probs, int count, hipStream_t s);

}  // namespace qg
