// Q8_0 weight-only GEMV and the fused LM-head projection + argmax for gfx950.
//
// Q8_0 (dotLLM README, Key Features / Performance: FP16, Q8_0, Q4_K_M blocks with
// fused scale x int dot products; news entry on the CUDA backend's quantized decode
// GEMV): a block is an fp16 scale d and 32 int8 quants, y_r += d * sum_l q_l x_l.
//
// Fused LM head ("Why Local LLMs Don't Need C++ or Python", section 2: the final
// projection and the argmax reduction run on the device and only one int32 token
// id crosses to the host): each workgroup computes the logits of its 16-row tile in
// registers, reduces them to (max, lowest index) and writes one 8-byte partial; a
// second, single-workgroup launch reduces the partials in a fixed order and writes
// the winning index and its logit. The logits never reach HBM.
//
// Packed layout (same size as the canonical 34-byte block stream): rows in tiles of
// 16; eight consecutive blocks form a 256-weight macro-block of 17 sixteen-byte
// segments (segment 0: the eight fp16 scales; segment 1+2k+h: quants 16h..16h+15 of
// block k). Segment s of macro-block mb of row i of a tile with rt rows sits at
//     tile_base + ((mb * 17 + s) * rt + i) * 16,   tile_base = tile * 16 * nbq * 34.
// When K/32 is not a multiple of 8, the remaining blocks of each row follow the
// macro-blocks of the tile, row after row, in canonical 34-byte form.
//
// Inner product, as in the Q4_K GEMV: a wavefront is four 16-lane DPP rows
// ("K-groups", lane = weight row); each K-group walks half macro-blocks (4 blocks,
// 128 weights) of its own. The int8 quants become signed fp16 subnormals
// q * 2^-24 in place (a byte bias, one byte permutation and one exact packed fp16
// addition per two quants: qg_q8_signed_masks), and v_dot2c_f32_f16 with a DPP
// row broadcast feeds each lane the fp16 activation pair it needs from the lane
// that holds it: per 4 weights 5 bit and fp16 operations and 2 dot2 operations.
// The products are exact and every partial sum is bounded by sum |q x|, so the
// result is within 2^-11 * sum|w x| plus fp32 accumulation error of the exact
// product (x rounded to fp16), also for rows whose quants are all zero.
#include <algorithm>
#include <climits>
#include <mutex>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;

struct Q8Prob {
    const uint8_t* w;
    const float* x;
    float* y;
    int32_t M, nbq, nmb, tb;  // rows, 32-blocks per row, macro-blocks, tail blocks
    int32_t tiles;
};

struct HalfIn {
    uint4 s[9];      // scale segment, then the 8 quant segments of blocks 4h..4h+3
    float4 xa, xb;   // this lane's 8 activations
};

// Half macro-block `u` (= 2*mb + h) of row `seg` (already offset to the row).
QG_DEV void load_half(HalfIn& d, const uint4* __restrict__ seg, const float* __restrict__ xk, int u, int rt) {
    const int mb = u >> 1, h = u & 1;
    const float* xb = xk + 128 * u;
    d.xa = *reinterpret_cast<const float4*>(xb);
    d.xb = *reinterpret_cast<const float4*>(xb + 4);
    const uint4* base = seg + (size_t)mb * 17 * rt;
    d.s[0] = base[0];  // the scales serve both halves: a cached load
#pragma unroll
    for (int s = 0; s < 8; ++s) d.s[1 + s] = qg_stream_load(base + (size_t)(1 + 8 * h + s) * rt);
}

// Contribution of half macro-block h for this lane's row: the signed quants as
// fp16 subnormals (qg_q8_signed_masks), so a block's product needs no activation
// sum and the block's term is d * 2^24 * S.
QG_DEV float half_dot(const HalfIn& d, int h) {
    const QgPairs4 xp = qg_cvt_pairs4(d.xa, d.xb);
    const uint4 x = make_uint4(xp.p[0], xp.p[1], xp.p[2], xp.p[3]);
    const uint32_t dw0 = h ? d.s[0].z : d.s[0].x;
    const uint32_t dw1 = h ? d.s[0].w : d.s[0].y;
    constexpr float two24 = 16777216.0f;
    const float dk[4] = {two24 * qg_half_lo(dw0), two24 * qg_half_hi(dw0), two24 * qg_half_lo(dw1),
                         two24 * qg_half_hi(dw1)};
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t m0[8], m1[8];
        qg_q8_signed_masks(m0, d.s[1 + 2 * k]);
        qg_q8_signed_masks(m1, d.s[2 + 2 * k]);
        float a[4] = {0.f, 0.f, 0.f, 0.f};
        switch (k) {
            case 0: qg_q8_seg8h_dot<0, false>(a, m0, x); qg_q8_seg8h_dot<2, true>(a, m1, x); break;
            case 1: qg_q8_seg8h_dot<4, false>(a, m0, x); qg_q8_seg8h_dot<6, true>(a, m1, x); break;
            case 2: qg_q8_seg8h_dot<8, false>(a, m0, x); qg_q8_seg8h_dot<10, true>(a, m1, x); break;
            default: qg_q8_seg8h_dot<12, false>(a, m0, x); qg_q8_seg8h_dot<14, true>(a, m1, x); break;
        }
        acc = fmaf(dk[k], (a[0] + a[1]) + (a[2] + a[3]), acc);
    }
    return acc;
}

// Remaining (K/32 mod 8) blocks of one row, canonical 34-byte form, 2-byte aligned.
QG_DEV float tail_dot(const uint8_t* __restrict__ rowtail, int tb, qg_uniform_f32 xs) {
    float acc = 0.f;
    for (int k = 0; k < tb; ++k) {
        const uint8_t* blk = rowtail + 34 * k;
        const uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
        const float dk = (float)__builtin_bit_cast(_Float16, dbits);
        float s = 0.f;
        for (int l = 0; l < 32; ++l) s = fmaf((float)(int8_t)blk[2 + l], xs[32 * k + l], s);
        acc = fmaf(dk, s, acc);
    }
    return acc;
}

// Dot products of the 16 rows of `tile` with x; the value for row (lane % 16) is
// returned in every lane of wavefront 0 (lanes 0..15 are the ones to use).
template <int W>
QG_DEV float tile_rows(const Q8Prob& P, int tile, int lane, int wave) {
    const int rt = min(T, P.M - tile * T);
    const int i = lane & 15;
    const int kg = 4 * wave + (lane >> 4);
    constexpr int G = 4 * W;
    const uint8_t* tbase = P.w + (size_t)tile * T * P.nbq * 34;
    const uint4* __restrict__ seg = reinterpret_cast<const uint4*>(tbase) + min(i, rt - 1);
    // activation slot: quant segment j = i/2 (block j/2, half j%2), dwords 2(i%2), +1
    const int j = i >> 1;
    const float* xk = P.x + 32 * (j >> 1) + 16 * (j & 1) + 8 * (i & 1);
    const int nu = 2 * P.nmb;  // half macro-blocks per row

    float acc = 0.f;
    if (nu > 0) {
        // Ping-pong between two register buffers over pairs of half macro-blocks:
        // the loads of one stay in flight while the other is computed. Loads are
        // unconditional (index clamped to the last one) and the pair loop has a
        // single exit, so every wait count is exact.
        const int niter = (nu + G - 1) / G;
        HalfIn b0, b1;
        load_half(b0, seg, xk, min(kg, nu - 1), rt);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            const int u = kg + G * it;
            load_half(b1, seg, xk, min(u + G, nu - 1), rt);
            __builtin_amdgcn_sched_barrier(0);  // issue the loads before any wait
            const float v0 = half_dot(b0, u & 1);
            acc += (u < nu) ? v0 : 0.f;
            load_half(b0, seg, xk, min(u + 2 * G, nu - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            const float v1 = half_dot(b1, (u + G) & 1);
            acc += (u + G < nu) ? v1 : 0.f;
        }
        if (it < niter) {
            const int u = kg + G * it;
            const float v0 = half_dot(b0, u & 1);
            acc += (u < nu) ? v0 : 0.f;
        }
    }
    if (P.tb > 0 && kg == 0 && i < rt) {
        const uint8_t* rowtail = tbase + (size_t)P.nmb * 17 * rt * 16 + (size_t)i * P.tb * 34;
        acc += tail_dot(rowtail, P.tb, (qg_uniform_f32)P.x + 256 * P.nmb);
    }
    float v = qg_sum_rows4(acc);
    if constexpr (W > 1) {
        __shared__ float red[W][T];
        if (lane < T) red[wave][lane] = v;
        __syncthreads();
        if (lane < T) {
            v = red[0][lane];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w][lane];
        }
    }
    return v;
}

template <int W>
__global__ __launch_bounds__(64 * W) void q8_0_gemv_kernel(Q8Prob P) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float v = tile_rows<W>(P, tile, lane, wave);
    const int rt = min(T, P.M - tile * T);
    if (wave == 0 && lane < rt) P.y[tile * T + lane] = v;
}

// (value, index) ordering for the argmax: larger value wins, equal values go to
// the lower index; NaN and missing rows carry -inf and INT_MAX.
QG_DEV bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

QG_DEV void argmax_xor(float& v, int& i, int off) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Stage 1: logits of one tile, reduced to one (max, index) partial per workgroup.
template <int W>
__global__ __launch_bounds__(64 * W) void lmhead_tile_kernel(Q8Prob P, float2* __restrict__ partials) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float v = tile_rows<W>(P, tile, lane, wave);
    if (wave != 0) return;
    const int rt = min(T, P.M - tile * T);
    int idx = tile * T + (lane & 15);
    if ((lane & 15) >= rt || v != v) {
        v = -__builtin_huge_valf();
        idx = INT_MAX;
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) argmax_xor(v, idx, off);
    if (lane == 0) partials[tile] = make_float2(v, __builtin_bit_cast(float, idx));
}

// Top-k stage 1: logits of one tile, written to the caller's logit vector, and
// the tile's (first maximum, row, sum of exp(z - max)) partial.
template <int W>
__global__ __launch_bounds__(64 * W) void lmhead_topk_tile_kernel(Q8Prob P, float* __restrict__ logits,
                                                                  float4* __restrict__ partials) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float v = tile_rows<W>(P, tile, lane, wave);
    if (wave != 0 || lane >= 16) return;
    const int rt = min(T, P.M - tile * T);
    if (lane < rt) logits[tile * T + lane] = v;
    const float4 st = qg_group16_stats(v, tile * T + lane, lane < rt);
    if (lane == 0) partials[tile] = st;
}

// Stage 2: one workgroup reduces the partials in a fixed order.
__global__ __launch_bounds__(1024) void lmhead_reduce_kernel(float2* __restrict__ partials, int n,
                                                              int32_t* out_index, float* out_value) {
    float bv = -__builtin_huge_valf();
    int bi = INT_MAX;
    // Pairs of partials per 16-byte load, eight loads in flight per thread before
    // any comparison (9504 partials: one round of loads for 1024 threads).
    float4* __restrict__ p4 = reinterpret_cast<float4*>(partials);
    const int n4 = n >> 1;
    for (int q0 = threadIdx.x; q0 < n4; q0 += 8 * blockDim.x) {
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = q0 + j * blockDim.x;
            v[j] = q < n4 ? p4[q] : make_float4(-__builtin_huge_valf(), __builtin_bit_cast(float, INT_MAX),
                                                -__builtin_huge_valf(), __builtin_bit_cast(float, INT_MAX));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = q0 + j * blockDim.x;
            if (q < n4) p4[q] = make_float4(0.f, 0.f, 0.f, 0.f);  // workspaces are left all-zero
            const int i0 = __builtin_bit_cast(int, v[j].y), i1 = __builtin_bit_cast(int, v[j].w);
            if (better(v[j].x, i0, bv, bi)) {
                bv = v[j].x;
                bi = i0;
            }
            if (better(v[j].z, i1, bv, bi)) {
                bv = v[j].z;
                bi = i1;
            }
        }
    }
    if ((n & 1) && threadIdx.x == 0) {  // odd count: the last partial
        const float2 pg = partials[n - 1];
        partials[n - 1] = make_float2(0.f, 0.f);
        const int gi = __builtin_bit_cast(int, pg.y);
        if (better(pg.x, gi, bv, bi)) {
            bv = pg.x;
            bi = gi;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) argmax_xor(bv, bi, off);
    __shared__ float sv[16];
    __shared__ int si[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nw = (blockDim.x + 63) / 64;
        for (int w = 1; w < nw; ++w)
            if (better(sv[w], si[w], bv, bi)) {
                bv = sv[w];
                bi = si[w];
            }
        out_index[0] = (bi == INT_MAX) ? -1 : bi;
        if (out_value) out_value[0] = bv;
    }
}

__global__ void q8_0_pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t M, int nbq) {
    const int nmb = nbq / 8, tb = nbq % 8;
    const int64_t rowbytes = (int64_t)nbq * 34;
    const int64_t tile_bytes = (int64_t)T * rowbytes;
    const int64_t total = M * rowbytes;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total; o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = o / tile_bytes;
        const int64_t in = o - t * tile_bytes;
        const int rt = (int)std::min<int64_t>(T, M - t * T);
        const int64_t macro = (int64_t)nmb * 17 * rt * 16;
        int64_t srcoff;
        if (in < macro) {
            const int64_t u = in / 16;
            const int e = (int)(in - u * 16);
            const int64_t ms = u / rt;  // mb * 17 + s
            const int i = (int)(u - ms * rt);
            const int64_t mb = ms / 17;
            const int s = (int)(ms - mb * 17);
            const int64_t r = t * T + i;
            if (s == 0) {
                srcoff = r * rowbytes + (8 * mb + e / 2) * 34 + (e & 1);
            } else {
                const int k = (s - 1) / 2, hh = (s - 1) % 2;
                srcoff = r * rowbytes + (8 * mb + k) * 34 + 2 + 16 * hh + e;
            }
        } else {
            const int64_t in2 = in - macro;
            const int i = (int)(in2 / ((int64_t)tb * 34));
            const int64_t rem = in2 - (int64_t)i * tb * 34;
            const int64_t r = t * T + i;
            srcoff = r * rowbytes + (int64_t)nmb * 8 * 34 + rem;
        }
        dst[o] = src[srcoff];
    }
}

qg_status validate(const void* w, const float* x, int64_t M, int64_t K) {
    if (!w || !x) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (K < 32 || K % 32 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 32 (<= 2^24)", (long long)K);
    if (!qg::aligned16(w) || !qg::aligned16(x)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    return QG_OK;
}

Q8Prob make_prob(const void* w, const float* x, float* y, int64_t M, int64_t K) {
    Q8Prob P{};
    P.w = (const uint8_t*)w;
    P.x = x;
    P.y = y;
    P.M = (int32_t)M;
    P.nbq = (int32_t)(K / 32);
    P.nmb = P.nbq / 8;
    P.tb = P.nbq % 8;
    P.tiles = (int32_t)qg::ceil_div(M, T);
    return P;
}

// Wavefronts per workgroup: more while the grid holds fewer than 640 wavefronts
// (measured, us per call: 11008 x 4096, 688 tiles: W = 1 9.43, 2 10.46, 8 9.71;
// 4096 x 11008, 256 tiles: W = 2 10.20, 4 10.04, 8 9.95) and each K-group keeps at
// least two half macro-blocks.
int choose_w(const Q8Prob& P) {
    int W = 1;
    while (W < 8 && (int64_t)P.tiles * W < 640 && 4 * (2 * W) <= 2 * P.nmb + 3) W *= 2;
    if (qg::launch_override().gemv_waves) W = qg::launch_override().gemv_waves;
    return W;
}

size_t lm_ws_bytes(const Q8Prob& P) { return qg::align_up((size_t)P.tiles * 8, 256); }

// Launches both stages of the LM-head argmax with its partials at `partials`.
qg_status lmhead_launch(const Q8Prob& P, float2* partials, int32_t* out_index, float* out_value, hipStream_t s) {
    const dim3 grid(P.tiles);
    switch (choose_w(P)) {
        case 1: hipLaunchKernelGGL(lmhead_tile_kernel<1>, grid, dim3(64), 0, s, P, partials); break;
        case 2: hipLaunchKernelGGL(lmhead_tile_kernel<2>, grid, dim3(128), 0, s, P, partials); break;
        case 4: hipLaunchKernelGGL(lmhead_tile_kernel<4>, grid, dim3(256), 0, s, P, partials); break;
        default: hipLaunchKernelGGL(lmhead_tile_kernel<8>, grid, dim3(512), 0, s, P, partials); break;
    }
    qg_status st = qg::launch_status("lmhead_argmax (tiles)");
    if (st) return st;
    const int threads = (int)std::min<int64_t>(1024, std::max<int64_t>(64, qg::ceil_div(P.tiles, 64) * 64));
    hipLaunchKernelGGL(lmhead_reduce_kernel, dim3(1), dim3(threads), 0, s, partials, P.tiles, out_index, out_value);
    return qg::launch_status("lmhead_argmax (reduce)");
}

}  // namespace

// Scratch of lmhead_argmax_noalloc: the per-tile (max, index) partials, 8 bytes
// per 16-row tile, in a device array of the library itself (one copy per GPU,
// held until the process ends). In host code `scratch` only names the symbol (a
// host-side stand-in, not a device address); its device address comes from
// hipGetSymbolAddress, once per device, and only that address reaches kernels.
constexpr size_t kLmScratchBytes = 256 * 1024;  // 32768 tiles: M <= 524288
static __device__ __align__(256) uint8_t scratch[kLmScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device: the device address of `scratch`

// Device address of the current device's scratch array, looked up on the first
// call on that device (with it current), or an error.
qg_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return qg::fail(QG_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return qg::fail(QG_ERR_DEVICE, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return qg::fail(QG_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QG_OK;
}

}  // namespace

extern "C" {

qg_status qgemv_q8_0(const void* w, const float* x, float* y, int64_t M, int64_t K, qg_stream_t stream) {
    qg::clear_error();
    qg_status st = validate(w, x, M, K);
    if (st) return st;
    if (!y) return qg::fail(QG_ERR_NULL, "y is NULL");
    if (!qg::aligned16(y)) return qg::fail(QG_ERR_ALIGN, "y not 16-byte aligned");
    Q8Prob P = make_prob(w, x, y, M, K);
    st = qg::check_device();
    if (st) return st;
    const dim3 grid(P.tiles);
    hipStream_t s = (hipStream_t)stream;
    switch (choose_w(P)) {
        case 1: hipLaunchKernelGGL(q8_0_gemv_kernel<1>, grid, dim3(64), 0, s, P); break;
        case 2: hipLaunchKernelGGL(q8_0_gemv_kernel<2>, grid, dim3(128), 0, s, P); break;
        case 4: hipLaunchKernelGGL(q8_0_gemv_kernel<4>, grid, dim3(256), 0, s, P); break;
        default: hipLaunchKernelGGL(q8_0_gemv_kernel<8>, grid, dim3(512), 0, s, P); break;
    }
    return qg::launch_status("qgemv_q8_0");
}

size_t lmhead_argmax_workspace_bytes(int64_t M, int64_t K) {
    if (M < 1 || M > INT32_MAX || K < 32 || K % 32 || K > (1 << 24)) return 0;
    return lm_ws_bytes(make_prob(nullptr, nullptr, nullptr, M, K));
}

qg_status lmhead_argmax(const void* w, const float* x, int64_t M, int64_t K, void* ws, size_t ws_bytes,
                  int32_t* out_index, float* out_value, qg_stream_t stream) {
    qg::clear_error();
    qg_status st = validate(w, x, M, K);
    if (st) return st;
    if (!out_index) return qg::fail(QG_ERR_NULL, "out_index is NULL");
    if ((reinterpret_cast<uintptr_t>(out_index) & 3) || (reinterpret_cast<uintptr_t>(out_value) & 3))
        return qg::fail(QG_ERR_ALIGN, "outputs must be 4-byte aligned");
    Q8Prob P = make_prob(w, x, nullptr, M, K);
    const size_t need = lm_ws_bytes(P);
    if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    st = qg::check_device();
    if (st) return st;
    return lmhead_launch(P, (float2*)ws, out_index, out_value, (hipStream_t)stream);
}

qg_status lmhead_argmax_noalloc(const void* w, const float* x, int64_t M, int64_t K, int32_t* out_index,
                                float* out_value, qg_stream_t stream) {
    qg::clear_error();
    qg_status st = validate(w, x, M, K);
    if (st) return st;
    if (!out_index) return qg::fail(QG_ERR_NULL, "out_index is NULL");
    if ((reinterpret_cast<uintptr_t>(out_index) & 3) || (reinterpret_cast<uintptr_t>(out_value) & 3))
        return qg::fail(QG_ERR_ALIGN, "outputs must be 4-byte aligned");
    Q8Prob P = make_prob(w, x, nullptr, M, K);
    if (lm_ws_bytes(P) > kLmScratchBytes)
        return qg::fail(QG_ERR_SHAPE, "M=%lld needs %zu bytes of partials; lmhead_argmax_noalloc holds %zu (M <= %zu)",
                        (long long)M, lm_ws_bytes(P), kLmScratchBytes, kLmScratchBytes / 8 * 16);
    st = qg::check_device();
    if (st) return st;
    void* ptr = nullptr;
    st = scratch_address(&ptr);
    if (st) return st;
    return lmhead_launch(P, (float2*)ptr, out_index, out_value, (hipStream_t)stream);
}

size_t lmhead_topk_workspace_bytes(int64_t M, int64_t K) {
    if (K < 32 || K % 32 || K > (1 << 24)) return 0;
    return qg::topk_ws_bytes(M);
}

qg_status lmhead_topk(const void* w, const float* x, int64_t M, int64_t K, int k, float* logits, const qg_sampler* sampler,
                void* ws, size_t ws_bytes, const qg_topk_out* out, qg_stream_t stream) {
    qg::clear_error();
    qg_status st = validate(w, x, M, K);
    if (st) return st;
    st = qg::validate_topk(M, k, sampler, out);
    if (st) return st;
    if (!logits) return qg::fail(QG_ERR_NULL, "logits is NULL");
    if (!qg::aligned16(logits)) return qg::fail(QG_ERR_ALIGN, "logits not 16-byte aligned");
    const size_t need = qg::topk_ws_bytes(M);
    if (!ws || ws_bytes < need)
        return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : 0);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    st = qg::check_device();
    if (st) return st;
    Q8Prob P = make_prob(w, x, nullptr, M, K);
    float4* partials = (float4*)ws;
    const dim3 grid(P.tiles);
    hipStream_t s = (hipStream_t)stream;
    switch (choose_w(P)) {
        case 1: hipLaunchKernelGGL(lmhead_topk_tile_kernel<1>, grid, dim3(64), 0, s, P, logits, partials); break;
        case 2: hipLaunchKernelGGL(lmhead_topk_tile_kernel<2>, grid, dim3(128), 0, s, P, logits, partials); break;
        case 4: hipLaunchKernelGGL(lmhead_topk_tile_kernel<4>, grid, dim3(256), 0, s, P, logits, partials); break;
        default: hipLaunchKernelGGL(lmhead_topk_tile_kernel<8>, grid, dim3(512), 0, s, P, logits, partials); break;
    }
    st = qg::launch_status("lmhead_topk (tiles)");
    if (st) return st;
    return qg::launch_topk_select(ws, P.tiles, logits, M, k, sampler, *out, s);
}

qg_status qg_pack_q8_0(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream) {
    qg::clear_error();
    if (!src || !dst) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX || K < 32 || K % 32 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "invalid Q8_0 shape M=%lld K=%lld", (long long)M, (long long)K);
    if (!qg::aligned16(src) || !qg::aligned16(dst)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t bytes = qg_q8_0_bytes(M, K);
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    if (s8 < d8 + bytes && d8 < s8 + bytes) return qg::fail(QG_ERR_SHAPE, "src and dst overlap");
    qg_status st = qg::check_device();
    if (st) return st;
    const int blocks = (int)std::min<int64_t>(qg::ceil_div((int64_t)bytes, 256), 65536);
    hipLaunchKernelGGL(q8_0_pack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)src,
                       (uint8_t*)dst, M, (int)(K / 32));
    return qg::launch_status("qg_pack_q8_0");
}

}  // extern "C"
