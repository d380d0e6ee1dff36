// Batched greedy verification on the LM head, for gfx950: N ≤ 32 activation
// columns (the drafted tokens plus one) against one pass over a Q8_0 vocabulary
// projection, each column reduced on the device to its first maximum.
//
// "Why Local LLMs Don't Need C++ or Python": section 2 (projection and argmax fused
// on the device, one int32 per decision crosses to the host) and section 4 (the K
// candidate tokens are verified in one batched pass, so the weights cross the bus
// once). For column n: out_index[n] = min{ i : logit_{i,n} = max_j logit_{j,n} },
// out_value[n] = that logit, logit = W x_n, W M x K in Q8_0 blocks (fp16 d and 32
// int8 q per block, weight = d q).
//
// Stage 1 (one workgroup per 16-row tile of the Q8_0 tile layout, q8_0_gemv.hip):
// for each 32-weight block, S'[n][r] = sum_k x[k][n] (q[r][k] + 128) is a
// 16 x 16 x 32 fp16 matrix-core product: the int8 quants are biased to bytes
// (q ^ 0x80 = q + 128) and enter the B operand in place as fp16 subnormals
// ((q + 128) * 2^-24, two per masked dword), the A operand carries 16 activation
// columns rounded to fp16; a product against an all-ones B gives the block's
// activation sums X[n], so logit += d (2^24 S' - 128 X) in fp32. The W wavefronts
// split K in units of two blocks and meet in LDS in a fixed order; the 16 rows of
// the tile then reduce per column to (max, lowest index) and one 8-byte partial
// per (column, tile) goes to the workspace. Stage 2 (one workgroup per column)
// reduces a column's partials in a fixed order, clears them and writes the id and
// its logit. K must be a multiple of 256 (whole macro-blocks of 8 blocks).
#include <algorithm>
#include <climits>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;

struct VaProb {
    const uint8_t* w;
    const float* X;
    int64_t ldx;
    float2* partials;  // [N][tiles]
    int32_t M, nmb, N, tiles;
};

// Inputs of one unit: blocks 2g and 2g + 1 of macro-block mb (u = 4 mb + g) of
// TW consecutive tiles, which share the unit's activations.
template <int C, int TW>
struct VaIn {
    uint4 sc[TW];        // the eight fp16 block scales of this lane's row
    uint2 q[TW][2];      // quants 8 (l / 16)..+7 of blocks 2g and 2g + 1
    float4 x[2][C][2];   // [block][column block][first / second 4 activations]
};

template <int C, int TW>
struct VaLane {
    __amdgpu_buffer_rsrc_t w[TW];  // one tile each
    int32_t rt[TW];                // rows of the tile
    uint32_t sc[TW], q[TW];        // byte offsets of this lane's scale segment / quant bytes
    uint32_t x[C];                 // per column block: byte offset of this lane's activations
};

template <int C, int TW>
QG_DEV void load_unit(VaIn<C, TW>& d, __amdgpu_buffer_rsrc_t xr, const VaLane<C, TW>& ln, int u) {
    const int mb = u >> 2, g = u & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int so = u * 256 + 128 * h;  // activations 64 u + 32 h + 8 (l / 16)
            d.x[h][c][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, ln.x[c], so, 0));
            d.x[h][c][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, ln.x[c], so + 16, 0));
        }
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int base = mb * 17 * 16 * ln.rt[t];
        // the scales serve the four units of the macro-block: a cached load
        const qg_u4v s = __builtin_amdgcn_raw_buffer_load_b128(ln.w[t], ln.sc[t], base, 0);
        d.sc[t] = make_uint4(s.x, s.y, s.z, s.w);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // block k = 2g + h: segment 1 + 2k + (l / 32)
            const qg_u2v q = __builtin_amdgcn_raw_buffer_load_b64(
                ln.w[t], ln.q[t], base + (1 + 2 * (2 * g + h)) * 16 * ln.rt[t], kQgNonTemporal);
            d.q[t][h] = make_uint2(q.x, q.y);
        }
    }
}

template <int C, int TW>
QG_DEV void unit_dot(qg_f4 (&acc)[TW][C], const VaIn<C, TW>& d, int u) {
    const int g = u & 3;
    const qg_h8 ones = qg_ones_h8();
    const qg_f4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        qg_h8 a[C];
        qg_f4 xs[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            a[c] = qg_a_operand(d.x[h][c][0], d.x[h][c][1]);
            xs[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[c], ones, zero, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            // scales of blocks 2g, 2g + 1
            const uint32_t dw = g == 0 ? d.sc[t].x : g == 1 ? d.sc[t].y : g == 2 ? d.sc[t].z : d.sc[t].w;
            const float dk = h ? qg_half_hi(dw) : qg_half_lo(dw);
            const float d24 = dk * 16777216.0f, dx = -128.0f * dk;
            const uint32_t w0 = d.q[t][h].x ^ 0x80808080u, w1 = d.q[t][h].y ^ 0x80808080u;
            const qg_h8 b = __builtin_bit_cast(qg_h8, make_uint4(w0 & 0x00ff00ffu, (w0 >> 8) & 0x00ff00ffu,
                                                                 w1 & 0x00ff00ffu, (w1 >> 8) & 0x00ff00ffu));
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const qg_f4 sp = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[c], b, zero, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[t][c][e] = fmaf(d24, sp[e], fmaf(dx, xs[c][e], acc[t][c][e]));
            }
        }
    }
}

// (value, index) order of the argmax: larger value wins, equal values go to the
// lower index; NaN and missing rows carry -inf and INT_MAX and never win.
QG_DEV bool va_better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

template <int C, int TW, int W>
__global__ __launch_bounds__(64 * W) void lmhead_verify_tile_kernel(VaProb P) {
    const int tile0 = blockIdx.x * TW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    const int K = P.nmb * 256;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + K) * 4), kQgRawBufferFlags);
    VaLane<C, TW> ln;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        // a tile past the matrix end re-reads the last tile, rows past a ragged
        // tile's end its last row; their results are dropped
        const int tc = min(tile0 + t, P.tiles - 1);
        ln.rt[t] = min(T, P.M - tc * T);
        ln.w[t] = __builtin_amdgcn_make_buffer_rsrc((void*)(P.w + (size_t)tc * T * P.nmb * 8 * 34), (short)0,
                                                    ln.rt[t] * P.nmb * 8 * 34, kQgRawBufferFlags);
        const uint32_t r = (uint32_t)min(i, ln.rt[t] - 1);
        ln.sc[t] = 16 * r;
        ln.q[t] = 16 * r + 8 * (s & 1) + (uint32_t)(s >> 1) * 16 * ln.rt[t];
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = 16 * c + i;
        ln.x[c] = n < P.N ? (uint32_t)(((int64_t)n * P.ldx + 8 * s) * 4) : kQgOutOfRange;
    }

    const int units = P.nmb * 4;
    const int niter = (units - wave + W - 1) / W;  // units wave, wave + W, ...
    qg_f4 acc[TW][C];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[t][c] = qg_f4{0.f, 0.f, 0.f, 0.f};
    // ping-pong over pairs of units with unconditional, clamped loads and a
    // single-exit loop, so every wait count is exact
    if (niter > 0) {
        const int ulast = wave + W * (niter - 1);
        VaIn<C, TW> b0, b1;
        load_unit<C, TW>(b0, xr, ln, wave);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            const int u0 = wave + W * it;
            load_unit<C, TW>(b1, xr, ln, u0 + W);
            __builtin_amdgcn_sched_barrier(0);
            unit_dot<C, TW>(acc, b0, u0);
            load_unit<C, TW>(b0, xr, ln, min(u0 + 2 * W, ulast));
            __builtin_amdgcn_sched_barrier(0);
            unit_dot<C, TW>(acc, b1, u0 + W);
        }
        if (it < niter) unit_dot<C, TW>(acc, b0, wave + W * it);
    }
    if constexpr (W > 1) {
        __shared__ float red[W][TW * C * 4][64];
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[wave][(t * C + c) * 4 + e][lane] = acc[t][c][e];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = red[0][(t * C + c) * 4 + e][lane];
#pragma unroll
                    for (int w = 1; w < W; ++w) v += red[w][(t * C + c) * 4 + e][lane];
                    acc[t][c][e] = v;
                }
    }
    // lane (i, s) holds row i of each tile, columns 16 c + 4 s + e: reduce over rows
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        if (tile0 + t >= P.tiles) break;  // wavefront-uniform
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = acc[t][c][e];
                int idx = (tile0 + t) * T + i;
                if (i >= ln.rt[t] || !(v == v)) {
                    v = -__builtin_huge_valf();
                    idx = INT_MAX;
                }
#pragma unroll
                for (int off = 8; off >= 1; off >>= 1) {
                    const float ov = __shfl_xor(v, off, 64);
                    const int oi = __shfl_xor(idx, off, 64);
                    if (va_better(ov, oi, v, idx)) {
                        v = ov;
                        idx = oi;
                    }
                }
                const int n = 16 * c + 4 * s + e;
                if (i == 0 && n < P.N)
                    P.partials[(int64_t)n * P.tiles + tile0 + t] = make_float2(v, __builtin_bit_cast(float, idx));
            }
    }
}

// Stage 2: workgroup n reduces column n's partials in a fixed order and clears them.
__global__ __launch_bounds__(1024) void lmhead_verify_reduce_kernel(float2* __restrict__ partials, int tiles,
                                                                    int32_t* out_index, float* out_value) {
    const int n = blockIdx.x;
    float2* col = partials + (int64_t)n * tiles;
    float bv = -__builtin_huge_valf();
    int bi = INT_MAX;
    for (int t0 = threadIdx.x; t0 < tiles; t0 += 8 * blockDim.x) {
        float2 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = t0 + j * blockDim.x;
            v[j] = t < tiles ? col[t] : make_float2(-__builtin_huge_valf(), __builtin_bit_cast(float, INT_MAX));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = t0 + j * blockDim.x;
            if (t < tiles) col[t] = make_float2(0.f, 0.f);  // workspaces are left all-zero
            const int vi = __builtin_bit_cast(int, v[j].y);
            if (va_better(v[j].x, vi, bv, bi)) {
                bv = v[j].x;
                bi = vi;
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (va_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
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
            if (va_better(sv[w], si[w], bv, bi)) {
                bv = sv[w];
                bi = si[w];
            }
        out_index[n] = (bi == INT_MAX) ? -1 : bi;
        if (out_value) out_value[n] = bv;
    }
}

int va_validate(const void* w, const float* X, int64_t ldx, int64_t M, int64_t K, int64_t N) {
    if (!w || !X) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (N < 1 || N > QG_SMALLN_MAX) return qg::fail(QG_ERR_SHAPE, "N=%lld not in [1, %d]", (long long)N, QG_SMALLN_MAX);
    if (ldx < K || ldx % 4) return qg::fail(QG_ERR_SHAPE, "ldx=%lld must be >= K and a multiple of 4", (long long)ldx);
    if ((N - 1) * ldx + K > INT32_MAX / 4) return qg::fail(QG_ERR_SHAPE, "X extent exceeds 2^31 bytes");
    if (!qg::aligned16(w) || !qg::aligned16(X)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    return QG_OK;
}

size_t va_ws_bytes(int64_t M, int64_t N) { return qg::align_up((size_t)qg::ceil_div(M, T) * N * 8, 256); }

template <int C, int TW>
void va_launch(const VaProb& P, int W, hipStream_t s) {
    const dim3 grid((unsigned)qg::ceil_div(P.tiles, TW));
    if (W == 8)
        hipLaunchKernelGGL((lmhead_verify_tile_kernel<C, TW, 8>), grid, dim3(512), 0, s, P);
    else
        hipLaunchKernelGGL((lmhead_verify_tile_kernel<C, TW, 4>), grid, dim3(256), 0, s, P);
}

}  // namespace

extern "C" {

size_t lmhead_argmax_verify_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || M > INT32_MAX || K < 256 || K % 256 || N < 1 || N > QG_SMALLN_MAX) return 0;
    return va_ws_bytes(M, N);
}

int lmhead_argmax_verify(const void* w, const float* X, int64_t ldx, int64_t M, int64_t K, int64_t N, void* ws,
                         size_t ws_bytes, int32_t* out_index, float* out_value, qg_stream_t stream) {
    qg::clear_error();
    int st = va_validate(w, X, ldx, M, K, N);
    if (st) return st;
    if (!out_index) return qg::fail(QG_ERR_NULL, "out_index is NULL");
    if ((reinterpret_cast<uintptr_t>(out_index) & 3) || (reinterpret_cast<uintptr_t>(out_value) & 3))
        return qg::fail(QG_ERR_ALIGN, "outputs must be 4-byte aligned");
    const size_t need = va_ws_bytes(M, N);
    if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    st = qg::check_device();
    if (st) return st;
    VaProb P{};
    P.w = (const uint8_t*)w;
    P.X = X;
    P.ldx = ldx;
    P.partials = (float2*)ws;
    P.M = (int32_t)M;
    P.nmb = (int32_t)(K / 256);
    P.N = (int32_t)N;
    P.tiles = (int32_t)qg::ceil_div(M, T);
    // W wavefronts split K (four for two column blocks, whose registers allow fewer
    // wavefronts per SIMD); TW tiles per workgroup share each unit's activations
    // (two while that leaves at least 1024 workgroups)
    int W = (P.nmb * 4 >= 16 && N <= 16) ? 8 : 4;
    int TW = P.tiles >= 2048 ? 2 : 1;
    // vocabulary-sized heads with one column block: four wavefronts over four tiles
    // (152064 x 3584, N = 5, interleaved A/B: 140.1 us against 143.0 for 8 x 2)
    if (N <= 16 && P.tiles >= 4096 && P.nmb * 4 >= 16) {
        W = 4;
        TW = 4;
    }
    int ew = 0, et = 0;
    if (qg::env_pair("QG_VA_CFG", &ew, &et)) {
        if (ew == 4 || ew == 8) W = ew;
        if (et == 1 || et == 2 || (et == 4 && N <= 16)) TW = et;  // four tiles of two column blocks spill
    }
    hipStream_t s = (hipStream_t)stream;
    const int key = 10 * (N > 16 ? 2 : 1) + TW;
    switch (key) {
        case 11: va_launch<1, 1>(P, W, s); break;
        case 12: va_launch<1, 2>(P, W, s); break;
        case 14: va_launch<1, 4>(P, W, s); break;
        case 21: va_launch<2, 1>(P, W, s); break;
        default: va_launch<2, 2>(P, W, s); break;
    }
    st = qg::launch_status("lmhead_argmax_verify (tiles)");
    if (st) return st;
    const int threads = (int)std::min<int64_t>(1024, std::max<int64_t>(64, qg::ceil_div(P.tiles, 8 * 64) * 64));
    hipLaunchKernelGGL(lmhead_verify_reduce_kernel, dim3((unsigned)N), dim3(threads), 0, s, P.partials, P.tiles,
                       out_index, out_value);
    return qg::launch_status("lmhead_argmax_verify (reduce)");
}

}  // extern "C"
