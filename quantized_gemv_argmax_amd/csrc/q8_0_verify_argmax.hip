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
// its logit. K must be a multiple of 256 (whole macro-blocks of 8 blocks). This
// matrix-core stage 1 serves N > 8 (and K > 4096 above 6 columns); the streamed
// form below takes N <= 8 with K <= 4096, the vector-ALU form the rest.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstring>

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

// Workgroup barrier: LDS operations complete first; pending global loads are not
// waited for.
QG_DEV void sw_vs_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

// Stage 2: workgroup n reduces column n's partials in a fixed order and clears them;
// the workgroups also clear `clr16` 16-byte words at `clr` (the vector-ALU form's
// activation pairs and sums, read by stage 1 only).
__global__ __launch_bounds__(1024) void lmhead_verify_reduce_kernel(float2* __restrict__ partials, int tiles,
                                                                    int32_t* out_index, float* out_value,
                                                                    uint4* __restrict__ clr, int clr16) {
    const int n = blockIdx.x;
    for (int w = n * blockDim.x + threadIdx.x; w < clr16; w += gridDim.x * blockDim.x) clr[w] = make_uint4(0, 0, 0, 0);
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

qg_status va_validate(const void* w, const float* X, int64_t ldx, int64_t M, int64_t K, int64_t N) {
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

// ---------------------------------------------------------------------------
// Vector-ALU form for N <= 6 fp32 columns (the default there): the work
// decomposition of the single-column LM head (lane = weight row, each DPP row a
// K-group over half macro-blocks of 128 weights), with the quants biased to bytes
// and read in place as fp16 subnormals as in q8_0_gemv.hip, and the masked words
// of a segment shared by all columns. A first launch rounds each column to fp16
// once, already in the pair order the masked words need ((x0, x2), (x1, x3),
// (x4, x6), (x5, x7) per 8 activations), and sums every 32-weight block's rounded
// activations in fp32 (X, which removes the bias exactly: logit += d (2^24 S' -
// 128 X)), stored as -128 * 2^-24 * X so that it can seed a product accumulator;
// both go to the workspace after the partials. Per column and block: 16
// v_dot2c_f32_f16 with DPP row broadcasts, 3 additions and 1 fma.

__global__ __launch_bounds__(256) void lmhead_verify_prep_kernel(const float* __restrict__ X, int64_t ldx, int K,
                                                                 int N, uint4* __restrict__ pairs,
                                                                 float* __restrict__ xsum) {
    const int g8 = K / 8;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= N * g8) return;  // whole quads only: N * g8 is a multiple of 32
    const int n = t / g8, g = t - n * g8;
    const float4* src = reinterpret_cast<const float4*>(X + (int64_t)n * ldx + 8 * g);
    const QgPairs4 p = qg_cvt_pairs4(src[0], src[1]);
    pairs[t] = make_uint4(p.p[0], p.p[1], p.p[2], p.p[3]);
    // the eight rounded values, in a fixed order: (x0 + x2) + (x1 + x3) + ...
    float v = ((qg_half_lo(p.p[0]) + qg_half_hi(p.p[0])) + (qg_half_lo(p.p[1]) + qg_half_hi(p.p[1]))) +
              ((qg_half_lo(p.p[2]) + qg_half_hi(p.p[2])) + (qg_half_lo(p.p[3]) + qg_half_hi(p.p[3])));
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    // stored as the bias term in the products' scale: -128 * 2^-24 * X
    if ((g & 3) == 0) xsum[(int64_t)n * (K / 32) + g / 4] = v * -7.62939453125e-06f;
}

struct VdProb {
    const uint8_t* w;
    const uint8_t* xp;  // N pair arrays of 2K bytes, then N block-sum arrays of K/8 bytes
    float2* partials;   // [N][tiles]
    int32_t xpb, xs_off, xsb, M, nmb, N, tiles;  // pair bytes per column, offset of the sums, sum bytes per column
};

template <int NC>
struct VdIn {
    uint4 s[9];    // scale segment, then the 8 quant segments of the half macro-block
    uint4 xp[NC];  // activations 8i .. 8i + 7 of the half as fp16 pairs (i = lane % 16), per column
    float xs[NC];  // bias term -128 * 2^-24 * X of block i % 4 of the half, per column
};

// The biased bytes of a quant segment, masked in place: per dword, bytes 0, 2
// then bytes 1, 3, each as two fp16 subnormals. One byte permutation each
// (selector byte 0x0c gives a zero byte): 3 operations per dword.
QG_DEV void seg8h_masks(uint32_t (&m)[8], const uint4 q) {
    const uint32_t w[4] = {q.x ^ 0x80808080u, q.y ^ 0x80808080u, q.z ^ 0x80808080u, q.w ^ 0x80808080u};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        m[2 * d] = __builtin_amdgcn_perm(w[d], w[d], 0x0c020c00u);
        m[2 * d + 1] = __builtin_amdgcn_perm(w[d], w[d], 0x0c030c01u);
    }
}

template <int NC>
QG_DEV void load_half_d(VdIn<NC>& d, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t xr, uint32_t vrow, int rt,
                        uint32_t vx, uint32_t vd, const VdProb& P, int u) {
    const int mb = u >> 1, h = u & 1;
    const uint32_t ox = vx + 256u * (uint32_t)u, od = vd + 16u * (uint32_t)u;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const qg_u4v a = __builtin_amdgcn_raw_buffer_load_b128(xr, ox, n * P.xpb, 0);
        d.xp[n] = make_uint4(a.x, a.y, a.z, a.w);
        d.xs[n] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, od, P.xs_off + n * P.xsb, 0));
    }
    const uint32_t vs = vrow + (uint32_t)mb * 17u * 16u * (uint32_t)rt;
    const qg_u4v sv = __builtin_amdgcn_raw_buffer_load_b128(wr, vs, 0, 0);  // scales: a cached load
    d.s[0] = make_uint4(sv.x, sv.y, sv.z, sv.w);
    const uint32_t vq = vs + (uint32_t)(8 * h) * 16u * (uint32_t)rt;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const qg_u4v v = __builtin_amdgcn_raw_buffer_load_b128(wr, vq, (1 + j) * 16 * rt, kQgNonTemporal);
        d.s[1 + j] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

template <int NC>
QG_DEV void half_dot_d(float (&acc)[NC], const VdIn<NC>& d, int h, bool live) {
    const uint32_t dw0 = h ? d.s[0].z : d.s[0].x;
    const uint32_t dw1 = h ? d.s[0].w : d.s[0].y;
    // a clamped re-read (live false) is scaled by zero; 2^24 undoes the subnormal scale
    constexpr float two24 = 16777216.0f;
    const float dk[4] = {live ? two24 * qg_half_lo(dw0) : 0.f, live ? two24 * qg_half_hi(dw0) : 0.f,
                         live ? two24 * qg_half_lo(dw1) : 0.f, live ? two24 * qg_half_hi(dw1) : 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t m0[8], m1[8];
        seg8h_masks(m0, d.s[1 + 2 * k]);
        seg8h_masks(m1, d.s[2 + 2 * k]);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            // the first accumulator starts at the block's bias term, so the sum is
            // 2^-24 (S' - 128 * 2^24 X)
            float a[4];
            switch (k) {
                case 0: a[0] = qg_bcast<0>(d.xs[n]); break;
                case 1: a[0] = qg_bcast<1>(d.xs[n]); break;
                case 2: a[0] = qg_bcast<2>(d.xs[n]); break;
                default: a[0] = qg_bcast<3>(d.xs[n]); break;
            }
            a[1] = a[2] = a[3] = 0.f;
            switch (k) {
                case 0: qg_q8_seg8h_dot<0, false>(a, m0, d.xp[n]); qg_q8_seg8h_dot<2, true>(a, m1, d.xp[n]); break;
                case 1: qg_q8_seg8h_dot<4, false>(a, m0, d.xp[n]); qg_q8_seg8h_dot<6, true>(a, m1, d.xp[n]); break;
                case 2: qg_q8_seg8h_dot<8, false>(a, m0, d.xp[n]); qg_q8_seg8h_dot<10, true>(a, m1, d.xp[n]); break;
                default: qg_q8_seg8h_dot<12, false>(a, m0, d.xp[n]); qg_q8_seg8h_dot<14, true>(a, m1, d.xp[n]); break;
            }
            acc[n] = fmaf(dk[k], (a[0] + a[1]) + (a[2] + a[3]), acc[n]);
        }
    }
}

template <int NC, int W>
__global__ __launch_bounds__(64 * W) void lmhead_verify_dot_kernel(VdProb P) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int kg = 4 * wave + (lane >> 4);
    constexpr int G = 4 * W;
    const int rt = min(T, P.M - tile * T);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(P.w + (size_t)tile * T * P.nmb * 272), (short)0, rt * P.nmb * 272, kQgRawBufferFlags);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.xp, (short)0, P.xs_off + P.N * P.xsb, kQgRawBufferFlags);
    const uint32_t vrow = 16u * (uint32_t)min(i, rt - 1);
    // the launch instantiates NC = N: every column is in range
    const uint32_t vx = (uint32_t)(16 * i), vd = (uint32_t)(4 * (i & 3));
    const int nu = 2 * P.nmb;
    float acc[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = 0.f;
    const int niter = (nu + G - 1) / G;
    VdIn<NC> b0, b1;
    load_half_d<NC>(b0, wr, xr, vrow, rt, vx, vd, P, min(kg, nu - 1));
    int it = 0;
    for (; it + 2 <= niter; it += 2) {
        const int u = kg + G * it;
        load_half_d<NC>(b1, wr, xr, vrow, rt, vx, vd, P, min(u + G, nu - 1));
        __builtin_amdgcn_sched_barrier(0);
        half_dot_d<NC>(acc, b0, u & 1, u < nu);
        load_half_d<NC>(b0, wr, xr, vrow, rt, vx, vd, P, min(u + 2 * G, nu - 1));
        __builtin_amdgcn_sched_barrier(0);
        half_dot_d<NC>(acc, b1, (u + G) & 1, u + G < nu);
    }
    if (it < niter) {
        const int u = kg + G * it;
        half_dot_d<NC>(acc, b0, u & 1, u < nu);
    }
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = qg_sum_rows4(acc[n]);
    if constexpr (W > 1) {
        __shared__ float red[W][NC][T];
#pragma unroll
        for (int n = 0; n < NC; ++n)
            if (lane < T) red[wave][n][lane] = acc[n];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            float v = red[0][n][i];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w][n][i];
            acc[n] = v;
        }
    }
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        float v = acc[n];
        int idx = tile * T + i;
        if (i >= rt || !(v == v)) {
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
        if (lane == 0) P.partials[(int64_t)n * P.tiles + tile] = make_float2(v, __builtin_bit_cast(float, idx));
    }
}

constexpr int kVdMaxCols = 6;  // above six columns the matrix-core form is faster

// Workspace of the vector-ALU form past the partials: 2K bytes of pairs and K/8
// bytes of block sums per column.
size_t vd_extra_bytes(int64_t K, int64_t N) { return qg::align_up((size_t)N * (size_t)(2 * K + K / 8), 256); }

template <int NC>
void vd_launch(const VdProb& P, int W, hipStream_t s) {
    const dim3 grid((unsigned)P.tiles);
    if (W == 4)
        hipLaunchKernelGGL((lmhead_verify_dot_kernel<NC, 4>), grid, dim3(256), 0, s, P);
    else
        hipLaunchKernelGGL((lmhead_verify_dot_kernel<NC, 1>), grid, dim3(64), 0, s, P);
}

// ---------------------------------------------------------------------------
// Streamed form (N <= 8, 2048 <= K <= 4096): the grid is sized to the resident
// workgroup slots, and workgroup j walks tiles j, j + G, j + 2G, ... The columns
// are staged into LDS once per workgroup (fp16, and the negated sums of every
// 32-weight block over the same fp16 values); the eight wavefronts take the (tile,
// macro-block) units of the walk in turn, with the next unit's loads in flight
// while one is computed, so the weight stream does not stop between tiles. The
// walk runs in rounds of two tiles: a wavefront keeps one accumulator per tile of
// the round, parks both at the round's end, and after the round's barrier two
// wavefronts (rotating with the round) add a tile's parked sums in a fixed order
// and fold the tile's rows into their running (max, lowest index) per column.
// At the end the running results meet in LDS and one 8-byte partial per (column,
// workgroup) goes to the workspace; stage 2 is lmhead_verify_reduce_kernel.
// Per block: S' = sum_k x[k][n] (q[r][k] + 128) as one 16 x 16 x 32 fp16
// matrix-core product (the biased quants as fp16 subnormals, one byte permutation
// per dword), logit += d 2^24 S' in fp32; the bias -128 d X[n] of four blocks is
// one v_mfma_f32_16x16x4_f32 (A the table entries -X, B 128 d of the lane's row),
// accumulated across the tile's units.
constexpr int kVsWaves = 8, kVsCols = 16;  // columns staged: 8 in one instance, 16 in the other
// The automatic choice for every N it takes (152064 x 3584, us, streamed / vector-ALU
// dot / matrix-core forms: N = 1 93.3 / 95.0 / 134.5, 2 92.2 / 96.4 / 135.7,
// 4 92.6 / 105.2 / 138.5, 5 93.2 / 115.8 / 139.2, 6 93.1 / 125.9 / 141.3,
// 8 94.4 / - / 142.9; the single-column argmax 94.7).
constexpr int kVsMinCols = 1;

struct VsProb {
    const uint8_t* w;
    const float* X;
    int64_t ldx;
    float2* partials;  // [N][G]
    int32_t M, nmb, N, tiles, G;
};

struct VsItem {
    uint4 sc;     // the eight fp16 block scales of this lane's row
    uint2 q[8];   // quant bytes 8 (l / 16)..+7 of blocks 0..7
};

// Loads of unit (tile t, macro-block mb); valid false: offsets past the resource,
// zeros without a memory access (every load is still issued: exact wait counts).
QG_DEV void vs_load(VsItem& it, __amdgpu_buffer_rsrc_t wr, const VsProb& P, int t, int mb, int i, int s,
                    bool valid) {
    const int rt = min(T, P.M - t * T);
    const uint32_t r = (uint32_t)min(i, rt - 1);
    const uint32_t vh = valid ? 16u * r : kQgOutOfRange;
    const uint32_t vq =
        valid ? 16u * r + 8u * (uint32_t)(s & 1) + (uint32_t)(s >> 1) * 16u * (uint32_t)rt : kQgOutOfRange;
    const int so = valid ? t * T * P.nmb * 272 + mb * 17 * 16 * rt : 0;
    const qg_u4v h = __builtin_amdgcn_raw_buffer_load_b128(wr, vh, so, 0);  // scales: a cached load
    it.sc = make_uint4(h.x, h.y, h.z, h.w);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const qg_u2v q = __builtin_amdgcn_raw_buffer_load_b64(wr, vq, so + (1 + 2 * k) * 16 * rt, kQgNonTemporal);
        it.q[k] = make_uint2(q.x, q.y);
    }
}

// One unit: a = LDS byte address of this lane's A operand for block 0 of the
// macro-block, xt = its table entry (block l / 16, column l % 16).
QG_DEV void vs_dot(qg_f4& acc, qg_f4& accm, const VsItem& it, const unsigned char* lds, uint32_t a, uint32_t xt,
                   int s) {
    const qg_f4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t dws[4] = {it.sc.x, it.sc.y, it.sc.z, it.sc.w};
    // bias: blocks s and 4 + s of the lane's row, 128 d each
    const uint32_t b0 = (s >> 1) ? it.sc.y : it.sc.x, b1 = (s >> 1) ? it.sc.w : it.sc.z;
    const float bm0 = 128.0f * ((s & 1) ? qg_half_hi(b0) : qg_half_lo(b0));
    const float bm1 = 128.0f * ((s & 1) ? qg_half_hi(b1) : qg_half_lo(b1));
    const float xa0 = *reinterpret_cast<const float*>(lds + xt);
    const float xa1 = *reinterpret_cast<const float*>(lds + xt + 256);
    accm = __builtin_amdgcn_mfma_f32_16x16x4f32(xa0, bm0, accm, 0, 0, 0);
    accm = __builtin_amdgcn_mfma_f32_16x16x4f32(xa1, bm1, accm, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t dw = dws[k >> 1];
        const float d24 = ((k & 1) ? qg_half_hi(dw) : qg_half_lo(dw)) * 16777216.0f;
        const qg_h8 av = *reinterpret_cast<const qg_h8*>(lds + a + 64 * k);
        const uint32_t w0 = it.q[k].x ^ 0x80808080u, w1 = it.q[k].y ^ 0x80808080u;
        const qg_h8 b = __builtin_bit_cast(
            qg_h8, make_uint4(__builtin_amdgcn_perm(w0, w0, 0x0c020c00u), __builtin_amdgcn_perm(w0, w0, 0x0c030c01u),
                              __builtin_amdgcn_perm(w1, w1, 0x0c020c00u), __builtin_amdgcn_perm(w1, w1, 0x0c030c01u)));
        const qg_f4 sp = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b, zero, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(d24, sp[e], acc[e]);
    }
}

template <int W, int NC>
__global__ __launch_bounds__(64 * W, NC == 8 ? 4 : 2) void lmhead_verify_stream_kernel(VsProb P) {
    // lanes holding real columns (column 4 (l / 16) + e of lane l): 32 for 8 columns,
    // all 64 for 16
    constexpr int LN = 4 * NC;
    extern __shared__ __align__(16) unsigned char lds[];
    const int j = blockIdx.x;
    const int G = P.G;
    const int nt = (P.tiles - j + G - 1) / G;  // tiles of this walk
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    const int nmb = P.nmb;
    const int K = nmb * 256;
    const int RB = (K + 8) * 2;
    const uint32_t xsb = (uint32_t)(P.N * RB);          // table of -X per block, 16 columns
    qg_f4* park = reinterpret_cast<qg_f4*>(lds + xsb + 2 * K);  // [2 buffers][2 slots][W][LN lanes]
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.w, (short)0, P.M * nmb * 272, kQgRawBufferFlags);

    // columns: thread tid takes 8-element group tid of every column (K <= 512 W)
    const int tid = threadIdx.x;
    const int gpr = K / 8;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + K) * 4), kQgRawBufferFlags);
    float4 v[NC][2];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const uint32_t off = (n < P.N && tid < gpr) ? (uint32_t)(((int64_t)n * P.ldx + 8 * tid) * 4) : kQgOutOfRange;
        v[n][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        v[n][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 16, 0));
    }

    // this wavefront's units: wave, wave + W, ... of the nt * nmb units of the walk;
    // (lt, lb) is the tile slot and macro-block of the unit being loaded
    const int U = nt * nmb;
    const int niter = (U - wave + W - 1) / W;
    int lt = wave / nmb, lb = wave - (wave / nmb) * nmb;
    auto advance = [&](int& t_, int& b_) {
        b_ += W;
        while (b_ >= nmb) {
            b_ -= nmb;
            ++t_;
        }
    };
    const int t_first = lt, b_first = lb;
    VsItem b0, b1;
    vs_load(b0, wr, P, j + min(lt, nt - 1) * G, lb, i, s, niter > 0);
    advance(lt, lb);

#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const qg_h8 h = qg_a_operand(v[n][0], v[n][1]);
        if (n < P.N && tid < gpr) *reinterpret_cast<qg_h8*>(lds + n * RB + 16 * tid) = h;
        const uint4 hw = __builtin_bit_cast(uint4, h);
        const float xsum = qg_quad_sum(qg_sum_pairs4(hw.x, hw.y, hw.z, hw.w));
        if ((tid & 3) == 0 && tid < gpr) *reinterpret_cast<float*>(lds + xsb + ((tid >> 2) * 16 + n) * 4) = -xsum;
    }
    if (NC == 8 && (tid & 3) == 0 && tid < gpr) {  // columns 8..15 of the table: zeros
        *reinterpret_cast<uint4*>(lds + xsb + ((tid >> 2) * 16 + 8) * 4) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(lds + xsb + ((tid >> 2) * 16 + 12) * 4) = make_uint4(0u, 0u, 0u, 0u);
    }
    sw_vs_barrier();

    const uint32_t an = (uint32_t)((i < P.N ? i : 0) * RB + 16 * s);
    const uint32_t xtl = xsb + (uint32_t)(s * 16 + i) * 4;
    // round accumulators (tile slots 2r and 2r + 1), running best per column of the
    // tiles this wavefront reduces
    qg_f4 acc[2] = {qg_f4{0.f, 0.f, 0.f, 0.f}, qg_f4{0.f, 0.f, 0.f, 0.f}};
    qg_f4 accm[2] = {qg_f4{0.f, 0.f, 0.f, 0.f}, qg_f4{0.f, 0.f, 0.f, 0.f}};
    float bv[4];
    int bi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bv[e] = -__builtin_huge_valf();
        bi[e] = INT_MAX;
    }
    int round = 0;
    // end of round `round`: park, barrier, reduce its tiles (wavefronts 2 round % W
    // and 2 round % W + 1), start the next
    auto end_round = [&]() {
        qg_f4* pb = park + (size_t)(round & 1) * 2 * W * LN;
        if (lane < LN) {
            pb[(0 * W + wave) * LN + lane] = acc[0] + accm[0];
            pb[(1 * W + wave) * LN + lane] = acc[1] + accm[1];
        }
        acc[0] = acc[1] = accm[0] = accm[1] = qg_f4{0.f, 0.f, 0.f, 0.f};
        sw_vs_barrier();
        const int q = wave - (2 * round) % W;  // this wavefront's slot in the round, if 0 or 1
        const int ts = 2 * round + q;
        if ((q == 0 || q == 1) && ts < nt && lane < LN) {
            qg_f4 sum = pb[(q * W) * LN + lane];
#pragma unroll
            for (int w = 1; w < W; ++w) sum += pb[(q * W + w) * LN + lane];
            const int t = j + ts * G;
            const int rt = min(T, P.M - t * T);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float vv = sum[e];
                int idx = t * T + i;
                if (i >= rt || !(vv == vv)) {
                    vv = -__builtin_huge_valf();
                    idx = INT_MAX;
                }
                if (va_better(vv, idx, bv[e], bi[e])) {
                    bv[e] = vv;
                    bi[e] = idx;
                }
            }
        }
        ++round;
    };

    int ct = t_first, cb = b_first;  // unit being computed
    auto unit = [&](const VsItem& it) {
        while (ct >= 2 * (round + 1)) end_round();  // the walk enters a later round
        if (ct & 1)
            vs_dot(acc[1], accm[1], it, lds, an + (uint32_t)(512 * cb), xtl + (uint32_t)(512 * cb), s);
        else
            vs_dot(acc[0], accm[0], it, lds, an + (uint32_t)(512 * cb), xtl + (uint32_t)(512 * cb), s);
        advance(ct, cb);
    };

    // ping-pong: unconditional loads, single-exit loop, exact wait counts
    int it = 0;
    for (; it + 2 <= niter; it += 2) {
        vs_load(b1, wr, P, j + min(lt, nt - 1) * G, lb, i, s, true);
        advance(lt, lb);
        __builtin_amdgcn_sched_barrier(0);
        unit(b0);
        vs_load(b0, wr, P, j + min(lt, nt - 1) * G, lb, i, s, it + 2 < niter);
        advance(lt, lb);
        __builtin_amdgcn_sched_barrier(0);
        unit(b1);
    }
    if (it < niter) unit(b0);
    // every wavefront ends every round, with or without units in it, so all meet
    // the same barriers
    const int nrounds = (nt + 1) / 2;
    while (round < nrounds) end_round();

    // the wavefronts' running results meet in LDS, over the columns and, for short
    // K, the parked sums, which the last round's reducing wavefronts may still be
    // reading: everyone waits for them first
    sw_vs_barrier();
    float* bvs = reinterpret_cast<float*>(lds);
    int* bis = reinterpret_cast<int*>(lds + W * LN * 4 * 4);
    if (lane < LN)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // rows first: the lanes i = 0..15 of column 4 s + e
            float vv = bv[e];
            int idx = bi[e];
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(vv, off, 64);
                const int oi = __shfl_xor(idx, off, 64);
                if (va_better(ov, oi, vv, idx)) {
                    vv = ov;
                    idx = oi;
                }
            }
            bvs[(wave * LN + lane) * 4 + e] = vv;
            bis[(wave * LN + lane) * 4 + e] = idx;
        }
    sw_vs_barrier();
    if (wave != 0 || i != 0 || lane >= LN) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float vv = bvs[lane * 4 + e];
        int idx = bis[lane * 4 + e];
#pragma unroll
        for (int w = 1; w < W; ++w) {
            const float ov = bvs[(w * LN + lane) * 4 + e];
            const int oi = bis[(w * LN + lane) * 4 + e];
            if (va_better(ov, oi, vv, idx)) {
                vv = ov;
                idx = oi;
            }
        }
        const int n = 4 * s + e;
        if (n < P.N) P.partials[(int64_t)n * G + j] = make_float2(vv, __builtin_bit_cast(float, idx));
    }
}

// Dynamic LDS of the streamed form: the columns, their block sums, the parked sums.
size_t vs_lds_bytes(int64_t K, int64_t N) {
    return (size_t)N * (K + 8) * 2 + 2 * (size_t)K + 2 * 2 * kVsWaves * (N <= 8 ? 32 : 64) * 16;
}

// ---------------------------------------------------------------------------
// Int8 activations: each column quantized Q8_1-style (qg_quantize_q8_1: a float32
// scale d_x and 32 int8 quants per block). Both operands are then signed int8, so
// a block's integer product S = sum_l q_w,l q_x,l comes straight from
// v_dot4c_i32_i8 with no bias term, and logit += d_w (d_x S). Work decomposition
// of the single-column LM head (q8_0_gemv.hip): lane = weight row, each DPP row a
// K-group walking half macro-blocks (4 blocks, 128 weights); the lane of slot i
// holds activation dwords 2i, 2i + 1 of the half for every column, and DPP row
// broadcasts feed them to the 16 rows. Per column and block: 8 v_dot4c_i32_i8,
// 7 integer and 4 float operations; the quant segments are used as loaded. Stage 2 is lmhead_verify_reduce_kernel, on the same partials layout.

struct VqProb {
    const uint8_t* w;
    const uint8_t* xq;  // N buffers of xb bytes
    float2* partials;   // [N][tiles]
    int32_t xb, q_off, M, nmb, N, tiles;
};

template <int NC>
struct VqIn {
    uint4 s[9];   // scale segment, then the 8 quant segments of the half macro-block
    uint2 x[NC];  // activation dwords 2i, 2i + 1 of the half (i = lane % 16), per column
    float dx[NC]; // scale of block i % 4 of the half, per column
};

// One block of one column: quant segments q0, q1 (weights 0..15, 16..31) against
// the activation dwords of lanes L, L + 1, L + 2, L + 3 (L = 4k). Four accumulators
// rotate, so none is re-read within two instructions of its last write; the block
// opens with two wait states (the accumulators may come from ordinary VALU code)
// and ends with s_nop 4 before ordinary VALU code reads them.
template <int L>
QG_DEV void blk_dot4(int (&a)[4], const uint4 q0, const uint4 q1, const uint2 x) {
    asm("s_nop 1\n\t"
        "v_dot4c_i32_i8_dpp %0, %12, %4 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %13, %5 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %12, %6 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %13, %7 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %12, %8 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %13, %9 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %12, %10 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %13, %11 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 4"
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
        : "v"(q0.x), "v"(q0.y), "v"(q0.z), "v"(q0.w), "v"(q1.x), "v"(q1.y), "v"(q1.z), "v"(q1.w), "v"(x.x),
          "v"(x.y), "n"(L), "n"(L + 1), "n"(L + 2), "n"(L + 3));
}

// Half macro-block u (macro-block u / 2, blocks 4 (u % 2) .. + 3) of this lane's
// row: `vrow` = 16 * row, `vx` / `vd` this lane's quant / scale offset within a
// column's buffer, `xb` the (uniform) distance between column buffers.
template <int NC>
QG_DEV void load_half_q(VqIn<NC>& d, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t xr, uint32_t vrow, int rt,
                        uint32_t vx, uint32_t vd, int xb, int u) {
    const int mb = u >> 1, h = u & 1;
    const uint32_t ox = vx + 128u * (uint32_t)u, od = vd + 16u * (uint32_t)u;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const qg_u2v a = __builtin_amdgcn_raw_buffer_load_b64(xr, ox, n * xb, 0);
        d.x[n] = make_uint2(a.x, a.y);
        d.dx[n] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, od, n * xb, 0));
    }
    const uint32_t vs = vrow + (uint32_t)mb * 17u * 16u * (uint32_t)rt;
    // the scales serve both halves: a cached load
    const qg_u4v sv = __builtin_amdgcn_raw_buffer_load_b128(wr, vs, 0, 0);
    d.s[0] = make_uint4(sv.x, sv.y, sv.z, sv.w);
    const uint32_t vq = vs + (uint32_t)(8 * h) * 16u * (uint32_t)rt;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const qg_u4v v = __builtin_amdgcn_raw_buffer_load_b128(wr, vq, (1 + j) * 16 * rt, kQgNonTemporal);
        d.s[1 + j] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// Column by column within each block (four integer accumulators live at a time).
// A half that is only a clamped re-read (live false) is scaled by zero: it adds
// nothing unless its activation scales are not finite, and then the same half's
// live pass has made the row's logit NaN already.
template <int NC>
QG_DEV void half_dot_q(float (&acc)[NC], const VqIn<NC>& d, int h, bool live) {
    const uint32_t dw0 = h ? d.s[0].z : d.s[0].x;
    const uint32_t dw1 = h ? d.s[0].w : d.s[0].y;
    const float dk[4] = {live ? qg_half_lo(dw0) : 0.f, live ? qg_half_hi(dw0) : 0.f, live ? qg_half_lo(dw1) : 0.f,
                         live ? qg_half_hi(dw1) : 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            int a[4] = {0, 0, 0, 0};
            switch (k) {
                case 0: blk_dot4<0>(a, d.s[1], d.s[2], d.x[n]); break;
                case 1: blk_dot4<4>(a, d.s[3], d.s[4], d.x[n]); break;
                case 2: blk_dot4<8>(a, d.s[5], d.s[6], d.x[n]); break;
                default: blk_dot4<12>(a, d.s[7], d.s[8], d.x[n]); break;
            }
            const int S = (a[0] + a[1]) + (a[2] + a[3]);  // |S| <= 32 * 128 * 127
            float dxk;
            switch (k) {
                case 0: dxk = qg_bcast<0>(d.dx[n]); break;
                case 1: dxk = qg_bcast<1>(d.dx[n]); break;
                case 2: dxk = qg_bcast<2>(d.dx[n]); break;
                default: dxk = qg_bcast<3>(d.dx[n]); break;
            }
            acc[n] = fmaf(dk[k], dxk * (float)S, acc[n]);
        }
    }
}

template <int NC, int W>
__global__ __launch_bounds__(64 * W) void lmhead_verify_q8_1_tile_kernel(VqProb P) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int kg = 4 * wave + (lane >> 4);
    constexpr int G = 4 * W;
    const int rt = min(T, P.M - tile * T);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(P.w + (size_t)tile * T * P.nmb * 272), (short)0, rt * P.nmb * 272, kQgRawBufferFlags);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.xq, (short)0, P.N * P.xb, kQgRawBufferFlags);
    const uint32_t vrow = 16u * (uint32_t)min(i, rt - 1);
    // the launch instantiates NC = N: every column is in range
    const uint32_t vx = (uint32_t)(P.q_off + 8 * i), vd = (uint32_t)(4 * (i & 3));
    const int nu = 2 * P.nmb;
    float acc[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = 0.f;
    // ping-pong over pairs of half macro-blocks with unconditional, clamped loads
    // and a single-exit loop, so every wait count is exact
    const int niter = (nu + G - 1) / G;
    VqIn<NC> b0, b1;
    load_half_q<NC>(b0, wr, xr, vrow, rt, vx, vd, P.xb, min(kg, nu - 1));
    int it = 0;
    for (; it + 2 <= niter; it += 2) {
        const int u = kg + G * it;
        load_half_q<NC>(b1, wr, xr, vrow, rt, vx, vd, P.xb, min(u + G, nu - 1));
        __builtin_amdgcn_sched_barrier(0);
        half_dot_q<NC>(acc, b0, u & 1, u < nu);
        load_half_q<NC>(b0, wr, xr, vrow, rt, vx, vd, P.xb, min(u + 2 * G, nu - 1));
        __builtin_amdgcn_sched_barrier(0);
        half_dot_q<NC>(acc, b1, (u + G) & 1, u + G < nu);
    }
    if (it < niter) {
        const int u = kg + G * it;
        half_dot_q<NC>(acc, b0, u & 1, u < nu);
    }
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = qg_sum_rows4(acc[n]);
    if constexpr (W > 1) {
        __shared__ float red[W][NC][T];
#pragma unroll
        for (int n = 0; n < NC; ++n)
            if (lane < T) red[wave][n][lane] = acc[n];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            float v = red[0][n][i];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w][n][i];
            acc[n] = v;
        }
    }
    // lanes i of each DPP row hold row i's logits: reduce over the 16 rows
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        float v = acc[n];
        int idx = tile * T + i;
        if (i >= rt || !(v == v)) {
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
        if (lane == 0 && n < P.N) P.partials[(int64_t)n * P.tiles + tile] = make_float2(v, __builtin_bit_cast(float, idx));
    }
}

constexpr int kVqMaxCols = 8;

template <int NC>
void vq_launch(const VqProb& P, int W, hipStream_t s) {
    const dim3 grid((unsigned)P.tiles);
    if (W == 4)
        hipLaunchKernelGGL((lmhead_verify_q8_1_tile_kernel<NC, 4>), grid, dim3(256), 0, s, P);
    else
        hipLaunchKernelGGL((lmhead_verify_q8_1_tile_kernel<NC, 1>), grid, dim3(64), 0, s, P);
}

}  // namespace

extern "C" {

size_t lmhead_argmax_verify_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || M > INT32_MAX || K < 256 || K % 256 || N < 1 || N > QG_SMALLN_MAX) return 0;
    return va_ws_bytes(M, N) + (N <= kVdMaxCols ? vd_extra_bytes(K, N) : 0);
}

qg_status lmhead_argmax_verify(const void* w, const float* X, int64_t ldx, int64_t M, int64_t K, int64_t N, void* ws,
                         size_t ws_bytes, int32_t* out_index, float* out_value, qg_stream_t stream) {
    qg::clear_error();
    qg_status st = va_validate(w, X, ldx, M, K, N);
    if (st) return st;
    if (!out_index) return qg::fail(QG_ERR_NULL, "out_index is NULL");
    if ((reinterpret_cast<uintptr_t>(out_index) & 3) || (reinterpret_cast<uintptr_t>(out_value) & 3))
        return qg::fail(QG_ERR_ALIGN, "outputs must be 4-byte aligned");
    const size_t need = lmhead_argmax_verify_workspace_bytes(M, K, N);
    if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    st = qg::check_device();
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const qg_launch_override& ov = qg::launch_override();
    // streamed form: up to 16 columns, K <= 4096 (one round of column loads), weights
    // under 2 GiB (one buffer resource)
    const bool vs_ok = N <= kVsCols && K <= 512 * kVsWaves && M * (K / 256) * 272 < (int64_t)INT32_MAX &&
                       vs_lds_bytes(K, N) <= 160 * 1024;
    const bool stream_form =
        vs_ok && (ov.verify_form == QG_FORM_VERIFY_STREAM || (ov.verify_form == QG_FORM_AUTO && N >= kVsMinCols));
    if (stream_form) {
        VsProb V{};
        V.w = (const uint8_t*)w;
        V.X = X;
        V.ldx = ldx;
        V.partials = (float2*)ws;
        V.M = (int32_t)M;
        V.nmb = (int32_t)(K / 256);
        V.N = (int32_t)N;
        V.tiles = (int32_t)qg::ceil_div(M, T);
        const size_t lds = vs_lds_bytes(K, N);
        const int per_cu = lds <= 80 * 1024 ? 2 : 1;
        V.G = (int32_t)std::min<int64_t>(V.tiles, (int64_t)per_cu * qg::device_cus());
        const auto kern = N <= 8 ? lmhead_verify_stream_kernel<kVsWaves, 8> : lmhead_verify_stream_kernel<kVsWaves, 16>;
        static std::atomic<bool> attr_set[2][64];  // per instance and device
        std::atomic<bool>* set = attr_set[N <= 8 ? 0 : 1];
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !set[dev].load(std::memory_order_acquire)) {
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            set[dev].store(true, std::memory_order_release);
        }
        hipLaunchKernelGGL(kern, dim3((unsigned)V.G), dim3(64 * kVsWaves), lds, s, V);
        st = qg::launch_status("lmhead_argmax_verify (tiles)");
        if (st) return st;
        const int threads = (int)std::min<int64_t>(1024, std::max<int64_t>(64, qg::ceil_div(V.G, 8 * 64) * 64));
        hipLaunchKernelGGL(lmhead_verify_reduce_kernel, dim3((unsigned)N), dim3(threads), 0, s, V.partials, V.G,
                           out_index, out_value, (uint4*)nullptr, 0);
        return qg::launch_status("lmhead_argmax_verify (reduce)");
    }
    const bool mfma = N > kVdMaxCols || ov.verify_form == QG_FORM_VERIFY_MFMA;
    if (!mfma) {
        // vector-ALU form: fp16 pairs and block sums, then one wavefront per tile on
        // grids that fill the chip, four that split K otherwise (152064 x 3584, us:
        // N = 1 95.5, 2 97.2, 4 111.3, 5 123.2, 6 133.7, 8 166.4 against 144.1, 135.9,
        // 138.6, 139.7, 141.3, 142.9 for the matrix-core form)
        const size_t pb = va_ws_bytes(M, N);
        uint8_t* xp = (uint8_t*)ws + pb;
        const int g8 = (int)(K / 8);
        hipLaunchKernelGGL(lmhead_verify_prep_kernel, dim3((unsigned)qg::ceil_div((int64_t)N * g8, 256)), dim3(256),
                           0, s, X, ldx, (int)K, (int)N, (uint4*)xp, (float*)(xp + (size_t)N * 2 * K));
        st = qg::launch_status("lmhead_argmax_verify (prep)");
        if (st) return st;
        VdProb D{};
        D.w = (const uint8_t*)w;
        D.xp = xp;
        D.partials = (float2*)ws;
        D.xpb = (int32_t)(2 * K);
        D.xs_off = (int32_t)(N * 2 * K);
        D.xsb = (int32_t)(K / 8);
        D.M = (int32_t)M;
        D.nmb = (int32_t)(K / 256);
        D.N = (int32_t)N;
        D.tiles = (int32_t)qg::ceil_div(M, T);
        int W = D.tiles >= 1024 ? 1 : 4;
        if (ov.verify_waves == 1 || ov.verify_waves == 4) W = ov.verify_waves;
        switch (N) {
            case 1: vd_launch<1>(D, W, s); break;
            case 2: vd_launch<2>(D, W, s); break;
            case 3: vd_launch<3>(D, W, s); break;
            case 4: vd_launch<4>(D, W, s); break;
            case 5: vd_launch<5>(D, W, s); break;
            default: vd_launch<6>(D, W, s); break;
        }
        st = qg::launch_status("lmhead_argmax_verify (tiles)");
        if (st) return st;
        const int threads = (int)std::min<int64_t>(1024, std::max<int64_t>(64, qg::ceil_div(D.tiles, 8 * 64) * 64));
        hipLaunchKernelGGL(lmhead_verify_reduce_kernel, dim3((unsigned)N), dim3(threads), 0, s, D.partials, D.tiles,
                           out_index, out_value, (uint4*)xp, (int)(N * (2 * K + K / 8) / 16));
        return qg::launch_status("lmhead_argmax_verify (reduce)");
    }
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
    if (ov.verify_waves == 4 || ov.verify_waves == 8) W = ov.verify_waves;
    const int et = ov.verify_tiles;
    if (et == 1 || et == 2 || (et == 4 && N <= 16)) TW = et;  // four tiles of two column blocks spill
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
                       out_index, out_value, (uint4*)nullptr, 0);
    return qg::launch_status("lmhead_argmax_verify (reduce)");
}

size_t lmhead_argmax_verify_q8_1_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || M > INT32_MAX || K < 256 || K % 256 || K > (1 << 24) || N < 1 || N > kVqMaxCols) return 0;
    return va_ws_bytes(M, N);
}

qg_status lmhead_argmax_verify_q8_1(const void* w, const void* xq, int64_t M, int64_t K, int64_t N, void* ws,
                              size_t ws_bytes, int32_t* out_index, float* out_value, qg_stream_t stream) {
    qg::clear_error();
    if (!w || !xq) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX - T) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (N < 1 || N > kVqMaxCols) return qg::fail(QG_ERR_SHAPE, "N=%lld not in [1, %d]", (long long)N, kVqMaxCols);
    if (!qg::aligned16(w) || !qg::aligned16(xq)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t xb = qg_q8_1_bytes(K);
    if ((int64_t)N * (int64_t)xb >= (int64_t)kQgOutOfRange)
        return qg::fail(QG_ERR_SHAPE, "activation buffers exceed 2^31 bytes");
    if (!out_index) return qg::fail(QG_ERR_NULL, "out_index is NULL");
    if ((reinterpret_cast<uintptr_t>(out_index) & 3) || (reinterpret_cast<uintptr_t>(out_value) & 3))
        return qg::fail(QG_ERR_ALIGN, "outputs must be 4-byte aligned");
    const size_t need = va_ws_bytes(M, N);
    if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    qg_status st = qg::check_device();
    if (st) return st;
    size_t q_off = 0, s_off = 0;
    qg::q8_1_offsets(K, &q_off, &s_off);
    VqProb P{};
    P.w = (const uint8_t*)w;
    P.xq = (const uint8_t*)xq;
    P.partials = (float2*)ws;
    P.xb = (int32_t)xb;
    P.q_off = (int32_t)q_off;
    P.M = (int32_t)M;
    P.nmb = (int32_t)(K / 256);
    P.N = (int32_t)N;
    P.tiles = (int32_t)qg::ceil_div(M, T);
    // one wavefront per tile on grids that fill the chip (vocabulary-sized heads),
    // four that split K otherwise
    int W = P.tiles >= 1024 ? 1 : 4;
    const qg_launch_override& ov = qg::launch_override();
    if (ov.verify_waves == 1 || ov.verify_waves == 4) W = ov.verify_waves;
    hipStream_t s = (hipStream_t)stream;
    switch (N) {
        case 1: vq_launch<1>(P, W, s); break;
        case 2: vq_launch<2>(P, W, s); break;
        case 3: vq_launch<3>(P, W, s); break;
        case 4: vq_launch<4>(P, W, s); break;
        case 5: vq_launch<5>(P, W, s); break;
        case 6: vq_launch<6>(P, W, s); break;
        case 7: vq_launch<7>(P, W, s); break;
        default: vq_launch<8>(P, W, s); break;
    }
    st = qg::launch_status("lmhead_argmax_verify_q8_1 (tiles)");
    if (st) return st;
    const int threads = (int)std::min<int64_t>(1024, std::max<int64_t>(64, qg::ceil_div(P.tiles, 8 * 64) * 64));
    hipLaunchKernelGGL(lmhead_verify_reduce_kernel, dim3((unsigned)N), dim3(threads), 0, s, P.partials, P.tiles,
                       out_index, out_value, (uint4*)nullptr, 0);
    return qg::launch_status("lmhead_argmax_verify_q8_1 (reduce)");
}

}  // extern "C"
