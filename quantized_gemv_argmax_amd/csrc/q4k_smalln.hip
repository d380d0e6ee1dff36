// Small-N Q4_K product Y = W X (N <= 32 columns) with one pass over the weights,
// for gfx950.
//
// Batched verification ("Why Local LLMs Don't Need C++ or Python", section 4: the
// candidate tokens are checked in a single batch pass, so the weights cross the
// memory bus once rather than once per token) and the 32-token prefill tile
// (section 3). Each weight byte is loaded from HBM once per call and applied to
// all N columns.
//
// Matrix-core formulation. For one 32-weight sub-block j of a 16-row tile,
//     S_j[n][r] = sum_k x[k][n] * q[r][k]
// is a 16 x 16 x 32 product: the A operand carries the activations of 16 columns
// (fp16), the B operand the 4-bit quants of the 16 rows. The quants enter B
// without any conversion: masking a dword with 0x000F000F leaves two fp16
// subnormals q * 2^-24 (0x00F000F0: 16q * 2^-24), which the fp16 matrix cores
// multiply exactly. A second product against an all-ones B gives the sub-block
// sums X_j[n] of the same fp16 activations, in the same output layout. The
// Q4_K affine form (dotLLM README, Key Features: fused scale x int dot products)
// is then applied per sub-block in fp32:
//     y[r][n] += 2^24 d sc_j S_j[n][r] - dmin m_j X_j[n].
// v_mfma_f32_16x16x32_f16 lane layout: lane l holds A[l % 16][8 (l / 16) + 0..7],
// B[8 (l / 16) + 0..7][l % 16] and D[4 (l / 16) + e][l % 16], e = 0..3; so lane
// l loads row l % 16 of the tile (its quant bytes 8 (l / 16)..+7 of each
// sub-block) and column l % 16 of the activations, and ends with row l % 16,
// columns 4 (l / 16) + e.
//
// Within a lane's 8-element K slice the order is that of the masked dwords:
// bytes 0, 2, 1, 3, 4, 6, 5, 7; the activations are packed in the same order.
//
// Grid: one workgroup per 16-row tile of the packed layout (q4k_gemv.hip), its W
// wavefronts splitting K in units of 256 / C weights (C = column blocks of 16);
// partial results meet in LDS in a fixed order, so results are deterministic. No
// workspace, no cross-workgroup traffic. Rows past a ragged tile's end and
// columns past N re-read the last row / column; their results are dropped.
#include <algorithm>
#include <climits>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;

typedef _Float16 qg_h8 __attribute__((ext_vector_type(8)));
typedef _Float16 qg_h2 __attribute__((ext_vector_type(2)));
typedef float qg_f4 __attribute__((ext_vector_type(4)));

struct SnProb {
    const uint8_t* w;
    const float* X;
    float* Y;
    int64_t ldx, ldy;
    int32_t M, nb, N, tiles, wg_begin;
};
struct SnArgs {
    int32_t begin[QG_MAX_BATCH];
    int32_t count;
    SnProb p[QG_MAX_BATCH];
};

// Inputs of one unit: super-block b, sub-block pairs g0 .. g0 + U - 1 (U = 4 / C).
template <int C>
struct SnIn {
    static constexpr int U = 4 / C;
    uint4 hdr;                 // d, dmin, 12 scale bytes of this lane's row
    uint2 q[U];                // quant bytes 8 (l / 16)..+7 of sub-blocks 2g and 2g + 1
    float4 x[U][2][C][2];      // [pair][low / high sub-block][column block][first / second 4]
};

template <int C>
QG_DEV void load_w(SnIn<C>& d, const uint4* __restrict__ seg, int rt, int u, int s) {
    constexpr int U = SnIn<C>::U;
    const int b = u / C, g0 = (u % C) * U;
    const uint4* sb = seg + (size_t)b * 9 * rt;
    d.hdr = qg_stream_load(sb);
#pragma unroll
    for (int gi = 0; gi < U; ++gi) {
        const uint4* sg = sb + (size_t)(1 + 2 * (g0 + gi) + (s >> 1)) * rt;
        const uint2* p = reinterpret_cast<const uint2*>(sg) + (s & 1);
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        const u2 v = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
        d.q[gi] = make_uint2(v.x, v.y);
    }
}

// xc[c] = start of column 16 c + (l % 16) (clamped to N - 1) at this lane's K slice.
template <int C>
QG_DEV void load_x(SnIn<C>& d, const float* const (&xc)[C], int u) {
    constexpr int U = SnIn<C>::U;
    const int b = u / C, g0 = (u % C) * U;
#pragma unroll
    for (int gi = 0; gi < U; ++gi)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const float* p = xc[c] + 256 * b + 64 * (g0 + gi) + 32 * h;
                d.x[gi][h][c][0] = *reinterpret_cast<const float4*>(p);
                d.x[gi][h][c][1] = *reinterpret_cast<const float4*>(p + 4);
            }
}

QG_DEV uint32_t pk_rne(float a, float b) {
    const qg_h2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Eight activations in the masked-dword order 0, 2, 1, 3, 4, 6, 5, 7, as fp16.
QG_DEV qg_h8 a_operand(const float4 lo, const float4 hi) {
    uint4 r;
    r.x = pk_rne(lo.x, lo.z);
    r.y = pk_rne(lo.y, lo.w);
    r.z = pk_rne(hi.x, hi.z);
    r.w = pk_rne(hi.y, hi.w);
    return __builtin_bit_cast(qg_h8, r);
}

// Byte k of a packed word, as float.
QG_DEV float byte_f(uint32_t v, int k) { return (float)((v >> (8 * k)) & 0xffu); }

template <int C>
QG_DEV void unit_dot(qg_f4 (&acc)[C], const SnIn<C>& d, int u) {
    constexpr int U = SnIn<C>::U;
    const int g0 = (u % C) * U;
    const float dd = qg_half_lo(d.hdr.x) * 16777216.0f;  // quants enter as q * 2^-24
    const float dm = qg_half_hi(d.hdr.x);
    const QgScales sc = qg_q4k_scales(d.hdr.y, d.hdr.z, d.hdr.w);
    const qg_h8 ones = __builtin_bit_cast(qg_h8, make_uint4(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u));
    const qg_f4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < U; ++gi) {
        const int g = g0 + gi;  // sub-blocks 2g (low nibbles) and 2g + 1 (high nibbles)
        const uint32_t scw = (g < 2) ? sc.sc03 : sc.sc47;
        const uint32_t mw = (g < 2) ? sc.m03 : sc.m47;
        const int kb = 2 * (g & 1);
        const float s_lo = dd * byte_f(scw, kb);
        const float s_hi = dd * 0.0625f * byte_f(scw, kb + 1);
        const float m_lo = dm * byte_f(mw, kb);
        const float m_hi = dm * byte_f(mw, kb + 1);

        const uint32_t w0 = d.q[gi].x, w1 = d.q[gi].y;
        const uint32_t w0s = w0 >> 8, w1s = w1 >> 8;
        const qg_h8 b_lo = __builtin_bit_cast(
            qg_h8, make_uint4(w0 & 0x000f000fu, w0s & 0x000f000fu, w1 & 0x000f000fu, w1s & 0x000f000fu));
        const qg_h8 b_hi = __builtin_bit_cast(
            qg_h8, make_uint4(w0 & 0x00f000f0u, w0s & 0x00f000f0u, w1 & 0x00f000f0u, w1s & 0x00f000f0u));
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const qg_h8 a_lo = a_operand(d.x[gi][0][c][0], d.x[gi][0][c][1]);
            const qg_h8 a_hi = a_operand(d.x[gi][1][c][0], d.x[gi][1][c][1]);
            const qg_f4 s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b_lo, zero, 0, 0, 0);
            const qg_f4 s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b_hi, zero, 0, 0, 0);
            const qg_f4 x0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, ones, zero, 0, 0, 0);
            const qg_f4 x1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, ones, zero, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = acc[c][e];
                v = fmaf(s_lo, s0[e], v);
                v = fmaf(s_hi, s1[e], v);
                v = fmaf(-m_lo, x0[e], v);
                v = fmaf(-m_hi, x1[e], v);
                acc[c][e] = v;
            }
        }
    }
}

template <int C, int W>
__global__ __launch_bounds__(64 * W) void q4k_smalln_kernel(SnArgs a) {
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SnProb P = a.p[k];

    const int tile = wg - P.wg_begin;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    const int rt = min(T, P.M - tile * T);
    const uint4* __restrict__ seg =
        reinterpret_cast<const uint4*>(P.w + (size_t)tile * T * P.nb * 144) + min(i, rt - 1);
    const float* xc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) xc[c] = P.X + (int64_t)min(16 * c + i, P.N - 1) * P.ldx + 8 * s;

    const int units = P.nb * C;
    const int niter = (units - wave + W - 1) / W;  // units wave, wave + W, ...
    qg_f4 acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = qg_f4{0.f, 0.f, 0.f, 0.f};

    if (niter > 0) {
        // ping-pong: the weight loads of the next unit are in flight while this one
        // is computed; activations (L2-resident) are loaded at the top of their own
        // iteration, before the next unit's weights, so waiting for them never waits
        // for those weights
        SnIn<C> b0, b1;
        load_w<C>(b0, seg, rt, wave, s);
        for (int it = 0;; it += 2) {
            const int u0 = wave + W * it;
            load_x<C>(b0, xc, u0);
            if (it + 1 < niter) load_w<C>(b1, seg, rt, u0 + W, s);
            unit_dot<C>(acc, b0, u0);
            if (it + 1 >= niter) break;
            load_x<C>(b1, xc, u0 + W);
            if (it + 2 < niter) load_w<C>(b0, seg, rt, u0 + 2 * W, s);
            unit_dot<C>(acc, b1, u0 + W);
            if (it + 2 >= niter) break;
        }
    }

    if constexpr (W > 1) {
        __shared__ float red[W][C * 4][64];
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][4 * c + e][lane] = acc[c][e];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = red[0][4 * c + e][lane];
#pragma unroll
                for (int w = 1; w < W; ++w) v += red[w][4 * c + e][lane];
                acc[c][e] = v;
            }
    }
    if (i < rt) {
        const int row = tile * T + i;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = 16 * c + 4 * s + e;
                if (n < P.N) P.Y[(int64_t)n * P.ldy + row] = acc[c][e];
            }
    }
}

// ------------------------------------------------------------------ host side
int sn_validate(const void* w, const float* X, int64_t ldx, const float* Y, int64_t ldy, int64_t M, int64_t K,
                int64_t N) {
    if (!w || !X || !Y) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (N < 1 || N > QG_SMALLN_MAX) return qg::fail(QG_ERR_SHAPE, "N=%lld not in [1, %d]", (long long)N, QG_SMALLN_MAX);
    if (ldx < K || ldy < M || ldx % 4 || ldy % 4)
        return qg::fail(QG_ERR_SHAPE, "ldx=%lld / ldy=%lld must be >= K / M and multiples of 4", (long long)ldx,
                        (long long)ldy);
    if (!qg::aligned16(w) || !qg::aligned16(X) || !qg::aligned16(Y))
        return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    return QG_OK;
}

SnProb make_sn(const void* w, const float* X, int64_t ldx, float* Y, int64_t ldy, int64_t M, int64_t K, int64_t N) {
    SnProb P{};
    P.w = (const uint8_t*)w;
    P.X = X;
    P.Y = Y;
    P.ldx = ldx;
    P.ldy = ldy;
    P.M = (int32_t)M;
    P.nb = (int32_t)(K / 256);
    P.N = (int32_t)N;
    P.tiles = (int32_t)qg::ceil_div(M, T);
    return P;
}

// Wavefronts per workgroup: enough K units per wavefront to pipeline, at most 8.
int choose_w(const SnArgs& a, int C) {
    int units = INT_MAX;
    for (int i = 0; i < a.count; ++i) units = std::min(units, a.p[i].nb * C);
    int W = 1;
    while (W < 4 && 2 * W <= units) W *= 2;
    int ew = 0, eu = 0;
    if (qg::env_pair("QG_SN_CFG", &ew, &eu) && (ew == 1 || ew == 2 || ew == 4 || ew == 8)) W = ew;
    return W;
}

template <int C>
void launch(const SnArgs& a, int grid, int W, hipStream_t s) {
    switch (W) {
        case 1: hipLaunchKernelGGL((q4k_smalln_kernel<C, 1>), dim3(grid), dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((q4k_smalln_kernel<C, 2>), dim3(grid), dim3(128), 0, s, a); break;
        case 4: hipLaunchKernelGGL((q4k_smalln_kernel<C, 4>), dim3(grid), dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((q4k_smalln_kernel<C, 8>), dim3(grid), dim3(512), 0, s, a); break;
    }
}

int run(const qg_gemm_problem* probs, int count, hipStream_t stream) {
    if (!probs) return qg::fail(QG_ERR_NULL, "NULL problem list");
    if (count < 1 || count > QG_MAX_BATCH)
        return qg::fail(QG_ERR_SHAPE, "count=%d not in [1, %d]", count, QG_MAX_BATCH);
    SnArgs a{};
    a.count = count;
    int64_t wgs = 0;
    int nmax = 0;
    for (int i = 0; i < count; ++i) {
        const qg_gemm_problem& q = probs[i];
        int st = sn_validate(q.w_packed, q.X, q.ldx, q.Y, q.ldy, q.M, q.K, q.N);
        if (st) return st;
        a.p[i] = make_sn(q.w_packed, q.X, q.ldx, q.Y, q.ldy, q.M, q.K, q.N);
        a.p[i].wg_begin = (int32_t)wgs;
        a.begin[i] = (int32_t)wgs;
        wgs += a.p[i].tiles;
        nmax = std::max(nmax, a.p[i].N);
    }
    if (wgs > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "too many tiles in one batch");
    int st = qg::check_device();
    if (st) return st;
    const int C = nmax > 16 ? 2 : 1;
    const int W = choose_w(a, C);
    if (C == 1)
        launch<1>(a, (int)wgs, W, stream);
    else
        launch<2>(a, (int)wgs, W, stream);
    return qg::launch_status("qgemm_q4k_smalln");
}

}  // namespace

extern "C" {

size_t qgemm_q4k_smalln_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    (void)M;
    (void)K;
    (void)N;
    return 0;  // each workgroup owns whole rows
}

int qgemm_q4k_smalln(const void* w, const float* X, int64_t ldx, float* Y, int64_t ldy, int64_t M, int64_t K,
                     int64_t N, void* ws, size_t ws_bytes, qg_stream_t stream) {
    (void)ws;
    (void)ws_bytes;
    qg::clear_error();
    const qg_gemm_problem p{w, X, ldx, Y, ldy, M, K, N};
    return run(&p, 1, (hipStream_t)stream);
}

size_t qgemm_q4k_smalln_batch_workspace_bytes(const qg_gemm_problem* problems, int count) {
    (void)problems;
    (void)count;
    return 0;
}

int qgemm_q4k_smalln_batch(const qg_gemm_problem* problems, int count, void* ws, size_t ws_bytes,
                           qg_stream_t stream) {
    (void)ws;
    (void)ws_bytes;
    qg::clear_error();
    return run(problems, count, (hipStream_t)stream);
}

}  // extern "C"
