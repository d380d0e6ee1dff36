// Small-N Q4_K product Y = W X (N <= 32 columns) with one pass over the weights,
// for gfx950.
//
// Batched verification ("Why Local LLMs Don't Need C++ or Python", section 4: the
// candidate tokens are checked in a single batch pass, so the weights cross the
// memory bus once rather than once per token) and the 32-token prefill tile
// (section 3). Each weight byte is loaded from HBM once per call and applied to
// all N columns.
//
// Both kernels read the 16-row-tile packed layout of q4k_gemv.hip and give a
// wavefront four consecutive tiles (64 rows, lane = 16 * tile + row for the vector
// kernel). A workgroup of W wavefronts owns those 64 rows and splits K among its
// wavefronts; partial results meet in LDS in a fixed order.
//
// N <= 8: vector-ALU kernel. Every lane accumulates its own row; the activations
// of the N columns are wavefront-uniform and arrive through scalar loads; fp32 FMA.
// N > 8: matrix-core kernel. Lane (i = lane % 16, s = lane / 16) loads quant
// segment 1 + 4t + s of row i of each of the four tiles, so the four lane groups
// cover half a super-block per round t; dword u of a lane's segment (4 low-nibble
// and 4 high-nibble weights) is that lane's 8-element K slice of MFMA step (t, u).
// The lane dequantizes those weights to fp16 in registers (d*sc*q - dmin*m in
// fp32, then one rounding); the B operand carries the matching 8 activations of
// each column, converted to fp16; v_mfma_f32_16x16x32_f16 accumulates in fp32.
#include <algorithm>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;

typedef _Float16 qg_h8 __attribute__((ext_vector_type(8)));
typedef float qg_f4 __attribute__((ext_vector_type(4)));

struct SnProb {
    const uint8_t* w;
    const float* X;
    float* Y;
    int64_t ldx, ldy;
    int32_t M, nb, N, tiles;
};

// Row i of tile `tile_in_group` of this wavefront's 64-row tile group, clamped
// into the matrix: returns the segment-0 pointer of super-block 0 and the segment
// stride (rows of its tile); `active` tells whether the row exists.
QG_DEV const uint4* row_base(const SnProb& P, int group, int tile_in_group, int i, int& stride, bool& active) {
    const int t = 4 * group + tile_in_group;
    const bool tile_ok = t < P.tiles;
    const int tc = tile_ok ? t : P.tiles - 1;
    const int rt = min(T, P.M - tc * T);
    active = tile_ok && i < rt;
    stride = rt;
    return reinterpret_cast<const uint4*>(P.w + (size_t)tc * T * P.nb * 144) + min(i, rt - 1);
}

// ------------------------------------------------------------------ VALU, N <= 8
template <int N>
struct SbN {
    uint4 s[9];
    float4 xv[N];  // this lane's 4 activations of each column (sub-block sums)
};

template <int N>
QG_DEV void load_sbn(SbN<N>& d, const uint4* __restrict__ seg, int stride, const SnProb& P, int b, int lane) {
#pragma unroll
    for (int n = 0; n < N; ++n) d.xv[n] = *reinterpret_cast<const float4*>(P.X + n * P.ldx + 256 * b + 4 * lane);
    const uint4* sb = seg + (size_t)b * 9 * stride;
#pragma unroll
    for (int s = 0; s < 9; ++s) d.s[s] = sb[s * stride];
}

// Sums of x over the eight 32-element sub-blocks (lane t holds x[4t..4t+3]).
QG_DEV void subblock_sums(const float4 xv, float (&X)[8]) {
    float s = ((xv.x + xv.y) + xv.z) + xv.w;
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
#pragma unroll
    for (int j = 0; j < 8; ++j) X[j] = qg_readlane(s, 8 * j);
}

template <int N>
QG_DEV void sb_dot_n(float (&acc)[N], const SbN<N>& d, const SnProb& P, int b) {
    float X[N][8];
#pragma unroll
    for (int n = 0; n < N; ++n) subblock_sums(d.xv[n], X[n]);
    float S[8][N];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int n = 0; n < N; ++n) S[j][n] = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int g = p >> 1, h = p & 1;
        const uint32_t qw[4] = {d.s[1 + p].x, d.s[1 + p].y, d.s[1 + p].z, d.s[1 + p].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t l4 = qg_opaque(qw[i] & 0x0f0f0f0fu);
            const uint32_t h4 = qg_opaque(qw[i] & 0xf0f0f0f0u);
            const float fl[4] = {qg_ub0(l4), qg_ub1(l4), qg_ub2(l4), qg_ub3(l4)};
            const float fh[4] = {qg_ub0(h4), qg_ub1(h4), qg_ub2(h4), qg_ub3(h4)};
#pragma unroll
            for (int n = 0; n < N; ++n) {
                qg_uniform_f32 xl = (qg_uniform_f32)(P.X + n * P.ldx) + 256 * b + 64 * g + 16 * h + 4 * i;
                qg_uniform_f32 xh = xl + 32;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    S[2 * g][n] = fmaf(fl[k], xl[k], S[2 * g][n]);
                    S[2 * g + 1][n] = fmaf(fh[k], xh[k], S[2 * g + 1][n]);
                }
            }
        }
    }
    const uint4 hd = d.s[0];
    const float dd = qg_half_lo(hd.x), dm = qg_half_hi(hd.x);
    const QgScales sc = qg_q4k_scales(hd.y, hd.z, hd.w);
    const float scf[8] = {qg_ub0(sc.sc03), qg_ub1(sc.sc03) * 0.0625f, qg_ub2(sc.sc03), qg_ub3(sc.sc03) * 0.0625f,
                          qg_ub0(sc.sc47), qg_ub1(sc.sc47) * 0.0625f, qg_ub2(sc.sc47), qg_ub3(sc.sc47) * 0.0625f};
    const float mf[8] = {qg_ub0(sc.m03), qg_ub1(sc.m03), qg_ub2(sc.m03), qg_ub3(sc.m03),
                         qg_ub0(sc.m47), qg_ub1(sc.m47), qg_ub2(sc.m47), qg_ub3(sc.m47)};
#pragma unroll
    for (int n = 0; n < N; ++n) {
        float t = scf[0] * S[0][n];
        float mn = mf[0] * X[n][0];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            t = fmaf(scf[j], S[j][n], t);
            mn = fmaf(mf[j], X[n][j], mn);
        }
        acc[n] += fmaf(dd, t, -dm * mn);
    }
}

template <int N, int W>
__global__ __launch_bounds__(64 * W) void q4k_smalln_valu_kernel(SnProb P) {
    const int group = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    int stride;
    bool active;
    const uint4* __restrict__ seg = row_base(P, group, lane >> 4, lane & 15, stride, active);
    const int row = group * 64 + lane;  // tiles of a group are consecutive rows
    const int wb0 = wave * nb / W, wb1 = (wave + 1) * nb / W;

    float acc[N];
#pragma unroll
    for (int n = 0; n < N; ++n) acc[n] = 0.f;
    if (wb0 < wb1) {
        SbN<N> cur, nxt;
        load_sbn<N>(cur, seg, stride, P, wb0, lane);
        for (int b = wb0; b < wb1 - 1; ++b) {
            load_sbn<N>(nxt, seg, stride, P, b + 1, lane);
            sb_dot_n<N>(acc, cur, P, b);
            cur = nxt;
        }
        sb_dot_n<N>(acc, cur, P, wb1 - 1);
    }
    if constexpr (W > 1) {
        __shared__ float red[W][N][64];
#pragma unroll
        for (int n = 0; n < N; ++n) red[wave][n][lane] = acc[n];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float v = red[0][n][lane];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w][n][lane];
            acc[n] = v;
        }
    }
    if (active)
#pragma unroll
        for (int n = 0; n < N; ++n) P.Y[n * P.ldy + row] = acc[n];
}

// ------------------------------------------------------------------ MFMA, N > 8
QG_DEV uint32_t pk_h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// 8 fp16 weights of one dword of quants: low nibbles (scale dsl, min dml) then
// high nibbles (dsh already divided by 16, min dmh).
QG_DEV qg_h8 dequant8(uint32_t w, float dsl, float dml, float dsh, float dmh) {
    const uint32_t l4 = qg_opaque(w & 0x0f0f0f0fu);
    const uint32_t h4 = qg_opaque(w & 0xf0f0f0f0u);
    uint4 r;
    r.x = pk_h2(fmaf(qg_ub0(l4), dsl, -dml), fmaf(qg_ub1(l4), dsl, -dml));
    r.y = pk_h2(fmaf(qg_ub2(l4), dsl, -dml), fmaf(qg_ub3(l4), dsl, -dml));
    r.z = pk_h2(fmaf(qg_ub0(h4), dsh, -dmh), fmaf(qg_ub1(h4), dsh, -dmh));
    r.w = pk_h2(fmaf(qg_ub2(h4), dsh, -dmh), fmaf(qg_ub3(h4), dsh, -dmh));
    return __builtin_bit_cast(qg_h8, r);
}

QG_DEV qg_h8 to_h8(const float4 a, const float4 b) {
    uint4 r;
    r.x = pk_h2(a.x, a.y);
    r.y = pk_h2(a.z, a.w);
    r.z = pk_h2(b.x, b.y);
    r.w = pk_h2(b.z, b.w);
    return __builtin_bit_cast(qg_h8, r);
}

struct MfW {
    uint4 hdr[4];
    uint4 q[2][4];  // [round t][tile r]
};

QG_DEV void load_mfw(MfW& d, const uint4* const (&base)[4], const int (&stride)[4], int b, int s) {
#pragma unroll
    for (int r = 0; r < 4; ++r) d.hdr[r] = base[r][(size_t)b * 9 * stride[r]];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) d.q[t][r] = base[r][((size_t)b * 9 + 1 + 4 * t + s) * stride[r]];
}

// Activations of one round of a super-block for column block c: 4 steps u, each
// a low and a high float4 (k0 = first low-nibble position of this lane group).
template <int C>
QG_DEV void load_x(float4 (&xs)[C][4][2], const float* const (&xcol)[C], int64_t k0) {
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xs[c][u][0] = *reinterpret_cast<const float4*>(xcol[c] + k0 + 4 * u);
            xs[c][u][1] = *reinterpret_cast<const float4*>(xcol[c] + k0 + 4 * u + 32);
        }
}

template <int C>
QG_DEV void mfma_round(qg_f4 (&D)[4][C], const MfW& d, const float4 (&xs)[C][4][2], const float (&cmask)[C], int t,
                       int s) {
    float dsl[4], dml[4], dsh[4], dmh[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float dd = qg_half_lo(d.hdr[r].x), dm = qg_half_hi(d.hdr[r].x);
        const QgScales sc = qg_q4k_scales(d.hdr[r].y, d.hdr[r].z, d.hdr[r].w);
        const int sh = 16 * (s >> 1);  // byte pair (2g, 2g+1) within the word
        const uint32_t scw = (t == 0 ? sc.sc03 : sc.sc47) >> sh;
        const uint32_t mw = (t == 0 ? sc.m03 : sc.m47) >> sh;
        dsl[r] = dd * qg_ub0(scw);
        dsh[r] = dd * qg_ub1(scw) * 0.0625f;
        dml[r] = dm * qg_ub0(mw);
        dmh[r] = dm * qg_ub1(mw);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        qg_h8 B[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const float m = cmask[c];
            const float4 lo = make_float4(xs[c][u][0].x * m, xs[c][u][0].y * m, xs[c][u][0].z * m, xs[c][u][0].w * m);
            const float4 hi = make_float4(xs[c][u][1].x * m, xs[c][u][1].y * m, xs[c][u][1].z * m, xs[c][u][1].w * m);
            B[c] = to_h8(lo, hi);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t qu = (&d.q[t][r].x)[u];
            const qg_h8 A = dequant8(qu, dsl[r], dml[r], dsh[r], dmh[r]);
#pragma unroll
            for (int c = 0; c < C; ++c) D[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[c], D[r][c], 0, 0, 0);
        }
    }
}

template <int C, int W>
__global__ __launch_bounds__(64 * W) void q4k_smalln_mfma_kernel(SnProb P) {
    const int group = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    const int nb = P.nb;
    const int wb0 = wave * nb / W, wb1 = (wave + 1) * nb / W;

    const uint4* base[4];
    int stride[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        bool act;
        base[r] = row_base(P, group, r, i, stride[r], act);
    }
    const float* xcol[C];
    float cmask[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = 16 * c + i;
        cmask[c] = n < P.N ? 1.f : 0.f;
        xcol[c] = P.X + (int64_t)(n < P.N ? n : 0) * P.ldx;
    }

    qg_f4 D[4][C];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) D[r][c] = qg_f4{0.f, 0.f, 0.f, 0.f};

    if (wb0 < wb1) {
        MfW cur, nxt;
        load_mfw(cur, base, stride, wb0, s);
        for (int b = wb0; b < wb1; ++b) {
            float4 xs[C][4][2];
            const int64_t k0 = 256 * (int64_t)b + 64 * (s >> 1) + 16 * (s & 1);
            // activations before the prefetch, so waiting for them never waits for it
            load_x<C>(xs, xcol, k0);
            mfma_round<C>(D, cur, xs, cmask, 0, s);
            load_x<C>(xs, xcol, k0 + 128);
            load_mfw(nxt, base, stride, min(b + 1, wb1 - 1), s);
            mfma_round<C>(D, cur, xs, cmask, 1, s);
            cur = nxt;
        }
    }

    // D[r][c] element e of lane (i, s): row 16r + 4s + e of the group, column 16c + i.
    if constexpr (W > 1) {
        __shared__ float red[W][4][C][4][64];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[wave][r][c][e][lane] = D[r][c][e];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = red[0][r][c][e][lane];
#pragma unroll
                    for (int w = 1; w < W; ++w) v += red[w][r][c][e][lane];
                    D[r][c][e] = v;
                }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = group * 64 + 16 * r + 4 * s + e;
                const int n = 16 * c + i;
                if (row < P.M && n < P.N) P.Y[(int64_t)n * P.ldy + row] = D[r][c][e];
            }
}

// ------------------------------------------------------------------ host side
int choose_w(const SnProb& P, bool mfma) {
    const int64_t groups = qg::ceil_div(P.M, 64);
    int W = 1;
    while (W < 8 && groups * W < 1024 && 2 * W <= P.nb) W *= 2;
    int ew = 0, eu = 0;
    if (qg::env_pair(mfma ? "QG_SNM_CFG" : "QG_SNV_CFG", &ew, &eu) && (ew == 1 || ew == 2 || ew == 4 || ew == 8)) W = ew;
    if (mfma && W > 4) W = 4;
    return W;
}

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

template <int N>
void launch_valu(const SnProb& P, int W, hipStream_t s) {
    const dim3 grid((unsigned)qg::ceil_div(P.M, 64));
    switch (W) {
        case 1: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 1>), grid, dim3(64), 0, s, P); break;
        case 2: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 2>), grid, dim3(128), 0, s, P); break;
        case 4: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 4>), grid, dim3(256), 0, s, P); break;
        default: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 8>), grid, dim3(512), 0, s, P); break;
    }
}

template <int C>
void launch_mfma(const SnProb& P, int W, hipStream_t s) {
    const dim3 grid((unsigned)qg::ceil_div(P.M, 64));
    switch (W) {
        case 1: hipLaunchKernelGGL((q4k_smalln_mfma_kernel<C, 1>), grid, dim3(64), 0, s, P); break;
        case 2: hipLaunchKernelGGL((q4k_smalln_mfma_kernel<C, 2>), grid, dim3(128), 0, s, P); break;
        default: hipLaunchKernelGGL((q4k_smalln_mfma_kernel<C, 4>), grid, dim3(256), 0, s, P); break;
    }
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
    int st = sn_validate(w, X, ldx, Y, ldy, M, K, N);
    if (st) return st;
    SnProb P = make_sn(w, X, ldx, Y, ldy, M, K, N);
    st = qg::check_device();
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const bool mfma = P.N > 8;
    const int W = choose_w(P, mfma);
    switch (P.N) {
        case 1: launch_valu<1>(P, W, s); break;
        case 2: launch_valu<2>(P, W, s); break;
        case 3: launch_valu<3>(P, W, s); break;
        case 4: launch_valu<4>(P, W, s); break;
        case 5: launch_valu<5>(P, W, s); break;
        case 6: launch_valu<6>(P, W, s); break;
        case 7: launch_valu<7>(P, W, s); break;
        case 8: launch_valu<8>(P, W, s); break;
        default:
            if (P.N <= 16)
                launch_mfma<1>(P, W, s);
            else
                launch_mfma<2>(P, W, s);
            break;
    }
    return qg::launch_status("qgemm_q4k_smalln");
}

}  // extern "C"
