// Small-N Q4_K product Y = W X (N <= 32 columns) with one pass over the weights,
// for gfx950.
//
// Batched verification ("Why Local LLMs Don't Need C++ or Python", section 4: the
// candidate tokens are checked in a single batch pass, so the weights cross the
// memory bus once rather than once per token) and the 32-token prefill tile
// (section 3). Each weight byte is loaded from HBM once per call and applied to
// all N columns.
//
// N <= 8: vector-ALU kernel, the GEMV's skeleton (lane = row, activations through
// scalar loads) with N accumulators per sub-block, fp32 FMA.
// N > 8: matrix-core kernel. A wavefront takes one 64-row packed tile as four
// 16-row MFMA tiles. Lane (i = lane % 16, s = lane / 16) loads quant segment
// 1 + 4t + s of row 16r + i, so the four lane groups cover the 128 weights of
// half a super-block per round t; dword u of a lane's segment (4 low-nibble and
// 4 high-nibble weights) is that lane's 8-element K slice of MFMA step (t, u).
// The lane dequantizes those weights to fp16 in registers (d*sc*q - dmin*m in
// fp32, then one rounding) and the B operand carries the matching 8 activations
// of each column, converted to fp16; v_mfma_f32_16x16x32_f16 accumulates in fp32.
// Split-K partials and the fixed-order last-arriver reduction are as in the GEMV.
#include <algorithm>

#include "qg_device.h"
#include "qg_host.h"

namespace {

typedef _Float16 qg_h8 __attribute__((ext_vector_type(8)));
typedef float qg_f4 __attribute__((ext_vector_type(4)));

struct SnProb {
    const uint8_t* w;
    const float* X;
    float* Y;
    int64_t ldx, ldy;
    int32_t M, nb, N, tiles, splits;
};

struct SbData {
    uint4 s[9];
};

QG_DEV void load_sb(SbData& d, const uint4* __restrict__ seg, int rt) {
#pragma unroll
    for (int s = 0; s < 9; ++s) d.s[s] = seg[s * rt];
}

// ------------------------------------------------------------------ VALU, N <= 8
template <int N>
QG_DEV void load_xv(float4 (&xv)[N], const SnProb& P, int b, int lane) {
#pragma unroll
    for (int n = 0; n < N; ++n) xv[n] = qg_x4(P.X + n * P.ldx + 256 * b, lane);
}

template <int N>
QG_DEV void sb_dot_n(float (&acc)[N], const SbData& d, const float4 (&xv)[N], const SnProb& P, int b) {
    QgSub8 X[N];
#pragma unroll
    for (int n = 0; n < N; ++n) X[n] = qg_subblock_sums(xv[n]);
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
        float mn = mf[0] * X[n].v[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            t = fmaf(scf[j], S[j][n], t);
            mn = fmaf(mf[j], X[n].v[j], mn);
        }
        acc[n] += fmaf(dd, t, -dm * mn);
    }
}

// Store or split-K-reduce N values per row held by wavefront 0 of the workgroup.
// vals[n] belongs to row `row`; returns after the output is written.
template <int N>
QG_DEV void finish_rows(const SnProb& P, float* __restrict__ part, uint32_t* cnt, int tile, int ks, int row,
                        bool active, const float (&vals)[N], int lane) {
    if (P.splits == 1) {
        if (active)
#pragma unroll
            for (int n = 0; n < N; ++n) P.Y[n * P.ldy + row] = vals[n];
        return;
    }
    if (active)
#pragma unroll
        for (int n = 0; n < N; ++n) part[((int64_t)ks * N + n) * P.M + row] = vals[n];
    __threadfence();
    const uint32_t old = qg_ticket(cnt + tile, lane);
    if (old != (uint32_t)(P.splits - 1)) return;
    __threadfence();
    if (active) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float s = 0.f;
            for (int j = 0; j < P.splits; ++j) s += __builtin_nontemporal_load(&part[((int64_t)j * N + n) * P.M + row]);
            P.Y[n * P.ldy + row] = s;
        }
    }
    qg_ticket_reset(cnt + tile, lane);
}

template <int N, int W>
__global__ __launch_bounds__(64 * W) void q4k_smalln_valu_kernel(SnProb P, float* __restrict__ part, uint32_t* cnt) {
    const int wg = blockIdx.x;
    const int tile = wg / P.splits;
    const int ks = wg - tile * P.splits;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    const int rt = min(qg::kTileRows, P.M - tile * qg::kTileRows);
    const bool active = lane < rt;
    const int row = tile * qg::kTileRows + lane;
    const int b0 = (int)((int64_t)ks * nb / P.splits);
    const int b1 = (int)((int64_t)(ks + 1) * nb / P.splits);
    const int wb0 = b0 + wave * (b1 - b0) / W;
    const int wb1 = b0 + (wave + 1) * (b1 - b0) / W;
    const uint4* __restrict__ seg =
        reinterpret_cast<const uint4*>(P.w + (size_t)tile * qg::kTileRows * nb * 144) + (active ? lane : rt - 1);

    float acc[N];
#pragma unroll
    for (int n = 0; n < N; ++n) acc[n] = 0.f;
    if (wb0 < wb1) {
        SbData cur, nxt;
        float4 xc[N], xn[N];
        load_xv<N>(xc, P, wb0, lane);
        load_sb(cur, seg + (size_t)wb0 * 9 * rt, rt);
        for (int b = wb0; b < wb1 - 1; ++b) {
            load_xv<N>(xn, P, b + 1, lane);
            load_sb(nxt, seg + (size_t)(b + 1) * 9 * rt, rt);
            sb_dot_n<N>(acc, cur, xc, P, b);
            cur = nxt;
#pragma unroll
            for (int n = 0; n < N; ++n) xc[n] = xn[n];
        }
        sb_dot_n<N>(acc, cur, xc, P, wb1 - 1);
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
    finish_rows<N>(P, part, cnt, tile, ks, row, active, acc, lane);
}

// ------------------------------------------------------------------ MFMA, N > 8
QG_DEV uint32_t pk_h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// 8 fp16 weights of one dword of quants: low nibbles (sub-block a) then high
// nibbles (sub-block b, scale pre-divided by 16).
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

QG_DEV qg_h8 x8(const float* __restrict__ col, int64_t k0, bool valid) {
    if (!valid) return __builtin_bit_cast(qg_h8, make_uint4(0, 0, 0, 0));
    const float4 a = *reinterpret_cast<const float4*>(col + k0);
    const float4 b = *reinterpret_cast<const float4*>(col + k0 + 32);
    uint4 r;
    r.x = pk_h2(a.x, a.y);
    r.y = pk_h2(a.z, a.w);
    r.z = pk_h2(b.x, b.y);
    r.w = pk_h2(b.z, b.w);
    return __builtin_bit_cast(qg_h8, r);
}

template <int C, int W>
__global__ __launch_bounds__(64 * W) void q4k_smalln_mfma_kernel(SnProb P, float* __restrict__ part, uint32_t* cnt) {
    const int wg = blockIdx.x;
    const int tile = wg / P.splits;
    const int ks = wg - tile * P.splits;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    const int nb = P.nb;
    const int rt = min(qg::kTileRows, P.M - tile * qg::kTileRows);
    const int b0 = (int)((int64_t)ks * nb / P.splits);
    const int b1 = (int)((int64_t)(ks + 1) * nb / P.splits);
    const int wb0 = b0 + wave * (b1 - b0) / W;
    const int wb1 = b0 + (wave + 1) * (b1 - b0) / W;
    const uint4* __restrict__ tbase = reinterpret_cast<const uint4*>(P.w + (size_t)tile * qg::kTileRows * nb * 144);

    bool rok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rok[r] = (16 * r + i) < rt;
    const float* xcol[C];
    bool cok[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = 16 * c + i;
        cok[c] = n < P.N;
        xcol[c] = P.X + (int64_t)(cok[c] ? n : 0) * P.ldx;
    }

    qg_f4 D[4][C];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) D[r][c] = qg_f4{0.f, 0.f, 0.f, 0.f};

    for (int b = wb0; b < wb1; ++b) {
        uint4 hdr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            hdr[r] = rok[r] ? tbase[((size_t)b * 9) * rt + 16 * r + i] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int p = 4 * t + s;        // quant segment of this lane
            const int g = p >> 1, h = p & 1;  // 64-weight group, half
            uint4 q[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                q[r] = rok[r] ? tbase[((size_t)b * 9 + 1 + p) * rt + 16 * r + i] : make_uint4(0, 0, 0, 0);
            float dsl[4], dml[4], dsh[4], dmh[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float dd = qg_half_lo(hdr[r].x), dm = qg_half_hi(hdr[r].x);
                const QgScales sc = qg_q4k_scales(hdr[r].y, hdr[r].z, hdr[r].w);
                const int sh = 16 * (s >> 1);  // byte pair (2g, 2g+1) within the word
                const uint32_t scw = (t == 0 ? sc.sc03 : sc.sc47) >> sh;
                const uint32_t mw = (t == 0 ? sc.m03 : sc.m47) >> sh;
                dsl[r] = dd * qg_ub0(scw);
                dsh[r] = dd * qg_ub1(scw) * 0.0625f;
                dml[r] = dm * qg_ub0(mw);
                dmh[r] = dm * qg_ub1(mw);
            }
            const int64_t kb = 256 * (int64_t)b + 64 * g + 16 * h;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                qg_h8 B[C];
#pragma unroll
                for (int c = 0; c < C; ++c) B[c] = x8(xcol[c], kb + 4 * u, cok[c]);
                const uint32_t qu[4] = {(&q[0].x)[u], (&q[1].x)[u], (&q[2].x)[u], (&q[3].x)[u]};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // m-term of a dequantized weight is -dmin*m even for q = 0; rows past the
                    // tile end load zero headers and so contribute exact zeros.
                    const qg_h8 A = dequant8(qu[r], dsl[r], dml[r], dsh[r], dmh[r]);
#pragma unroll
                    for (int c = 0; c < C; ++c) D[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[c], D[r][c], 0, 0, 0);
                }
            }
        }
    }

    // D[r][c] element e of lane (i, s): row 16r + 4s + e, column 16c + i.
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

    if (P.splits == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int lr = 16 * r + 4 * s + e;
                    const int n = 16 * c + i;
                    if (lr < rt && n < P.N) P.Y[(int64_t)n * P.ldy + tile * qg::kTileRows + lr] = D[r][c][e];
                }
        return;
    }
    const int NP = 16 * C;  // partial columns per split
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int lr = 16 * r + 4 * s + e;
                const int n = 16 * c + i;
                if (lr < rt && n < P.N)
                    part[((int64_t)ks * NP + n) * P.M + tile * qg::kTileRows + lr] = D[r][c][e];
            }
    __threadfence();
    const uint32_t old = qg_ticket(cnt + tile, lane);
    if (old != (uint32_t)(P.splits - 1)) return;
    __threadfence();
    // lane = row of the tile; loop over columns
    if (lane < rt) {
        const int row = tile * qg::kTileRows + lane;
        for (int n = 0; n < P.N; ++n) {
            float v = 0.f;
            for (int j = 0; j < P.splits; ++j) v += __builtin_nontemporal_load(&part[((int64_t)j * NP + n) * P.M + row]);
            P.Y[(int64_t)n * P.ldy + row] = v;
        }
    }
    qg_ticket_reset(cnt + tile, lane);
}

// ------------------------------------------------------------------ host side
struct SnPlan {
    int W = 2;
    int64_t part_floats = 0;
};

void plan_sn(SnProb& P, SnPlan* pl) {
    const bool mfma = P.N > 8;
    int W = mfma ? 1 : 2, wpt = 0, ew = 0, es = 0;
    if (qg::env_pair(mfma ? "QG_SNM_CFG" : "QG_SNV_CFG", &ew, &es) && (ew == 1 || ew == 2 || ew == 4 || ew == 8) && es >= 1) {
        W = ew;
        wpt = es;
    }
    if (!wpt) wpt = (int)qg::ceil_div(mfma ? 1024 : 2048, P.tiles);
    wpt = std::max(1, std::min(wpt, P.nb));
    int splits = std::max(1, std::min((int)qg::ceil_div(wpt, W), P.nb));
    if (P.tiles > qg::kCounterSlots) splits = 1;
    P.splits = splits;
    pl->W = W;
    const int ncols = mfma ? (P.N > 16 ? 32 : 16) : P.N;
    pl->part_floats = splits > 1 ? (int64_t)splits * ncols * P.M : 0;
}

size_t sn_ws_bytes(const SnPlan& pl) {
    if (!pl.part_floats) return 0;
    return (size_t)QG_WORKSPACE_COUNTER_BYTES + qg::align_up((size_t)pl.part_floats * 4, 256);
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
    P.tiles = (int32_t)qg::ceil_div(M, qg::kTileRows);
    return P;
}

template <int N>
void launch_valu(const SnProb& P, int W, float* part, uint32_t* cnt, hipStream_t s) {
    const dim3 grid(P.tiles * P.splits);
    switch (W) {
        case 1: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 1>), grid, dim3(64), 0, s, P, part, cnt); break;
        case 2: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 2>), grid, dim3(128), 0, s, P, part, cnt); break;
        case 4: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 4>), grid, dim3(256), 0, s, P, part, cnt); break;
        default: hipLaunchKernelGGL((q4k_smalln_valu_kernel<N, 8>), grid, dim3(512), 0, s, P, part, cnt); break;
    }
}

template <int C>
void launch_mfma(const SnProb& P, int W, float* part, uint32_t* cnt, hipStream_t s) {
    const dim3 grid(P.tiles * P.splits);
    switch (W) {
        case 1: hipLaunchKernelGGL((q4k_smalln_mfma_kernel<C, 1>), grid, dim3(64), 0, s, P, part, cnt); break;
        case 2: hipLaunchKernelGGL((q4k_smalln_mfma_kernel<C, 2>), grid, dim3(128), 0, s, P, part, cnt); break;
        default: hipLaunchKernelGGL((q4k_smalln_mfma_kernel<C, 4>), grid, dim3(256), 0, s, P, part, cnt); break;
    }
}

}  // namespace

extern "C" {

size_t qgemm_q4k_smalln_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || M > INT32_MAX || K < 256 || K % 256 || K > (1 << 24) || N < 1 || N > QG_SMALLN_MAX) return 0;
    SnProb P = make_sn(nullptr, nullptr, K, nullptr, M, M, K, N);
    SnPlan pl;
    plan_sn(P, &pl);
    return sn_ws_bytes(pl);
}

int qgemm_q4k_smalln(const void* w, const float* X, int64_t ldx, float* Y, int64_t ldy, int64_t M, int64_t K,
                     int64_t N, void* ws, size_t ws_bytes, qg_stream_t stream) {
    qg::clear_error();
    int st = sn_validate(w, X, ldx, Y, ldy, M, K, N);
    if (st) return st;
    SnProb P = make_sn(w, X, ldx, Y, ldy, M, K, N);
    SnPlan pl;
    plan_sn(P, &pl);
    const size_t need = sn_ws_bytes(pl);
    if (need) {
        if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
        if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
        if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    }
    st = qg::check_device();
    if (st) return st;
    uint32_t* cnt = (uint32_t*)ws;
    float* part = need ? (float*)((uint8_t*)ws + QG_WORKSPACE_COUNTER_BYTES) : nullptr;
    hipStream_t s = (hipStream_t)stream;
    switch (P.N) {
        case 1: launch_valu<1>(P, pl.W, part, cnt, s); break;
        case 2: launch_valu<2>(P, pl.W, part, cnt, s); break;
        case 3: launch_valu<3>(P, pl.W, part, cnt, s); break;
        case 4: launch_valu<4>(P, pl.W, part, cnt, s); break;
        case 5: launch_valu<5>(P, pl.W, part, cnt, s); break;
        case 6: launch_valu<6>(P, pl.W, part, cnt, s); break;
        case 7: launch_valu<7>(P, pl.W, part, cnt, s); break;
        case 8: launch_valu<8>(P, pl.W, part, cnt, s); break;
        default:
            if (P.N <= 16)
                launch_mfma<1>(P, pl.W, part, cnt, s);
            else
                launch_mfma<2>(P, pl.W, part, cnt, s);
            break;
    }
    return qg::launch_status("qgemm_q4k_smalln");
}

}  // extern "C"
