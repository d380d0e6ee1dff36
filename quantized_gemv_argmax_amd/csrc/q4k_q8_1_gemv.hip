// Q4_K GEMV against int8 activations (Q8_1-style input quantization), for gfx950.
//
// Method (dotLLM README, news entries on Q8_1 / Q8_K input quantization: a float32
// scale per block of activations with precomputed block sums, feeding fused
// K-quant dot products; the "scale x int" dot product of Key Features taken
// literally). The activations are quantized once per vector, per block c of 32
// (one block per Q4_K sub-block):
//     d_c = max|x| / 127,  q_k = round-half-even(x_k / d_c),  s_c = sum of the 32 q,
// and the product of row r over super-block b (sub-blocks j, blocks c = 8b + j) is
//     y_r += d * sum_j d_c sc_j S_j  -  dmin * sum_j d_c m_j s_c,
//     S_j = sum_l w4_{j,l} q_{32c+l}  (an exact integer).
// A scale per 256 activations (the Q8_K block) was measured to push the
// quantization error past 1e-3 * sum|w x| on some rows at K = 3584; per 32 it
// stays below 0.63 of it.
//
// Quantized activation buffer (qg_q8_1_bytes(K) bytes, nc = K / 32):
//     float d[nc] at 0;  int8 q[K] at q_off = align16(4 nc);
//     int16 s[nc] at s_off = align16(q_off + K).
//
// GEMV: the tile, K-group and pipeline structure of the fp32-activation Q4_K
// kernel on the same packed weights. Each lane holds 16 int8 activations of its
// slot (8 of a low-nibble sub-block, 8 of the matching high-nibble one); per
// quant dword, two masks give eight unsigned 4-bit quants as bytes and two
// v_dot4c_i32_i8 with the DPP row broadcast add four products each: per 8 weights
// 3 bit operations and 2 dot operations, against 5 and 4 with fp16 activations.
#include <algorithm>
#include <cstdlib>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;

struct Q81Layout {
    size_t q_off, s_off, total;
};
Q81Layout q81_layout(int64_t K) {
    const size_t nc = (size_t)(K / 32);
    Q81Layout L;
    L.q_off = qg::align_up(4 * nc, 16);
    L.s_off = qg::align_up(L.q_off + (size_t)K, 16);
    L.total = qg::align_up(L.s_off + 2 * nc, 16);
    return L;
}

struct XqArgs {
    const float* d;
    const int8_t* q;
    const int16_t* s;
};

// One wavefront per 256 activations of one column (eight blocks: lanes 8c ..
// 8c+7 hold block c), four per workgroup; column n reads x + n * ldx and writes
// the buffer at xq + n * xqb (q at q_off, sums at s_off within it).
__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float* __restrict__ x, int64_t ldx, int n256,
                                                            int N, uint8_t* __restrict__ xq, int64_t xqb,
                                                            int32_t q_off, int32_t s_off) {
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (gw >= n256 * N) return;  // whole wavefronts
    const int n = gw / n256, b = gw - n * n256;
    uint8_t* out = xq + (int64_t)n * xqb;
    float* d = reinterpret_cast<float*>(out);
    int8_t* q = reinterpret_cast<int8_t*>(out + q_off);
    int16_t* s = reinterpret_cast<int16_t*>(out + s_off);
    const float4 v = reinterpret_cast<const float4*>(x + (int64_t)n * ldx + 256 * (int64_t)b)[lane];
    float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    // maximum over the eight lanes of the block: quad swaps, then the 8-lane mirror
    am = fmaxf(am, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, am), 0xb1, 0xf, 0xf, true)));
    am = fmaxf(am, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, am), 0x4e, 0xf, 0xf, true)));
    am = fmaxf(am, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, am), 0x141, 0xf, 0xf, true)));
    const float dc = __fdiv_rn(am, 127.0f);
    auto qz = [dc](float e) -> int {
        if (dc == 0.f) return 0;
        const float r = rintf(__fdiv_rn(e, dc));
        return (int)fminf(fmaxf(r, -127.f), 127.f);
    };
    const int q0 = qz(v.x), q1 = qz(v.y), q2 = qz(v.z), q3 = qz(v.w);
    reinterpret_cast<uint32_t*>(q + 256 * (size_t)b)[lane] =
        (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
    int t = q0 + q1 + q2 + q3;
    t += __builtin_amdgcn_mov_dpp(t, 0xb1, 0xf, 0xf, true);
    t += __builtin_amdgcn_mov_dpp(t, 0x4e, 0xf, 0xf, true);
    t += __builtin_amdgcn_mov_dpp(t, 0x141, 0xf, 0xf, true);
    if ((lane & 7) == 0) {
        const size_t c = 8 * (size_t)b + (lane >> 3);
        d[c] = dc;
        s[c] = (int16_t)t;
    }
}

struct SbIn8 {
    uint4 s[9];
    uint2 xl, xh;  // this lane's activations: low run, high run
    float4 d0, d1;  // the super-block's eight block scales
    uint4 bs;       // and eight block sums (int16)
};

QG_DEV void load_sb8(SbIn8& v, const uint4* __restrict__ seg, const XqArgs& xa, int lo_off, int b, int rt) {
    const int8_t* xb = xa.q + 256 * (size_t)b + lo_off;
    v.xl = *reinterpret_cast<const uint2*>(xb);
    v.xh = *reinterpret_cast<const uint2*>(xb + 32);
    const float4* dp = reinterpret_cast<const float4*>(xa.d + 8 * (size_t)b);
    v.d0 = dp[0];
    v.d1 = dp[1];
    v.bs = *reinterpret_cast<const uint4*>(xa.s + 8 * (size_t)b);
    const uint4* sb = seg + (size_t)b * 9 * rt;
#pragma unroll
    for (int s = 0; s < 9; ++s) v.s[s] = qg_stream_load(sb + s * rt);
}

QG_DEV int lo16(uint32_t w) { return (int)(int16_t)(w & 0xffffu); }
QG_DEV int hi16(uint32_t w) { return (int)(int16_t)(w >> 16); }

QG_DEV float sb_dot8(const SbIn8& v) {
    const uint32_t x[4] = {v.xl.x, v.xl.y, v.xh.x, v.xh.y};
    int S[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        int lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0;
        switch (g) {
            case 0:
                qg_q4_seg_dot_i8<0, 1>(lo0, hi0, lo1, hi1, v.s[1], x);
                qg_q4_seg_dot_i8<2, 3>(lo0, hi0, lo1, hi1, v.s[2], x);
                break;
            case 1:
                qg_q4_seg_dot_i8<4, 5>(lo0, hi0, lo1, hi1, v.s[3], x);
                qg_q4_seg_dot_i8<6, 7>(lo0, hi0, lo1, hi1, v.s[4], x);
                break;
            case 2:
                qg_q4_seg_dot_i8<8, 9>(lo0, hi0, lo1, hi1, v.s[5], x);
                qg_q4_seg_dot_i8<10, 11>(lo0, hi0, lo1, hi1, v.s[6], x);
                break;
            default:
                qg_q4_seg_dot_i8<12, 13>(lo0, hi0, lo1, hi1, v.s[7], x);
                qg_q4_seg_dot_i8<14, 15>(lo0, hi0, lo1, hi1, v.s[8], x);
                break;
        }
        S[2 * g] = lo0 + lo1;
        S[2 * g + 1] = hi0 + hi1;
    }
    const uint4 hd = v.s[0];
    const float dd = qg_half_lo(hd.x), dm = qg_half_hi(hd.x);
    const QgScales sc = qg_q4k_scales(hd.y, hd.z, hd.w);
    const uint32_t scw[2] = {sc.sc03, sc.sc47}, mw[2] = {sc.m03, sc.m47};
    const float dc[8] = {v.d0.x, v.d0.y, v.d0.z, v.d0.w, v.d1.x, v.d1.y, v.d1.z, v.d1.w};
    const uint32_t sw[4] = {v.bs.x, v.bs.y, v.bs.z, v.bs.w};
    float t = 0.f, u = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int scj = (int)((scw[j >> 2] >> (8 * (j & 3))) & 0xff);
        const int mj = (int)((mw[j >> 2] >> (8 * (j & 3))) & 0xff);
        const int sj = (j & 1) ? hi16(sw[j >> 1]) : lo16(sw[j >> 1]);
        t = fmaf(dc[j], (float)(scj * S[j]), t);  // |sc S| < 2^22: exact in fp32
        u = fmaf(dc[j], (float)(mj * sj), u);
    }
    return fmaf(dd, t, -dm * u);
}

struct Q81Prob {
    const uint8_t* w;
    XqArgs xq;
    float* y;
    int32_t M, nb, wg_begin;
};

// Up to QG_MAX_BATCH problems in one grid; a workgroup finds its problem from the
// compact array of first tiles.
struct Q81Args {
    int32_t begin[QG_MAX_BATCH];
    int32_t count;
    Q81Prob p[QG_MAX_BATCH];
};

template <int W, int MODE>
__global__ __launch_bounds__(64 * W) void q4k_q8_1_gemv_kernel(Q81Args A) {
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < A.count && (int)blockIdx.x >= A.begin[i]) k = i;
    const Q81Prob P = A.p[k];
    const int tile = blockIdx.x - P.wg_begin;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    const int rt = min(T, P.M - tile * T);
    const int i = lane & 15;
    const int kg = 4 * wave + (lane >> 4);
    constexpr int G = 4 * W;
    // activation slot: quant segment p = i/2 of group g = p/2, bytes 8(i%2) .. +7
    const int p = i >> 1;
    const int lo_off = 64 * (p >> 1) + 16 * (p & 1) + 8 * (i & 1);
    const uint4* __restrict__ seg =
        reinterpret_cast<const uint4*>(P.w + (size_t)tile * T * nb * 144) + min(i, rt - 1);

    float acc = 0.f;
    if constexpr (MODE == 0) {
        SbIn8 b0;
        load_sb8(b0, seg, P.xq, lo_off, min(kg, nb - 1), rt);
        const float v0 = sb_dot8(b0);
        acc = (kg < nb) ? v0 : 0.f;
    } else {
        const int niter = (nb + G - 1) / G;
        SbIn8 b0, b1;
        load_sb8(b0, seg, P.xq, lo_off, min(kg, nb - 1), rt);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            load_sb8(b1, seg, P.xq, lo_off, min(kg + G * (it + 1), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            const float v0 = sb_dot8(b0);
            acc += (kg + G * it < nb) ? v0 : 0.f;
            load_sb8(b0, seg, P.xq, lo_off, min(kg + G * (it + 2), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            const float v1 = sb_dot8(b1);
            acc += (kg + G * (it + 1) < nb) ? v1 : 0.f;
        }
        if (it < niter) {
            const float v0 = sb_dot8(b0);
            acc += (kg + G * it < nb) ? v0 : 0.f;
        }
    }
    float v = qg_sum_rows4(acc);
    if constexpr (W > 1) {
        __shared__ float red[W][T];
        if (lane < T) red[wave][lane] = v;
        __syncthreads();
        if (wave != 0) return;
        if (lane < T) {
            v = red[0][lane];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w][lane];
        }
    }
    if (lane < rt) P.y[tile * T + lane] = v;
}

template <int W>
void launch(const Q81Args& a, int tiles, int nb_max, hipStream_t s) {
    if (nb_max <= 4 * W)
        hipLaunchKernelGGL((q4k_q8_1_gemv_kernel<W, 0>), dim3(tiles), dim3(64 * W), 0, s, a);
    else
        hipLaunchKernelGGL((q4k_q8_1_gemv_kernel<W, 2>), dim3(tiles), dim3(64 * W), 0, s, a);
}

bool k_ok(int64_t K) { return K >= 256 && K % 256 == 0 && K <= (1 << 24); }

}  // namespace

void qg::q8_1_offsets(int64_t K, size_t* q_off, size_t* s_off) {
    const Q81Layout L = q81_layout(K);
    *q_off = L.q_off;
    *s_off = L.s_off;
}

extern "C" {

size_t qg_q8_1_bytes(int64_t K) { return k_ok(K) ? q81_layout(K).total : 0; }

qg_status qg_quantize_q8_1_columns(const float* X, int64_t ldx, int64_t K, int64_t N, void* xq, qg_stream_t stream) {
    qg::clear_error();
    if (!X || !xq) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (!k_ok(K)) return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (N < 1 || N > QG_SMALLN_MAX) return qg::fail(QG_ERR_SHAPE, "N=%lld not in [1, %d]", (long long)N, QG_SMALLN_MAX);
    if (N > 1 && (ldx < K || ldx % 4 || (N - 1) * ldx + K > (int64_t)1 << 29))
        return qg::fail(QG_ERR_SHAPE, "ldx=%lld must be a multiple of 4, >= K, with (N-1)*ldx + K < 2^29",
                        (long long)ldx);
    if (!qg::aligned16(X) || !qg::aligned16(xq)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const Q81Layout L = q81_layout(K);
    const uint8_t* x8 = (const uint8_t*)X;
    const uint8_t* q8 = (const uint8_t*)xq;
    const int64_t xspan = 4 * ((N - 1) * (N > 1 ? ldx : 0) + K);
    if (x8 < q8 + N * L.total && q8 < x8 + xspan) return qg::fail(QG_ERR_SHAPE, "X and xq overlap");
    qg_status st = qg::check_device();
    if (st) return st;
    const int n256 = (int)(K / 256);
    hipLaunchKernelGGL(q8_1_quantize_kernel, dim3((unsigned)qg::ceil_div((int64_t)n256 * N, 4)), dim3(256), 0,
                       (hipStream_t)stream, X, N > 1 ? ldx : 0, n256, (int)N, (uint8_t*)xq, (int64_t)L.total,
                       (int32_t)L.q_off, (int32_t)L.s_off);
    return qg::launch_status("qg_quantize_q8_1");
}

qg_status qg_quantize_q8_1(const float* x, int64_t K, void* xq, qg_stream_t stream) {
    return qg_quantize_q8_1_columns(x, K, K, 1, xq, stream);
}

qg_status qgemv_q4k_q8_1_batch(const qg_gemv_q8_1_problem* pr, int count, qg_stream_t stream) {
    qg::clear_error();
    if (!pr) return qg::fail(QG_ERR_NULL, "problem list is NULL");
    if (count < 1 || count > QG_MAX_BATCH)
        return qg::fail(QG_ERR_SHAPE, "batch count %d not in [1, %d]", count, QG_MAX_BATCH);
    Q81Args a{};
    int tiles = 0, nb_max = 1;
    for (int i = 0; i < count; ++i) {
        const qg_gemv_q8_1_problem& p = pr[i];
        if (!p.w_packed || !p.xq || !p.y) return qg::fail(QG_ERR_NULL, "problem %d: NULL pointer", i);
        if (p.M < 1 || p.M > INT32_MAX - T) return qg::fail(QG_ERR_SHAPE, "problem %d: M=%lld out of range", i, (long long)p.M);
        if (!k_ok(p.K))
            return qg::fail(QG_ERR_SHAPE, "problem %d: K=%lld must be a positive multiple of 256 (<= 2^24)", i, (long long)p.K);
        if (!qg::aligned16(p.w_packed) || !qg::aligned16(p.xq) || !qg::aligned16(p.y))
            return qg::fail(QG_ERR_ALIGN, "problem %d: pointers must be 16-byte aligned", i);
        const Q81Layout L = q81_layout(p.K);
        const uint8_t* b = (const uint8_t*)p.xq;
        Q81Prob& P = a.p[i];
        P.w = (const uint8_t*)p.w_packed;
        P.xq = XqArgs{(const float*)b, (const int8_t*)(b + L.q_off), (const int16_t*)(b + L.s_off)};
        P.y = p.y;
        P.M = (int32_t)p.M;
        P.nb = (int32_t)(p.K / 256);
        P.wg_begin = tiles;
        a.begin[i] = tiles;
        const int64_t t = qg::ceil_div(p.M, T);
        if ((int64_t)tiles + t > INT32_MAX / 2) return qg::fail(QG_ERR_SHAPE, "batch too large");
        tiles += (int)t;
        nb_max = std::max(nb_max, (int)P.nb);
    }
    a.count = count;
    qg_status st = qg::check_device();
    if (st) return st;
    int W = 1;
    while (W < 4 && 4 * W < nb_max) W *= 2;
    if (qg::launch_override().gemv_waves) W = qg::launch_override().gemv_waves;
    hipStream_t s = (hipStream_t)stream;
    switch (W) {
        case 1: launch<1>(a, tiles, nb_max, s); break;
        case 2: launch<2>(a, tiles, nb_max, s); break;
        case 4: launch<4>(a, tiles, nb_max, s); break;
        default: launch<8>(a, tiles, nb_max, s); break;
    }
    return qg::launch_status("qgemv_q4k_q8_1");
}

qg_status qgemv_q4k_q8_1(const void* w, const void* xq, float* y, int64_t M, int64_t K, qg_stream_t stream) {
    qg_gemv_q8_1_problem p{w, xq, y, M, K};
    return qgemv_q4k_q8_1_batch(&p, 1, stream);
}

}  // extern "C"
