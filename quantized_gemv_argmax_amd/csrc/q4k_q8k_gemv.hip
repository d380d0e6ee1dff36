// Q4_K GEMV against int8 activations (Q8_K-style input quantization), for gfx950.
//
// Method (dotLLM README, news entries on Q8_1 / Q8_K input quantization: a float32
// scale per 256-element block and precomputed block sums, feeding fused K-quant
// dot products; the "scale x int" dot product of Key Features taken literally).
// The activations are quantized once per vector, per super-block b:
//     d_b = max|x| / 127,  q_k = round-half-even(x_k / d_b),  bsums_i = sum of 16 q,
// and the product of row r is
//     y_r = sum_b d_b * ( d * sum_j sc_j * S_j  -  dmin * sum_j m_j * B_j ),
//     S_j = sum_l w4_{j,l} q_{32j+l}  (integer),  B_j = bsums_{2j} + bsums_{2j+1},
// with everything inside the parentheses but the two float scales exact integers.
//
// Quantized activation buffer (qg_q8k_bytes(K) bytes, nb = K / 256):
//     float d[nb] at 0;  int8 q[K] at q_off = align16(4 nb);
//     int16 bsums[K / 16] at b_off = align16(q_off + K).
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

struct Q8kLayout {
    size_t q_off, b_off, total;
};
Q8kLayout q8k_layout(int64_t K) {
    const size_t nb = (size_t)(K / 256);
    Q8kLayout L;
    L.q_off = qg::align_up(4 * nb, 16);
    L.b_off = qg::align_up(L.q_off + (size_t)K, 16);
    L.total = qg::align_up(L.b_off + 2 * (size_t)(K / 16), 16);
    return L;
}

struct XqArgs {
    const float* d;
    const int8_t* q;
    const int16_t* bsums;
};

// One wavefront per 256-element block, four per workgroup.
__global__ __launch_bounds__(256) void q8k_quantize_kernel(const float* __restrict__ x, int nb, float* __restrict__ d,
                                                           int8_t* __restrict__ q, int16_t* __restrict__ bsums) {
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (b >= nb) return;  // whole wavefronts
    const float4 v = reinterpret_cast<const float4*>(x + 256 * (size_t)b)[lane];
    float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
    const float db = __fdiv_rn(am, 127.0f);
    auto qz = [db](float e) -> int {
        if (db == 0.f) return 0;
        const float r = rintf(__fdiv_rn(e, db));
        return (int)fminf(fmaxf(r, -127.f), 127.f);
    };
    const int q0 = qz(v.x), q1 = qz(v.y), q2 = qz(v.z), q3 = qz(v.w);
    reinterpret_cast<uint32_t*>(q + 256 * (size_t)b)[lane] =
        (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
    // lanes 4i .. 4i+3 hold elements 16i .. 16i+15
    int s = q0 + q1 + q2 + q3;
    s += __builtin_amdgcn_mov_dpp(s, 0xb1, 0xf, 0xf, true);  // quad_perm [1,0,3,2]
    s += __builtin_amdgcn_mov_dpp(s, 0x4e, 0xf, 0xf, true);  // quad_perm [2,3,0,1]
    if ((lane & 3) == 0) bsums[16 * (size_t)b + (lane >> 2)] = (int16_t)s;
    if (lane == 0) d[b] = db;
}

struct SbIn8 {
    uint4 s[9];
    uint2 xl, xh;   // this lane's activations: low run, high run
    float dx;
    uint4 bs0, bs1;  // the super-block's 16 block sums
};

QG_DEV void load_sb8(SbIn8& v, const uint4* __restrict__ seg, const XqArgs& xa, int lo_off, int b, int rt) {
    const int8_t* xb = xa.q + 256 * (size_t)b + lo_off;
    v.xl = *reinterpret_cast<const uint2*>(xb);
    v.xh = *reinterpret_cast<const uint2*>(xb + 32);
    v.dx = xa.d[b];
    const uint4* bs = reinterpret_cast<const uint4*>(xa.bsums + 16 * (size_t)b);
    v.bs0 = bs[0];
    v.bs1 = bs[1];
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
    const uint32_t bsw[8] = {v.bs0.x, v.bs0.y, v.bs0.z, v.bs0.w, v.bs1.x, v.bs1.y, v.bs1.z, v.bs1.w};
    int it = 0, mn = 0;  // exact: |it| < 2^25, |mn| < 2^21
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int scj = (int)((scw[j >> 2] >> (8 * (j & 3))) & 0xff);
        const int mj = (int)((mw[j >> 2] >> (8 * (j & 3))) & 0xff);
        it += scj * S[j];
        mn += mj * (lo16(bsw[j]) + hi16(bsw[j]));
    }
    return v.dx * fmaf(dd, (float)it, -dm * (float)mn);
}

struct Q48Args {
    const uint8_t* w;
    XqArgs xq;
    float* y;
    int32_t M, nb;
};

template <int W, int MODE>
__global__ __launch_bounds__(64 * W) void q4k_q8k_gemv_kernel(Q48Args P) {
    const int tile = blockIdx.x;
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
void launch(const Q48Args& a, int tiles, hipStream_t s) {
    if (a.nb <= 4 * W)
        hipLaunchKernelGGL((q4k_q8k_gemv_kernel<W, 0>), dim3(tiles), dim3(64 * W), 0, s, a);
    else
        hipLaunchKernelGGL((q4k_q8k_gemv_kernel<W, 2>), dim3(tiles), dim3(64 * W), 0, s, a);
}

bool k_ok(int64_t K) { return K >= 256 && K % 256 == 0 && K <= (1 << 24); }

}  // namespace

extern "C" {

size_t qg_q8k_bytes(int64_t K) { return k_ok(K) ? q8k_layout(K).total : 0; }

int qg_quantize_q8k(const float* x, int64_t K, void* xq, qg_stream_t stream) {
    qg::clear_error();
    if (!x || !xq) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (!k_ok(K)) return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (!qg::aligned16(x) || !qg::aligned16(xq)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const Q8kLayout L = q8k_layout(K);
    const uint8_t* x8 = (const uint8_t*)x;
    const uint8_t* q8 = (const uint8_t*)xq;
    if (x8 < q8 + L.total && q8 < x8 + 4 * K) return qg::fail(QG_ERR_SHAPE, "x and xq overlap");
    int st = qg::check_device();
    if (st) return st;
    const int nb = (int)(K / 256);
    uint8_t* b = (uint8_t*)xq;
    hipLaunchKernelGGL(q8k_quantize_kernel, dim3((unsigned)qg::ceil_div(nb, 4)), dim3(256), 0, (hipStream_t)stream, x,
                       nb, (float*)b, (int8_t*)(b + L.q_off), (int16_t*)(b + L.b_off));
    return qg::launch_status("qg_quantize_q8k");
}

size_t qgemv_q4k_q8k_workspace_bytes(int64_t M, int64_t K) {
    (void)M;
    (void)K;
    return 0;
}

int qgemv_q4k_q8k(const void* w, const void* xq, float* y, int64_t M, int64_t K, void* ws, size_t ws_bytes,
                  qg_stream_t stream) {
    (void)ws;
    (void)ws_bytes;
    qg::clear_error();
    if (!w || !xq || !y) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX - T) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (!k_ok(K)) return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (!qg::aligned16(w) || !qg::aligned16(xq) || !qg::aligned16(y))
        return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    int st = qg::check_device();
    if (st) return st;
    const Q8kLayout L = q8k_layout(K);
    const uint8_t* b = (const uint8_t*)xq;
    Q48Args a{(const uint8_t*)w, {(const float*)b, (const int8_t*)(b + L.q_off), (const int16_t*)(b + L.b_off)}, y,
              (int32_t)M, (int32_t)(K / 256)};
    int W = 1;
    while (W < 4 && 4 * W < a.nb) W *= 2;
    int ew = 0, eu = 0;
    if (qg::env_pair("QG_Q4K8_CFG", &ew, &eu) && (ew == 1 || ew == 2 || ew == 4 || ew == 8)) W = ew;
    const int tiles = (int)qg::ceil_div(M, T);
    hipStream_t s = (hipStream_t)stream;
    switch (W) {
        case 1: launch<1>(a, tiles, s); break;
        case 2: launch<2>(a, tiles, s); break;
        case 4: launch<4>(a, tiles, s); break;
        default: launch<8>(a, tiles, s); break;
    }
    return qg::launch_status("qgemv_q4k_q8k");
}

}  // extern "C"
