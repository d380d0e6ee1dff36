// Q6_K weight-only GEMV for gfx950 (CDNA4), plus the Q6_K load-time repack.
//
// Method (dotLLM README: the CUDA backend's custom quantized decode GEMV, which
// names Q6_K beside Q8_0 and Q4_K, and the "Q4_K_M dequantization and vec_dot
// kernels" entry, which lists Q6_K among the K-quant formats with a fused dot).
// The block reading is the GGUF one: a super-block of 256 weights holds 128 bytes
// of low nibbles ql, 64 bytes of two-bit high parts qh, sixteen int8 sub-scales
// and an fp16 d, and weight k of sub-block j = k / 16 is d * sc_j * (q_k - 32)
// with the six-bit q_k. In half h (weights 128h..128h+127), for l < 32 and
// p < 4, weight 128h + 32p + l takes its low four bits from ql byte
// 64h + 32(p % 2) + l (low nibble for p < 2, high nibble otherwise) and its top
// two bits from bits 2p, 2p+1 of qh byte 32h + l. For row r and super-block b,
//     y_r += d * sum_j sc_j * (S_j - 32 X_j),
//     S_j = sum_l q_{j,l} x_{256b+16j+l},   X_j = sum_l x_{256b+16j+l},
// the per-sub-block activation sums carrying the -32 offset, as the mins of Q4_K.
//
// Packed layout (a same-size byte permutation of the canonical row-major block
// stream). Rows are grouped in tiles of 16. The first 208 bytes of a super-block
// are 13 sixteen-byte segments (0..7: ql bytes 16s.., 8..11: qh bytes
// 16(s-8).., 12: the sub-scales), the last 2 bytes its d. Within a tile of rt rows,
//     segment s of super-block b of row i:  tile_base + ((b * 13 + s) * rt + i) * 16,
//     d of super-block b of row i:          tile_base + nb * 13 * rt * 16 + (b * rt + i) * 2,
// with tile_base = tile * 16 * nb * 210.
//
// Work decomposition as for Q4_K: a 16-lane DPP row is a K-group walking its own
// super-blocks for the 16 rows of the tile (lane i = weight row i), a workgroup of
// W wavefronts owns one tile and all of K, and the 4W K-groups meet through
// cross-row shuffles and LDS in a fixed order.
//
// Inner product. Lane i of a K-group holds the activations of ql segment s = i/2,
// dwords 2(i%2), 2(i%2)+1: eight of the low-nibble run (weights 128h + 32pp + 16c
// + 8(i%2) + 0..7 with s = 4h + 2pp + c) and the eight of the high-nibble run 64
// weights further on, as fp16 pairs broadcast by DPP to the 16 rows. The six-bit
// quants are assembled in place with one bit-field insert per four weights and
// masked to fp16 subnormals q * 2^-24 (qg_q6_seg_dot); one segment call yields
// S_j of two sub-blocks. The 2^24 factor and the -32 offset are applied per
// super-block, with activation sums taken over the same fp16 values, so fp16
// rounding of x changes each product by at most 2^-11 relative (x in the fp16
// normal range); accumulation is fp32.
#include <algorithm>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;
constexpr int kSegs = 13;        // sixteen-byte segments per super-block
constexpr int kBlockBytes = 210;

struct Q6Args {
    const uint8_t* w;
    const float* x;
    float* y;
    int32_t M, nb;
};

struct Q6In {
    uint4 s[kSegs];
    uint32_t d;               // fp16 bits in the low half
    float4 xa, xb, xc, xd;    // low run dwords 0, 1, then high run dwords 0, 1
};

// Raw buffer loads: one resource for the tile and one for x, a per-lane byte
// offset, the segment and activation offsets as scalar operands.
struct Q6Src {
    __amdgpu_buffer_rsrc_t w, x;
    uint32_t vrow, vd, vx;  // this lane's row in the segments / in the d region, its x slot
};

QG_DEV void load_q6(Q6In& v, const Q6Src& q, int b, int rt) {
    const uint32_t vxb = q.vx + (uint32_t)b * 1024u;
    v.xa = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(q.x, vxb, 0, 0));
    v.xb = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(q.x, vxb, 16, 0));
    v.xc = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(q.x, vxb, 256, 0));
    v.xd = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(q.x, vxb, 272, 0));
    const uint32_t vb = q.vrow + (uint32_t)b * (uint32_t)kSegs * (uint32_t)rt * 16u;
#pragma unroll
    for (int s = 0; s < kSegs; ++s) {
        const qg_u4v t = __builtin_amdgcn_raw_buffer_load_b128(q.w, vb, s * rt * 16, kQgNonTemporal);
        v.s[s] = make_uint4(t.x, t.y, t.z, t.w);
    }
    v.d = __builtin_amdgcn_raw_buffer_load_b16(q.w, q.vd + (uint32_t)b * (uint32_t)rt * 2u, 0, kQgNonTemporal);
}

QG_DEV float sc_i8(const uint4& sc, int j) {
    const uint32_t w = j < 4 ? sc.x : j < 8 ? sc.y : j < 12 ? sc.z : sc.w;
    return (float)(int8_t)(uint8_t)(w >> (8 * (j & 3)));
}

// Segment s of this super-block (ql segment s with its qh segment) into S[j_lo],
// S[j_lo + 4], j_lo = 8h + 2pp + c.
template <int S>
QG_DEV void q6_seg(float (&Sj)[16], const Q6In& v, const uint32_t (&x)[8], uint32_t m4) {
    constexpr int h = S >> 2, pp = (S >> 1) & 1, c = S & 1;
    constexpr int jlo = 8 * h + 2 * pp + c;
    float lo0 = 0.f, hi0 = 0.f, lo1 = 0.f, hi1 = 0.f;
    qg_q6_seg_dot<2 * S, 2 * S + 1, pp>(lo0, hi0, lo1, hi1, v.s[S], v.s[8 + 2 * h + c], x, m4);
    Sj[jlo] = lo0 + lo1;
    Sj[jlo + 4] = hi0 + hi1;
}

// Contribution of one super-block for this lane's row.
QG_DEV float q6_dot(const Q6In& v) {
    const uint32_t m4 = __builtin_amdgcn_readfirstlane(0x0F0F0F0Fu);
    const QgPairs8 xp = qg_cvt_pairs(v.xa, v.xc, v.xb, v.xd);
    // this lane holds 8 values of sub-block j_lo(s) and 8 of j_lo(s) + 4; the
    // lane pair 2s, 2s+1 holds all 16 of both
    // (the sums are taken over the same fp16 values the dot products use: low run
    // pairs 0, 1, 4, 5, high run pairs 2, 3, 6, 7)
    float slo = qg_sum_pairs4(xp.p[0], xp.p[1], xp.p[4], xp.p[5]);
    float shi = qg_sum_pairs4(xp.p[2], xp.p[3], xp.p[6], xp.p[7]);
    slo += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, slo), 0xb1, 0xf, 0xf, true));
    shi += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, shi), 0xb1, 0xf, 0xf, true));

    float Sj[16];
    q6_seg<0>(Sj, v, xp.p, m4);
    q6_seg<1>(Sj, v, xp.p, m4);
    q6_seg<2>(Sj, v, xp.p, m4);
    q6_seg<3>(Sj, v, xp.p, m4);
    q6_seg<4>(Sj, v, xp.p, m4);
    q6_seg<5>(Sj, v, xp.p, m4);
    q6_seg<6>(Sj, v, xp.p, m4);
    q6_seg<7>(Sj, v, xp.p, m4);

    const uint4 sc = v.s[12];
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaf(sc_i8(sc, j), Sj[j], a);
    // X_j from lane 2s: j_lo(s) = s + 4 (s / 4) from slo, j_lo(s) + 4 from shi
    float bx = sc_i8(sc, 0) * qg_bcast<0>(slo);
    bx = fmaf(sc_i8(sc, 1), qg_bcast<2>(slo), bx);
    bx = fmaf(sc_i8(sc, 2), qg_bcast<4>(slo), bx);
    bx = fmaf(sc_i8(sc, 3), qg_bcast<6>(slo), bx);
    bx = fmaf(sc_i8(sc, 4), qg_bcast<0>(shi), bx);
    bx = fmaf(sc_i8(sc, 5), qg_bcast<2>(shi), bx);
    bx = fmaf(sc_i8(sc, 6), qg_bcast<4>(shi), bx);
    bx = fmaf(sc_i8(sc, 7), qg_bcast<6>(shi), bx);
    bx = fmaf(sc_i8(sc, 8), qg_bcast<8>(slo), bx);
    bx = fmaf(sc_i8(sc, 9), qg_bcast<10>(slo), bx);
    bx = fmaf(sc_i8(sc, 10), qg_bcast<12>(slo), bx);
    bx = fmaf(sc_i8(sc, 11), qg_bcast<14>(slo), bx);
    bx = fmaf(sc_i8(sc, 12), qg_bcast<8>(shi), bx);
    bx = fmaf(sc_i8(sc, 13), qg_bcast<10>(shi), bx);
    bx = fmaf(sc_i8(sc, 14), qg_bcast<12>(shi), bx);
    bx = fmaf(sc_i8(sc, 15), qg_bcast<14>(shi), bx);
    const float d = qg_half_lo(v.d);
    // quants entered as q * 2^-24
    return d * fmaf(16777216.0f, a, -32.0f * bx);
}

// MODE 0: one super-block per K-group; 2: several, two register buffers
// (ping-pong prefetch over pairs of super-blocks, single-exit loop and
// unconditional clamped loads, as in the Q4_K kernel).
template <int W, int MODE>
__global__ __launch_bounds__(64 * W) void q6k_gemv_kernel(Q6Args P) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    const int rt = min(T, P.M - tile * T);
    const int i = lane & 15;
    const int kg = 4 * wave + (lane >> 4);
    constexpr int G = 4 * W;

    // activation slot of this lane: ql segment s = i/2 = 4h + 2pp + c, dwords 2(i%2), +1
    const int s = i >> 1;
    Q6Src src;
    src.vx = 4u * (uint32_t)(128 * (s >> 2) + 32 * ((s >> 1) & 1) + 16 * (s & 1) + 8 * (i & 1));
    // rows past a ragged tile's end re-read the last row; their results are dropped
    const uint32_t r = (uint32_t)min(i, rt - 1);
    src.w = __builtin_amdgcn_make_buffer_rsrc((void*)(P.w + (size_t)tile * T * nb * kBlockBytes), (short)0,
                                              rt * nb * kBlockBytes, kQgRawBufferFlags);
    src.x = __builtin_amdgcn_make_buffer_rsrc((void*)P.x, (short)0, nb * 1024, kQgRawBufferFlags);
    src.vrow = 16u * r;
    src.vd = (uint32_t)nb * kSegs * (uint32_t)rt * 16u + 2u * r;

    float acc = 0.f;
    if constexpr (MODE == 0) {
        Q6In b0;
        load_q6(b0, src, min(kg, nb - 1), rt);
        const float v0 = q6_dot(b0);
        acc = (kg < nb) ? v0 : 0.f;
    } else {
        const int niter = (nb + G - 1) / G;
        Q6In b0, b1;
        load_q6(b0, src, min(kg, nb - 1), rt);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            load_q6(b1, src, min(kg + G * (it + 1), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            const float v0 = q6_dot(b0);
            acc += (kg + G * it < nb) ? v0 : 0.f;
            load_q6(b0, src, min(kg + G * (it + 2), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            const float v1 = q6_dot(b1);
            acc += (kg + G * (it + 1) < nb) ? v1 : 0.f;
        }
        if (it < niter) {
            const float v0 = q6_dot(b0);
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

// One item per sixteen-byte segment or d value of the packed output. The
// canonical stream is only 2-byte aligned per block, so it is read as halfwords.
__global__ void q6k_pack_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t M, int nb) {
    const int64_t per_row = (int64_t)nb * (kSegs + 1);
    const int64_t items = M * per_row;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < items; o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = o / (T * per_row);
        const int64_t in = o - t * T * per_row;
        const int rt = (int)std::min<int64_t>(T, M - t * T);
        uint8_t* tb = dst + t * T * nb * kBlockBytes;
        const int64_t nseg = (int64_t)nb * kSegs * rt;
        if (in < nseg) {
            const int64_t bs = in / rt;  // b * 13 + s
            const int i = (int)(in - bs * rt);
            const int64_t b = bs / kSegs, s = bs - b * kSegs;
            const uint16_t* p = src + ((t * T + i) * nb * kBlockBytes + b * kBlockBytes + 16 * s) / 2;
            uint4 u;
            u.x = p[0] | ((uint32_t)p[1] << 16);
            u.y = p[2] | ((uint32_t)p[3] << 16);
            u.z = p[4] | ((uint32_t)p[5] << 16);
            u.w = p[6] | ((uint32_t)p[7] << 16);
            reinterpret_cast<uint4*>(tb)[in] = u;
        } else {
            const int64_t e = in - nseg;  // b * rt + i
            const int64_t b = e / rt;
            const int i = (int)(e - b * rt);
            reinterpret_cast<uint16_t*>(tb + nseg * 16)[e] = src[((t * T + i) * nb * kBlockBytes + b * kBlockBytes + 208) / 2];
        }
    }
}

int choose_w(int nb) {
    // enough K-groups that every super-block of a row has its own, up to 4 wavefronts
    int W = 1;
    while (W < 4 && 4 * W < nb) W *= 2;
    if (qg::launch_override().gemv_waves) W = qg::launch_override().gemv_waves;
    return W;
}

template <int W>
void launch(const Q6Args& a, int tiles, hipStream_t s) {
    if (a.nb <= 4 * W)
        hipLaunchKernelGGL((q6k_gemv_kernel<W, 0>), dim3(tiles), dim3(64 * W), 0, s, a);
    else
        hipLaunchKernelGGL((q6k_gemv_kernel<W, 2>), dim3(tiles), dim3(64 * W), 0, s, a);
}

}  // namespace

extern "C" {

size_t qg_q6k_bytes(int64_t M, int64_t K) {
    if (M < 1 || K < 256 || K % 256) return 0;
    return (size_t)M * (size_t)(K / 256) * (size_t)kBlockBytes;
}

// Every workgroup owns whole rows: no workspace.
qg_status qgemv_q6k(const void* w, const float* x, float* y, int64_t M, int64_t K, qg_stream_t stream) {
    qg::clear_error();
    if (!w || !x || !y) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX - T) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (!qg::aligned16(w) || !qg::aligned16(x) || !qg::aligned16(y))
        return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    qg_status st = qg::check_device();
    if (st) return st;
    Q6Args a{(const uint8_t*)w, x, y, (int32_t)M, (int32_t)(K / 256)};
    const int tiles = (int)qg::ceil_div(M, T);
    hipStream_t s = (hipStream_t)stream;
    switch (choose_w(a.nb)) {
        case 1: launch<1>(a, tiles, s); break;
        case 2: launch<2>(a, tiles, s); break;
        case 4: launch<4>(a, tiles, s); break;
        default: launch<8>(a, tiles, s); break;
    }
    return qg::launch_status("qgemv_q6k");
}

qg_status qg_pack_q6k(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream) {
    qg::clear_error();
    if (!src || !dst) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX || K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "invalid Q6_K shape M=%lld K=%lld", (long long)M, (long long)K);
    if (!qg::aligned16(src) || !qg::aligned16(dst)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t bytes = qg_q6k_bytes(M, K);
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    if (s8 < d8 + bytes && d8 < s8 + bytes) return qg::fail(QG_ERR_SHAPE, "src and dst overlap");
    qg_status st = qg::check_device();
    if (st) return st;
    const int64_t items = M * (K / 256) * (kSegs + 1);
    const int blocks = (int)std::min<int64_t>(qg::ceil_div(items, 256), 65536);
    hipLaunchKernelGGL(q6k_pack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint16_t*)src,
                       (uint8_t*)dst, M, (int)(K / 256));
    return qg::launch_status("qg_pack_q6k");
}

}  // extern "C"
