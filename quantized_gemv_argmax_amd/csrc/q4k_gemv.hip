// Q4_K weight-only GEMV for gfx950 (CDNA4), plus the Q4_K load-time repack.
//
// Method (dotLLM README: Key Features / Performance, "Quantized inference" with
// fused scale x int dot products run on the quantized blocks; news entries
// "Q4_K_M dequantization and vec_dot kernels" and the CUDA backend's "custom
// quantized GEMV for decode"): for row r and super-block b, with sub-block j of
// 32 weights,
//     y_r += d * sum_j sc_j * S_j  -  dmin * sum_j m_j * X_j,
//     S_j = sum_l q_{j,l} x_{256b+32j+l},   X_j = sum_l x_{256b+32j+l},
// which equals sum_k (d*sc*q - dmin*m) * x_k. The mins are applied through
// per-sub-block activation sums (the README's precomputed block sums).
//
// Packed layout (a same-size byte permutation of the canonical row-major block
// stream; the README's load-time row-interleaved repacking, sized for DPP rows):
// rows are grouped in tiles of 16. A super-block is 9 sixteen-byte segments
// (segment 0: d, dmin and the 12 scale bytes; segment 1+p: quant bytes
// 16p..16p+15). Within a tile of rt rows, segment s of super-block b of row i is at
//     tile_base + ((b * 9 + s) * rt + i) * 16,   tile_base = tile * 16 * nb * 144.
//
// Work decomposition. A wavefront is four 16-lane DPP rows; each DPP row is a
// "K-group" that walks its own super-blocks for the 16 rows of the tile (lane i of
// the DPP row = weight row i), so a segment load is one contiguous 256-byte run per
// K-group. A workgroup of W wavefronts owns one tile and all of K: its 4W K-groups
// take super-blocks kg, kg + 4W, ... and are summed at the end through cross-row
// shuffles and LDS, in a fixed order. No workgroup talks to another.
//
// Inner product. Each lane of a K-group loads 16 of the super-block's 256
// activations and converts them to eight fp16 pairs; v_dot2c_f32_f16 with a DPP
// row broadcast (row_newbcast) then feeds every lane the pair it needs from the
// lane that holds it, so activations cost no extra instruction per weight. The
// 4-bit quants are used in place as fp16 subnormals: masking a word with
// 0x000F000F leaves two quants q as the binary16 values q * 2^-24, with
// 0x00F000F0 two high nibbles as 16q * 2^-24; the 2^24 and 1/16 factors go into
// the sub-block scales. Per 8 weights: 5 bit operations and 4 dot2 operations.
// The sub-block sums X_j are taken over the same fp16 values, so the result is the
// exact product of W with the rounded x up to fp32 accumulation: rounding x to
// fp16 changes each product by at most 2^-11 relative (x in the fp16 normal
// range), well inside the 1e-3 * sum|w*x| bound.
#include <algorithm>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;

struct Q4Prob {
    const uint8_t* w;
    const float* x;
    float* y;
    int32_t M, nb, tiles, wg_begin;
};

// Kernel arguments. The first tile of every problem is repeated in a compact
// array at the front, so a workgroup finds its problem with one scalar load.
struct Q4Args {
    int32_t begin[QG_MAX_BATCH];
    int32_t count;
    Q4Prob p[QG_MAX_BATCH];
};

struct SbIn {
    uint4 s[9];
    float4 xa, xb, xc, xd;  // activations: low-nibble dwords i0, i0+1, then high-nibble ones
};

// Loads of super-block b: raw buffer loads with one resource per tile (weights)
// and one for x, a per-lane byte offset and the segment / activation offsets as
// scalar operands, so that a super-block costs one vector address operation
// instead of one 64-bit address per load. A K-group past the end of K (valid
// false) gets an offset beyond both resources: the loads return zeros without a
// memory access, and every load is still issued, so the wait counts stay exact.
QG_DEV void load_sb_buf(SbIn& d, __amdgpu_buffer_rsrc_t wr, uint32_t vrow, __amdgpu_buffer_rsrc_t xr, uint32_t vx,
                        int b, int rt, bool valid) {
    const uint32_t vxb = valid ? vx + (uint32_t)b * 1024u : kQgOutOfRange;
    d.xa = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, vxb, 0, 0));
    d.xb = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, vxb, 16, 0));
    d.xc = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, vxb, 128, 0));
    d.xd = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, vxb, 144, 0));
    const uint32_t vb = valid ? vrow + (uint32_t)b * 9u * (uint32_t)rt * 16u : kQgOutOfRange;
#pragma unroll
    for (int s = 0; s < 9; ++s) {
        const qg_u4v v = __builtin_amdgcn_raw_buffer_load_b128(wr, vb, s * rt * 16, kQgNonTemporal);
        d.s[s] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// Contribution of one super-block for this lane's row.
QG_DEV float sb_dot(const SbIn& d) {
    // activation pairs in the order the dot products consume them
    const QgPairs8 xp = qg_cvt_pairs(d.xa, d.xc, d.xb, d.xd);
    // sub-block sums of the same fp16 values: this lane holds 8 of sub-block 2g
    // (pairs 0, 1, 4, 5) and 8 of 2g+1 (pairs 2, 3, 6, 7), g = (lane % 16) / 4, so a
    // quad reduction gives X_{2g}, X_{2g+1}
    const float Xlo = qg_quad_sum(qg_sum_pairs4(xp.p[0], xp.p[1], xp.p[4], xp.p[5]));
    const float Xhi = qg_quad_sum(qg_sum_pairs4(xp.p[2], xp.p[3], xp.p[6], xp.p[7]));

    // S_{2g} (low nibbles) and S_{2g+1} (high nibbles, x16) from quant segments 2g, 2g+1
    float S[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float lo0 = 0.f, hi0 = 0.f, lo1 = 0.f, hi1 = 0.f;
        switch (g) {
            case 0:
                qg_q4_seg_dot<0, 1>(lo0, hi0, lo1, hi1, d.s[1], xp.p);
                qg_q4_seg_dot<2, 3>(lo0, hi0, lo1, hi1, d.s[2], xp.p);
                break;
            case 1:
                qg_q4_seg_dot<4, 5>(lo0, hi0, lo1, hi1, d.s[3], xp.p);
                qg_q4_seg_dot<6, 7>(lo0, hi0, lo1, hi1, d.s[4], xp.p);
                break;
            case 2:
                qg_q4_seg_dot<8, 9>(lo0, hi0, lo1, hi1, d.s[5], xp.p);
                qg_q4_seg_dot<10, 11>(lo0, hi0, lo1, hi1, d.s[6], xp.p);
                break;
            default:
                qg_q4_seg_dot<12, 13>(lo0, hi0, lo1, hi1, d.s[7], xp.p);
                qg_q4_seg_dot<14, 15>(lo0, hi0, lo1, hi1, d.s[8], xp.p);
                break;
        }
        S[2 * g] = lo0 + lo1;
        S[2 * g + 1] = hi0 + hi1;
    }

    const uint4 hd = d.s[0];
    const float dd = qg_half_lo(hd.x), dm = qg_half_hi(hd.x);
    const QgScales sc = qg_q4k_scales(hd.y, hd.z, hd.w);
    float te = qg_ub0(sc.sc03) * S[0];
    te = fmaf(qg_ub2(sc.sc03), S[2], te);
    te = fmaf(qg_ub0(sc.sc47), S[4], te);
    te = fmaf(qg_ub2(sc.sc47), S[6], te);
    float to = qg_ub1(sc.sc03) * S[1];
    to = fmaf(qg_ub3(sc.sc03), S[3], to);
    to = fmaf(qg_ub1(sc.sc47), S[5], to);
    to = fmaf(qg_ub3(sc.sc47), S[7], to);
    const float t = fmaf(to, 0.0625f, te);  // high nibbles were 16q
    // X_j of all eight sub-blocks from the quads that hold them
    float mn = qg_ub0(sc.m03) * qg_bcast<0>(Xlo);
    mn = fmaf(qg_ub1(sc.m03), qg_bcast<0>(Xhi), mn);
    mn = fmaf(qg_ub2(sc.m03), qg_bcast<4>(Xlo), mn);
    mn = fmaf(qg_ub3(sc.m03), qg_bcast<4>(Xhi), mn);
    mn = fmaf(qg_ub0(sc.m47), qg_bcast<8>(Xlo), mn);
    mn = fmaf(qg_ub1(sc.m47), qg_bcast<8>(Xhi), mn);
    mn = fmaf(qg_ub2(sc.m47), qg_bcast<12>(Xlo), mn);
    mn = fmaf(qg_ub3(sc.m47), qg_bcast<12>(Xhi), mn);
    // quants entered as q * 2^-24
    return fmaf(dd * 16777216.0f, t, -dm * mn);
}

// MODE 0: one super-block per K-group; 2: several, two register buffers
// (ping-pong prefetch).
template <int W, int MODE>
__global__ __launch_bounds__(64 * W) void q4k_gemv_kernel(Q4Args a) {
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const Q4Prob P = a.p[k];

    const int tile = wg - P.wg_begin;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    const int rt = min(T, P.M - tile * T);
    const int i = lane & 15;   // weight row within the tile, and activation slot
    const int kg = 4 * wave + (lane >> 4);
    constexpr int G = 4 * W;

    // activation slot of this lane: quant segment p = i/2, dwords 2(i%2), +1
    const int p = i >> 1;
    const uint32_t vx = 4u * (uint32_t)(64 * (p >> 1) + 16 * (p & 1) + 8 * (i & 1));
    // rows past a ragged tile's end re-read the last row; their results are dropped
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(P.w + (size_t)tile * T * nb * 144), (short)0, rt * nb * 144, kQgRawBufferFlags);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.x, (short)0, nb * 1024, kQgRawBufferFlags);
    const uint32_t vrow = 16u * (uint32_t)min(i, rt - 1);

    float acc = 0.f;
    if constexpr (MODE == 0) {  // one super-block per K-group (4W >= K/256)
        SbIn b0;
        load_sb_buf(b0, wr, vrow, xr, vx, kg, rt, kg < nb);
        const float v0 = sb_dot(b0);
        acc = (kg < nb) ? v0 : 0.f;
    } else {
        const int niter = (nb + G - 1) / G;
        // Ping-pong between two register buffers over pairs of super-blocks: the
        // loads of one stay in flight while the other is computed. The loads are
        // unconditional (past the end of K they read zeros without a memory access)
        // and the pair loop has a single exit, so the loop-carried load state, and
        // with it every wait count, is exact: waiting for one super-block never
        // waits for the next.
        SbIn b0, b1;
        load_sb_buf(b0, wr, vrow, xr, vx, kg, rt, kg < nb);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            load_sb_buf(b1, wr, vrow, xr, vx, kg + G * (it + 1), rt, kg + G * (it + 1) < nb);
            __builtin_amdgcn_sched_barrier(0);  // issue the loads before any wait
            const float v0 = sb_dot(b0);
            acc += (kg + G * it < nb) ? v0 : 0.f;
            load_sb_buf(b0, wr, vrow, xr, vx, kg + G * (it + 2), rt, kg + G * (it + 2) < nb);
            __builtin_amdgcn_sched_barrier(0);
            const float v1 = sb_dot(b1);
            acc += (kg + G * (it + 1) < nb) ? v1 : 0.f;
        }
        if (it < niter) {
            const float v0 = sb_dot(b0);
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

__global__ void q4k_pack_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t M, int nb) {
    const int64_t units = M * nb * 9;
    const int64_t tile_units = (int64_t)T * nb * 9;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < units;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = o / tile_units;
        const int64_t in = o - t * tile_units;
        const int rt = (int)std::min<int64_t>(T, M - t * T);
        const int64_t bs = in / rt;  // b * 9 + s
        const int i = (int)(in - bs * rt);
        const int64_t r = t * T + i;
        dst[o] = src[r * nb * 9 + bs];
    }
}

// Launch plan: one workgroup per 16-row tile; W wavefronts (4W K-groups) each.
struct Plan {
    int W = 1;
    int total_wg = 0;  // tiles over all problems
};

void plan_batch(const qg_gemv_problem* pr, int count, Q4Args* args, Plan* plan) {
    int64_t tiles_total = 0;
    int nb_max = 1;
    for (int i = 0; i < count; ++i) {
        tiles_total += qg::ceil_div(pr[i].M, T);
        nb_max = std::max(nb_max, (int)(pr[i].K / 256));
    }
    // Enough K-groups per tile that every super-block of a row has its own
    // (all of a tile's weights are requested at once), up to 4 wavefronts; a
    // measured sweep over the 7B decode shapes put W = 4 first for every stage.
    (void)tiles_total;
    int W = 1;
    while (W < 4 && 4 * W < nb_max) W *= 2;
    if (qg::launch_override().gemv_waves) W = qg::launch_override().gemv_waves;
    plan->W = W;
    int wg = 0;
    for (int i = 0; i < count; ++i) {
        Q4Prob& P = args->p[i];
        P.w = (const uint8_t*)pr[i].w_packed;
        P.x = pr[i].x;
        P.y = pr[i].y;
        P.M = (int32_t)pr[i].M;
        P.nb = (int32_t)(pr[i].K / 256);
        P.tiles = (int32_t)qg::ceil_div(pr[i].M, T);
        P.wg_begin = wg;
        args->begin[i] = wg;
        wg += P.tiles;
    }
    args->count = count;
    plan->total_wg = wg;
}

qg_status validate(const qg_gemv_problem* pr, int count) {
    if (!pr) return qg::fail(QG_ERR_NULL, "problem list is NULL");
    if (count < 1 || count > QG_MAX_BATCH) return qg::fail(QG_ERR_SHAPE, "batch count %d not in [1, %d]", count, QG_MAX_BATCH);
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
        const qg_gemv_problem& p = pr[i];
        if (!p.w_packed || !p.x || !p.y) return qg::fail(QG_ERR_NULL, "problem %d: NULL pointer", i);
        if (p.M < 1 || p.M > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "problem %d: M=%lld out of range", i, (long long)p.M);
        if (p.K < 256 || p.K % 256 || p.K > (1 << 24))
            return qg::fail(QG_ERR_SHAPE, "problem %d: K=%lld must be a positive multiple of 256 (<= 2^24)", i, (long long)p.K);
        if (!qg::aligned16(p.w_packed) || !qg::aligned16(p.x) || !qg::aligned16(p.y))
            return qg::fail(QG_ERR_ALIGN, "problem %d: pointers must be 16-byte aligned", i);
        tiles += qg::ceil_div(p.M, T);
    }
    if (tiles > INT32_MAX / 2) return qg::fail(QG_ERR_SHAPE, "batch too large");
    return QG_OK;
}

template <int W>
void launch(const Q4Args& a, int tiles, hipStream_t s) {
    bool multi = false;  // some K-group walks more than one super-block
    for (int i = 0; i < a.count; ++i) multi = multi || a.p[i].nb > 4 * W;
    if (!multi)
        hipLaunchKernelGGL((q4k_gemv_kernel<W, 0>), dim3(tiles), dim3(64 * W), 0, s, a);
    else
        hipLaunchKernelGGL((q4k_gemv_kernel<W, 2>), dim3(tiles), dim3(64 * W), 0, s, a);
}

}  // namespace

extern "C" {

// Every workgroup owns whole rows: no cross-workgroup reduction, no workspace.
qg_status qgemv_q4k_batch(const qg_gemv_problem* problems, int count, qg_stream_t stream) {
    qg::clear_error();
    qg_status st = validate(problems, count);
    if (st) return st;
    Q4Args a{};
    Plan p;
    plan_batch(problems, count, &a, &p);
    st = qg::check_device();
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    switch (p.W) {
        case 1: launch<1>(a, p.total_wg, s); break;
        case 2: launch<2>(a, p.total_wg, s); break;
        case 4: launch<4>(a, p.total_wg, s); break;
        default: launch<8>(a, p.total_wg, s); break;
    }
    return qg::launch_status("qgemv_q4k");
}

qg_status qgemv_q4k(const void* w, const float* x, float* y, int64_t M, int64_t K, qg_stream_t stream) {
    qg_gemv_problem p{w, x, y, M, K};
    return qgemv_q4k_batch(&p, 1, stream);
}

qg_status qg_pack_q4k(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream) {
    qg::clear_error();
    if (!src || !dst) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX || K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "invalid Q4_K shape M=%lld K=%lld", (long long)M, (long long)K);
    if (!qg::aligned16(src) || !qg::aligned16(dst)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t bytes = qg_q4k_bytes(M, K);
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    if (s8 < d8 + bytes && d8 < s8 + bytes) return qg::fail(QG_ERR_SHAPE, "src and dst overlap");
    qg_status st = qg::check_device();
    if (st) return st;
    const int64_t units = (int64_t)(bytes / 16);
    const int blocks = (int)std::min<int64_t>(qg::ceil_div(units, 256), 65536);
    hipLaunchKernelGGL(q4k_pack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                       (uint4*)dst, M, (int)(K / 256));
    return qg::launch_status("qg_pack_q4k");
}

}  // extern "C"
