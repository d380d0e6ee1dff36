// Small-N Q4_K product against int8 activations (N <= 8 columns, each quantized
// Q8_1-style as for qgemv_q4k_q8_1), for gfx950, with the weights read once for
// all N columns.
//
// Batched verification ("Why Local LLMs Don't Need C++ or Python", section 4: the
// candidate tokens are checked in one batch pass, so the weights cross the memory
// bus once) on the integer path of the dotLLM README's news entries (Q8_1 / Q8_K
// input quantization with a float32 scale and a precomputed sum per block,
// feeding fused K-quant dot products). Per row r, super-block b, column n and
// sub-block j (activation block c = 8b + j of column n),
//     Y[r][n] += d * sum_j d_cn sc_j S_jn  -  dmin * sum_j d_cn m_j s_cn,
//     S_jn = sum_l w4_{j,l} q_{32c+l, n}   (an exact integer).
//
// Tiles, K-groups, packed layout and per-column arithmetic are those of
// qgemv_q4k_q8_1 (four wavefronts per 16-row tile, DPP row broadcasts of the
// activation dwords, the same summation order), so each column equals that
// kernel's result bit for bit when it also runs four wavefronts. The nibble masks
// of a quant segment are computed once and shared by the columns: per 8 weights,
// 3 bit operations plus 2 v_dot4c_i32_i8 per column (5 + 4 per column with fp16
// activations, q4k_smalln_dot.hip). The next super-block's weights stay in flight
// while one is computed; its activations (quants, block scales and sums of every
// column) are requested before the next weights, so no wait covers later loads.
// Columns past a problem's N read zeros through an out-of-range offset and are
// not stored.
#include <algorithm>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;
constexpr int W = 4;      // wavefronts per workgroup
constexpr int G = 4 * W;  // K-groups per workgroup

struct QnProb {
    const uint8_t* w;
    const uint8_t* xq;  // N quantized activation buffers, xb bytes apart
    float* Y;
    int32_t xb, q_off, s_off, ldy, M, nb, N, wg_begin;
};
struct QnArgs {
    int32_t begin[QG_MAX_BATCH];
    int32_t count;
    QnProb p[QG_MAX_BATCH];
};

// 8 v_dot4c_i32_i8 of one quant segment for one column: masked bytes m (low and
// high nibbles of dwords 0..3) against the activation dwords x of lanes LA
// (quant dwords 0, 1) and LB (2, 3), in the order of qg_q4_seg_dot_i8. The masks
// come from ordinary VALU code, so the block opens with two wait states; the four
// accumulators rotate; TAIL blocks end with s_nop 4 before ordinary VALU code
// reads the accumulators.
#define QG_SEG8I_TEXT \
    "s_nop 1\n\t" \
    "v_dot4c_i32_i8_dpp %0, %12, %4 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot4c_i32_i8_dpp %1, %14, %5 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot4c_i32_i8_dpp %2, %13, %6 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot4c_i32_i8_dpp %3, %15, %7 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot4c_i32_i8_dpp %0, %12, %8 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot4c_i32_i8_dpp %1, %14, %9 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot4c_i32_i8_dpp %2, %13, %10 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot4c_i32_i8_dpp %3, %15, %11 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
template <int LA, int LB, bool TAIL>
QG_DEV void seg_dot4_m(int& lo0, int& hi0, int& lo1, int& hi1, const uint32_t (&m)[8], const uint32_t (&x)[4]) {
    if constexpr (TAIL)
        asm(QG_SEG8I_TEXT "s_nop 4"
            : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1)
            : "v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]), "v"(m[4]), "v"(m[5]), "v"(m[6]), "v"(m[7]), "v"(x[0]),
              "v"(x[1]), "v"(x[2]), "v"(x[3]), "n"(LA), "n"(LB));
    else
        asm(QG_SEG8I_TEXT ""
            : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1)
            : "v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]), "v"(m[4]), "v"(m[5]), "v"(m[6]), "v"(m[7]), "v"(x[0]),
              "v"(x[1]), "v"(x[2]), "v"(x[3]), "n"(LA), "n"(LB));
}

// Low and high nibbles of each dword of a quant segment, as unsigned bytes.
QG_DEV void seg_masks8(uint32_t (&m)[8], const uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        m[2 * d] = w[d] & 0x0f0f0f0fu;
        m[2 * d + 1] = (w[d] >> 4) & 0x0f0f0f0fu;
    }
}

template <int NC>
struct XqIn {
    uint2 xl[NC], xh[NC];   // this lane's activations: low run, high run
    float4 d0[NC], d1[NC];  // the super-block's eight block scales
    uint4 bs[NC];           // and eight block sums (int16)
};

QG_DEV void load_w(uint4 (&s)[9], __amdgpu_buffer_rsrc_t wr, uint32_t vrow, int b, int rt) {
    const uint32_t vb = vrow + (uint32_t)b * 9u * (uint32_t)rt * 16u;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const qg_u4v v = __builtin_amdgcn_raw_buffer_load_b128(wr, vb, k * rt * 16, kQgNonTemporal);
        s[k] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// coff[n]: byte offset of column n's buffer (out of range past N); vq: this
// lane's quant offset within a buffer; b: super-block.
template <int NC>
QG_DEV void load_xq(XqIn<NC>& x, __amdgpu_buffer_rsrc_t xr, const QnProb& P, uint32_t vq, int b, const int (&coff)[NC]) {
    const uint32_t q = vq + (uint32_t)b * 256u;
    const uint32_t dof = 32u * (uint32_t)b;             // 8 floats
    const uint32_t sof = (uint32_t)P.s_off + 16u * (uint32_t)b;  // 8 int16
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const qg_u2v a = __builtin_amdgcn_raw_buffer_load_b64(xr, q, coff[n], 0);
        const qg_u2v c = __builtin_amdgcn_raw_buffer_load_b64(xr, q + 32u, coff[n], 0);
        x.xl[n] = make_uint2(a.x, a.y);
        x.xh[n] = make_uint2(c.x, c.y);
        x.d0[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, dof, coff[n], 0));
        x.d1[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, dof + 16u, coff[n], 0));
        const qg_u4v s = __builtin_amdgcn_raw_buffer_load_b128(xr, sof, coff[n], 0);
        x.bs[n] = make_uint4(s.x, s.y, s.z, s.w);
    }
}

QG_DEV float f4at(const float4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

QG_DEV int lo16(uint32_t w) { return (int)(int16_t)(w & 0xffffu); }
QG_DEV int hi16(uint32_t w) { return (int)(int16_t)(w >> 16); }

// Contribution of one super-block to this lane's row, for every column.
template <int NC>
QG_DEV void sb_dot8_n(float (&out)[NC], const uint4 (&s)[9], const XqIn<NC>& x) {
    const uint4 hd = s[0];
    const QgScales sc = qg_q4k_scales(hd.y, hd.z, hd.w);
    const uint32_t scw[2] = {sc.sc03, sc.sc47}, mw[2] = {sc.m03, sc.m47};
    float t[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) t[n] = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        int lo0[NC], hi0[NC], lo1[NC], hi1[NC];
#pragma unroll
        for (int n = 0; n < NC; ++n) lo0[n] = hi0[n] = lo1[n] = hi1[n] = 0;
        uint32_t m[8];
        seg_masks8(m, s[1 + 2 * g]);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint32_t xv[4] = {x.xl[n].x, x.xl[n].y, x.xh[n].x, x.xh[n].y};
            switch (g) {
                case 0: seg_dot4_m<0, 1, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
                case 1: seg_dot4_m<4, 5, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
                case 2: seg_dot4_m<8, 9, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
                default: seg_dot4_m<12, 13, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
            }
        }
        seg_masks8(m, s[2 + 2 * g]);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint32_t xv[4] = {x.xl[n].x, x.xl[n].y, x.xh[n].x, x.xh[n].y};
            switch (g) {
                case 0: seg_dot4_m<2, 3, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
                case 1: seg_dot4_m<6, 7, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
                case 2: seg_dot4_m<10, 11, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
                default: seg_dot4_m<14, 15, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xv); break;
            }
        }
        // sub-blocks j = 2g (low nibbles) and 2g + 1 (high nibbles)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = 2 * g + h;
            const int scj = (int)((scw[j >> 2] >> (8 * (j & 3))) & 0xff);
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const float dc = (j < 4) ? f4at(x.d0[n], j) : f4at(x.d1[n], j - 4);
                const int S = h ? hi0[n] + hi1[n] : lo0[n] + lo1[n];
                t[n] = fmaf(dc, (float)(scj * S), t[n]);  // |sc S| < 2^22: exact in fp32
            }
        }
    }
    const float dd = qg_half_lo(hd.x), dm = qg_half_hi(hd.x);
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const uint32_t sw[4] = {x.bs[n].x, x.bs[n].y, x.bs[n].z, x.bs[n].w};
        float u = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int mj = (int)((mw[j >> 2] >> (8 * (j & 3))) & 0xff);
            const int sj = (j & 1) ? hi16(sw[j >> 1]) : lo16(sw[j >> 1]);
            const float dc = (j < 4) ? f4at(x.d0[n], j) : f4at(x.d1[n], j - 4);
            u = fmaf(dc, (float)(mj * sj), u);
        }
        out[n] = fmaf(dd, t[n], -dm * u);
    }
}

// MODE 0: one super-block per K-group (K <= 4096); 1: several, weights of the next
// one in flight.
template <int MODE, int NC>
__global__ __launch_bounds__(64 * W) void q4k_q8_1_smalln_kernel(QnArgs a) {
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const QnProb P = a.p[k];
    const int tile = wg - P.wg_begin;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    const int rt = min(T, P.M - tile * T);
    const int i = lane & 15;
    const int kg = 4 * wave + (lane >> 4);
    // activation slot: quant segment p = i/2 of group p/2, bytes 8(i%2) .. +7
    const int p = i >> 1;
    const uint32_t vq = (uint32_t)P.q_off + (uint32_t)(64 * (p >> 1) + 16 * (p & 1) + 8 * (i & 1));
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(P.w + (size_t)tile * T * nb * 144), (short)0, rt * nb * 144, kQgRawBufferFlags);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.xq, (short)0, P.N * P.xb, kQgRawBufferFlags);
    const uint32_t vrow = 16u * (uint32_t)min(i, rt - 1);
    int coff[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) coff[n] = n < P.N ? n * P.xb : (int)kQgOutOfRange;

    float acc[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = 0.f;
    if constexpr (MODE == 0) {
        uint4 w0[9];
        XqIn<NC> x;
        const int b = min(kg, nb - 1);
        load_w(w0, wr, vrow, b, rt);
        load_xq<NC>(x, xr, P, vq, b, coff);
        float v[NC];
        sb_dot8_n<NC>(v, w0, x);
#pragma unroll
        for (int n = 0; n < NC; ++n) acc[n] = (kg < nb) ? v[n] : 0.f;
    } else {
        // Two weight buffers over pairs of super-blocks; loads unconditional (indices
        // clamped to the last super-block), one exit: the wait counts are the same on
        // every turn.
        const int niter = (nb + G - 1) / G;
        uint4 w0[9], w1[9];
        XqIn<NC> x;
        load_w(w0, wr, vrow, min(kg, nb - 1), rt);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            load_xq<NC>(x, xr, P, vq, min(kg + G * it, nb - 1), coff);
            load_w(w1, wr, vrow, min(kg + G * (it + 1), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            float v[NC];
            sb_dot8_n<NC>(v, w0, x);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * it < nb) ? v[n] : 0.f;
            load_xq<NC>(x, xr, P, vq, min(kg + G * (it + 1), nb - 1), coff);
            load_w(w0, wr, vrow, min(kg + G * (it + 2), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            sb_dot8_n<NC>(v, w1, x);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * (it + 1) < nb) ? v[n] : 0.f;
        }
        if (it < niter) {
            load_xq<NC>(x, xr, P, vq, min(kg + G * it, nb - 1), coff);
            float v[NC];
            sb_dot8_n<NC>(v, w0, x);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * it < nb) ? v[n] : 0.f;
        }
    }

    __shared__ float red[W][NC][T];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const float v = qg_sum_rows4(acc[n]);
        if (lane < T) red[wave][n][lane] = v;
    }
    __syncthreads();
    if (wave != 0) return;
    const int r = lane & 15;
#pragma unroll
    for (int n0 = 0; n0 < NC; n0 += 4) {
        const int n = n0 + (lane >> 4);
        if (n < NC && n < P.N && r < rt) {
            float v = red[0][n][r];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w][n][r];
            P.Y[(size_t)n * P.ldy + tile * T + r] = v;
        }
    }
}

template <int NC>
void launch_nc(const QnArgs& a, int grid, bool multi, hipStream_t s) {
    if (multi)
        hipLaunchKernelGGL((q4k_q8_1_smalln_kernel<1, NC>), dim3(grid), dim3(64 * W), 0, s, a);
    else
        hipLaunchKernelGGL((q4k_q8_1_smalln_kernel<0, NC>), dim3(grid), dim3(64 * W), 0, s, a);
}

constexpr int kMaxCols = 8;

}  // namespace

extern "C" {

qg_status qgemm_q4k_q8_1_smalln_batch(const qg_gemm_q8_1_problem* pr, int count, qg_stream_t stream) {
    qg::clear_error();
    if (!pr) return qg::fail(QG_ERR_NULL, "problem list is NULL");
    if (count < 1 || count > QG_MAX_BATCH)
        return qg::fail(QG_ERR_SHAPE, "batch count %d not in [1, %d]", count, QG_MAX_BATCH);
    QnArgs a{};
    int tiles = 0, nmax = 1;
    bool multi = false;
    for (int i = 0; i < count; ++i) {
        const qg_gemm_q8_1_problem& q = pr[i];
        if (!q.w_packed || !q.xq || !q.Y) return qg::fail(QG_ERR_NULL, "problem %d: NULL pointer", i);
        if (q.M < 1 || q.M > INT32_MAX - T) return qg::fail(QG_ERR_SHAPE, "problem %d: M=%lld out of range", i, (long long)q.M);
        if (q.K < 256 || q.K % 256 || q.K > (1 << 24))
            return qg::fail(QG_ERR_SHAPE, "problem %d: K=%lld must be a positive multiple of 256 (<= 2^24)", i,
                            (long long)q.K);
        if (q.N < 1 || q.N > kMaxCols)
            return qg::fail(QG_ERR_SHAPE, "problem %d: N=%lld not in [1, %d]", i, (long long)q.N, kMaxCols);
        if (q.ldy < q.M || q.ldy % 4) return qg::fail(QG_ERR_SHAPE, "problem %d: ldy must be >= M and a multiple of 4", i);
        if (!qg::aligned16(q.w_packed) || !qg::aligned16(q.xq) || !qg::aligned16(q.Y))
            return qg::fail(QG_ERR_ALIGN, "problem %d: pointers must be 16-byte aligned", i);
        size_t q_off = 0, s_off = 0;
        qg::q8_1_offsets(q.K, &q_off, &s_off);
        const size_t xb = qg_q8_1_bytes(q.K);
        if ((int64_t)q.N * (int64_t)xb >= (int64_t)kQgOutOfRange)
            return qg::fail(QG_ERR_SHAPE, "problem %d: activation buffers exceed 2^31 bytes", i);
        QnProb& P = a.p[i];
        P.w = (const uint8_t*)q.w_packed;
        P.xq = (const uint8_t*)q.xq;
        P.Y = q.Y;
        P.xb = (int32_t)xb;
        P.q_off = (int32_t)q_off;
        P.s_off = (int32_t)s_off;
        P.ldy = (int32_t)std::min<int64_t>(q.ldy, INT32_MAX);
        P.M = (int32_t)q.M;
        P.nb = (int32_t)(q.K / 256);
        P.N = (int32_t)q.N;
        P.wg_begin = tiles;
        a.begin[i] = tiles;
        const int64_t t = qg::ceil_div(q.M, T);
        if ((int64_t)tiles + t > INT32_MAX / 2) return qg::fail(QG_ERR_SHAPE, "batch too large");
        if ((int64_t)(q.N - 1) * q.ldy + q.M > INT32_MAX)
            return qg::fail(QG_ERR_SHAPE, "problem %d: Y extent exceeds 2^31 elements", i);
        tiles += (int)t;
        nmax = std::max(nmax, (int)q.N);
        multi = multi || P.nb > G;
    }
    a.count = count;
    qg_status st = qg::check_device();
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    switch (nmax) {
        case 1: launch_nc<1>(a, tiles, multi, s); break;
        case 2: launch_nc<2>(a, tiles, multi, s); break;
        case 3: launch_nc<3>(a, tiles, multi, s); break;
        case 4: launch_nc<4>(a, tiles, multi, s); break;
        case 5: launch_nc<5>(a, tiles, multi, s); break;
        case 6: launch_nc<6>(a, tiles, multi, s); break;
        case 7: launch_nc<7>(a, tiles, multi, s); break;
        default: launch_nc<8>(a, tiles, multi, s); break;
    }
    return qg::launch_status("qgemm_q4k_q8_1_smalln");
}

qg_status qgemm_q4k_q8_1_smalln(const void* w_packed, const void* xq, float* Y, int64_t ldy, int64_t M, int64_t K,
                                int64_t N, qg_stream_t stream) {
    const qg_gemm_q8_1_problem p{w_packed, xq, Y, ldy, M, K, N};
    return qgemm_q4k_q8_1_smalln_batch(&p, 1, stream);
}

}  // extern "C"
