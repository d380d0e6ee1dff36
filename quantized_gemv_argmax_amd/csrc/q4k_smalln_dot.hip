// Small-N Q4_K product Y = W X for a few columns (N <= 8) on the vector ALUs, for
// gfx950: the dot-product form of the single-column GEMV (q4k_gemv.hip) with the
// weights read once for all N columns.
//
// Batched verification ("Why Local LLMs Don't Need C++ or Python", section 4:
// the candidate tokens are checked in a single batch pass, so the weights cross
// the memory bus once for all of them). Per row r, super-block b and column n,
//     Y[r][n] += d * sum_j sc_j * S_jn  -  dmin * sum_j m_j * X_jn,
//     S_jn = sum_l q_{j,l} x_{256b+32j+l, n},   X_jn = sum_l x_{256b+32j+l, n},
// the Q4_K affine form (dotLLM README, Key Features: fused scale x int dot
// products on the quantized blocks).
//
// Same tiles, K-groups and packed layout as the single-column kernel: a workgroup
// of W = 4 wavefronts owns one 16-row tile and all of K; each 16-lane DPP row is
// a K-group walking super-blocks kg, kg + 16, ...; lane i of a K-group is weight
// row i and holds activation slot i of every column. Per quant dword the four
// masked words (two fp16-subnormal quants each) are computed once and shared by
// the N columns; each column then costs four v_dot2c_f32_f16 with the DPP row
// broadcast of the lane holding its activation pair: per 8 weights, 5 bit
// operations plus 4 N dot operations, against 5 + 4 for a single column.
//
// Loads: the weights of the next super-block are kept in flight while the
// current one is computed (two register buffers); a super-block's activations
// are requested just before the next weights, so that waiting for them never
// waits for those weights. Columns past a problem's N read zeros through an
// out-of-range buffer offset and are not stored.
#include <algorithm>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;
constexpr int W = 4;        // wavefronts per workgroup
constexpr int G = 4 * W;    // K-groups per workgroup

struct SdProb {
    const uint8_t* w;
    const float* X;
    float* Y;
    int64_t ldy;
    int32_t ldx, M, nb, N, wg_begin;  // (N - 1) * ldx + K < 2^29 (checked by the entry points)
};
struct SdArgs {
    int32_t begin[QG_MAX_BATCH];
    int32_t count;
    SdProb p[QG_MAX_BATCH];
};

// 16 dot2 of one quant segment for one column: the masked words m (four per
// dword, dwords 0..3) against the activation pairs x of lanes LA (dwords 0, 1)
// and LB (dwords 2, 3), in the order of qg_q4_seg_dot. The masks come from
// ordinary VALU code, so the block opens with two wait states before the first
// DPP read; the four accumulators rotate, so each is re-read four instructions
// after its last write. TAIL blocks (the last segment of a sub-block pair) end
// with s_nop 4 before ordinary VALU code reads the accumulators.
#define QG_SEG16_TEXT \
    "s_nop 1\n\t" \
    "v_dot2c_f32_f16_dpp %0, %20, %4 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %1, %22, %5 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %2, %21, %6 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %3, %23, %7 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %0, %24, %8 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %1, %26, %9 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %2, %25, %10 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %3, %27, %11 row_newbcast:%28 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %0, %20, %12 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %1, %22, %13 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %2, %21, %14 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %3, %23, %15 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %0, %24, %16 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %1, %26, %17 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %2, %25, %18 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %3, %27, %19 row_newbcast:%29 row_mask:0xf bank_mask:0xf\n\t"
template <int LA, int LB, bool TAIL>
QG_DEV void seg_dot_m(float& lo0, float& hi0, float& lo1, float& hi1, const uint32_t (&m)[16], const uint32_t (&x)[8]) {
    if constexpr (TAIL)
        asm(QG_SEG16_TEXT "s_nop 4"
        : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1)
        : "v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]), "v"(m[4]), "v"(m[5]), "v"(m[6]), "v"(m[7]), "v"(m[8]),
          "v"(m[9]), "v"(m[10]), "v"(m[11]), "v"(m[12]), "v"(m[13]), "v"(m[14]), "v"(m[15]), "v"(x[0]), "v"(x[1]),
          "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "n"(LA), "n"(LB));
    else
        asm(QG_SEG16_TEXT ""
        : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1)
        : "v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]), "v"(m[4]), "v"(m[5]), "v"(m[6]), "v"(m[7]), "v"(m[8]),
          "v"(m[9]), "v"(m[10]), "v"(m[11]), "v"(m[12]), "v"(m[13]), "v"(m[14]), "v"(m[15]), "v"(x[0]), "v"(x[1]),
          "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "n"(LA), "n"(LB));
}

// The four masked words of each dword of a quant segment: low nibbles of bytes
// 0, 2; high nibbles of bytes 0, 2; low and high nibbles of bytes 1, 3.
QG_DEV void seg_masks(uint32_t (&m)[16], const uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t t = w[d] >> 8;
        m[4 * d + 0] = w[d] & 0x000f000fu;
        m[4 * d + 1] = w[d] & 0x00f000f0u;
        m[4 * d + 2] = t & 0x000f000fu;
        m[4 * d + 3] = t & 0x00f000f0u;
    }
}

template <int NC>
struct XIn {
    float4 a[NC], b[NC], c[NC], d[NC];  // low-run dwords i0, i0+1, then the high run, per column
};

QG_DEV void load_w(uint4 (&s)[9], __amdgpu_buffer_rsrc_t wr, uint32_t vrow, int b, int rt) {
    const uint32_t vb = vrow + (uint32_t)b * 9u * (uint32_t)rt * 16u;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const qg_u4v v = __builtin_amdgcn_raw_buffer_load_b128(wr, vb, k * rt * 16, kQgNonTemporal);
        s[k] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

template <int NC>
QG_DEV void load_x(XIn<NC>& x, __amdgpu_buffer_rsrc_t xr, uint32_t vx, int b, const int (&coff)[NC]) {
    const uint32_t v = vx + (uint32_t)b * 1024u;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        x.a[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, v, coff[n], 0));
        x.b[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, v, coff[n] + 16, 0));
        x.c[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, v, coff[n] + 128, 0));
        x.d[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, v, coff[n] + 144, 0));
    }
}

// Contribution of one super-block to this lane's row, for every column.
template <int NC>
QG_DEV void sb_dot_n(float (&out)[NC], const uint4 (&s)[9], const XIn<NC>& x) {
    QgPairs8 xp[NC];
    float Xlo[NC], Xhi[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        xp[n] = qg_cvt_pairs(x.a[n], x.c[n], x.b[n], x.d[n]);
        // sub-block sums over the same fp16 values (low run pairs 0, 1, 4, 5;
        // high run pairs 2, 3, 6, 7), as in the single-column kernel
        Xlo[n] = qg_quad_sum(qg_sum_pairs4(xp[n].p[0], xp[n].p[1], xp[n].p[4], xp[n].p[5]));
        Xhi[n] = qg_quad_sum(qg_sum_pairs4(xp[n].p[2], xp[n].p[3], xp[n].p[6], xp[n].p[7]));
    }
    const uint4 hd = s[0];
    const QgScales sc = qg_q4k_scales(hd.y, hd.z, hd.w);
    const uint32_t scw[2] = {sc.sc03, sc.sc47};
    float te[NC], to[NC];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float lo0[NC], hi0[NC], lo1[NC], hi1[NC];
#pragma unroll
        for (int n = 0; n < NC; ++n) lo0[n] = hi0[n] = lo1[n] = hi1[n] = 0.f;
        uint32_t m[16];
        seg_masks(m, s[1 + 2 * g]);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            switch (g) {
                case 0: seg_dot_m<0, 1, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
                case 1: seg_dot_m<4, 5, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
                case 2: seg_dot_m<8, 9, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
                default: seg_dot_m<12, 13, false>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
            }
        }
        seg_masks(m, s[2 + 2 * g]);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            switch (g) {
                case 0: seg_dot_m<2, 3, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
                case 1: seg_dot_m<6, 7, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
                case 2: seg_dot_m<10, 11, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
                default: seg_dot_m<14, 15, true>(lo0[n], hi0[n], lo1[n], hi1[n], m, xp[n].p); break;
            }
        }
        // sub-blocks 2g (low nibbles) and 2g + 1 (high nibbles, entered as 16q)
        const uint32_t sw = scw[g >> 1];
        const float sce = (float)((sw >> (16 * (g & 1))) & 0xffu);
        const float sco = (float)((sw >> (16 * (g & 1) + 8)) & 0xffu);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const float Se = lo0[n] + lo1[n], So = hi0[n] + hi1[n];
            te[n] = g == 0 ? sce * Se : fmaf(sce, Se, te[n]);
            to[n] = g == 0 ? sco * So : fmaf(sco, So, to[n]);
        }
    }
    const float dd = qg_half_lo(hd.x), dm = qg_half_hi(hd.x);
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const float t = fmaf(to[n], 0.0625f, te[n]);
        float mn = qg_ub0(sc.m03) * qg_bcast<0>(Xlo[n]);
        mn = fmaf(qg_ub1(sc.m03), qg_bcast<0>(Xhi[n]), mn);
        mn = fmaf(qg_ub2(sc.m03), qg_bcast<4>(Xlo[n]), mn);
        mn = fmaf(qg_ub3(sc.m03), qg_bcast<4>(Xhi[n]), mn);
        mn = fmaf(qg_ub0(sc.m47), qg_bcast<8>(Xlo[n]), mn);
        mn = fmaf(qg_ub1(sc.m47), qg_bcast<8>(Xhi[n]), mn);
        mn = fmaf(qg_ub2(sc.m47), qg_bcast<12>(Xlo[n]), mn);
        mn = fmaf(qg_ub3(sc.m47), qg_bcast<12>(Xhi[n]), mn);
        out[n] = fmaf(dd * 16777216.0f, t, -dm * mn);  // quants entered as q * 2^-24
    }
}

// MODE 0: one super-block per K-group (K <= 4096); 1: several, weights of the next
// one in flight; 2: several, weights and activations of the next one in flight
// (two full register buffers; used for one column, where it measured faster on
// the 3584 x 18944 down projection, 10.4 -> 9.8 us, and slower for two, 13.5 ->
// 14.2 us).
template <int MODE, int NC>
__global__ __launch_bounds__(64 * W) void q4k_smalln_dot_kernel(SdArgs a) {
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SdProb P = a.p[k];
    const int tile = wg - P.wg_begin;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    const int rt = min(T, P.M - tile * T);
    const int i = lane & 15;
    const int kg = 4 * wave + (lane >> 4);

    const int p = i >> 1;
    const uint32_t vx = 4u * (uint32_t)(64 * (p >> 1) + 16 * (p & 1) + 8 * (i & 1));
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(P.w + (size_t)tile * T * nb * 144), (short)0, rt * nb * 144, kQgRawBufferFlags);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, ((P.N - 1) * P.ldx + nb * 256) * 4, kQgRawBufferFlags);
    const uint32_t vrow = 16u * (uint32_t)min(i, rt - 1);
    int coff[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) coff[n] = n < P.N ? n * P.ldx * 4 : (int)kQgOutOfRange;

    float acc[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = 0.f;
    if constexpr (MODE == 0) {
        uint4 w0[9];
        XIn<NC> x;
        const int b = min(kg, nb - 1);
        load_w(w0, wr, vrow, b, rt);
        load_x<NC>(x, xr, vx, b, coff);
        float v[NC];
        sb_dot_n<NC>(v, w0, x);
#pragma unroll
        for (int n = 0; n < NC; ++n) acc[n] = (kg < nb) ? v[n] : 0.f;
    } else if constexpr (MODE == 1) {
        const int niter = (nb + G - 1) / G;
        // Two weight buffers over pairs of super-blocks; each super-block's
        // activations are requested before the next weights, so every wait is for
        // loads issued earlier only. All loads are unconditional (indices clamped
        // to the last super-block) and the pair loop has one exit, so the wait
        // counts are the same on every turn.
        uint4 w0[9], w1[9];
        XIn<NC> x;
        load_w(w0, wr, vrow, min(kg, nb - 1), rt);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            load_x<NC>(x, xr, vx, min(kg + G * it, nb - 1), coff);
            load_w(w1, wr, vrow, min(kg + G * (it + 1), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            float v[NC];
            sb_dot_n<NC>(v, w0, x);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * it < nb) ? v[n] : 0.f;
            load_x<NC>(x, xr, vx, min(kg + G * (it + 1), nb - 1), coff);
            load_w(w0, wr, vrow, min(kg + G * (it + 2), nb - 1), rt);
            __builtin_amdgcn_sched_barrier(0);
            sb_dot_n<NC>(v, w1, x);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * (it + 1) < nb) ? v[n] : 0.f;
        }
        if (it < niter) {
            load_x<NC>(x, xr, vx, min(kg + G * it, nb - 1), coff);
            float v[NC];
            sb_dot_n<NC>(v, w0, x);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * it < nb) ? v[n] : 0.f;
        }
    }
    if constexpr (MODE == 2) {
        const int niter = (nb + G - 1) / G;
        uint4 w0[9], w1[9];
        XIn<NC> x0, x1;
        load_w(w0, wr, vrow, min(kg, nb - 1), rt);
        load_x<NC>(x0, xr, vx, min(kg, nb - 1), coff);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            load_w(w1, wr, vrow, min(kg + G * (it + 1), nb - 1), rt);
            load_x<NC>(x1, xr, vx, min(kg + G * (it + 1), nb - 1), coff);
            __builtin_amdgcn_sched_barrier(0);
            float v[NC];
            sb_dot_n<NC>(v, w0, x0);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * it < nb) ? v[n] : 0.f;
            load_w(w0, wr, vrow, min(kg + G * (it + 2), nb - 1), rt);
            load_x<NC>(x0, xr, vx, min(kg + G * (it + 2), nb - 1), coff);
            __builtin_amdgcn_sched_barrier(0);
            sb_dot_n<NC>(v, w1, x1);
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] += (kg + G * (it + 1) < nb) ? v[n] : 0.f;
        }
        if (it < niter) {
            float v[NC];
            sb_dot_n<NC>(v, w0, x0);
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
    // lane = 16 * (column within a group of four) + row
    const int r = lane & 15;
#pragma unroll
    for (int n0 = 0; n0 < NC; n0 += 4) {
        const int n = n0 + (lane >> 4);
        if (n < NC && n < P.N && r < rt) {
            float v = red[0][n][r];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w][n][r];
            P.Y[n * P.ldy + tile * T + r] = v;
        }
    }
}

template <int NC>
void launch_nc(const SdArgs& a, int grid, bool multi, hipStream_t s) {
    if constexpr (NC == 1) {
        if (multi) {
            hipLaunchKernelGGL((q4k_smalln_dot_kernel<2, NC>), dim3(grid), dim3(64 * W), 0, s, a);
            return;
        }
    }
    if (multi)
        hipLaunchKernelGGL((q4k_smalln_dot_kernel<1, NC>), dim3(grid), dim3(64 * W), 0, s, a);
    else
        hipLaunchKernelGGL((q4k_smalln_dot_kernel<0, NC>), dim3(grid), dim3(64 * W), 0, s, a);
}

}  // namespace

namespace qg {

// Launches the dot-product form for problems already validated by the small-N
// entry points (N <= 8 each; ldx, ldy and the activation extent checked there).
qg_status smalln_dot_launch(const qg_gemm_problem* probs, int count, hipStream_t s) {
    SdArgs a{};
    a.count = count;
    int wg = 0, nmax = 0;
    bool multi = false;
    for (int i = 0; i < count; ++i) {
        const qg_gemm_problem& q = probs[i];
        SdProb& P = a.p[i];
        P.w = (const uint8_t*)q.w_packed;
        P.X = q.X;
        P.Y = q.Y;
        P.ldx = q.N > 1 ? (int32_t)q.ldx : 0;  // the first column needs no stride
        P.ldy = q.ldy;
        P.M = (int32_t)q.M;
        P.nb = (int32_t)(q.K / 256);
        P.N = (int32_t)q.N;
        P.wg_begin = wg;
        a.begin[i] = wg;
        wg += (int32_t)ceil_div(q.M, T);
        nmax = std::max(nmax, P.N);
        multi = multi || P.nb > G;
    }
    switch (nmax) {
        case 1: launch_nc<1>(a, wg, multi, s); break;
        case 2: launch_nc<2>(a, wg, multi, s); break;
        case 3: launch_nc<3>(a, wg, multi, s); break;
        case 4: launch_nc<4>(a, wg, multi, s); break;
        case 5: launch_nc<5>(a, wg, multi, s); break;
        case 6: launch_nc<6>(a, wg, multi, s); break;
        case 7: launch_nc<7>(a, wg, multi, s); break;
        default: launch_nc<8>(a, wg, multi, s); break;
    }
    return launch_status("qgemm_q4k_smalln");
}

}  // namespace qg
