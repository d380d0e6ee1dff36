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
// For up to four columns the vector-ALU dot-product form (q4k_smalln_dot.hip)
// runs instead: per 8 weights it costs 5 bit operations and 4 dot2 operations per
// column, which stays below the matrix-core forms' per-sub-block scaling work
// while N is small.
//
// Two forms share this arithmetic. The LDS-staged form (the default, further
// down) stages the activations in LDS and streams the weights with deep queues.
// The register-staged form, described here: one workgroup per TW consecutive
// 16-row tiles of the packed layout (q4k_gemv.hip); its W wavefronts split K in
// units of 64 weights (two sub-blocks), each wavefront applying one unit's
// activations to all TW tiles.
// Partial results meet in LDS in a fixed order, so results are deterministic. No
// workspace, no cross-workgroup traffic. Rows past a ragged tile's end and tiles
// past the matrix end re-read the last row / tile, columns past N read zeros;
// their results are dropped.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdlib>
#include <string>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;

struct SnProb {
    const uint8_t* w;
    const float* X;
    float* Y;
    int64_t ldx, ldy;
    int32_t M, nb, N, tiles, wg_begin;
    int32_t wgs;        // streamed and walk forms: workgroups (walk: tile groups) of this problem
    int32_t slices;
    int32_t hfast;  // workgroups ordered slice fastest (else tile group fastest)     // walk form: K slices (workgroups = wgs * slices)
    int32_t slice_sbs;  // super-blocks per K slice
    float* part;        // walk form with K slices: partial sums (qg_f4 per lane) instead of Y
    uint32_t* ctr;      // and one arrival counter per tile group (zero between calls)
};
struct SnArgs {
    int32_t begin[QG_MAX_BATCH];
    int32_t count;
    SnProb p[QG_MAX_BATCH];
};

// Inputs of one unit: sub-blocks 2g and 2g + 1 of super-block b (u = 4 b + g) of
// TW consecutive tiles.
template <int C, int TW>
struct SnIn {
    uint4 hdr[TW];        // d, dmin, 12 scale bytes of this lane's row in each tile
    uint2 q[TW];          // quant bytes 8 (l / 16)..+7 of sub-blocks 2g and 2g + 1
    float4 x[2][C][2];    // [low / high sub-block][column block][first / second 4]
};

// All loads are raw buffer loads: a wavefront-uniform resource and unit offset
// (scalar registers) plus a fixed per-lane offset, so no vector instruction
// computes an address inside the K loop. Activation lanes of columns past N get
// an offset beyond the resource's range: the hardware returns zeros for them
// without a memory access (their products land in output columns that are not
// stored).
constexpr uint32_t kOutOfRange = kQgOutOfRange;
constexpr int kNonTemporal = kQgNonTemporal;

template <int C, int TW>
struct SnLane {
    uint32_t hdr[TW], q[TW];  // per tile: byte offset of this lane's header / quant bytes
    uint32_t x[C];            // per column block: byte offset of this lane's activations
};

template <int TW>
struct SnTiles {
    __amdgpu_buffer_rsrc_t w[TW];  // one tile each
    int32_t rt[TW];                // rows of the tile
};

template <int C, int TW>
QG_DEV void load_w(SnIn<C, TW>& d, const SnTiles<TW>& tl, const SnLane<C, TW>& ln, int u) {
    const int b = u >> 2, g = u & 3;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int sb = b * 9 * 16 * tl.rt[t];
        const qg_u4v h = __builtin_amdgcn_raw_buffer_load_b128(tl.w[t], ln.hdr[t], sb, kNonTemporal);
        d.hdr[t] = make_uint4(h.x, h.y, h.z, h.w);
        const qg_u2v q = __builtin_amdgcn_raw_buffer_load_b64(tl.w[t], ln.q[t], sb + (1 + 2 * g) * 16 * tl.rt[t],
                                                              kNonTemporal);
        d.q[t] = make_uint2(q.x, q.y);
    }
}

template <int C, int TW>
QG_DEV void load_x(SnIn<C, TW>& d, __amdgpu_buffer_rsrc_t xr, const SnLane<C, TW>& ln, int u) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int so = u * 256 + 128 * h;
            const qg_u4v v0 = __builtin_amdgcn_raw_buffer_load_b128(xr, ln.x[c], so, 0);
            const qg_u4v v1 = __builtin_amdgcn_raw_buffer_load_b128(xr, ln.x[c], so + 16, 0);
            d.x[h][c][0] = __builtin_bit_cast(float4, v0);
            d.x[h][c][1] = __builtin_bit_cast(float4, v1);
        }
}

template <int C, int TW>
QG_DEV void unit_dot(qg_f4 (&acc)[TW][C], const SnIn<C, TW>& d, int u) {
    const int g = u & 3;  // sub-blocks 2g (low nibbles) and 2g + 1 (high nibbles)
    const qg_h8 ones = qg_ones_h8();
    const qg_f4 zero = {0.f, 0.f, 0.f, 0.f};
    // activations and their sub-block sums, shared by the TW tiles
    qg_h8 a_lo[C], a_hi[C];
    qg_f4 x_lo[C], x_hi[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        a_lo[c] = qg_a_operand(d.x[0][c][0], d.x[0][c][1]);
        a_hi[c] = qg_a_operand(d.x[1][c][0], d.x[1][c][1]);
        x_lo[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[c], ones, zero, 0, 0, 0);
        x_hi[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[c], ones, zero, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const uint4 hd = d.hdr[t];
        const float dd = qg_half_lo(hd.x) * 16777216.0f;  // quants enter as q * 2^-24
        const float dm = qg_half_hi(hd.x);
        // 6-bit scale and min of sub-blocks 2g, 2g + 1 (both forms computed and
        // selected, so that no branch splits the wait counts)
        const uint32_t sc03 = hd.y & 0x3f3f3f3fu, m03 = hd.z & 0x3f3f3f3fu;
        const uint32_t sc47 = (hd.w & 0x0f0f0f0fu) | ((hd.y >> 2) & 0x30303030u);
        const uint32_t m47 = ((hd.w >> 4) & 0x0f0f0f0fu) | ((hd.z >> 2) & 0x30303030u);
        const uint32_t scw = qg_opaque(g < 2 ? sc03 : sc47);
        const uint32_t mw = qg_opaque(g < 2 ? m03 : m47);
        const int kb = 2 * (g & 1);
        const float s_lo = dd * qg_byte_f(scw, kb);
        const float s_hi = dd * 0.0625f * qg_byte_f(scw, kb + 1);
        const float m_lo = dm * qg_byte_f(mw, kb);
        const float m_hi = dm * qg_byte_f(mw, kb + 1);

        const uint32_t w0 = d.q[t].x, w1 = d.q[t].y;
        const uint32_t w0s = w0 >> 8, w1s = w1 >> 8;
        const qg_h8 b_lo = __builtin_bit_cast(
            qg_h8, make_uint4(w0 & 0x000f000fu, w0s & 0x000f000fu, w1 & 0x000f000fu, w1s & 0x000f000fu));
        const qg_h8 b_hi = __builtin_bit_cast(
            qg_h8, make_uint4(w0 & 0x00f000f0u, w0s & 0x00f000f0u, w1 & 0x00f000f0u, w1s & 0x00f000f0u));
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const qg_f4 s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[c], b_lo, zero, 0, 0, 0);
            const qg_f4 s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[c], b_hi, zero, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = acc[t][c][e];
                v = fmaf(s_lo, s0[e], v);
                v = fmaf(s_hi, s1[e], v);
                v = fmaf(-m_lo, x_lo[c][e], v);
                v = fmaf(-m_hi, x_hi[c][e], v);
                acc[t][c][e] = v;
            }
        }
    }
}

template <int C, int TW, int W>
__global__ __launch_bounds__(64 * W) void q4k_smalln_kernel(SnArgs a) {
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SnProb P = a.p[k];

    const int tile0 = (wg - P.wg_begin) * TW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    SnTiles<TW> tl;
    SnLane<C, TW> ln;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        // a tile past the matrix end (TW > 1, ragged tile count) re-reads the last tile
        const int tc = min(tile0 + t, P.tiles - 1);
        tl.rt[t] = min(T, P.M - tc * T);
        tl.w[t] = __builtin_amdgcn_make_buffer_rsrc((void*)(P.w + (size_t)tc * T * P.nb * 144), (short)0,
                                                    tl.rt[t] * P.nb * 144, kQgRawBufferFlags);
        const uint32_t r = (uint32_t)min(i, tl.rt[t] - 1);
        ln.hdr[t] = 16 * r;
        ln.q[t] = 16 * r + 8 * (s & 1) + (uint32_t)(s >> 1) * 16 * tl.rt[t];
    }
    // activations: column n = 16 c + i of X, this lane's 8-element K slice
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + (int64_t)P.nb * 256) * 4), kQgRawBufferFlags);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = 16 * c + i;
        ln.x[c] = n < P.N ? (uint32_t)(((int64_t)n * P.ldx + 8 * s) * 4) : kOutOfRange;
    }
    // the K units, split among the wavefronts round-robin
    const int units = P.nb * 4;
    const int niter = (units - wave + W - 1) / W;  // units wave, wave + W, ...
    qg_f4 acc[TW][C];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[t][c] = qg_f4{0.f, 0.f, 0.f, 0.f};

    // Ping-pong over pairs of units: the inputs of the next unit are in flight
    // while one is computed (activations first, so waiting for one unit's inputs
    // never waits for the next unit's). The loads are unconditional (the unit index
    // is clamped to the wavefront's last unit) and the pair loop has a single exit,
    // so the loop-carried load state, and with it every wait count, is exact.
    if (niter > 0) {
        const int ufirst = wave, ulast = ufirst + W * (niter - 1);
        SnIn<C, TW> b0, b1;
        load_x<C, TW>(b0, xr, ln, ufirst);
        load_w<C, TW>(b0, tl, ln, ufirst);
        int it = 0;
        for (; it + 2 <= niter; it += 2) {
            const int u0 = ufirst + W * it;
            load_x<C, TW>(b1, xr, ln, u0 + W);
            load_w<C, TW>(b1, tl, ln, u0 + W);
            __builtin_amdgcn_sched_barrier(0);  // issue the loads before any wait
            unit_dot<C, TW>(acc, b0, u0);
            const int u2 = min(u0 + 2 * W, ulast);
            load_x<C, TW>(b0, xr, ln, u2);
            load_w<C, TW>(b0, tl, ln, u2);
            __builtin_amdgcn_sched_barrier(0);
            unit_dot<C, TW>(acc, b1, u0 + W);
        }
        if (it < niter) unit_dot<C, TW>(acc, b0, ufirst + W * it);
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
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        if (tile0 + t < P.tiles && i < tl.rt[t]) {
            const int row = (tile0 + t) * T + i;
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = 16 * c + 4 * s + e;
                    if (n >= P.N) continue;
                    P.Y[(int64_t)n * P.ldy + row] = acc[t][c][e];
                }
        }
    }
}

// ------------------------------------------------------------ LDS-staged form
// The kernel above keeps each wavefront's activations in registers (16 per lane
// and column block for every 64-weight unit), which leaves room for only two units
// of weights in flight per wavefront: too few bytes per CU to cover the HBM
// latency. Here the activations go through LDS instead, and the two kinds of work
// are given to different wavefronts, since a wavefront's loads complete in issue
// order and a wait for an activation load would also wait for every weight load
// issued before it:
//   - WP producer wavefronts stage the activations of a chunk of WC super-blocks
//     (256 WC values per column, all columns) into LDS, already rounded to fp16 and
//     in the element order of the A operand; two chunk buffers alternate;
//   - WC consumer wavefronts each take one super-block of the chunk for the TW
//     tiles; their weight loads run D chunks ahead in a ring of register buffers
//     and never wait behind an activation load.
// One s_barrier per chunk separates the staging of chunk q + 1 from the use of
// chunk q; it does not wait for outstanding memory loads, so the weight queues
// stay full across it. LDS row layout: buffer 0 holds columns 0..N-1, buffer 1
// columns N..2N-1, then one row of zeros, which lanes of columns past N (and every
// lane of a super-block past the end of K) read instead. Rows are padded by 16
// bytes so that the sixteen rows read by one instruction start in different banks.
template <int WC>
struct SwGeom {
    static constexpr int kRowBytes = (WC * 256 + 8) * 2;
};

template <int TW>
struct SwItem {
    uint4 hdr[TW];   // d, dmin, 12 scale bytes of this lane's row
    uint2 q[TW][4];  // quant words: sw_load's layout (bytes 8 (l / 16)..+7 of groups 0..3), or st_load's
};

template <int C, int TW>
QG_DEV void sw_load(SwItem<TW>& it, const SnTiles<TW>& tl, const SnLane<C, TW>& ln, int b) {
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int sb = b * 9 * 16 * tl.rt[t];
        const qg_u4v h = __builtin_amdgcn_raw_buffer_load_b128(tl.w[t], ln.hdr[t], sb, kNonTemporal);
        it.hdr[t] = make_uint4(h.x, h.y, h.z, h.w);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const qg_u2v q =
                __builtin_amdgcn_raw_buffer_load_b64(tl.w[t], ln.q[t], sb + (1 + 2 * g) * 16 * tl.rt[t], kNonTemporal);
            it.q[t][g] = make_uint2(q.x, q.y);
        }
    }
}

// One super-block for the TW tiles: a[c] is the LDS byte address of this lane's
// first A operand (column block c, sub-block 0).
template <int C, int TW>
QG_DEV void sw_dot(qg_f4 (&acc)[TW][C], const SwItem<TW>& it, const unsigned char* lds, const uint32_t (&a)[C]) {
    const qg_h8 ones = qg_ones_h8();
    const qg_f4 zero = {0.f, 0.f, 0.f, 0.f};
    // per tile: d (x 2^24: the quants enter as q * 2^-24), dmin and the 6-bit
    // scales and mins of the eight sub-blocks
    float dd[TW], dm[TW];
    uint32_t sc03[TW], m03[TW], sc47[TW], m47[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const uint4 hd = it.hdr[t];
        dd[t] = qg_half_lo(hd.x) * 16777216.0f;
        dm[t] = qg_half_hi(hd.x);
        sc03[t] = hd.y & 0x3f3f3f3fu;
        m03[t] = hd.z & 0x3f3f3f3fu;
        sc47[t] = (hd.w & 0x0f0f0f0fu) | ((hd.y >> 2) & 0x30303030u);
        m47[t] = ((hd.w >> 4) & 0x0f0f0f0fu) | ((hd.z >> 2) & 0x30303030u);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        qg_h8 a_lo[C], a_hi[C];
        qg_f4 x_lo[C], x_hi[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            a_lo[c] = *reinterpret_cast<const qg_h8*>(lds + a[c] + 128 * g);
            a_hi[c] = *reinterpret_cast<const qg_h8*>(lds + a[c] + 128 * g + 64);
            x_lo[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[c], ones, zero, 0, 0, 0);
            x_hi[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[c], ones, zero, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const uint32_t scw = g < 2 ? sc03[t] : sc47[t];
            const uint32_t mw = g < 2 ? m03[t] : m47[t];
            const int kb = 2 * (g & 1);
            const float s_lo = dd[t] * qg_byte_f(scw, kb);
            const float s_hi = dd[t] * 0.0625f * qg_byte_f(scw, kb + 1);
            const float m_lo = dm[t] * qg_byte_f(mw, kb);
            const float m_hi = dm[t] * qg_byte_f(mw, kb + 1);
            const uint32_t w0 = it.q[t][g].x, w1 = it.q[t][g].y;
            const uint32_t w0s = w0 >> 8, w1s = w1 >> 8;
            const qg_h8 b_lo = __builtin_bit_cast(
                qg_h8, make_uint4(w0 & 0x000f000fu, w0s & 0x000f000fu, w1 & 0x000f000fu, w1s & 0x000f000fu));
            const qg_h8 b_hi = __builtin_bit_cast(
                qg_h8, make_uint4(w0 & 0x00f000f0u, w0s & 0x00f000f0u, w1 & 0x00f000f0u, w1s & 0x00f000f0u));
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const qg_f4 s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[c], b_lo, zero, 0, 0, 0);
                const qg_f4 s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[c], b_hi, zero, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = acc[t][c][e];
                    v = fmaf(s_lo, s0[e], v);
                    v = fmaf(s_hi, s1[e], v);
                    v = fmaf(-m_lo, x_lo[c][e], v);
                    v = fmaf(-m_hi, x_hi[c][e], v);
                    acc[t][c][e] = v;
                }
            }
        }
    }
}

// Workgroup barrier for the chunk hand-over: LDS operations complete first; pending
// global loads are not waited for.
QG_DEV void sw_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Producer: activations of chunk q (super-blocks q WC .. q WC + WC - 1, the last
// chunk possibly shorter) into the LDS rows starting at `row0`. A pass covers CPP
// columns, lane pl taking 8-element group pl % LPC of column pl / LPC; PB passes
// have their loads in flight together.
template <int WC, int WP>
QG_DEV void sw_stage(unsigned char* lds, uint32_t row0, __amdgpu_buffer_rsrc_t xr, const SnProb& P, int q, int pl) {
    constexpr int RB = SwGeom<WC>::kRowBytes;
    constexpr int LPC = 32 * WC;  // 8-element groups per column and chunk
    static_assert((64 * WP) % LPC == 0, "producer lanes must cover whole chunk rows");
    constexpr int CPP = 64 * WP / LPC;
    constexpr int PB = 8;
    const int k0 = q * WC * 256;
    const int g8n = min(WC, P.nb - q * WC) * 32;
    const int g = pl % LPC;
    const int passes = (P.N + CPP - 1) / CPP;
    for (int p0 = 0; p0 < passes; p0 += PB) {
        float4 v[PB][2];
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int n = (p0 + j) * CPP + pl / LPC;
            const uint32_t off =
                (n < P.N && g < g8n) ? (uint32_t)(((int64_t)n * P.ldx + k0 + 8 * g) * 4) : kOutOfRange;
            v[j][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            v[j][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 16, 0));
        }
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int n = (p0 + j) * CPP + pl / LPC;
            if (n < P.N && g < g8n)
                *reinterpret_cast<qg_h8*>(lds + row0 + n * RB + 16 * g) = qg_a_operand(v[j][0], v[j][1]);
        }
    }
}

// The same staging split in two, for chunks that take a single round of PB passes
// (N <= PB * CPP): sw_issue requests chunk q's activations into registers,
// sw_write waits for them and stores them. The producer issues chunk q + 2 right
// after writing chunk q + 1, so the loads have a whole chunk interval to arrive.
template <int WC, int WP>
struct SwRegs {
    static constexpr int kPB = 8;
    float4 v[kPB][2];
};

template <int WC, int WP>
QG_DEV void sw_issue(SwRegs<WC, WP>& r, __amdgpu_buffer_rsrc_t xr, const SnProb& P, int q, int pl) {
    constexpr int LPC = 32 * WC;
    constexpr int CPP = 64 * WP / LPC;
    const int k0 = q * WC * 256;
    const int g8n = min(WC, P.nb - q * WC) * 32;
    const int g = pl % LPC;
#pragma unroll
    for (int j = 0; j < SwRegs<WC, WP>::kPB; ++j) {
        const int n = j * CPP + pl / LPC;
        const uint32_t off = (n < P.N && g < g8n) ? (uint32_t)(((int64_t)n * P.ldx + k0 + 8 * g) * 4) : kOutOfRange;
        r.v[j][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        r.v[j][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 16, 0));
    }
}

template <int WC, int WP>
QG_DEV void sw_write(const SwRegs<WC, WP>& r, unsigned char* lds, uint32_t row0, const SnProb& P, int q, int pl) {
    constexpr int RB = SwGeom<WC>::kRowBytes;
    constexpr int LPC = 32 * WC;
    constexpr int CPP = 64 * WP / LPC;
    const int g8n = min(WC, P.nb - q * WC) * 32;
    const int g = pl % LPC;
#pragma unroll
    for (int j = 0; j < SwRegs<WC, WP>::kPB; ++j) {
        const int n = j * CPP + pl / LPC;
        if (n < P.N && g < g8n) *reinterpret_cast<qg_h8*>(lds + row0 + n * RB + 16 * g) = qg_a_operand(r.v[j][0], r.v[j][1]);
    }
}

template <int C, int TW, int WC, int WP, int D>
__global__ __launch_bounds__(64 * (WC + WP)) void q4k_smalln_lds_kernel(SnArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int RB = SwGeom<WC>::kRowBytes;
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SnProb P = a.p[k];
    const int tile0 = (wg - P.wg_begin) * TW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nq = (P.nb + WC - 1) / WC;
    const uint32_t zrow = (uint32_t)(2 * P.N * RB);

    qg_f4 acc[TW][C];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[t][c] = qg_f4{0.f, 0.f, 0.f, 0.f};
    const int i = lane & 15, s = lane >> 4;

    if (wave >= WC) {
        // ---------------- producer
        const int pl = (wave - WC) * 64 + lane;
        for (int o = 16 * pl; o < RB; o += 16 * 64 * WP)
            *reinterpret_cast<uint4*>(lds + zrow + o) = make_uint4(0u, 0u, 0u, 0u);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + (int64_t)P.nb * 256) * 4), kQgRawBufferFlags);
        constexpr int CPP = 64 * WP / (32 * WC);
        if (P.N <= SwRegs<WC, WP>::kPB * CPP) {
            // one round per chunk: software-pipelined, loads one interval ahead
            SwRegs<WC, WP> r;
            sw_issue<WC, WP>(r, xr, P, 0, pl);
            sw_write<WC, WP>(r, lds, 0, P, 0, pl);
            if (1 < nq) sw_issue<WC, WP>(r, xr, P, 1, pl);
            sw_barrier();
            for (int q = 0; q < nq; q += D) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    // during chunk q + j: store chunk q + j + 1 (requested during the
                    // previous interval) into the other buffer, request chunk q + j + 2
                    const int qs = q + j + 1;
                    if (qs < nq) {
                        sw_write<WC, WP>(r, lds, (qs & 1) * P.N * RB, P, qs, pl);
                        if (qs + 1 < nq) sw_issue<WC, WP>(r, xr, P, qs + 1, pl);
                    }
                    sw_barrier();
                }
            }
        } else {
            sw_stage<WC, WP>(lds, 0, xr, P, 0, pl);
            sw_barrier();
            for (int q = 0; q < nq; q += D) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    // during chunk q + j: stage chunk q + j + 1 into the other buffer
                    if (q + j + 1 < nq) sw_stage<WC, WP>(lds, ((q + j + 1) & 1) * P.N * RB, xr, P, q + j + 1, pl);
                    sw_barrier();
                }
            }
        }
    } else {
        // ---------------- consumers: wavefront w takes super-block q WC + w of chunk q
        const int w = wave;
        SnTiles<TW> tl;
        SnLane<C, TW> ln;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int tc = min(tile0 + t, P.tiles - 1);
            tl.rt[t] = min(T, P.M - tc * T);
            tl.w[t] = __builtin_amdgcn_make_buffer_rsrc((void*)(P.w + (size_t)tc * T * P.nb * 144), (short)0,
                                                        tl.rt[t] * P.nb * 144, kQgRawBufferFlags);
            const uint32_t r = (uint32_t)min(i, tl.rt[t] - 1);
            ln.hdr[t] = 16 * r;
            ln.q[t] = 16 * r + 8 * (s & 1) + (uint32_t)(s >> 1) * 16 * tl.rt[t];
        }
        // this lane's A-operand byte offsets: column n = 16 c + i, elements
        // 256 w + 8 s.. of the chunk (+ 64 g, + 32 for the high sub-block)
        const uint32_t kw = (uint32_t)(256 * w + 8 * s) * 2;
        uint32_t a0[C], a1[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int n = 16 * c + i;
            a0[c] = (n < P.N ? (uint32_t)(n * RB) : zrow) + kw;
            a1[c] = (n < P.N ? (uint32_t)((P.N + n) * RB) : zrow) + kw;
        }
        const uint32_t az = zrow + kw;
        SwItem<TW> ring[D];
#pragma unroll
        for (int j = 0; j < D; ++j) sw_load<C, TW>(ring[j], tl, ln, min(j * WC + w, P.nb - 1));
        sw_barrier();
        for (int q = 0; q < nq; q += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const int qq = q + j;
                // a super-block past the end of K (or a chunk past the last) reads
                // the zero row: its products are exact zeros
                const bool valid = qq * WC + w < P.nb;
                uint32_t ad[C];
#pragma unroll
                for (int c = 0; c < C; ++c) ad[c] = valid ? ((qq & 1) ? a1[c] : a0[c]) : az;
                sw_dot<C, TW>(acc, ring[j], lds, ad);
                sw_load<C, TW>(ring[j], tl, ln, min((qq + D) * WC + w, P.nb - 1));
                sw_barrier();
            }
        }
    }

    // partial sums of the WC consumers meet in LDS (the chunk buffers are free now)
    float* red = reinterpret_cast<float*>(lds);
    if (wave < WC) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[(wave * TW * C * 4 + (t * C + c) * 4 + e) * 64 + lane] = acc[t][c][e];
    }
    sw_barrier();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        if (tile0 + t < P.tiles && i < min(T, P.M - (tile0 + t) * T)) {
            const int row = (tile0 + t) * T + i;
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = 16 * c + 4 * s + e;
                    if (n >= P.N) continue;
                    float v = red[((t * C + c) * 4 + e) * 64 + lane];
#pragma unroll
                    for (int w = 1; w < WC; ++w) v += red[(w * TW * C * 4 + (t * C + c) * 4 + e) * 64 + lane];
                    P.Y[(int64_t)n * P.ldy + row] = v;
                }
        }
    }
}

// Single-pass form for short K and few columns: when the activations of the whole
// K range fit in LDS (fp16, N rows and the zero row), every wavefront first
// requests its share of them, then the weights of all its super-blocks at once
// (W wavefronts take super-blocks w, w + W, ...; at most IMAX each), waits for the
// activations only, stores them converted to LDS, and after one barrier computes
// as the weights arrive: one memory round trip per workgroup, as in the GEMV.
constexpr int kS1Waves = 8, kS1Items = 2, kS1Cols = 8;

template <int C, int TW, int W, int IMAX>
__global__ __launch_bounds__(64 * W) void q4k_smalln_lds1_kernel(SnArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SnProb P = a.p[k];
    const int tile0 = (wg - P.wg_begin) * TW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    const int K = P.nb * 256;
    const int RB = (K + 8) * 2;  // bytes per LDS row
    const uint32_t zrow = (uint32_t)(P.N * RB);

    SnTiles<TW> tl;
    SnLane<C, TW> ln;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int tc = min(tile0 + t, P.tiles - 1);
        tl.rt[t] = min(T, P.M - tc * T);
        tl.w[t] = __builtin_amdgcn_make_buffer_rsrc((void*)(P.w + (size_t)tc * T * P.nb * 144), (short)0,
                                                    tl.rt[t] * P.nb * 144, kQgRawBufferFlags);
        const uint32_t r = (uint32_t)min(i, tl.rt[t] - 1);
        ln.hdr[t] = 16 * r;
        ln.q[t] = 16 * r + 8 * (s & 1) + (uint32_t)(s >> 1) * 16 * tl.rt[t];
    }

    // activation groups of 8 (column n, group g): thread tid takes group tid of every
    // column (the launcher guarantees K <= 512 W and N <= kS1Cols: a single round).
    // They are requested before the weights, so that waiting for them waits for
    // nothing else.
    const int tid = threadIdx.x;
    const int g = tid;
    const int gpr = K / 8;  // groups per column
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + K) * 4), kQgRawBufferFlags);
    float4 v[kS1Cols][2];
#pragma unroll
    for (int n = 0; n < kS1Cols; ++n) {
        const uint32_t off = (n < P.N && g < gpr) ? (uint32_t)(((int64_t)n * P.ldx + 8 * g) * 4) : kOutOfRange;
        v[n][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        v[n][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 16, 0));
    }
    SwItem<TW> items[IMAX];
#pragma unroll
    for (int j = 0; j < IMAX; ++j) sw_load<C, TW>(items[j], tl, ln, min(wave + j * W, P.nb - 1));
#pragma unroll
    for (int n = 0; n < kS1Cols; ++n)
        if (n < P.N && g < gpr) *reinterpret_cast<qg_h8*>(lds + n * RB + 16 * g) = qg_a_operand(v[n][0], v[n][1]);
    for (int o = 16 * tid; o < RB; o += 16 * 64 * W)
        *reinterpret_cast<uint4*>(lds + zrow + o) = make_uint4(0u, 0u, 0u, 0u);
    sw_barrier();

    qg_f4 acc[TW][C];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[t][c] = qg_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < IMAX; ++j) {
        // a super-block past the end of K reads the zero row: exact zeros
        const int b = wave + j * W;
        const uint32_t kb = (uint32_t)(256 * b + 8 * s) * 2;
        uint32_t ad[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int n = 16 * c + i;
            ad[c] = (b < P.nb && n < P.N) ? (uint32_t)(n * RB) + kb : zrow + (uint32_t)(16 * s);
        }
        sw_dot<C, TW>(acc, items[j], lds, ad);
    }

    // the W partial sums meet in LDS, after every wavefront is done with the
    // activations
    sw_barrier();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(wave * TW * C * 4 + (t * C + c) * 4 + e) * 64 + lane] = acc[t][c][e];
    sw_barrier();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        if (tile0 + t < P.tiles && i < min(T, P.M - (tile0 + t) * T)) {
            const int row = (tile0 + t) * T + i;
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = 16 * c + 4 * s + e;
                    if (n >= P.N) continue;
                    float v = red[((t * C + c) * 4 + e) * 64 + lane];
#pragma unroll
                    for (int w = 1; w < W; ++w) v += red[(w * TW * C * 4 + (t * C + c) * 4 + e) * 64 + lane];
                    P.Y[(int64_t)n * P.ldy + row] = v;
                }
        }
    }
}

// Streamed single-pass form, for the same shapes as the single-pass form when the
// batch has more tiles than the chip holds workgroups: the grid is sized to the
// resident workgroup slots, and workgroup j of a problem with G workgroups walks
// tiles j, j + G, j + 2G, ... (at most st_tiles(W)). The activations of the whole K
// range go to LDS once per workgroup, as in the single-pass form; the W
// wavefronts then take the (tile, super-block) units of the walk in turn, each
// with the next unit's loads in flight while one is computed, so a CU's weight
// stream does not stop between tiles and no partly filled last generation of
// workgroups is left at the end. A wavefront accumulates the units of one tile in
// registers and parks the sum in LDS when its walk moves to the next tile; the
// parked sums of the W wavefronts meet once, at the end, in a fixed order.
// LDS: the N activation rows (lanes of columns past N read column 0: their
// products only reach output columns that are not stored), the negated sub-block
// sums of the activations (K / 32 entries of 16 columns, those past N zero), then
// one parked sum per tile slot and wavefront, for the 32 lanes that hold columns
// 0..7 (N <= 8); a tile adds the parks of the wavefronts that had one of its units.
// Two shapes: W = 8 wavefronts, two workgroups per CU, at most 5 tiles each; and
// for batches of many tiles W = 16, one workgroup per CU, at most 10 tiles, which
// stages the activations once per CU instead of twice (7B gate/up, 2368 tiles:
// N = 5 about 21.5 -> 20.7 us, N = 8 24 -> 22).
constexpr int st_per_cu(int W) { return W >= 16 ? 1 : 2; }  // resident workgroups per CU
constexpr int st_tiles(int W) { return W >= 16 ? 10 : 5; }  // most tiles per workgroup
#ifndef QG_ST_RING
#define QG_ST_RING 2
#endif

// Loads of unit (tile t, super-block b) for the streamed, walk and slice forms;
// valid false: offsets past the resource, zeros without a memory access (so every
// load is still issued and the wait counts stay exact). The caller passes a tile
// inside the matrix either way. Lane (i, s) takes quant segments 1 + s and 5 + s
// of row i whole (two 16-byte loads instead of four 8-byte ones: the CU issues
// fewer load instructions per unit), so its words q[g], g = 2h + c, hold quant
// bytes 8c..8c+7 of segment 1 + s + 4h: weights 16 (s % 2) + 8c .. + 7 of group
// 2h + s / 2, low nibbles in sub-block 2 (2h + s / 2), high ones in the next.
// The products take the matching activations (st_alane) and scales (st_scale_sel).
QG_DEV void st_load(SwItem<1>& it, __amdgpu_buffer_rsrc_t wr, const SnProb& P, int t, int b, int i, int s,
                    bool valid) {
    const int rt = min(T, P.M - t * T);
    const uint32_t r = (uint32_t)min(i, rt - 1);
    const uint32_t vh = valid ? 16u * r : kOutOfRange;
    const uint32_t vq = valid ? 16u * r + (uint32_t)s * 16u * (uint32_t)rt : kOutOfRange;
    const int so = valid ? t * T * P.nb * 144 + b * 9 * 16 * rt : 0;
    const qg_u4v h = __builtin_amdgcn_raw_buffer_load_b128(wr, vh, so, kNonTemporal);
    it.hdr[0] = make_uint4(h.x, h.y, h.z, h.w);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const qg_u4v q = __builtin_amdgcn_raw_buffer_load_b128(wr, vq, so + (1 + 4 * h2) * 16 * rt, kNonTemporal);
        it.q[0][2 * h2] = make_uint2(q.x, q.y);
        it.q[0][2 * h2 + 1] = make_uint2(q.z, q.w);
    }
}

// LDS offset of lane (., s)'s activations within a super-block of an fp16
// activation row, for the words st_load gives it: the staged row holds, per
// group g of 64 weights (128 bytes), the 32 low-nibble weights and then the 32
// high-nibble ones, 8 per 16 bytes in the order the quant words unpack; word
// q[2h + c] of lane s is group 2h + s / 2, eight-weight chunk 2 (s % 2) + c,
// at 256 h + 16 c past this offset (+64 for the high nibbles).
QG_DEV uint32_t st_alane(int s) { return 128u * (uint32_t)(s >> 1) + 32u * (uint32_t)(s & 1); }

// v_perm selectors putting this lane's low- and high-nibble sub-block scales
// (bytes 2 (s / 2) and 2 (s / 2) + 1 of sc03 for words q[0], q[1], of sc47 for
// q[2], q[3]) into both 16-bit halves; sh = 8 s.
QG_DEV uint32_t st_scale_sel(uint32_t sh) {
    const uint32_t kb = (sh >> 3) & 2u;
    return 0x0c000c00u | (kb << 16) | kb;
}

// One super-block of one tile for the streamed form (a: this lane's activations in
// the super-block's LDS row, st_alane), with the sub-block scales inside the
// matrix-core operands:
//   - B carries q * sc_j instead of q (at most 15 * 63 = 945, still an exact fp16
//     subnormal, one packed 16-bit multiply per dword), so the eight products of
//     the super-block accumulate in the matrix core and d is applied once; each
//     lane scales its own sub-block, so one product may span two sub-blocks;
//   - the min term sum_j (dmin m_j) X_j[n] is a 16 x 16 x 8 product in fp32, two
//     v_mfma_f32_16x16x4_f32 with A = -X_j[n] from the workgroup's table (xt: byte
//     address of this lane's entry, column l % 16, sub-block l / 16) and B = dmin m_j
//     of this lane's row, accumulated into the same running sum as the products.
typedef unsigned short qg_u16x2 __attribute__((ext_vector_type(2)));

QG_DEV uint32_t st_mul16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(qg_u16x2, a) * __builtin_bit_cast(qg_u16x2, b));
}

// The top nibble of each 16-bit half (a packed 16-bit shift: no mask needed).
QG_DEV uint32_t st_hi4(uint32_t a) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(qg_u16x2, a) >> qg_u16x2{12, 12});
}

QG_DEV void st_dot2(qg_f4& acc, const SwItem<1>& it, const unsigned char* lds, uint32_t a, uint32_t xt, uint32_t sh) {
    const uint4 hd = it.hdr[0];
    const float dd = qg_half_lo(hd.x) * 16777216.0f;  // quants enter as q * 2^-24
    const float dm = qg_half_hi(hd.x);
    const uint32_t sc03 = hd.y & 0x3f3f3f3fu, m03 = hd.z & 0x3f3f3f3fu;
    const uint32_t sc47 = (hd.w & 0x0f0f0f0fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t m47 = ((hd.w >> 4) & 0x0f0f0f0fu) | ((hd.z >> 2) & 0x30303030u);
    // min term: B = dmin m_j, j = l / 16 (first product) and 4 + l / 16 (second)
    const float bm0 = dm * (float)((m03 >> sh) & 0xffu);
    const float bm1 = dm * (float)((m47 >> sh) & 0xffu);
    const float xa0 = *reinterpret_cast<const float*>(lds + xt);
    const float xa1 = *reinterpret_cast<const float*>(lds + xt + 256);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa0, bm0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa1, bm1, acc, 0, 0, 0);

    qg_f4 p = {0.f, 0.f, 0.f, 0.f};
    constexpr uint32_t M = 0x000f000fu;
    const uint32_t sel = st_scale_sel(sh);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t ao = 256u * (uint32_t)(g >> 1) + 16u * (uint32_t)(g & 1);
        const qg_h8 a_lo = *reinterpret_cast<const qg_h8*>(lds + a + ao);
        const qg_h8 a_hi = *reinterpret_cast<const qg_h8*>(lds + a + ao + 64);
        const uint32_t scw = g < 2 ? sc03 : sc47;
        // this lane's sub-block scales in both 16-bit halves
        const uint32_t s_lo = __builtin_amdgcn_perm(0u, scw, sel);
        const uint32_t s_hi = __builtin_amdgcn_perm(0u, scw, sel + 0x00010001u);
        const uint32_t w0 = it.q[0][g].x, w1 = it.q[0][g].y;
        const qg_h8 b_lo = __builtin_bit_cast(
            qg_h8, make_uint4(st_mul16(w0 & M, s_lo), st_mul16((w0 >> 8) & M, s_lo), st_mul16(w1 & M, s_lo),
                              st_mul16((w1 >> 8) & M, s_lo)));
        const qg_h8 b_hi = __builtin_bit_cast(
            qg_h8, make_uint4(st_mul16((w0 >> 4) & M, s_hi), st_mul16(st_hi4(w0), s_hi),
                              st_mul16((w1 >> 4) & M, s_hi), st_mul16(st_hi4(w1), s_hi)));
        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b_lo, p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b_hi, p, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(dd, p[e], acc[e]);
}

template <int W, int R>
__global__ __launch_bounds__(64 * W, 4) void q4k_smalln_stream_kernel(SnArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SnProb P = a.p[k];
    const int j = wg - P.wg_begin;
    const int G = P.wgs;
    const int nt = (P.tiles - j + G - 1) / G;  // tiles of this walk, 1..st_tiles(W)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, s = lane >> 4;
    const int nb = P.nb;
    const int K = nb * 256;
    const int RB = (K + 8) * 2;  // bytes per LDS row
    const uint32_t xsb = (uint32_t)(P.N * RB);  // sub-block sums -X_j[n], 16 columns per j
    qg_f4* park = reinterpret_cast<qg_f4*>(lds + xsb + 2 * K);
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.w, (short)0, P.M * nb * 144, kQgRawBufferFlags);

    // activations: thread tid takes 8-element group tid of every column (K <= 512 W);
    // wavefronts holding no group, and columns past N, issue no loads (the columns
    // past N only reach output columns that are not stored)
    const int tid = threadIdx.x;
    const int gpr = K / 8;
    const bool xw = 64 * wave < gpr;  // this wavefront holds activation groups
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + K) * 4), kQgRawBufferFlags);
    float4 v[kS1Cols][2];
#pragma unroll
    for (int n = 0; n < kS1Cols; ++n) {
        if (n < P.N && xw) {
            const uint32_t off = tid < gpr ? (uint32_t)(((int64_t)n * P.ldx + 8 * tid) * 4) : kOutOfRange;
            v[n][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            v[n][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 16, 0));
        }
    }

    // this wavefront's units: wave, wave + W, ... of the nt * nb units of the walk;
    // (lt, lb) is the tile slot and super-block of the unit being loaded
    const int U = nt * nb;
    const int niter = (U - wave + W - 1) / W;
    int lt = wave / nb, lb = wave - (wave / nb) * nb;
    auto advance = [&](int& t_, int& b_) {
        b_ += W;
        while (b_ >= nb) {
            b_ -= nb;
            ++t_;
        }
    };
    // a ring of R unit buffers: units 0..R-2 are requested before the activations
    // are stored
    const int t_first = lt, b_first = lb;
    SwItem<1> ring[R];
#pragma unroll
    for (int r = 0; r + 1 < R; ++r) {
        st_load(ring[r], wr, P, j + min(lt, nt - 1) * G, lb, i, s, r < niter);
        advance(lt, lb);
    }

    // fp16 activations, and the sums of each 32-element sub-block over the same
    // fp16 values (a quad of threads holds one sub-block of a column); the table's
    // columns past N are zeros
#pragma unroll
    for (int n = 0; n < kS1Cols; ++n) {
        if (n < P.N && xw) {
            const qg_h8 h = qg_a_operand(v[n][0], v[n][1]);
            if (tid < gpr) *reinterpret_cast<qg_h8*>(lds + n * RB + 16 * tid) = h;
            const uint4 hw = __builtin_bit_cast(uint4, h);
            const float xsum = qg_quad_sum(qg_sum_pairs4(hw.x, hw.y, hw.z, hw.w));
            if ((tid & 3) == 0 && tid < gpr) *reinterpret_cast<float*>(lds + xsb + ((tid >> 2) * 16 + n) * 4) = -xsum;
        } else if ((tid & 3) == 0 && tid < gpr) {
            *reinterpret_cast<float*>(lds + xsb + ((tid >> 2) * 16 + n) * 4) = 0.f;
        }
    }
    if ((tid & 3) == 0 && tid < gpr) {  // columns 8..15 of the table: zeros
        *reinterpret_cast<uint4*>(lds + xsb + ((tid >> 2) * 16 + 8) * 4) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(lds + xsb + ((tid >> 2) * 16 + 12) * 4) = make_uint4(0u, 0u, 0u, 0u);
    }
    sw_barrier();

    const uint32_t an = (uint32_t)((i < P.N ? i : 0) * RB) + st_alane(s);
    const uint32_t xtl = xsb + (uint32_t)(s * 16 + i) * 4;  // sub-block s of a super-block, column i
    const uint32_t msh = 8u * (uint32_t)s;
    qg_f4 cur[1][1] = {{qg_f4{0.f, 0.f, 0.f, 0.f}}};
    int ct = t_first, cb = b_first;  // unit being computed
    auto unit = [&](const SwItem<1>& it) {
        st_dot2(cur[0][0], it, lds, an + (uint32_t)(512 * cb), xtl + (uint32_t)(512 * cb), msh);
        const int pt = ct;
        advance(ct, cb);
        if (ct != pt) {  // the walk moves to the next tile: park this one's sum
            if (lane < 32) park[(pt * W + wave) * 32 + lane] = cur[0][0];
            cur[0][0] = qg_f4{0.f, 0.f, 0.f, 0.f};
        }
    };

    // Each step requests unit it + R - 1 and computes unit it. The loads are
    // unconditional (past the wavefront's last unit they read zeros) and the loop
    // has a single exit, so the loop-carried load state, and with it every wait
    // count, is exact: waiting for one unit never waits for a later one.
    for (int it = 0; it < niter; it += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            st_load(ring[(r + R - 1) % R], wr, P, j + min(lt, nt - 1) * G, lb, i, s, it + r + R - 1 < niter);
            advance(lt, lb);
            __builtin_amdgcn_sched_barrier(0);
            if (it + r < niter) unit(ring[r]);
        }
    }
    // (the position after a wavefront's last unit lies past the walk's last tile,
    // so every tile's sum has been parked)
    sw_barrier();
    if (wave >= nt) return;
    const int t = j + wave * G;
    const int rt = min(T, P.M - t * T);
    if (lane >= 32) return;
    // only wavefronts with a unit in this tile slot parked a sum for it: wavefront w
    // takes units w, w + W, ..., so it has one of the slot's units wave nb ..
    // wave nb + nb - 1 when nb >= W or when (w - wave nb) mod W < nb
    const int r0 = (wave * nb) % W;
    qg_f4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < W; ++w)
        if (nb >= W || (w - r0 + W) % W < nb) sum += park[(wave * W + w) * 32 + lane];
    if (i < rt) {
        const int row = t * T + i;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int n = 4 * s + e;
            if (n < P.N) P.Y[(int64_t)n * P.ldy + row] = sum[e];
        }
    }
}

// Chunked walk form, for batches of many tiles with up to 32 columns: one
// workgroup of 16 wavefronts per CU walks up to kWkTiles tiles (j, j + G, j + 2G,
// ...) chunk by chunk along K. The activations of a chunk of KC super-blocks (all N
// columns) are staged into LDS as fp16 once per workgroup, with the sums of their
// 32-element sub-blocks, one chunk ahead in two buffers, and serve every tile of
// the walk: a workgroup reads X once, not once per tile. In each chunk, wavefront w
// computes super-block w % KC of the chunk for the tile slots (w + 16 m) / KC, m =
// 0, 1, ...: the same tile slots in every chunk, so its per-tile sums stay in
// registers until the end, and with KC C = 4 the four SIMDs get equal work for any
// number of tiles. The weights of a wavefront's units in the next chunk are
// requested right after the same units of this chunk are computed. Products as in
// the streamed form (scales inside the matrix-core operands, the min term as an
// fp32 matrix-core product); every column block c of 16 columns reuses one B.
constexpr int kWkWaves = 16, kWkTiles = 10;
constexpr int64_t kWkAutoTiles = 1024;
constexpr int kSpMaxSlices = 16, kSpAutoCols = 3, kSpAutoK1 = 8192, kSpAutoColsShortK = 12;
constexpr size_t kSpCtrBytes = 4096;  // the workspace's counter block


template <int C, int KC_, int TMAX>
struct WkGeom {
    static constexpr int KC = KC_;                                     // super-blocks per chunk
    static constexpr int MU = (TMAX * KC + kWkWaves - 1) / kWkWaves;  // units per wavefront and chunk
    static constexpr int RB = (KC * 256 + 8) * 2;                          // bytes per activation row
    static constexpr int TB = KC * 8 * 16 * C * 4;                          // sub-block sum table bytes
    static constexpr int GC = KC * 32;                                      // 8-element groups per column
};

// Activations of chunk q of the K slice [kb0, kb1) (super-blocks) into registers:
// thread tid takes groups tid and tid + 1024 of the chunk (group g: column g / GC,
// elements 8 (g % GC)..+7 of the chunk; the launcher keeps N GC <= 2048). Groups past N or past the
// slice read zeros without a memory access.
template <int C, int KC_>
QG_DEV void wk_issue(float4 (&v)[2][2], __amdgpu_buffer_rsrc_t xr, const SnProb& P, int kb0, int kb1, int q,
                     int tid) {
    constexpr int KC = WkGeom<C, KC_, 1>::KC, GC = WkGeom<C, KC_, 1>::GC;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int g = tid + 1024 * r;
        const int n = g / GC, k8 = g % GC;
        const int kk = (kb0 + q * KC) * 256 + 8 * k8;
        const uint32_t off =
            (n < P.N && kk < kb1 * 256) ? (uint32_t)(((int64_t)n * P.ldx + kk) * 4) : kOutOfRange;
        v[r][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        v[r][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 16, 0));
    }
}

// ... and from registers into a chunk buffer: fp16 rows of RB bytes per column,
// then the table of -X_j[n] (16 C columns per sub-block j of the chunk, from the
// same fp16 values; a quad of threads holds one sub-block of a column).
template <int C, int KC_>
QG_DEV void wk_write(const float4 (&v)[2][2], unsigned char* buf, const SnProb& P, int tid) {
    constexpr int RB = WkGeom<C, KC_, 1>::RB, GC = WkGeom<C, KC_, 1>::GC;
    float* table = reinterpret_cast<float*>(buf + P.N * RB);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int g = tid + 1024 * r;
        const int n = g / GC, k8 = g % GC;
        const qg_h8 h = qg_a_operand(v[r][0], v[r][1]);
        if (n < P.N) *reinterpret_cast<qg_h8*>(buf + n * RB + 16 * k8) = h;
        const uint4 hw = __builtin_bit_cast(uint4, h);
        const float xs = qg_quad_sum(qg_sum_pairs4(hw.x, hw.y, hw.z, hw.w));
        if ((k8 & 3) == 0) table[(k8 >> 2) * 16 * C + n] = -xs;
    }
}

// One super-block of one tile for C column blocks, products as in st_dot2 (a[c]:
// LDS byte address of this lane's activations in the super-block of column block
// c, st_alane; xt: this lane's table entry, sub-block l / 16 of the super-block,
// column l % 16 of block 0).
template <int C>
QG_DEV void wk_dot(qg_f4 (&acc)[C], const SwItem<1>& it, const unsigned char* buf, const uint32_t (&a)[C],
                   uint32_t xt, uint32_t sh) {
    const uint4 hd = it.hdr[0];
    const float dd = qg_half_lo(hd.x) * 16777216.0f;  // quants enter as q * 2^-24
    const float dm = qg_half_hi(hd.x);
    const uint32_t sc03 = hd.y & 0x3f3f3f3fu, m03 = hd.z & 0x3f3f3f3fu;
    const uint32_t sc47 = (hd.w & 0x0f0f0f0fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t m47 = ((hd.w >> 4) & 0x0f0f0f0fu) | ((hd.z >> 2) & 0x30303030u);
    const float bm0 = dm * (float)((m03 >> sh) & 0xffu);
    const float bm1 = dm * (float)((m47 >> sh) & 0xffu);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const float xa0 = *reinterpret_cast<const float*>(buf + xt + 64 * c);
        const float xa1 = *reinterpret_cast<const float*>(buf + xt + 64 * c + 256 * C);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa0, bm0, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa1, bm1, acc[c], 0, 0, 0);
    }
    qg_f4 p[C];
#pragma unroll
    for (int c = 0; c < C; ++c) p[c] = qg_f4{0.f, 0.f, 0.f, 0.f};
    constexpr uint32_t M = 0x000f000fu;
    const uint32_t sel = st_scale_sel(sh);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t ao = 256u * (uint32_t)(g >> 1) + 16u * (uint32_t)(g & 1);
        const uint32_t scw = g < 2 ? sc03 : sc47;
        const uint32_t s_lo = __builtin_amdgcn_perm(0u, scw, sel);
        const uint32_t s_hi = __builtin_amdgcn_perm(0u, scw, sel + 0x00010001u);
        const uint32_t w0 = it.q[0][g].x, w1 = it.q[0][g].y;
        const qg_h8 b_lo = __builtin_bit_cast(
            qg_h8, make_uint4(st_mul16(w0 & M, s_lo), st_mul16((w0 >> 8) & M, s_lo), st_mul16(w1 & M, s_lo),
                              st_mul16((w1 >> 8) & M, s_lo)));
        const qg_h8 b_hi = __builtin_bit_cast(
            qg_h8, make_uint4(st_mul16((w0 >> 4) & M, s_hi), st_mul16(st_hi4(w0), s_hi),
                              st_mul16((w1 >> 4) & M, s_hi), st_mul16(st_hi4(w1), s_hi)));
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const qg_h8 a_lo = *reinterpret_cast<const qg_h8*>(buf + a[c] + ao);
            const qg_h8 a_hi = *reinterpret_cast<const qg_h8*>(buf + a[c] + ao + 64);
            p[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b_lo, p[c], 0, 0, 0);
            p[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b_hi, p[c], 0, 0, 0);
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[c][e] = fmaf(dd, p[c][e], acc[c][e]);
}

template <int C>
QG_DEV void wk_finish(qg_f4 (&sum)[C], unsigned char* lds, const SnProb& P, int j, int h, int nt, int G, int wave,
                      int lane);

// End of the walk and slice forms: the per-tile partial sums of the KC
// wavefronts of each tile meet in LDS (every wavefront has finished reading the
// activations), wavefront w < nt adds those of tile slot w, and the sums go to Y,
// or, for one of several K slices, to the workspace for the slices' last
// workgroup to add.
template <int C, int KC, int MU>
QG_DEV void wk_tail(const qg_f4 (&acc)[MU][C], unsigned char* lds, const SnProb& P, int j, int h, int nt, int G,
                    int wave, int lane) {
    qg_f4* park = reinterpret_cast<qg_f4*>(lds);
#pragma unroll
    for (int m = 0; m < MU; ++m) {
        const int u = wave + kWkWaves * m;
        if (u / KC < nt)
#pragma unroll
            for (int c = 0; c < C; ++c) park[(u * C + c) * 64 + lane] = acc[m][c];
    }
    sw_barrier();
    // wavefront w < nt owns tile slot w from here on
    qg_f4 sum[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        sum[c] = park[((min(wave, nt - 1) * KC) * C + c) * 64 + lane];
#pragma unroll
        for (int b2 = 1; b2 < KC; ++b2) sum[c] += park[((min(wave, nt - 1) * KC + b2) * C + c) * 64 + lane];
    }
    wk_finish<C>(sum, lds, P, j, h, nt, G, wave, lane);
}

// Sums of tile slot w < nt (wavefront w) to Y, or, for one of several K slices,
// to the workspace for the slices' last workgroup to add.
template <int C>
QG_DEV void wk_finish(qg_f4 (&sum)[C], unsigned char* lds, const SnProb& P, int j, int h, int nt, int G, int wave,
                      int lane) {
    const int i = lane & 15, s = lane >> 4;
    const int t = j + min(wave, nt - 1) * G;
    const int rt = min(T, P.M - t * T);
    if (P.part) {
        // One of several K slices. Its partial sums go to the workspace with
        // device-coherent stores; after every wavefront's stores have completed, one
        // lane counts the workgroup in on its tile group's counter, and the group's
        // last workgroup (which saw the others' arrivals, hence their completed
        // stores) adds the slices' partial sums in slice order with device-coherent
        // loads and writes Y, then returns the counter to zero. No workgroup waits
        // for another.
        // partial sums: one buffer resource over the problem's slices; cache policy
        // sc1 makes the stores and loads device-coherent (other XCDs' L2 caches are
        // not consulted)
        constexpr int kCoherent = 0x10;
        const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)P.part, (short)0, P.slices * P.tiles * C * 1024, kQgRawBufferFlags);
        // (only lanes holding real columns store and load)
        if (wave < nt)
#pragma unroll
            for (int c = 0; c < C; ++c)
                if (16 * c + 4 * s < P.N)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(qg_u4v, sum[c]), pr,
                                                       (uint32_t)lane * 16u,
                                                       ((h * P.tiles + t) * C + c) * 1024, kCoherent);
        __builtin_amdgcn_s_waitcnt(0);
        int* last = reinterpret_cast<int*>(lds);  // the parked sums have all been read
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t old = __hip_atomic_fetch_add(P.ctr + j, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *last = old == (uint32_t)(P.slices - 1);
            if (*last) __hip_atomic_store(P.ctr + j, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!*last || wave >= nt) return;
        // rounds of LS slices, the loads of every column block of a round in flight
        // at once (one memory round trip for up to LS slices), each column's sums
        // added in slice order
        constexpr int LS = kSpMaxSlices / C;
        qg_f4 v[C];
#pragma unroll
        for (int q = 0; q < C; ++q) {
            if (q * LS >= P.slices) break;
            qg_u4v pv[C][LS];
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int r = 0; r < LS; ++r) {
                    const int h2 = q * LS + r;
                    pv[c][r] = __builtin_amdgcn_raw_buffer_load_b128(
                        pr, h2 < P.slices && 16 * c + 4 * s < P.N ? (uint32_t)lane * 16u : kOutOfRange,
                        h2 < P.slices ? ((h2 * P.tiles + t) * C + c) * 1024 : 0, kCoherent);
                }
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int r = 0; r < LS; ++r) {
                    const int h2 = q * LS + r;
                    if (h2 == 0)
                        v[c] = __builtin_bit_cast(qg_f4, pv[c][0]);
                    else if (h2 < P.slices)
                        v[c] += __builtin_bit_cast(qg_f4, pv[c][r]);
                }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) sum[c] = v[c];
    }
    if (wave >= nt) return;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (i < rt) {
            const int row = t * T + i;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = 16 * c + 4 * s + e;
                if (n < P.N) P.Y[(int64_t)n * P.ldy + row] = sum[c][e];
            }
        }
    }
}

template <int C, int KC_, int TMAX>
__global__ __launch_bounds__(64 * kWkWaves, 4) void q4k_smalln_walk_kernel(SnArgs a) {
    using Gm = WkGeom<C, KC_, TMAX>;
    constexpr int KC = Gm::KC, MU = Gm::MU, RB = Gm::RB, TB = Gm::TB;
    extern __shared__ __align__(16) unsigned char lds[];
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SnProb P = a.p[k];
    const int G = P.wgs;
    const int j = P.hfast ? (wg - P.wg_begin) / P.slices : (wg - P.wg_begin) % G;  // tile group: tiles j, j + G, ...
    const int h = P.hfast ? (wg - P.wg_begin) % P.slices : (wg - P.wg_begin) / G;  // K slice
    const int nt = (P.tiles - j + G - 1) / G;  // tiles of this walk, 1..TMAX
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tid = threadIdx.x;
    const int i = lane & 15, s = lane >> 4;
    const int nb = P.nb;
    const int kb0 = h * P.slice_sbs, kb1 = min(nb, kb0 + P.slice_sbs);  // super-blocks of the slice
    const int nq = (kb1 - kb0 + KC - 1) / KC;
    const uint32_t BS = ((uint32_t)(P.N * RB + TB) + 15u) & ~15u;  // bytes per chunk buffer
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.w, (short)0, P.M * nb * 144, kQgRawBufferFlags);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + (int64_t)nb * 256) * 4), kQgRawBufferFlags);
    const int sb = wave % KC;  // this wavefront's super-block within every chunk

    // chunk 0: activations, and the weights of this wavefront's units
    float4 vx[2][2];
    wk_issue<C, KC>(vx, xr, P, kb0, kb1, 0, tid);
    SwItem<1> ring[MU];
#pragma unroll
    for (int m = 0; m < MU; ++m) {
        const int ts = (wave + kWkWaves * m) / KC;
        st_load(ring[m], wr, P, j + min(ts, nt - 1) * G, min(kb0 + sb, nb - 1), i, s, ts < nt && kb0 + sb < kb1);
    }
    wk_write<C, KC>(vx, lds, P, tid);
    sw_barrier();

    uint32_t an[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = 16 * c + i;
        an[c] = (uint32_t)((n < P.N ? n : 0) * RB + 512 * sb) + st_alane(s);
    }
    const uint32_t xt = (uint32_t)(P.N * RB) + (uint32_t)(((sb * 8 + s) * 16 * C + i) * 4);
    const uint32_t sh = 8u * (uint32_t)s;
    qg_f4 acc[MU][C];
#pragma unroll
    for (int m = 0; m < MU; ++m)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[m][c] = qg_f4{0.f, 0.f, 0.f, 0.f};

    for (int q = 0; q < nq; ++q) {
        const unsigned char* cur = lds + (q & 1) * BS;
        wk_issue<C, KC>(vx, xr, P, kb0, kb1, q + 1, tid);  // past the last chunk: zeros, no memory access
        const int b = kb0 + q * KC + sb;
#pragma unroll
        for (int m = 0; m < MU; ++m) {
            const int ts = (wave + kWkWaves * m) / KC;
            if (ts < nt && b < kb1) wk_dot<C>(acc[m], ring[m], cur, an, xt, sh);
            st_load(ring[m], wr, P, j + min(ts, nt - 1) * G, min(b + KC, nb - 1), i, s, ts < nt && b + KC < kb1);
        }
        wk_write<C, KC>(vx, lds + ((q + 1) & 1) * BS, P, tid);
        sw_barrier();
    }

    wk_tail<C, KC, MU>(acc, lds, P, j, h, nt, G, wave, lane);
}

// K-slice form for up to 16 columns (one column block): tile groups of TMAX
// tiles and K slices as in the walk form, but the activations of the whole slice
// (at most NG 8-element groups per thread: N times the slice's super-blocks at
// most 32 NG) are staged into LDS once, before any weight is requested, so that
// they arrive first, and the walk over the weights has no staging and no
// barrier. Wavefront w keeps tile slot w % TMAX and takes super-blocks w / TMAX,
// w / TMAX + 16 / TMAX, ... of the slice into one accumulator, the next
// super-block's weights in flight while it computes one. Slice h covers
// super-blocks [h nb / H, (h + 1) nb / H) of the H slices. Measured on the 7B
// down projection (N = 5): weights requested before the activations delay them
// (staged at 3.7 us instead of 2.2), and deeper weight queues (two to four units
// ahead) or units claimed through an LDS counter were slower (14.1 us against
// 15.0, 16.0, 16.7 and 15.2).
constexpr int kSlGroups = 5, kSlTiles = 4, kSl1Tiles = 2;

template <int TMAX, int NG>
__global__ __launch_bounds__(64 * kWkWaves, 4) void q4k_smalln_slice_kernel(SnArgs a) {
    constexpr int R = 2;  // units in the ring: one computed, one in flight
    static_assert(kWkWaves % TMAX == 0, "tile slots must divide the wavefronts");
    constexpr int SS = kWkWaves / TMAX;  // super-block stride of a wavefront
    extern __shared__ __align__(16) unsigned char lds[];
    const int wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int i = 1; i < QG_MAX_BATCH; ++i)
        if (i < a.count && wg >= a.begin[i]) k = i;
    const SnProb P = a.p[k];
    const int G = P.wgs;
    const int j = P.hfast ? (wg - P.wg_begin) / P.slices : (wg - P.wg_begin) % G;  // tile group: tiles j, j + G, ...
    const int h = P.hfast ? (wg - P.wg_begin) % P.slices : (wg - P.wg_begin) / G;  // K slice
    const int nt = (P.tiles - j + G - 1) / G;  // tiles of this walk, 1..TMAX
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tid = threadIdx.x;
    const int i = lane & 15, s = lane >> 4;
    const int nb = P.nb;
    const int kb0 = (int)((int64_t)h * nb / P.slices), kb1 = (int)((int64_t)(h + 1) * nb / P.slices);
    const int ns = kb1 - kb0;                            // super-blocks of the slice
    const int GS = 32 * ns;                              // 8-element groups per column of the slice
    const uint32_t RB = (uint32_t)(ns * 256 + 8) * 2;    // bytes per activation row
    const uint32_t XT = (uint32_t)P.N * RB;              // table of -X_j[n], 16 columns per sub-block
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.w, (short)0, P.M * nb * 144, kQgRawBufferFlags);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)P.X, (short)0, (int)(((int64_t)(P.N - 1) * P.ldx + (int64_t)nb * 256) * 4), kQgRawBufferFlags);
    const int ts = wave % TMAX, s0 = wave / TMAX;
    const int nu = ts < nt && s0 < ns ? (ns - s0 + SS - 1) / SS : 0;  // this wavefront's units
    const int t = j + min(ts, nt - 1) * G;

    // the slice's activations (group g: column g / GS, elements 8 (g % GS)..+7 of
    // the slice; groups past N columns read zeros without a memory access)
    float4 v[NG][2];
#pragma unroll
    for (int r = 0; r < NG; ++r) {
        const int g = tid + 64 * kWkWaves * r;
        const int n = g / GS, k8 = g - n * GS;
        const uint32_t off = n < P.N ? (uint32_t)(((int64_t)n * P.ldx + kb0 * 256 + 8 * k8) * 4) : kOutOfRange;
        v[r][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        v[r][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 16, 0));
    }
    SwItem<1> ring[R];
    // fp16 activations, and the sums of each 32-element sub-block over the same
    // fp16 values (a quad of threads holds one sub-block of a column)
    float* table = reinterpret_cast<float*>(lds + XT);
#pragma unroll
    for (int r = 0; r < NG; ++r) {
        const int g = tid + 64 * kWkWaves * r;
        const int n = g / GS, k8 = g - n * GS;
        const qg_h8 hx = qg_a_operand(v[r][0], v[r][1]);
        if (n < P.N) *reinterpret_cast<qg_h8*>(lds + n * RB + 16 * k8) = hx;
        const uint4 hw = __builtin_bit_cast(uint4, hx);
        const float xs = qg_quad_sum(qg_sum_pairs4(hw.x, hw.y, hw.z, hw.w));
        if (n < P.N && (k8 & 3) == 0) table[(k8 >> 2) * 16 + n] = -xs;
    }
    sw_barrier();
    // then the weights of this wavefront's first R - 1 units
#pragma unroll
    for (int r = 0; r + 1 < R; ++r)
        st_load(ring[r], wr, P, t, min(kb0 + s0 + SS * r, nb - 1), i, s, r < nu);

    const uint32_t an0 = (uint32_t)((i < P.N ? i : 0) * RB) + st_alane(s);
    const uint32_t xt0 = XT + (uint32_t)(s * 16 + i) * 4;
    const uint32_t sh = 8u * (uint32_t)s;
    qg_f4 acc[1] = {qg_f4{0.f, 0.f, 0.f, 0.f}};
    // Each step requests unit it + R - 1 and computes unit it. The loads are
    // unconditional (past the wavefront's last unit they read zeros without a
    // memory access), so every wait count is exact.
    for (int it = 0; it < nu; it += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int u = it + r;
            st_load(ring[(r + R - 1) % R], wr, P, t, min(kb0 + s0 + SS * (u + R - 1), nb - 1), i, s, u + R - 1 < nu);
            __builtin_amdgcn_sched_barrier(0);
            if (u < nu) {
                const uint32_t sl = (uint32_t)(s0 + SS * u);  // super-block within the slice
                const uint32_t an[1] = {an0 + 512u * sl};
                wk_dot<1>(acc, ring[r], lds, an, xt0 + 512u * sl, sh);
            }
        }
    }
    // wavefronts of one tile slot meet in LDS (every wavefront has finished
    // reading the activations)
    sw_barrier();
    qg_f4* park = reinterpret_cast<qg_f4*>(lds);
    park[wave * 64 + lane] = acc[0];
    sw_barrier();
    qg_f4 sum[1] = {park[min(wave, TMAX - 1) * 64 + lane]};
#pragma unroll
    for (int w2 = 1; w2 < SS; ++w2) sum[0] += park[(min(wave, TMAX - 1) + TMAX * w2) * 64 + lane];
    wk_finish<1>(sum, lds, P, j, h, nt, G, wave, lane);
}

// ------------------------------------------------------------------ host side
qg_status sn_validate(const void* w, const float* X, int64_t ldx, const float* Y, int64_t ldy, int64_t M, int64_t K,
                int64_t N) {
    if (!w || !X || !Y) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 256 (<= 2^24)", (long long)K);
    if (N < 1 || N > QG_SMALLN_MAX) return qg::fail(QG_ERR_SHAPE, "N=%lld not in [1, %d]", (long long)N, QG_SMALLN_MAX);
    if (ldx < K || ldy < M || ldx % 4 || ldy % 4)
        return qg::fail(QG_ERR_SHAPE, "ldx=%lld / ldy=%lld must be >= K / M and multiples of 4", (long long)ldx,
                        (long long)ldy);
    // the activations are read through one buffer resource whose 32-bit range must
    // stay below the out-of-range offset used for columns past N
    if ((N - 1) * ldx + K > INT32_MAX / 4) return qg::fail(QG_ERR_SHAPE, "X extent exceeds 2^31 bytes");
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
    P.slices = 1;
    P.hfast = 0;
    P.slice_sbs = P.nb;
    P.part = nullptr;
    P.ctr = nullptr;
    return P;
}

// Launch shape. TW tiles per wavefront: sharing one unit's activations among TW
// tiles divides the activation traffic (which for 16-row tiles exceeds the weight
// traffic once N > 2) by TW, at the price of TW times fewer workgroups: one tile
// up to 256 tiles in the batch (about one workgroup per CU), two above that, and
// for more than 16 columns four above 1024 tiles. W wavefronts per workgroup (up
// to 8, 4 with four tiles), each with at least two units. (Splitting K among
// workgroups, their partial sums meeting through atomic exchanges, was measured
// slower at every 7B shape: the device-scope round trips at the end of every
// workgroup cost more than the added parallelism gains.)
// Batches of at least this many tiles take the streamed form from three columns.
constexpr int64_t kStAutoTiles = 1024;

// Dynamic LDS of the streamed form: nmax activation rows and the parked sums.
size_t stream_lds_bytes(int nmax, int kmax, int W) {
    return (size_t)nmax * (kmax + 8) * 2 + 2 * (size_t)kmax + (size_t)st_tiles(W) * W * 32 * 16;
}

struct SnCfg {
    int W, TW;
    bool lds;   // chunked LDS-staged kernel
    int D;      // its weight-queue depth in chunks
    bool lds1;  // single-pass LDS kernel (short K, N <= 8)
    bool dot;   // vector-ALU dot-product kernel (N <= 8, q4k_smalln_dot.hip)
    int stream;   // streamed single-pass kernel (single-pass shapes): its wavefronts per workgroup, or 0
    bool walk;    // chunked walk kernel (many tiles, up to 32 columns)
    bool split;   // groups of tiles and K slices (workspace), the last workgroup of a group adding them
    bool slice;   // ... in the slice kernel where it fits, else in the walk kernel
    bool slice1;  // the slice kernel without K slices, groups of kSl1Tiles tiles
};
bool slice_plan_fits(const SnArgs& a, int cus);  // below, with the slice form's plan

SnCfg choose_cfg(const SnArgs& a, int C, bool ws, int cus) {
    const qg_launch_override& ov = qg::launch_override();
    const int form = ov.smalln_form;
    int units = INT_MAX;
    int64_t tiles = 0;
    int ncol = 0;
    for (int i = 0; i < a.count; ++i) {
        units = std::min(units, a.p[i].nb * 4);
        tiles += a.p[i].tiles;
        ncol = std::max(ncol, (int)a.p[i].N);
    }
    SnCfg c{1, tiles > 256 ? 2 : 1, false, 2, false, false, false, false, false, false, false};
    if (C == 2 && tiles > 1024) c.TW = 4;
    // Form selection, from measurements on the 7B shapes (stage times in us, register
    // form -> chosen form), in the order tested below:
    //   - with a workspace, K slices for few tiles and long K or many columns: the
    //     slice form where each slice's activations fit its staging, else the
    //     K-sliced walk (reasons and times beside the rule below);
    //   - the slice form without slices, two tiles per workgroup, for more tiles
    //     than CUs but at most twice as many (q/k/v, 4 to 8 columns);
    //   - the vector-ALU dot-product form for up to four columns (196 decode
    //     matrices, ms per step against the matrix-core forms: N = 1 0.93 / 1.57,
    //     2 1.13 / 1.58, 3 1.29 / 1.63, 4 1.52 / 1.67, 5 1.83 / 1.74);
    //   - the single-pass LDS form for K <= 4096 and N <= 8 (N = 5: q/k/v 9.05 ->
    //     8.75, o 6.85 -> 6.44, gate/up 29.7 -> 26.6), in its streamed variant
    //     (N = 5: q/k/v 8.86 -> 8.49, o 6.36 -> 5.48, gate/up 27.2 -> 21.1; N = 8
    //     gate/up 28.4 -> 23.4), with 16 wavefronts per workgroup from 1024 tiles;
    //   - the chunked LDS form for K >= 8192 (down projection: N = 5 23.6 -> 21.6,
    //     N = 32 72.3 -> 44.7) and for more than 16 columns over at most 1024 tiles
    //     (N = 32: q/k/v 18.2 -> 14.2, o 16.6 -> 12.0);
    //   - the chunked walk form for more columns over at least kWkAutoTiles tiles
    //     (N = 32 gate/up, 2368 tiles: 56.7 -> 28.3; with few tiles per CU it idles
    //     most of its wavefronts: N = 32 q/k/v 15.5 -> 32.9);
    //   - the register form otherwise (N = 5 short K: 29.7 against 37.0 for the
    //     chunked LDS form).
    // A launch override (qg_set_launch_override) can force a form within the range
    // it supports, and the launch shape.
    // the walk form reads the weights through one buffer resource per matrix
    bool wk = true;
    int kmin = INT_MAX;
    for (int i = 0; i < a.count; ++i) {
        wk = wk && (int64_t)a.p[i].M * a.p[i].nb * 144 < (int64_t)INT32_MAX;
        kmin = std::min(kmin, a.p[i].nb * 256);
    }
    // K slices need a workspace for their partial sums. Automatic choice: fewer
    // tiles than the many-tile walk takes, and two column blocks or long K
    // (measured on the 7B stages: N = 32 down 41.7 -> 22.2, q/k/v 15.3 -> 12.2; N = 16
    // down 30.2 -> 22.9, N = 8 down 20.1 -> 17.1, N = 5 down 19.6 -> 16.3, N = 4 down
    // 17.7 (dot form) -> 16.0; but N = 3 down 15.4 (dot) -> 16.0; with one column
    // block and short K the K-sliced walk lost: N = 16 q/k/v 11.2 -> 13.1, o 9.9 ->
    // 10.6), or one column block of at least kSpAutoColsShortK columns on short K
    // where the slice form's staging fits (q/k/v and o against the unsliced forms:
    // N = 12 10.1 -> 9.0 and 8.8 -> 8.4 us, N = 14 10.4 -> 9.5 and 9.1 -> 8.4, N = 16
    // 11.2 -> 9.5 and 9.9 -> 8.5; at N = 10 o went 8.1 -> 8.4)
    const bool short_slice = form == QG_FORM_AUTO && C == 1 && ncol >= kSpAutoColsShortK && kmin < kSpAutoK1;
    c.split = c.walk = ws && wk &&
                       (form == QG_FORM_SMALLN_SPLIT || form == QG_FORM_SMALLN_SLICE ||
                        (form == QG_FORM_AUTO && tiles < kWkAutoTiles && ncol >= kSpAutoCols &&
                         (C == 2 || kmin >= kSpAutoK1 || (short_slice && slice_plan_fits(a, cus)))));
    c.slice = c.split && form != QG_FORM_SMALLN_SPLIT;
    if (c.walk) return c;
    // The slice form without K slices, in groups of two tiles, for batches of more
    // tiles than CUs but at most twice as many, where the streamed form puts two
    // workgroups on some CUs (q/k/v, 288 tiles: N = 4 7.9 -> 7.3 us (dot form
    // before), N = 5 8.75 -> 7.3, N = 8 9.1 -> 7.8; N = 3 stays with the dot form,
    // 6.9 against 7.2); every problem's activations within the staging, and N <= 8
    // as measured. Forced without a workspace, it needs only the fit.
    bool s1fit = C == 1 && wk;
    for (int i = 0; i < a.count; ++i)
        s1fit = s1fit && (int64_t)a.p[i].N * a.p[i].nb * 32 <= (int64_t)kSlGroups * 64 * kWkWaves &&
                (int64_t)a.p[i].N * (a.p[i].nb * 256 + 8) * 2 + (int64_t)a.p[i].nb * 512 <= 160 * 1024;
    c.slice1 = s1fit && ((form == QG_FORM_AUTO && ncol >= 4 && ncol <= 8 && tiles > cus && tiles <= 2 * (int64_t)cus) ||
                         (form == QG_FORM_SMALLN_SLICE && !ws));
    if (c.slice1) return c;
    // (three and four columns over many tiles go to the streamed form below: gate/up,
    // 2368 tiles, N = 3 23.6 -> 20.7 us, N = 4 26.6 -> 20.1)
    const bool many_short = tiles >= kStAutoTiles && ncol >= 3;
    c.dot = (form == QG_FORM_AUTO && ncol <= 4 && !many_short) || (form == QG_FORM_SMALLN_DOT && ncol <= 8);
    if (c.dot) return c;
    c.walk = wk && form == QG_FORM_SMALLN_WALK;
    if (c.walk) return c;
    // Single-pass form: every problem with K <= 512 * 8 and N <= 8 (one round of
    // activation loads per lane, all super-blocks of a row in flight at once).
    bool s1 = C == 1;
    for (int i = 0; i < a.count; ++i)
        s1 = s1 && a.p[i].N <= kS1Cols && a.p[i].nb * 32 <= 64 * kS1Waves && a.p[i].nb <= kS1Items * kS1Waves;
    // the streamed form reads the weights through one buffer resource per matrix,
    // and its LDS must fit (automatic choice: two workgroups per CU)
    bool st = s1;
    int kmax = 0;
    for (int i = 0; i < a.count; ++i) {
        st = st && (int64_t)a.p[i].M * a.p[i].nb * 144 < (int64_t)INT32_MAX;
        kmax = std::max(kmax, a.p[i].nb * 256);
    }
    // automatic choice: the 16-wavefront shape for batches of many tiles, else the
    // 8-wavefront shape where two workgroups fit a CU's LDS; forced, the 8-wavefront
    // shape wherever its LDS fits
    const size_t st8 = stream_lds_bytes(ncol, kmax, 8), st16 = stream_lds_bytes(ncol, kmax, 16);
    if (st && form == QG_FORM_AUTO && tiles >= kStAutoTiles && st16 <= 160 * 1024)
        c.stream = 16;
    else if (st && ((form == QG_FORM_AUTO && st8 <= 160 * 1024 / st_per_cu(8)) ||
                    (form == QG_FORM_SMALLN_STREAM && st8 <= 160 * 1024)))
        c.stream = 8;
    if (c.stream) return c;
    c.lds1 = s1 && (form == QG_FORM_AUTO || form == QG_FORM_SMALLN_LDS1 || form == QG_FORM_SMALLN_STREAM);
    if (c.lds1) {
        c.TW = tiles > 1024 ? 2 : 1;
        if (ov.smalln_tiles == 1 || ov.smalln_tiles == 2) c.TW = ov.smalln_tiles;
        return c;
    }
    // many tiles, more columns than the single-pass forms take: the chunked walk
    c.walk = wk && form == QG_FORM_AUTO && tiles >= kWkAutoTiles;
    if (c.walk) return c;
    c.lds = form == QG_FORM_SMALLN_LDS ||
            (form != QG_FORM_SMALLN_REGS && (units >= 32 * 4 || (C == 2 && tiles <= 1024)));
    if (c.lds) {
        c.TW = tiles > 1024 || (C == 2 && tiles > 256) ? 2 : 1;
        c.D = 2;
        if (ov.smalln_tiles == 1 || ov.smalln_tiles == 2) c.TW = ov.smalln_tiles;
        if (ov.smalln_depth >= 2 && ov.smalln_depth <= (C == 2 ? 3 : 4)) c.D = ov.smalln_depth;
        return c;
    }
    // register form
    if (ov.smalln_tiles) c.TW = ov.smalln_tiles;
    const int wmax = c.TW == 4 ? 4 : 8;
    while (c.W < wmax && 2 * c.W <= units / 2) c.W *= 2;
    if (ov.smalln_waves && (ov.smalln_waves < 8 || c.TW < 4)) c.W = ov.smalln_waves;
    return c;
}

// Consumer and producer wavefronts per workgroup: eight consumers for up to 16
// columns, four above (the chunk buffers of 32 columns fill the LDS with four
// super-blocks per chunk); as many producers as stage a chunk of up to 16 / 32
// columns with one round of loads per lane.
template <int C>
constexpr int sw_consumers() {
    return C == 1 ? 8 : 4;
}
template <int C>
constexpr int sw_producers() {
    return C == 1 ? 4 : 8;
}

// Dynamic LDS of the LDS-staged kernel: two chunk buffers of N rows and the zero
// row, or the consumers' partial sums if larger.
size_t sw_lds_bytes(int C, int TW, int nmax) {
    const int WC = C == 1 ? sw_consumers<1>() : sw_consumers<2>();
    const size_t rb = (size_t)(WC * 256 + 8) * 2;
    return std::max((2 * (size_t)nmax + 1) * rb, (size_t)WC * TW * C * 4 * 64 * 4);
}

template <int C, int TW, int D>
void launch_lds(const SnArgs& a, int grid, size_t lds, hipStream_t s) {
    constexpr int WC = sw_consumers<C>();
    constexpr int WP = sw_producers<C>();
    const auto kern = q4k_smalln_lds_kernel<C, TW, WC, WP, D>;
    // the dynamic LDS limit is raised once per device (more than 64 KB are used)
    static std::atomic<bool> attr[64];
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr[dev].load(std::memory_order_acquire)) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * (WC + WP)), lds, s, a);
}

template <int TW>
void launch_s1(const SnArgs& a, int grid, size_t lds, hipStream_t s) {
    const auto kern = q4k_smalln_lds1_kernel<1, TW, kS1Waves, kS1Items>;
    static std::atomic<bool> attr[64];
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr[dev].load(std::memory_order_acquire)) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kS1Waves), lds, s, a);
}

template <int W>
void launch_stream(const SnArgs& a, int grid, size_t lds, hipStream_t s) {
    const auto kern = q4k_smalln_stream_kernel<W, QG_ST_RING>;
    static std::atomic<bool> attr[64];
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr[dev].load(std::memory_order_acquire)) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * W), lds, s, a);
}

// Workgroups per problem for the streamed form: the resident slots (per_cu
// workgroups per CU) shared in proportion to the tiles, at most tmax tiles
// per workgroup. Fills wg_begin, wgs and the compact begin array; returns the grid.
int64_t stream_grid(SnArgs& a, int cus, int per_cu, int tmax) {
    int64_t tiles = 0;
    for (int i = 0; i < a.count; ++i) tiles += a.p[i].tiles;
    const int64_t slots = per_cu * (int64_t)std::max(cus, 1);
    int64_t wgs = 0;
    for (int i = 0; i < a.count; ++i) {
        const int64_t t = a.p[i].tiles;
        int64_t g = (slots * t + tiles - 1) / tiles;
        g = std::max<int64_t>(g, qg::ceil_div(t, tmax));
        g = std::min<int64_t>(std::max<int64_t>(g, 1), t);
        a.p[i].wg_begin = (int32_t)wgs;
        a.p[i].wgs = (int32_t)g;
        a.begin[i] = (int32_t)wgs;
        wgs += g;
    }
    return wgs;
}

template <int C, int KC, int TMAX>
void launch_walk(const SnArgs& a, int grid, size_t lds, hipStream_t s) {
    const auto kern = q4k_smalln_walk_kernel<C, KC, TMAX>;
    static std::atomic<bool> attr[64];
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr[dev].load(std::memory_order_acquire)) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kWkWaves), lds, s, a);
}

// Walk-form shapes: column blocks, super-blocks per chunk, most tiles per
// workgroup, and tiles per group when K is sliced (KC C = 4 for up to 32 columns;
// KC = 8 for up to 8 columns, where groups of four tiles give every wavefront two
// units per chunk: N = 5 down projection 19.7 -> 16.7 us, against 18.9 with
// groups of two).
struct WkShape {
    int C, KC, TMAX, T;
};

// Dynamic LDS of the walk form: two chunk buffers, or the parked sums if larger.
size_t walk_lds_bytes(const WkShape& w, int nmax) {
    const size_t rb = (size_t)(w.KC * 256 + 8) * 2;
    const size_t tb = (size_t)w.KC * 8 * 16 * w.C * 4;
    const size_t bs = (nmax * rb + tb + 15) / 16 * 16;
    return std::max(2 * bs, (size_t)w.TMAX * w.KC * w.C * 1024);
}

WkShape walk_shape(int C, int nmax, bool split) {
    if (C == 2) return WkShape{2, 2, kWkTiles, 8};
    if (split && nmax <= 8) return WkShape{1, 8, 4, 4};
    return WkShape{1, 4, kWkTiles, 4};
}

// The slice form serves a batch whose every slice fits its activation staging
// and LDS.
size_t slice_lds_bytes(const SnArgs& a);
bool slice_fits(const SnArgs& a) {
    for (int i = 0; i < a.count; ++i)
        if ((int64_t)a.p[i].N * a.p[i].slice_sbs * 32 > (int64_t)kSlGroups * 64 * kWkWaves) return false;
    return slice_lds_bytes(a) <= 160 * 1024;
}

// Dynamic LDS of the slice form: the slice's activation rows and sub-block sums,
// or the parked sums if larger.
size_t slice_lds_bytes(const SnArgs& a) {
    size_t b = (size_t)kWkWaves * 1024;
    for (int i = 0; i < a.count; ++i) {
        const size_t ns = (size_t)a.p[i].slice_sbs;
        b = std::max(b, (size_t)a.p[i].N * (ns * 256 + 8) * 2 + ns * 512);
    }
    return b;
}

template <int TMAX, int NG>
void launch_slice(const SnArgs& a, int grid, size_t lds, hipStream_t s) {
    const auto kern = q4k_smalln_slice_kernel<TMAX, NG>;
    static std::atomic<bool> attr[64];
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr[dev].load(std::memory_order_acquire)) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kWkWaves), lds, s, a);
}

// Activation groups per thread the batch's slices need: three (the smaller
// instance, enough at N <= 5 on the 7B shapes) or kSlGroups; tmax tiles per group
// (kSlTiles with K slices, kSl1Tiles without).
void launch_slice_any(const SnArgs& a, int grid, int tmax, hipStream_t s) {
    int64_t g = 0;
    for (int i = 0; i < a.count; ++i) g = std::max<int64_t>(g, (int64_t)a.p[i].N * a.p[i].slice_sbs * 32);
    const size_t lds = slice_lds_bytes(a);
    const bool small = g <= 3 * 64 * kWkWaves;
    if (tmax == kSl1Tiles)
        small ? launch_slice<kSl1Tiles, 3>(a, grid, lds, s) : launch_slice<kSl1Tiles, kSlGroups>(a, grid, lds, s);
    else
        small ? launch_slice<kSlTiles, 3>(a, grid, lds, s) : launch_slice<kSlTiles, kSlGroups>(a, grid, lds, s);
}

// The slice form without K slices: groups of kSl1Tiles tiles, one workgroup each,
// writing Y directly. Fills wgs, slices, slice_sbs, wg_begin and begin; returns
// the grid.
int64_t slice1_grid(SnArgs& a) {
    int64_t wgs = 0;
    for (int i = 0; i < a.count; ++i) {
        SnProb& P = a.p[i];
        P.wgs = (int32_t)qg::ceil_div(P.tiles, kSl1Tiles);
        P.slices = 1;
        P.slice_sbs = P.nb;
        P.part = nullptr;
        P.ctr = nullptr;
        P.wg_begin = (int32_t)wgs;
        a.begin[i] = (int32_t)wgs;
        wgs += P.wgs;
    }
    return wgs;
}

void launch_walk_any(const WkShape& w, const SnArgs& a, int grid, int nmax, hipStream_t s) {
    const size_t lds = walk_lds_bytes(w, nmax);
    if (w.C == 2)
        launch_walk<2, 2, kWkTiles>(a, grid, lds, s);
    else if (w.KC == 8)
        launch_walk<1, 8, 4>(a, grid, lds, s);
    else
        launch_walk<1, 4, kWkTiles>(a, grid, lds, s);
}

// Tile groups and K slices of the walk form with a workspace: per problem, groups
// of w.T tiles (enough units per chunk for the 16 wavefronts), and as many K slices
// as give the problem its share of one workgroup per CU (at most kSpMaxSlices).
// Problems left with one slice write Y directly. Workspace: a block of
// kSpCtrBytes at its start for one counter per tile group of the sliced problems,
// then their partial sums. The counter block has the same place and size for every
// batch, so a call's counters always fall where earlier calls on the workspace,
// whatever their shapes, left zeros (their partial sums never reach it). A sliced
// problem has at least two slices, so G <= share / 2 tile groups, and the shares
// add up to at most CUs + count: (256 + 8) / 2 = 132 counters on MI355X, against
// the block's 1024. Fills wgs, slices, slice_sbs, part, ctr, wg_begin and begin;
// returns the grid and the workspace bytes, or -1 if the counters would not fit.
// Workgroup order of a sliced problem, and its slice count. Slice fastest, with a
// power-of-two slice count: with workgroups dealt to the XCDs in turn, each XCD
// then runs whole slices only, and its L2 fetches the activations of those
// slices instead of all of them. Measured on the 7B stages: the slice form (N = 5
// small-N step 1.053 -> 1.036 times its algorithmic bytes, down projection time
// unchanged) and the walk form on long K (N = 32 step 1.393 -> 1.268 times, down
// projection 23.0 -> 22.7 us); on q/k/v at N = 32 the fewer slices cost more than
// the traffic saves (12.4 -> 13.7 us), so the walk keeps its order there.
constexpr int kHfWalkNb = 32;  // the walk form's threshold: K >= 8192
int32_t hfast(bool slice, const SnProb& P) { return slice || P.nb >= kHfWalkNb; }

int64_t split_grid(SnArgs& a, int cus, const WkShape& w, void* ws, size_t* need, bool slice) {
    const int C = w.C;
    int64_t tiles = 0;
    for (int i = 0; i < a.count; ++i) tiles += a.p[i].tiles;
    int64_t wgs = 0;
    size_t nctr = 0, npart = 0;
    for (int i = 0; i < a.count; ++i) {
        SnProb& P = a.p[i];
        const int64_t G = qg::ceil_div(P.tiles, w.T);
        const int64_t share = std::max<int64_t>(1, (int64_t)std::max(cus, 1) * P.tiles / tiles);
        int64_t H = std::min<int64_t>({std::max<int64_t>(share / G, 1), kSpMaxSlices, P.nb});
        if (hfast(slice, P))
            while (H & (H - 1)) H &= H - 1;  // a power of two: each XCD then holds whole slices
        P.slice_sbs = (int32_t)qg::ceil_div(P.nb, H);
        H = qg::ceil_div(P.nb, P.slice_sbs);
        P.wgs = (int32_t)G;
        P.slices = (int32_t)H;
        P.hfast = hfast(slice, P);
        P.wg_begin = (int32_t)wgs;
        a.begin[i] = (int32_t)wgs;
        wgs += G * H;
        if (H > 1) {
            nctr += (size_t)G;
            npart += (size_t)H * P.tiles * C * 1024;
        }
    }
    if (nctr * 4 > kSpCtrBytes) return -1;
    const size_t ctr_bytes = kSpCtrBytes;
    size_t co = 0, po = ctr_bytes;
    for (int i = 0; i < a.count; ++i) {
        SnProb& P = a.p[i];
        P.part = nullptr;
        P.ctr = nullptr;
        if (P.slices > 1 && ws) {
            P.ctr = (uint32_t*)ws + co;
            P.part = (float*)((char*)ws + po);
        }
        if (P.slices > 1) {
            co += (size_t)P.wgs;
            po += (size_t)P.slices * P.tiles * C * 1024;
        }
    }
    *need = npart ? ctr_bytes + npart : 0;
    return wgs;
}

// Plan of a batch with a workspace: tile groups and K slices for the slice form
// where it may serve (one column block, every slice's activations within its
// staging), else for the walk form. Returns the grid; *slice tells which form.
int64_t split_plan(SnArgs& a, int cus, int C, int nmax, bool slice_ok, void* ws, size_t* need, bool* slice) {
    if (slice_ok && C == 1) {
        SnArgs b = a;
        const int64_t grid = split_grid(b, cus, WkShape{1, 8, kSlTiles, kSlTiles}, ws, need, true);
        if (grid >= 0 && slice_fits(b)) {
            a = b;
            *slice = true;
            return grid;
        }
    }
    *slice = false;
    return split_grid(a, cus, walk_shape(C, nmax, true), ws, need, false);
}

// Whether the slice form's plan (tile groups and K slices, one column block) fits
// every slice's activations in its staging.
bool slice_plan_fits(const SnArgs& a, int cus) {
    SnArgs b = a;
    size_t need = 0;
    return split_grid(b, cus, WkShape{1, 8, kSlTiles, kSlTiles}, nullptr, &need, true) >= 0 && slice_fits(b);
}

void launch_lds_any(const SnArgs& a, int grid, int C, int TW, int D, size_t lds, hipStream_t s) {
    switch (100 * C + 10 * TW + D) {
        case 112: launch_lds<1, 1, 2>(a, grid, lds, s); break;
        case 113: launch_lds<1, 1, 3>(a, grid, lds, s); break;
        case 114: launch_lds<1, 1, 4>(a, grid, lds, s); break;
        case 122: launch_lds<1, 2, 2>(a, grid, lds, s); break;
        case 123: launch_lds<1, 2, 3>(a, grid, lds, s); break;
        case 124: launch_lds<1, 2, 4>(a, grid, lds, s); break;
        case 212: launch_lds<2, 1, 2>(a, grid, lds, s); break;
        case 213: launch_lds<2, 1, 3>(a, grid, lds, s); break;
        case 222: launch_lds<2, 2, 2>(a, grid, lds, s); break;
        default: launch_lds<2, 2, 3>(a, grid, lds, s); break;
    }
}

template <int C, int TW>
void launch(const SnArgs& a, int grid, int W, hipStream_t s) {
    switch (W) {
        case 1: hipLaunchKernelGGL((q4k_smalln_kernel<C, TW, 1>), dim3(grid), dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((q4k_smalln_kernel<C, TW, 2>), dim3(grid), dim3(128), 0, s, a); break;
        case 4: hipLaunchKernelGGL((q4k_smalln_kernel<C, TW, 4>), dim3(grid), dim3(256), 0, s, a); break;
        default:
            if constexpr (TW < 4) hipLaunchKernelGGL((q4k_smalln_kernel<C, TW, 8>), dim3(grid), dim3(512), 0, s, a);
            break;
    }
}

// CUs of the current device (256, as on MI355X, where there is none: the plan a
// workspace query makes on the host matches the one a launch makes).
int plan_cus() {
    if (qg::check_device() == QG_OK) return qg::device_cus();
    qg::clear_error();
    return 256;
}

// Validates the problems and fills the kernel arguments and launch shape.
qg_status plan(const qg_gemm_problem* probs, int count, SnArgs& a, SnCfg& cfg, int& C, int64_t& wgs, int& nmax,
               bool ws = false) {
    if (!probs) return qg::fail(QG_ERR_NULL, "NULL problem list");
    if (count < 1 || count > QG_MAX_BATCH)
        return qg::fail(QG_ERR_SHAPE, "count=%d not in [1, %d]", count, QG_MAX_BATCH);
    a = SnArgs{};
    a.count = count;
    nmax = 0;
    for (int i = 0; i < count; ++i) {
        const qg_gemm_problem& q = probs[i];
        qg_status st = sn_validate(q.w_packed, q.X, q.ldx, q.Y, q.ldy, q.M, q.K, q.N);
        if (st) return st;
        a.p[i] = make_sn(q.w_packed, q.X, q.ldx, q.Y, q.ldy, q.M, q.K, q.N);
        nmax = std::max(nmax, a.p[i].N);
    }
    C = nmax > 16 ? 2 : 1;
    cfg = choose_cfg(a, C, ws, plan_cus());
    wgs = 0;
    for (int i = 0; i < count; ++i) {
        a.p[i].wg_begin = (int32_t)wgs;
        a.begin[i] = (int32_t)wgs;
        wgs += qg::ceil_div(a.p[i].tiles, cfg.TW);
    }
    if (wgs > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "too many tiles in one batch");
    return QG_OK;
}

// Workspace bytes the batch needs on the current device (0: none).
size_t split_bytes(const qg_gemm_problem* probs, int count) {
    SnArgs a;
    SnCfg cfg;
    int C, nmax;
    int64_t wgs;
    if (plan(probs, count, a, cfg, C, wgs, nmax, true) || !cfg.split) return 0;
    const int cus = plan_cus();
    size_t need = 0;
    bool slice = false;
    split_plan(a, cus, C, nmax, cfg.slice, nullptr, &need, &slice);
    return need;
}

qg_status run(const qg_gemm_problem* probs, int count, hipStream_t stream, void* ws = nullptr, size_t ws_bytes = 0,
              bool ws_mode = false) {
    SnArgs a;
    SnCfg cfg;
    int C, nmax;
    int64_t wgs;
    qg_status st = plan(probs, count, a, cfg, C, wgs, nmax, ws_mode);
    if (st) return st;
    st = qg::check_device();
    if (st) return st;
    if (cfg.split) {
        size_t need = 0;
        bool slice = false;
        const int64_t grid = split_plan(a, qg::device_cus(), C, nmax, cfg.slice, ws, &need, &slice);
        if (grid < 0) return qg::fail(QG_ERR_SHAPE, "more tile groups than the workspace's counter block holds");
        if (need > 0 && (!ws || ws_bytes < need))
            return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
        if (need > 0 && !qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
        if (slice)
            launch_slice_any(a, (int)grid, kSlTiles, stream);
        else
            launch_walk_any(walk_shape(C, nmax, true), a, (int)grid, nmax, stream);
        return qg::launch_status("qgemm_q4k_smalln_batch_ws");
    }
    if (cfg.slice1) {
        const int64_t grid = slice1_grid(a);
        launch_slice_any(a, (int)grid, kSl1Tiles, stream);
        return qg::launch_status("qgemm_q4k_smalln");
    }
    if (cfg.dot) return qg::smalln_dot_launch(probs, count, stream);
    if (cfg.lds) {
        launch_lds_any(a, (int)wgs, C, cfg.TW, cfg.D, sw_lds_bytes(C, cfg.TW, nmax), stream);
        return qg::launch_status("qgemm_q4k_smalln");
    }
    if (cfg.walk) {
        const WkShape w = walk_shape(C, nmax, false);
        const int64_t grid = stream_grid(a, qg::device_cus(), 1, w.TMAX);
        launch_walk_any(w, a, (int)grid, nmax, stream);
        return qg::launch_status("qgemm_q4k_smalln");
    }
    if (cfg.stream) {
        const int W = cfg.stream;
        const int64_t grid = stream_grid(a, qg::device_cus(), st_per_cu(W), st_tiles(W));
        int kmax = 0;
        for (int i = 0; i < count; ++i) kmax = std::max(kmax, a.p[i].nb * 256);
        if (W == 16)
            launch_stream<16>(a, (int)grid, stream_lds_bytes(nmax, kmax, 16), stream);
        else
            launch_stream<8>(a, (int)grid, stream_lds_bytes(nmax, kmax, 8), stream);
        return qg::launch_status("qgemm_q4k_smalln");
    }
    if (cfg.lds1) {
        int kmax = 0;
        for (int i = 0; i < count; ++i) kmax = std::max(kmax, a.p[i].nb * 256);
        const size_t lds = std::max((size_t)(nmax + 1) * (kmax + 8) * 2, (size_t)kS1Waves * cfg.TW * 4 * 64 * 4);
        if (cfg.TW == 2)
            launch_s1<2>(a, (int)wgs, lds, stream);
        else
            launch_s1<1>(a, (int)wgs, lds, stream);
        return qg::launch_status("qgemm_q4k_smalln");
    }
    const int key = 10 * C + cfg.TW;
    switch (key) {
        case 11: launch<1, 1>(a, (int)wgs, cfg.W, stream); break;
        case 12: launch<1, 2>(a, (int)wgs, cfg.W, stream); break;
        case 14: launch<1, 4>(a, (int)wgs, cfg.W, stream); break;
        case 21: launch<2, 1>(a, (int)wgs, cfg.W, stream); break;
        case 22: launch<2, 2>(a, (int)wgs, cfg.W, stream); break;
        default: launch<2, 4>(a, (int)wgs, cfg.W, stream); break;
    }
    return qg::launch_status("qgemm_q4k_smalln");
}

}  // namespace

extern "C" {

qg_status qgemm_q4k_smalln(const void* w, const float* X, int64_t ldx, float* Y, int64_t ldy, int64_t M, int64_t K,
                           int64_t N, qg_stream_t stream) {
    qg::clear_error();
    const qg_gemm_problem p{w, X, ldx, Y, ldy, M, K, N};
    return run(&p, 1, (hipStream_t)stream);
}

qg_status qgemm_q4k_smalln_batch(const qg_gemm_problem* problems, int count, qg_stream_t stream) {
    qg::clear_error();
    return run(problems, count, (hipStream_t)stream);
}

size_t qgemm_q4k_smalln_batch_workspace_bytes(const qg_gemm_problem* problems, int count) {
    qg::clear_error();
    return split_bytes(problems, count);
}

qg_status qgemm_q4k_smalln_batch_ws(const qg_gemm_problem* problems, int count, void* workspace,
                                    size_t workspace_bytes, qg_stream_t stream) {
    qg::clear_error();
    return run(problems, count, (hipStream_t)stream, workspace, workspace_bytes, true);
}

}  // extern "C"
