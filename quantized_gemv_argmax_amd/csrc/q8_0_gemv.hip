// Q8_0 weight-only GEMV and the fused LM-head projection + argmax for gfx950.
//
// Q8_0 (dotLLM README, Key Features / Performance: FP16, Q8_0, Q4_K_M blocks with
// fused scale x int dot products; news entry on the CUDA backend's quantized decode
// GEMV): a block is an fp16 scale d and 32 int8 quants, y_r += d * sum_l q_l x_l.
// The int8 quants are biased to unsigned bytes (q ^ 0x80 = q + 128) so one
// v_cvt_f32_ubyte converts each; the bias is removed per block with the block's
// activation sum: d * (sum (q+128) x - 128 * X).
//
// Fused LM head ("Why Local LLMs Don't Need C++ or Python", section 2: the final
// projection and the argmax reduction run on the device and only one int32 token
// id crosses to the host): each workgroup computes the logits of its 64-row tile
// in registers, reduces them to (max, lowest index) and writes one 8-byte partial;
// the last workgroup to finish (agent-scope ticket) reduces the partials in a
// fixed order and writes the winning index and its logit. The logits never reach
// HBM.
//
// Packed layout (same size as the canonical 34-byte block stream): rows in tiles
// of 64; eight consecutive blocks form a 256-weight macro-block of 17 sixteen-byte
// segments (segment 0: the eight fp16 scales; segment 1+2k+h: quants 16h..16h+15
// of block k). Segment s of macro-block mb of row i of a tile with rt rows sits at
//     tile_base + ((mb * 17 + s) * rt + i) * 16,   tile_base = tile * 64 * nbq * 34.
// When K/32 is not a multiple of 8, the remaining blocks of each row follow the
// macro-blocks of the tile, row after row, in canonical 34-byte form.
#include <algorithm>
#include <climits>

#include "qg_device.h"
#include "qg_host.h"

namespace {

struct Q8Prob {
    const uint8_t* w;
    const float* x;
    float* y;
    int32_t M, nbq, nmb, tb;  // rows, 32-blocks per row, macro-blocks, tail blocks
    int32_t tiles, splits;
};

// Half a macro-block: the scale segment and the 8 quant segments of blocks
// 4h..4h+3 (the scale segment is fetched for both halves; the second fetch hits
// the cache). Keeps the in-flight register footprint of a lane at 9 segments.
struct HalfMb {
    float2 xv;  // this lane's 2 activations of the half macro-block (block sums)
    uint4 s[9];
};

QG_DEV void load_half(HalfMb& d, const uint4* __restrict__ seg, const float* __restrict__ x, int unit, int rt,
                      int lane) {
    const int mb = unit >> 1, h = unit & 1;
    d.xv = *reinterpret_cast<const float2*>(x + 128 * unit + 2 * lane);
    const uint4* base = seg + (size_t)mb * 17 * rt;
    d.s[0] = base[0];
#pragma unroll
    for (int s = 0; s < 8; ++s) d.s[1 + s] = base[(size_t)(1 + 8 * h + s) * rt];
}

QG_DEV float blk_dot(const uint4 a, const uint4 b, qg_uniform_f32 xs) {
    const uint32_t qw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t u = qg_opaque(qw[i] ^ 0x80808080u);
        s = fmaf(qg_ub0(u), xs[4 * i + 0], s);
        s = fmaf(qg_ub1(u), xs[4 * i + 1], s);
        s = fmaf(qg_ub2(u), xs[4 * i + 2], s);
        s = fmaf(qg_ub3(u), xs[4 * i + 3], s);
    }
    return s;
}

// Sums of x over four 32-element blocks (lane t holds x[2t], x[2t+1]; lanes
// 16k..16k+15 cover block k).
struct QgSub4 {
    float v[4];
};
QG_DEV QgSub4 block_sums4(const float2 xv) {
    float s = xv.x + xv.y;
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
    s += __shfl_xor(s, 8, 64);
    QgSub4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r.v[k] = qg_readlane(s, 16 * k);
    return r;
}

// Dot of half a macro-block (Q8_0 blocks 4h..4h+3 of macro-block mb) with the
// 128 activations at xs / xb.
QG_DEV float half_dot(const HalfMb& d, int h, qg_uniform_f32 xs) {
    const QgSub4 X = block_sums4(d.xv);
    const uint32_t dw0 = h ? d.s[0].z : d.s[0].x;
    const uint32_t dw1 = h ? d.s[0].w : d.s[0].y;
    const float dk[4] = {qg_half_lo(dw0), qg_half_hi(dw0), qg_half_lo(dw1), qg_half_hi(dw1)};
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float sk = blk_dot(d.s[1 + 2 * k], d.s[2 + 2 * k], xs + 32 * k);
        acc = fmaf(dk[k], fmaf(-128.f, X.v[k], sk), acc);
    }
    return acc;
}

// Remaining (K/32 mod 8) blocks of one row, canonical 34-byte form, 2-byte aligned.
QG_DEV float tail_dot(const uint8_t* __restrict__ rowtail, int tb, qg_uniform_f32 xs) {
    float acc = 0.f;
    for (int k = 0; k < tb; ++k) {
        const uint8_t* blk = rowtail + 34 * k;
        const uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
        const float dk = (float)__builtin_bit_cast(_Float16, dbits);
        float s = 0.f;
        for (int l = 0; l < 32; ++l) s = fmaf((float)(int8_t)blk[2 + l], xs[32 * k + l], s);
        acc = fmaf(dk, s, acc);
    }
    return acc;
}

// Row dot product over the workgroup's macro-block range [m0, m1) plus (when
// with_tail) the tail blocks; W wavefronts split the range.
template <int W>
QG_DEV float row_partial(const Q8Prob& P, int tile, int m0, int m1, bool with_tail, int lane, int wave) {
    const int rt = min(qg::kTileRows, P.M - tile * qg::kTileRows);
    const bool active = lane < rt;
    const uint8_t* tbase = P.w + (size_t)tile * qg::kTileRows * P.nbq * 34;
    const uint4* __restrict__ seg = reinterpret_cast<const uint4*>(tbase) + (active ? lane : rt - 1);
    qg_uniform_f32 xs = (qg_uniform_f32)P.x;
    // units are half macro-blocks: [2*m0, 2*m1)
    const int u0 = 2 * m0, u1 = 2 * m1;
    const int wu0 = u0 + wave * (u1 - u0) / W;
    const int wu1 = u0 + (wave + 1) * (u1 - u0) / W;
    float acc = 0.f;
    if (wu0 < wu1) {
        HalfMb cur, nxt;
        load_half(cur, seg, P.x, wu0, rt, lane);
        for (int u = wu0; u < wu1 - 1; ++u) {
            load_half(nxt, seg, P.x, u + 1, rt, lane);
            acc += half_dot(cur, u & 1, xs + 128 * u);
            cur = nxt;
        }
        acc += half_dot(cur, (wu1 - 1) & 1, xs + 128 * (wu1 - 1));
    }
    if (with_tail && P.tb > 0 && wave == W - 1 && active) {
        const uint8_t* rowtail = tbase + (size_t)P.nmb * 17 * rt * 16 + (size_t)lane * P.tb * 34;
        acc += tail_dot(rowtail, P.tb, xs + 256 * P.nmb);
    }
    return acc;
}

template <int W>
QG_DEV float wg_reduce(float acc, int lane, int wave) {
    if constexpr (W == 1) {
        return acc;
    } else {
        __shared__ float red[W][64];
        red[wave][lane] = acc;
        __syncthreads();
        float v = red[0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[w][lane];
        return v;  // meaningful in wave 0
    }
}

template <int W>
__global__ __launch_bounds__(64 * W) void q8_0_gemv_kernel(Q8Prob P, float* __restrict__ part, uint32_t* cnt) {
    const int wg = blockIdx.x;
    const int tile = wg / P.splits;
    const int ks = wg - tile * P.splits;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m0 = (int)((int64_t)ks * P.nmb / P.splits);
    const int m1 = (int)((int64_t)(ks + 1) * P.nmb / P.splits);
    const float acc = row_partial<W>(P, tile, m0, m1, ks == P.splits - 1, lane, wave);
    const float v = wg_reduce<W>(acc, lane, wave);
    if (wave != 0) return;
    const int rt = min(qg::kTileRows, P.M - tile * qg::kTileRows);
    const bool active = lane < rt;
    const int row = tile * qg::kTileRows + lane;
    if (P.splits == 1) {
        if (active) P.y[row] = v;
        return;
    }
    if (active) part[(int64_t)ks * P.M + row] = v;
    __threadfence();
    const uint32_t old = qg_ticket(cnt + tile, lane);
    if (old != (uint32_t)(P.splits - 1)) return;
    __threadfence();
    if (active) {
        float s = 0.f;
        for (int j = 0; j < P.splits; ++j) s += __builtin_nontemporal_load(&part[(int64_t)j * P.M + row]);
        P.y[row] = s;
    }
    qg_ticket_reset(cnt + tile, lane);
}

// (value, index) pair ordering for the argmax: larger value wins, equal values go
// to the lower index; NaN (and inactive lanes) carry index INT_MAX and -inf.
QG_DEV bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

QG_DEV void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off, 64);
        const int oi = __shfl_xor(i, off, 64);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

template <int W>
__global__ __launch_bounds__(64 * W) void lmhead_argmax_kernel(Q8Prob P, float2* __restrict__ partials,
                                                                 uint32_t* cnt, int32_t* out_index,
                                                                 float* out_value) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float acc = row_partial<W>(P, tile, 0, P.nmb, true, lane, wave);
    float v = wg_reduce<W>(acc, lane, wave);
    if (wave != 0) return;
    const int rt = min(qg::kTileRows, P.M - tile * qg::kTileRows);
    int idx = tile * qg::kTileRows + lane;
    if (lane >= rt || v != v) {
        v = -__builtin_huge_valf();
        idx = INT_MAX;
    }
    wave_argmax(v, idx);
    if (lane == 0) partials[tile] = make_float2(v, __builtin_bit_cast(float, idx));
    __threadfence();
    const uint32_t old = qg_ticket(cnt, lane);
    if (old != (uint32_t)(gridDim.x - 1)) return;
    __threadfence();
    float bv = -__builtin_huge_valf();
    int bi = INT_MAX;
    for (int g = lane; g < (int)gridDim.x; g += 64) {
        const uint64_t raw = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(partials + g));
        const float gv = __builtin_bit_cast(float, (uint32_t)raw);
        const int gi = (int)(uint32_t)(raw >> 32);
        if (better(gv, gi, bv, bi)) {
            bv = gv;
            bi = gi;
        }
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
        out_index[0] = (bi == INT_MAX) ? -1 : bi;
        if (out_value) out_value[0] = bv;
    }
    qg_ticket_reset(cnt, lane);
}

__global__ void q8_0_pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t M, int nbq) {
    const int nmb = nbq / 8, tb = nbq % 8;
    const int64_t rowbytes = (int64_t)nbq * 34;
    const int64_t tile_bytes = (int64_t)qg::kTileRows * rowbytes;
    const int64_t total = M * rowbytes;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total; o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = o / tile_bytes;
        const int64_t in = o - t * tile_bytes;
        const int rt = (int)std::min<int64_t>(qg::kTileRows, M - t * qg::kTileRows);
        const int64_t macro = (int64_t)nmb * 17 * rt * 16;
        int64_t srcoff;
        if (in < macro) {
            const int64_t u = in / 16;
            const int e = (int)(in - u * 16);
            const int64_t ms = u / rt;  // mb * 17 + s
            const int i = (int)(u - ms * rt);
            const int64_t mb = ms / 17;
            const int s = (int)(ms - mb * 17);
            const int64_t r = t * qg::kTileRows + i;
            if (s == 0) {
                srcoff = r * rowbytes + (8 * mb + e / 2) * 34 + (e & 1);
            } else {
                const int k = (s - 1) / 2, hh = (s - 1) % 2;
                srcoff = r * rowbytes + (8 * mb + k) * 34 + 2 + 16 * hh + e;
            }
        } else {
            const int64_t in2 = in - macro;
            const int i = (int)(in2 / ((int64_t)tb * 34));
            const int64_t rem = in2 - (int64_t)i * tb * 34;
            const int64_t r = t * qg::kTileRows + i;
            srcoff = r * rowbytes + (int64_t)nmb * 8 * 34 + rem;
        }
        dst[o] = src[srcoff];
    }
}

int validate(const void* w, const float* x, int64_t M, int64_t K) {
    if (!w || !x) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "M=%lld out of range", (long long)M);
    if (K < 32 || K % 32 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "K=%lld must be a positive multiple of 32 (<= 2^24)", (long long)K);
    if (!qg::aligned16(w) || !qg::aligned16(x)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    return QG_OK;
}

Q8Prob make_prob(const void* w, const float* x, float* y, int64_t M, int64_t K) {
    Q8Prob P{};
    P.w = (const uint8_t*)w;
    P.x = x;
    P.y = y;
    P.M = (int32_t)M;
    P.nbq = (int32_t)(K / 32);
    P.nmb = P.nbq / 8;
    P.tb = P.nbq % 8;
    P.tiles = (int32_t)qg::ceil_div(M, qg::kTileRows);
    return P;
}

void plan_q8(Q8Prob& P, int* W) {
    int w = 2, wpt = 0, ew = 0, es = 0;
    if (qg::env_pair("QG_Q8_CFG", &ew, &es) && (ew == 1 || ew == 2 || ew == 4 || ew == 8) && es >= 1) {
        w = ew;
        wpt = es;
    }
    if (!wpt) wpt = (int)qg::ceil_div(2048, P.tiles);
    wpt = std::max(1, std::min(wpt, std::max(P.nmb, 1)));
    int splits = (int)qg::ceil_div(wpt, w);
    splits = std::max(1, std::min(splits, std::max(P.nmb, 1)));
    if (P.tiles > qg::kCounterSlots) splits = 1;
    P.splits = splits;
    *W = w;
}

size_t q8_ws_bytes(const Q8Prob& P) {
    if (P.splits <= 1) return 0;
    return (size_t)QG_WORKSPACE_COUNTER_BYTES + qg::align_up((size_t)P.splits * P.M * 4, 256);
}

int lm_W(const Q8Prob& P) {
    int w = 2, ew = 0, es = 0;
    if (qg::env_pair("QG_LM_CFG", &ew, &es) && (ew == 1 || ew == 2 || ew == 4 || ew == 8)) w = ew;
    (void)P;
    return w;
}

size_t lm_ws_bytes(const Q8Prob& P) {
    return (size_t)QG_WORKSPACE_COUNTER_BYTES + qg::align_up((size_t)P.tiles * 8, 256);
}

}  // namespace

extern "C" {

size_t qgemv_q8_0_workspace_bytes(int64_t M, int64_t K) {
    if (M < 1 || M > INT32_MAX || K < 32 || K % 32 || K > (1 << 24)) return 0;
    Q8Prob P = make_prob(nullptr, nullptr, nullptr, M, K);
    int W;
    plan_q8(P, &W);
    return q8_ws_bytes(P);
}

int qgemv_q8_0(const void* w, const float* x, float* y, int64_t M, int64_t K, void* ws, size_t ws_bytes,
               qg_stream_t stream) {
    qg::clear_error();
    int st = validate(w, x, M, K);
    if (st) return st;
    if (!y) return qg::fail(QG_ERR_NULL, "y is NULL");
    if (!qg::aligned16(y)) return qg::fail(QG_ERR_ALIGN, "y not 16-byte aligned");
    Q8Prob P = make_prob(w, x, y, M, K);
    int W;
    plan_q8(P, &W);
    const size_t need = q8_ws_bytes(P);
    if (need) {
        if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
        if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
        if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    }
    st = qg::check_device();
    if (st) return st;
    uint32_t* cnt = (uint32_t*)ws;
    float* part = need ? (float*)((uint8_t*)ws + QG_WORKSPACE_COUNTER_BYTES) : nullptr;
    const dim3 grid(P.tiles * P.splits);
    hipStream_t s = (hipStream_t)stream;
    switch (W) {
        case 1: hipLaunchKernelGGL(q8_0_gemv_kernel<1>, grid, dim3(64), 0, s, P, part, cnt); break;
        case 2: hipLaunchKernelGGL(q8_0_gemv_kernel<2>, grid, dim3(128), 0, s, P, part, cnt); break;
        case 4: hipLaunchKernelGGL(q8_0_gemv_kernel<4>, grid, dim3(256), 0, s, P, part, cnt); break;
        default: hipLaunchKernelGGL(q8_0_gemv_kernel<8>, grid, dim3(512), 0, s, P, part, cnt); break;
    }
    return qg::launch_status("qgemv_q8_0");
}

size_t lmhead_argmax_workspace_bytes(int64_t M, int64_t K) {
    if (M < 1 || M > INT32_MAX || K < 32 || K % 32 || K > (1 << 24)) return 0;
    Q8Prob P = make_prob(nullptr, nullptr, nullptr, M, K);
    return lm_ws_bytes(P);
}

int lmhead_argmax(const void* w, const float* x, int64_t M, int64_t K, void* ws, size_t ws_bytes,
                  int32_t* out_index, float* out_value, qg_stream_t stream) {
    qg::clear_error();
    int st = validate(w, x, M, K);
    if (st) return st;
    if (!out_index) return qg::fail(QG_ERR_NULL, "out_index is NULL");
    if ((reinterpret_cast<uintptr_t>(out_index) & 3) || (reinterpret_cast<uintptr_t>(out_value) & 3))
        return qg::fail(QG_ERR_ALIGN, "outputs must be 4-byte aligned");
    Q8Prob P = make_prob(w, x, nullptr, M, K);
    P.splits = 1;
    const size_t need = lm_ws_bytes(P);
    if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    st = qg::check_device();
    if (st) return st;
    uint32_t* cnt = (uint32_t*)ws;
    float2* partials = (float2*)((uint8_t*)ws + QG_WORKSPACE_COUNTER_BYTES);
    const dim3 grid(P.tiles);
    hipStream_t s = (hipStream_t)stream;
    switch (lm_W(P)) {
        case 1: hipLaunchKernelGGL(lmhead_argmax_kernel<1>, grid, dim3(64), 0, s, P, partials, cnt, out_index, out_value); break;
        case 2: hipLaunchKernelGGL(lmhead_argmax_kernel<2>, grid, dim3(128), 0, s, P, partials, cnt, out_index, out_value); break;
        case 4: hipLaunchKernelGGL(lmhead_argmax_kernel<4>, grid, dim3(256), 0, s, P, partials, cnt, out_index, out_value); break;
        default: hipLaunchKernelGGL(lmhead_argmax_kernel<8>, grid, dim3(512), 0, s, P, partials, cnt, out_index, out_value); break;
    }
    return qg::launch_status("lmhead_argmax");
}

int qg_pack_q8_0(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream) {
    qg::clear_error();
    if (!src || !dst) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX || K < 32 || K % 32 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "invalid Q8_0 shape M=%lld K=%lld", (long long)M, (long long)K);
    if (!qg::aligned16(src) || !qg::aligned16(dst)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t bytes = qg_q8_0_bytes(M, K);
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    if (s8 < d8 + bytes && d8 < s8 + bytes) return qg::fail(QG_ERR_SHAPE, "src and dst overlap");
    int st = qg::check_device();
    if (st) return st;
    const int blocks = (int)std::min<int64_t>(qg::ceil_div((int64_t)bytes, 256), 65536);
    hipLaunchKernelGGL(q8_0_pack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)src,
                       (uint8_t*)dst, M, (int)(K / 32));
    return qg::launch_status("qg_pack_q8_0");
}

}  // extern "C"
