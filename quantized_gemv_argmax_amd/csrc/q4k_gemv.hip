// Q4_K weight-only GEMV for gfx950 (CDNA4), plus the Q4_K load-time repack.
//
// Method (dotLLM README: Key Features / Performance, "Quantized inference" with
// fused scale x int dot products run on the quantized blocks; news entries
// "Q4_K_M dequantization and vec_dot kernels" and "CUDA GPU backend ... custom
// quantized GEMV for decode"): for row r and super-block b, with sub-block j of
// 32 weights,
//     y_r += d * sum_j sc_j * S_j  -  dmin * sum_j m_j * X_j,
//     S_j = sum_l q_{j,l} x_{256b+32j+l},   X_j = sum_l x_{256b+32j+l},
// which equals sum_k (d*sc*q - dmin*m) * x_k. The mins are applied through the
// per-sub-block activation sums, as the README's "precomputed block sums" of the
// Q8_1 / Q8_K input path do.
//
// Packed layout (a same-size byte permutation of the canonical row-major block
// stream; cf. the README's load-time row-interleaved repacking): rows are grouped
// in tiles of 64. A super-block is 9 sixteen-byte segments (segment 0: d, dmin and
// the 12 scale bytes; segment 1+p: quant bytes 16p..16p+15). Within a tile of rt
// rows, segment s of super-block b of row i sits at
//     tile_base + ((b * 9 + s) * rt + i) * 16,   tile_base = tile * 64 * nb * 144,
// so one wavefront (lane = row) reading one segment issues a single contiguous
// 1 KiB request, and a wavefront's super-block is one contiguous 9 KiB run.
//
// Work decomposition: a workgroup of W wavefronts owns one row tile and a range
// of super-blocks; its wavefronts split that range, every lane accumulates its
// own row. Activations are wavefront-uniform and come through scalar loads.
// When a tile's K range is split over several workgroups (to fill 256 CUs with
// narrow matrices), partial sums go to the workspace and the last workgroup to
// arrive (an agent-scope ticket per tile) adds them in a fixed order, so the
// result is deterministic.
#include <algorithm>

#include "qg_device.h"
#include "qg_host.h"

namespace {

struct Q4Prob {
    const uint8_t* w;
    const float* x;
    float* y;
    int32_t M, nb, tiles, splits;
    int32_t wg_begin, cnt_base;
    int64_t part_off;  // floats, into the workspace partial area
};

struct Q4Args {
    Q4Prob p[QG_MAX_BATCH];
    float* part;
    uint32_t* cnt;
    int32_t count;
};

struct SbData {
    float4 xv;  // this lane's 4 activations of the super-block (for the sub-block sums)
    uint4 s[9];
};

QG_DEV void load_sb(SbData& d, const uint4* __restrict__ seg, const float* __restrict__ xb, int rt, int lane) {
    d.xv = qg_x4(xb, lane);
#pragma unroll
    for (int s = 0; s < 9; ++s) d.s[s] = seg[s * rt];
}

// Dot product of one super-block row segment set with x[256b .. 256b+255].
QG_DEV float sb_dot(const SbData& d, qg_uniform_f32 xs) {
    const QgSub8 X = qg_subblock_sums(d.xv);
    float S[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) S[j] = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int g = p >> 1, h = p & 1;
        qg_uniform_f32 xl = xs + 64 * g + 16 * h;  // low nibbles: sub-block 2g
        qg_uniform_f32 xh = xl + 32;               // high nibbles: sub-block 2g+1
        const uint32_t qw[4] = {d.s[1 + p].x, d.s[1 + p].y, d.s[1 + p].z, d.s[1 + p].w};
        float lo = S[2 * g], hi = S[2 * g + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t l4 = qg_opaque(qw[i] & 0x0f0f0f0fu);
            const uint32_t h4 = qg_opaque(qw[i] & 0xf0f0f0f0u);  // 16 * q per byte
            lo = fmaf(qg_ub0(l4), xl[4 * i + 0], lo);
            lo = fmaf(qg_ub1(l4), xl[4 * i + 1], lo);
            lo = fmaf(qg_ub2(l4), xl[4 * i + 2], lo);
            lo = fmaf(qg_ub3(l4), xl[4 * i + 3], lo);
            hi = fmaf(qg_ub0(h4), xh[4 * i + 0], hi);
            hi = fmaf(qg_ub1(h4), xh[4 * i + 1], hi);
            hi = fmaf(qg_ub2(h4), xh[4 * i + 2], hi);
            hi = fmaf(qg_ub3(h4), xh[4 * i + 3], hi);
        }
        S[2 * g] = lo;
        S[2 * g + 1] = hi;
    }
    const uint4 hd = d.s[0];
    const float dd = qg_half_lo(hd.x), dm = qg_half_hi(hd.x);
    const QgScales sc = qg_q4k_scales(hd.y, hd.z, hd.w);
    // even sub-blocks come from low nibbles, odd ones from high nibbles (x16)
    float te = qg_ub0(sc.sc03) * S[0];
    te = fmaf(qg_ub2(sc.sc03), S[2], te);
    te = fmaf(qg_ub0(sc.sc47), S[4], te);
    te = fmaf(qg_ub2(sc.sc47), S[6], te);
    float to = qg_ub1(sc.sc03) * S[1];
    to = fmaf(qg_ub3(sc.sc03), S[3], to);
    to = fmaf(qg_ub1(sc.sc47), S[5], to);
    to = fmaf(qg_ub3(sc.sc47), S[7], to);
    const float t = fmaf(to, 0.0625f, te);
    float mn = qg_ub0(sc.m03) * X.v[0];
    mn = fmaf(qg_ub1(sc.m03), X.v[1], mn);
    mn = fmaf(qg_ub2(sc.m03), X.v[2], mn);
    mn = fmaf(qg_ub3(sc.m03), X.v[3], mn);
    mn = fmaf(qg_ub0(sc.m47), X.v[4], mn);
    mn = fmaf(qg_ub1(sc.m47), X.v[5], mn);
    mn = fmaf(qg_ub2(sc.m47), X.v[6], mn);
    mn = fmaf(qg_ub3(sc.m47), X.v[7], mn);
    return fmaf(dd, t, -dm * mn);
}

template <int W>
__global__ __launch_bounds__(64 * W) void q4k_gemv_kernel(Q4Args a) {
    const int wg = blockIdx.x;
    int k = 0;
    for (int i = 1; i < a.count; ++i)
        if (wg >= a.p[i].wg_begin) k = i;
    const Q4Prob P = a.p[k];

    const int local = wg - P.wg_begin;
    const int tile = local / P.splits;
    const int ks = local - tile * P.splits;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.nb;
    const int rt = min(qg::kTileRows, P.M - tile * qg::kTileRows);
    const bool active = lane < rt;
    const int row = tile * qg::kTileRows + lane;

    const int b0 = (int)((int64_t)ks * nb / P.splits);
    const int b1 = (int)((int64_t)(ks + 1) * nb / P.splits);
    const int wb0 = b0 + wave * (b1 - b0) / W;
    const int wb1 = b0 + (wave + 1) * (b1 - b0) / W;

    // lanes past a ragged tile's end re-read the tile's last row (no divergent
    // branches around the loads, so the loads stay counted and pipelined)
    const uint4* __restrict__ seg =
        reinterpret_cast<const uint4*>(P.w + (size_t)tile * qg::kTileRows * nb * 144) + (active ? lane : rt - 1);
    qg_uniform_f32 xs = (qg_uniform_f32)P.x;

    float acc = 0.f;
    if (wb0 < wb1) {
        SbData cur, nxt;
        load_sb(cur, seg + (size_t)wb0 * 9 * rt, P.x + 256 * wb0, rt, lane);
        for (int b = wb0; b < wb1 - 1; ++b) {
            load_sb(nxt, seg + (size_t)(b + 1) * 9 * rt, P.x + 256 * (b + 1), rt, lane);
            acc += sb_dot(cur, xs + 256 * b);
            cur = nxt;
        }
        acc += sb_dot(cur, xs + 256 * (wb1 - 1));
    }

    float v = acc;
    if constexpr (W > 1) {
        __shared__ float red[W][64];
        red[wave][lane] = acc;
        __syncthreads();
        if (wave != 0) return;
        v = red[0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[w][lane];
    }

    if (P.splits == 1) {
        if (active) P.y[row] = v;
        return;
    }
    float* part = a.part + P.part_off;
    if (active) part[(int64_t)ks * P.M + row] = v;
    __threadfence();
    uint32_t* cnt = a.cnt + P.cnt_base + tile;
    const uint32_t old = qg_ticket(cnt, lane);
    if (old != (uint32_t)(P.splits - 1)) return;
    __threadfence();
    if (active) {
        float s = 0.f;
        for (int j = 0; j < P.splits; ++j) s += __builtin_nontemporal_load(&part[(int64_t)j * P.M + row]);
        P.y[row] = s;
    }
    qg_ticket_reset(cnt, lane);
}

__global__ void q4k_pack_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t M, int nb) {
    const int64_t units = M * nb * 9;
    const int64_t tile_units = (int64_t)qg::kTileRows * nb * 9;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < units;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = o / tile_units;
        const int64_t in = o - t * tile_units;
        const int rt = (int)std::min<int64_t>(qg::kTileRows, M - t * qg::kTileRows);
        const int64_t bs = in / rt;  // b * 9 + s
        const int i = (int)(in - bs * rt);
        const int64_t r = t * qg::kTileRows + i;
        dst[o] = src[r * nb * 9 + bs];
    }
}

// Launch plan for a batch of Q4_K GEMVs.
struct Plan {
    int W = 2;
    int total_wg = 0;
    int64_t part_floats = 0;
    int counters = 0;
};

int plan_batch(const qg_gemv_problem* pr, int count, Q4Args* args, Plan* plan) {
    int64_t tiles_total = 0;
    for (int i = 0; i < count; ++i) tiles_total += qg::ceil_div(pr[i].M, qg::kTileRows);
    // Target about 2048 wavefronts (8 per CU), at least one super-block each.
    const int64_t target_waves = 2048;
    int W = 2;
    int fixed_wpt = 0;
    int ew = 0, es = 0;
    if (qg::env_pair("QG_Q4K_CFG", &ew, &es) && (ew == 1 || ew == 2 || ew == 4 || ew == 8 || ew == 16) && es >= 1) {
        W = ew;
        fixed_wpt = es;  // wavefronts per tile
    }
    plan->W = W;
    int wg = 0, cnt = 0;
    int64_t part = 0;
    for (int i = 0; i < count; ++i) {
        Q4Prob& P = args->p[i];
        const int nb = (int)(pr[i].K / 256);
        const int tiles = (int)qg::ceil_div(pr[i].M, qg::kTileRows);
        int64_t wpt = fixed_wpt ? fixed_wpt : qg::ceil_div(target_waves, tiles_total);
        wpt = std::max<int64_t>(1, std::min<int64_t>(wpt, nb));
        int splits = (int)qg::ceil_div(wpt, W);
        splits = std::min(splits, nb);
        if (splits > 1 && cnt + tiles > qg::kCounterSlots) splits = 1;
        P.w = (const uint8_t*)pr[i].w_packed;
        P.x = pr[i].x;
        P.y = pr[i].y;
        P.M = (int32_t)pr[i].M;
        P.nb = nb;
        P.tiles = tiles;
        P.splits = splits;
        P.wg_begin = wg;
        P.cnt_base = cnt;
        P.part_off = part;
        wg += tiles * splits;
        if (splits > 1) {
            cnt += tiles;
            part += (int64_t)splits * pr[i].M;
        }
    }
    args->count = count;
    plan->total_wg = wg;
    plan->part_floats = part;
    plan->counters = cnt;
    return QG_OK;
}

size_t plan_ws_bytes(const Plan& p) {
    if (p.part_floats == 0) return 0;
    return (size_t)QG_WORKSPACE_COUNTER_BYTES + qg::align_up((size_t)p.part_floats * 4, 256);
}

int validate(const qg_gemv_problem* pr, int count) {
    if (!pr) return qg::fail(QG_ERR_NULL, "problem list is NULL");
    if (count < 1 || count > QG_MAX_BATCH) return qg::fail(QG_ERR_SHAPE, "batch count %d not in [1, %d]", count, QG_MAX_BATCH);
    int64_t wg_total = 0;
    for (int i = 0; i < count; ++i) {
        const qg_gemv_problem& p = pr[i];
        if (!p.w_packed || !p.x || !p.y) return qg::fail(QG_ERR_NULL, "problem %d: NULL pointer", i);
        if (p.M < 1 || p.M > INT32_MAX) return qg::fail(QG_ERR_SHAPE, "problem %d: M=%lld out of range", i, (long long)p.M);
        if (p.K < 256 || p.K % 256 || p.K > (1 << 24))
            return qg::fail(QG_ERR_SHAPE, "problem %d: K=%lld must be a positive multiple of 256 (<= 2^24)", i, (long long)p.K);
        if (!qg::aligned16(p.w_packed) || !qg::aligned16(p.x) || !qg::aligned16(p.y))
            return qg::fail(QG_ERR_ALIGN, "problem %d: pointers must be 16-byte aligned", i);
        wg_total += qg::ceil_div(p.M, qg::kTileRows) * (p.K / 256);
    }
    if (wg_total > INT32_MAX / 2) return qg::fail(QG_ERR_SHAPE, "batch too large");
    return QG_OK;
}

template <int W>
void launch(const Q4Args& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL(q4k_gemv_kernel<W>, dim3(grid), dim3(64 * W), 0, s, a);
}

}  // namespace

extern "C" {

size_t qgemv_q4k_batch_workspace_bytes(const qg_gemv_problem* problems, int count) {
    if (validate(problems, count) != QG_OK) return 0;
    Q4Args a{};
    Plan p;
    plan_batch(problems, count, &a, &p);
    return plan_ws_bytes(p);
}

int qgemv_q4k_batch(const qg_gemv_problem* problems, int count, void* ws, size_t ws_bytes, qg_stream_t stream) {
    qg::clear_error();
    int st = validate(problems, count);
    if (st) return st;
    Q4Args a{};
    Plan p;
    plan_batch(problems, count, &a, &p);
    const size_t need = plan_ws_bytes(p);
    if (need > 0) {
        if (!ws) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
        if (ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
        if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
        a.cnt = (uint32_t*)ws;
        a.part = (float*)((uint8_t*)ws + QG_WORKSPACE_COUNTER_BYTES);
    }
    st = qg::check_device();
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    switch (p.W) {
        case 1: launch<1>(a, p.total_wg, s); break;
        case 2: launch<2>(a, p.total_wg, s); break;
        case 4: launch<4>(a, p.total_wg, s); break;
        case 8: launch<8>(a, p.total_wg, s); break;
        default: launch<16>(a, p.total_wg, s); break;
    }
    return qg::launch_status("qgemv_q4k");
}

size_t qgemv_q4k_workspace_bytes(int64_t M, int64_t K) {
    qg_gemv_problem p{(const void*)16, (const float*)16, (float*)16, M, K};
    return qgemv_q4k_batch_workspace_bytes(&p, 1);
}

int qgemv_q4k(const void* w, const float* x, float* y, int64_t M, int64_t K, void* ws, size_t ws_bytes,
              qg_stream_t stream) {
    qg_gemv_problem p{w, x, y, M, K};
    return qgemv_q4k_batch(&p, 1, ws, ws_bytes, stream);
}

int qg_pack_q4k(const void* src, void* dst, int64_t M, int64_t K, qg_stream_t stream) {
    qg::clear_error();
    if (!src || !dst) return qg::fail(QG_ERR_NULL, "NULL pointer");
    if (M < 1 || M > INT32_MAX || K < 256 || K % 256 || K > (1 << 24))
        return qg::fail(QG_ERR_SHAPE, "invalid Q4_K shape M=%lld K=%lld", (long long)M, (long long)K);
    if (!qg::aligned16(src) || !qg::aligned16(dst)) return qg::fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t bytes = qg_q4k_bytes(M, K);
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    if (s8 < d8 + bytes && d8 < s8 + bytes) return qg::fail(QG_ERR_SHAPE, "src and dst overlap");
    int st = qg::check_device();
    if (st) return st;
    const int64_t units = (int64_t)(bytes / 16);
    const int blocks = (int)std::min<int64_t>(qg::ceil_div(units, 256), 65536);
    hipLaunchKernelGGL(q4k_pack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                       (uint4*)dst, M, (int)(K / 256));
    return qg::launch_status("qg_pack_q4k");
}

}  // extern "C"
