// Top-k, log-softmax and the top-k sampler over a logit vector, for gfx950.
//
// Method (dotLLM README: the news entry on log-probabilities, which returns the
// top_logprobs (0..20) alternatives from the per-token log-softmax taken before
// sampling; Key Features, composable sampling: temperature -> top-k -> top-p ->
// min-p -> categorical draw). Here the whole step runs on the device so that the
// 608 KB logit vector of a 152064-token head never crosses to the host.
//
// Stages.
//  1. Per 16-row tile: the first maximum (value, row) and the sum of
//     exp(z - tile max). For the LM head this is fused into the projection kernel
//     (q8_0_gemv.hip); for a given logit vector topk_tile_stats_kernel computes it.
//  2. topk_group_kernel, one 256-thread workgroup per 1024 tiles: the group's
//     log-sum-exp partial (max, sum of exp(m_t - max) s_t) and its k best tiles by
//     their (max, row) key. Every element of the top k is at least as good as the
//     k-th best tile maximum (the k best tile maxima are k distinct elements), and
//     a tile whose maximum ranks below the k best holds no top-k element, so the k
//     best tiles contain the answer; the same holds within each group.
//  3. topk_final_kernel, one workgroup: the k best of the groups' tiles, their
//     16k rows as candidates, the k best candidates, a 64-lane bitonic sort of the
//     winners by (value, lower row), log-probabilities, and optionally one draw of
//     the sampler chain.
// Selections find the k-th largest 64-bit key (order-preserving value bits, then
// the complement of the row) by radix selection over 8-bit digits with an LDS
// histogram, stopping as soon as the chosen digit's bucket holds exactly the keys
// still needed. Wave-level reductions, scans and the sort's lane exchanges use DPP
// and the gfx950 lane-swap instructions rather than LDS shuffles.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;
constexpr int kWG = 256;           // threads per selection workgroup (4 wavefronts)
constexpr int kGroupTiles = 1024;  // tiles per group (4 per thread)
constexpr int kMaxGroups = QG_TOPK_MAX_ROWS / T / kGroupTiles;

struct FinArgs {
    uint64_t* gkeys;  // [groups][QG_TOPK_MAX], zero where a group has fewer
    float2* glse;     // [groups]: (max, sum)
    int32_t groups;
    int32_t nkeys;    // nonzero group keys: sum over groups of min(k, tiles in group)
    int32_t tiles;
    int32_t M;
    const float* logits;
    int32_t k;
    int32_t sample;
    float temperature, top_p, min_p;
    const float* u;
    qg_topk_out out;
};

QG_DEV uint64_t elem_key(float v, int row) { return ((uint64_t)qg_ord(v) << 32) | (uint32_t)(0xffffffffu - (uint32_t)row); }
QG_DEV float key_value(uint64_t key) { return qg_unord((uint32_t)(key >> 32)); }
QG_DEV int key_row(uint64_t key) { return (int)(0xffffffffu - (uint32_t)key); }

QG_DEV int lane_id() { return __lane_id(); }

template <int CTRL>
QG_DEV uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}

// The value of lane (this lane ^ S), S a power of two below 64.
template <int S>
QG_DEV uint32_t lane_xor(uint32_t v) {
    if constexpr (S == 1) {
        return dpp<0xb1>(v);  // quad_perm [1,0,3,2]
    } else if constexpr (S == 2) {
        return dpp<0x4e>(v);  // quad_perm [2,3,0,1]
    } else if constexpr (S == 4 || S == 8) {
        const uint32_t up = dpp<0x100 + S>(v);  // row_shl:S, lane i reads i + S
        const uint32_t dn = dpp<0x110 + S>(v);  // row_shr:S, lane i reads i - S
        return (lane_id() & S) ? dn : up;
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane_id() & 16) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane_id() & 32) ? r[0] : r[1];
    }
}

template <int S>
QG_DEV uint64_t lane_xor64(uint64_t v) {
    return ((uint64_t)lane_xor<S>((uint32_t)(v >> 32)) << 32) | lane_xor<S>((uint32_t)v);
}

QG_DEV float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Wave-uniform maximum / sum (fixed order: within quads, 8-lane and 16-lane
// mirrors, then the four rows in order).
QG_DEV float wave_max_u(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0xb1>(__builtin_bit_cast(uint32_t, v))));
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0x4e>(__builtin_bit_cast(uint32_t, v))));
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(uint32_t, v))));
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0x140>(__builtin_bit_cast(uint32_t, v))));
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
QG_DEV float wave_sum_u(float v) {
    v += __builtin_bit_cast(float, dpp<0xb1>(__builtin_bit_cast(uint32_t, v)));
    v += __builtin_bit_cast(float, dpp<0x4e>(__builtin_bit_cast(uint32_t, v)));
    v += __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(uint32_t, v)));
    v += __builtin_bit_cast(float, dpp<0x140>(__builtin_bit_cast(uint32_t, v)));
    return ((readlane_f(v, 0) + readlane_f(v, 16)) + readlane_f(v, 32)) + readlane_f(v, 48);
}

template <int C, typename V>
QG_DEV V dpp_v(V x) {
    return __builtin_bit_cast(V, dpp<C>(__builtin_bit_cast(uint32_t, x)));
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each
// 16-lane row, then the row totals carried by row broadcasts.
template <typename V>
QG_DEV V wave_incl_scan(V v) {
    v += dpp_v<0x111>(v);
    v += dpp_v<0x112>(v);
    v += dpp_v<0x114>(v);
    v += dpp_v<0x118>(v);
    // row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3; other rows add 0
    v += __builtin_bit_cast(V, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
    v += __builtin_bit_cast(V, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
    return v;
}

// The k-th largest of the workgroup's keys (R per thread; 0 marks an empty slot
// and never ranks among the k as long as at least k keys are nonzero). Returns a
// threshold t such that exactly k keys are >= t when the nonzero keys are distinct.
template <int R>
QG_DEV uint64_t kth_largest(const uint64_t (&key)[R], uint32_t k, uint32_t* hist, uint32_t* sc) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint64_t prefix = 0, pmask = 0;
    uint32_t kk = k;
    for (int round = 0; round < 8; ++round) {
        const int shift = 56 - 8 * round;
        hist[tid] = 0;  // kWG == 256 bins
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            bool act = (key[r] & pmask) == prefix;
            const uint32_t dg = (uint32_t)(key[r] >> shift) & 255u;
            // leading digits of similar values collide: up to two distinct digits of
            // the wavefront are counted with one atomic each, the rest lane by lane
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const uint64_t pending = __ballot(act);
                if (pending) {
                    const int leader = __builtin_ctzll(pending);
                    const uint32_t ldg = __builtin_amdgcn_readlane(dg, leader);
                    const uint64_t same = __ballot(act && dg == ldg);
                    if (lane == leader) atomicAdd(&hist[ldg], (uint32_t)__builtin_popcountll(same));
                    if (dg == ldg) act = false;
                }
            }
            if (act) atomicAdd(&hist[dg], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds digits 255-4l .. 252-4l; counts accumulate from the top digit down
            const uint32_t c0 = hist[255 - 4 * lane], c1 = hist[254 - 4 * lane];
            const uint32_t c2 = hist[253 - 4 * lane], c3 = hist[252 - 4 * lane];
            const uint32_t tot = c0 + c1 + c2 + c3;
            const uint32_t incl = wave_incl_scan(tot);
            const uint32_t excl = incl - tot;
            if (excl < kk && kk <= incl) {
                uint32_t above = excl, cnt = c0;
                int dg = 255 - 4 * lane;
                if (kk > above + c0) {
                    above += c0;
                    dg -= 1;
                    cnt = c1;
                    if (kk > above + c1) {
                        above += c1;
                        dg -= 1;
                        cnt = c2;
                        if (kk > above + c2) {
                            above += c2;
                            dg -= 1;
                            cnt = c3;
                        }
                    }
                }
                sc[0] = (uint32_t)dg;
                sc[1] = above;
                sc[2] = cnt;
            }
        }
        __syncthreads();
        const uint32_t dg = sc[0], above = sc[1], cnt = sc[2];
        prefix |= (uint64_t)dg << shift;
        pmask |= (uint64_t)0xff << shift;
        kk -= above;
        if (cnt == kk) break;  // the whole bucket is needed: keys >= prefix are the k
    }
    return prefix;
}

template <int STRIDE, int SIZE>
QG_DEV uint64_t bitonic_step(uint64_t x) {
    const uint64_t o = lane_xor64<STRIDE>(x);
    const int lane = lane_id();
    const bool lower = (lane & STRIDE) == 0;
    const bool desc = (lane & SIZE) == 0;  // block direction; the final block is descending
    return (lower == desc) ? (x > o ? x : o) : (x < o ? x : o);
}

template <int SIZE, int STRIDE>
QG_DEV uint64_t bitonic_merge(uint64_t x) {
    x = bitonic_step<STRIDE, SIZE>(x);
    if constexpr (STRIDE > 1) x = bitonic_merge<SIZE, STRIDE / 2>(x);
    return x;
}

// Bitonic sort of one key per lane over the 64 lanes, largest first.
QG_DEV uint64_t wave_sort_desc(uint64_t x) {
    x = bitonic_merge<2, 1>(x);
    x = bitonic_merge<4, 2>(x);
    x = bitonic_merge<8, 4>(x);
    x = bitonic_merge<16, 8>(x);
    x = bitonic_merge<32, 16>(x);
    return bitonic_merge<64, 32>(x);
}

// Stage 1 for a given logit vector: 16 tiles per 256-thread workgroup.
__global__ __launch_bounds__(256) void topk_tile_stats_kernel(const float* __restrict__ logits, int M, int tiles,
                                                              float4* __restrict__ partials) {
    const int g = blockIdx.x * 256 + threadIdx.x;
    const bool valid = g < M;
    const float v = valid ? logits[g] : 0.f;
    const float4 st = qg_group16_stats(v, g, valid);
    if ((threadIdx.x & 15) == 0 && (g >> 4) < tiles) partials[g >> 4] = st;
}

// Stage 2: per group of 1024 tiles, the log-sum-exp partial and the k best tile
// keys (written unordered to the group's 64 slots; the others stay zero).
__global__ __launch_bounds__(kWG) void topk_group_kernel(float4* __restrict__ partials, int tiles, int k,
                                                         uint64_t* __restrict__ gkeys, float2* __restrict__ glse) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sc[4];
    __shared__ float red[kWG / 64];
    __shared__ uint32_t cnt;
    constexpr int R = kGroupTiles / kWG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.x;
    const int base = g * kGroupTiles;
    const int n = min(kGroupTiles, tiles - base);
    const float ninf = -__builtin_huge_valf();

    float4 p[R];
#pragma unroll
    for (int r = 0; r < R; ++r) p[r] = partials[base + min(tid + kWG * r, n - 1)];  // loads first, clamped
    uint64_t key[R];
    float m[R], s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = tid + kWG * r < n;
        m[r] = in ? p[r].x : ninf;
        s[r] = in ? p[r].z : 0.f;
        key[r] = in ? elem_key(p[r].x, __builtin_bit_cast(int, p[r].y)) : 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (tid + kWG * r < n) partials[base + tid + kWG * r] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid == 0) cnt = 0;

    float mx = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
    mx = wave_max_u(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc += (m[r] == ninf) ? 0.f : s[r] * __expf(m[r] - mx);
    acc = wave_sum_u(acc);
    __syncthreads();  // red has been read
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (tid == 0) glse[g] = make_float2(mx, ((red[0] + red[1]) + red[2]) + red[3]);

    uint64_t* out = gkeys + (size_t)g * QG_TOPK_MAX;
    if (n <= k) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (tid + kWG * r < n) out[tid + kWG * r] = key[r];
        return;
    }
    const uint64_t t = kth_largest<R>(key, (uint32_t)k, hist, sc);
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (key[r] != 0 && key[r] >= t) {
            const uint32_t pos = atomicAdd(&cnt, 1u);  // exactly k keys reach t
            if (pos < QG_TOPK_MAX) out[pos] = key[r];
        }
}

// Stage 3: one workgroup.
__global__ __launch_bounds__(kWG) void topk_final_kernel(FinArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sc[4];
    __shared__ int32_t sel_tiles[QG_TOPK_MAX];
    __shared__ uint64_t winners[QG_TOPK_MAX];
    __shared__ uint32_t counts[2];
    __shared__ float lse_s;
    constexpr int R = QG_TOPK_MAX * kMaxGroups / kWG;  // group keys per thread (4)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float ninf = -__builtin_huge_valf();
    const int nslots = a.groups * QG_TOPK_MAX;

    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + kWG * r;
        key[r] = i < nslots ? a.gkeys[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + kWG * r;
        if (i < nslots) a.gkeys[i] = 0;
    }
    if (tid < 2) counts[tid] = 0;
    if (wave == 0) {  // log-sum-exp from the group partials, fixed order
        const float2 gp = lane < a.groups ? a.glse[lane] : make_float2(ninf, 0.f);
        if (lane < a.groups) a.glse[lane] = make_float2(0.f, 0.f);
        const float mx = wave_max_u(gp.x);
        const float tot = wave_sum_u(gp.x == ninf ? 0.f : gp.y * __expf(gp.x - mx));
        if (lane == 0) lse_s = (mx == ninf) ? ninf : mx + __logf(tot);
    }
    __syncthreads();  // counts are zero

    // the k best tiles (all of them when there are no more than k)
    const int nsel = min(a.tiles, a.k);
    if (a.nkeys <= a.k) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (key[r] != 0) {
                const uint32_t pos = atomicAdd(&counts[0], 1u);
                if (pos < QG_TOPK_MAX) sel_tiles[pos] = key_row(key[r]) / T;
            }
    } else {
        const uint64_t t = kth_largest<R>(key, (uint32_t)a.k, hist, sc);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (key[r] != 0 && key[r] >= t) {
                const uint32_t pos = atomicAdd(&counts[0], 1u);
                if (pos < QG_TOPK_MAX) sel_tiles[pos] = key_row(key[r]) / T;
            }
    }
    __syncthreads();

    // their rows are the candidates, 16 per tile
    constexpr int RC = QG_TOPK_MAX * T / kWG;
    uint64_t ck[RC];
#pragma unroll
    for (int r = 0; r < RC; ++r) {
        const int c = tid + kWG * r;
        ck[r] = 0;
        if (c < T * nsel) {
            const int row = sel_tiles[c >> 4] * T + (c & 15);
            if (row < a.M) ck[r] = elem_key(a.logits[row], row);
        }
    }
    const uint64_t t2 = kth_largest<RC>(ck, (uint32_t)a.k, hist, sc);
#pragma unroll
    for (int r = 0; r < RC; ++r)
        if (ck[r] != 0 && ck[r] >= t2) {
            const uint32_t pos = atomicAdd(&counts[1], 1u);
            if (pos < QG_TOPK_MAX) winners[pos] = ck[r];
        }
    __syncthreads();
    if (wave != 0) return;

    const float lse = lse_s;
    const uint64_t x = wave_sort_desc(lane < a.k ? winners[lane] : 0);
    const float v = key_value(x);
    const int row = key_row(x);
    if (lane < a.k) {
        a.out.index[lane] = row;
        if (a.out.logit) a.out.logit[lane] = v;
        if (a.out.logprob) a.out.logprob[lane] = v - lse;
    }
    if (lane == 0 && a.out.lse) a.out.lse[0] = lse;
    if (!a.sample) return;

    // sampler chain over the sorted k: weights, top-p prefix, min-p, inverse CDF
    const float z0 = readlane_f(v, 0);
    int pick = 0;
    if (a.temperature > 0.f && a.k > 1 && z0 != ninf) {
        const bool in = lane < a.k;
        const float q = in ? __expf((v - z0) / a.temperature) : 0.f;
        const float c = wave_incl_scan(q);
        const float ctot = readlane_f(c, a.k - 1);
        int n = a.k;
        if (a.top_p < 1.f) {
            const uint64_t reach = __ballot(in && c >= a.top_p * ctot);
            if (reach) n = __builtin_ctzll(reach) + 1;
        }
        const uint64_t keep = __ballot(lane < n && q >= a.min_p);  // q of the first entry is 1
        const int mk = keep ? 64 - __builtin_clzll(keep) : 1;
        const float kept = readlane_f(c, mk - 1);
        const float target = a.u[0] * kept;
        const uint64_t past = __ballot(lane < mk && c > target);
        pick = past ? __builtin_ctzll(past) : mk - 1;
    }
    const int tok = __builtin_amdgcn_readlane(row, pick);
    if (lane == 0 && a.out.token) a.out.token[0] = tok;
}

struct WsLayout {
    size_t partials, gkeys, glse, total;
};
WsLayout ws_layout(int64_t M) {
    const int64_t tiles = qg::ceil_div(M, T);
    const int64_t groups = qg::ceil_div(tiles, kGroupTiles);
    WsLayout w;
    w.partials = 0;
    w.gkeys = qg::align_up((size_t)tiles * 16, 256);
    w.glse = w.gkeys + (size_t)groups * QG_TOPK_MAX * 8;
    w.total = qg::align_up(w.glse + (size_t)groups * 8, 256);
    return w;
}

}  // namespace

namespace qg {

size_t topk_ws_bytes(int64_t M) {
    if (M < 1 || M > QG_TOPK_MAX_ROWS) return 0;
    return ws_layout(M).total;
}

qg_status validate_topk(int64_t M, int k, const qg_sampler* sampler, const qg_topk_out* out) {
    if (!out) return fail(QG_ERR_NULL, "output descriptor is NULL");
    if (!out->index) return fail(QG_ERR_NULL, "out->index is NULL");
    if (M < 1 || M > QG_TOPK_MAX_ROWS)
        return fail(QG_ERR_SHAPE, "M=%lld not in [1, %d]", (long long)M, QG_TOPK_MAX_ROWS);
    if (k < 1 || k > QG_TOPK_MAX || k > M) return fail(QG_ERR_SHAPE, "k=%d not in [1, min(%d, M)]", k, QG_TOPK_MAX);
    const void* ptrs[5] = {out->index, out->logit, out->logprob, out->lse, out->token};
    for (const void* p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) & 3) return fail(QG_ERR_ALIGN, "outputs must be 4-byte aligned");
    if (sampler) {
        if (!sampler->u) return fail(QG_ERR_NULL, "sampler->u is NULL");
        if (!out->token) return fail(QG_ERR_NULL, "out->token is NULL while a sampler is given");
        if (reinterpret_cast<uintptr_t>(sampler->u) & 3) return fail(QG_ERR_ALIGN, "sampler->u not 4-byte aligned");
        if (!(sampler->temperature == sampler->temperature) || !(sampler->top_p > 0.f && sampler->top_p <= 1.f) ||
            !(sampler->min_p >= 0.f && sampler->min_p <= 1.f))
            return fail(QG_ERR_SHAPE, "sampler needs a non-NaN temperature, 0 < top_p <= 1, 0 <= min_p <= 1");
    }
    return QG_OK;
}

qg_status launch_topk_select(void* ws, int tiles, const float* logits, int64_t M, int k, const qg_sampler* sampler,
                       const qg_topk_out& out, hipStream_t s) {
    const WsLayout L = ws_layout(M);
    uint8_t* w8 = (uint8_t*)ws;
    const int groups = (int)ceil_div(tiles, kGroupTiles);
    uint64_t* gkeys = (uint64_t*)(w8 + L.gkeys);
    float2* glse = (float2*)(w8 + L.glse);
    hipLaunchKernelGGL(topk_group_kernel, dim3(groups), dim3(kWG), 0, s, (float4*)(w8 + L.partials), tiles, k, gkeys,
                       glse);
    qg_status st = launch_status("top-k selection (groups)");
    if (st) return st;
    FinArgs a{};
    a.gkeys = gkeys;
    a.glse = glse;
    a.groups = groups;
    a.nkeys = 0;
    for (int g = 0; g < groups; ++g) a.nkeys += std::min(k, std::min(kGroupTiles, tiles - g * kGroupTiles));
    a.tiles = tiles;
    a.M = (int32_t)M;
    a.logits = logits;
    a.k = k;
    a.sample = sampler ? 1 : 0;
    if (sampler) {
        a.temperature = sampler->temperature;
        a.top_p = sampler->top_p;
        a.min_p = sampler->min_p;
        a.u = sampler->u;
    }
    a.out = out;
    hipLaunchKernelGGL(topk_final_kernel, dim3(1), dim3(kWG), 0, s, a);
    return launch_status("top-k selection (final)");
}

}  // namespace qg

extern "C" {

size_t logits_topk_workspace_bytes(int64_t M) { return qg::topk_ws_bytes(M); }

qg_status logits_topk(const float* logits, int64_t M, int k, const qg_sampler* sampler, void* ws, size_t ws_bytes,
                const qg_topk_out* out, qg_stream_t stream) {
    qg::clear_error();
    if (!logits) return qg::fail(QG_ERR_NULL, "logits is NULL");
    qg_status st = qg::validate_topk(M, k, sampler, out);
    if (st) return st;
    if (!qg::aligned16(logits)) return qg::fail(QG_ERR_ALIGN, "logits not 16-byte aligned");
    const size_t need = qg::topk_ws_bytes(M);
    if (!ws || ws_bytes < need)
        return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : 0);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    st = qg::check_device();
    if (st) return st;
    const int tiles = (int)qg::ceil_div(M, T);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(topk_tile_stats_kernel, dim3((unsigned)qg::ceil_div(tiles, 16)), dim3(256), 0, s, logits,
                       (int)M, tiles, (float4*)ws);
    st = qg::launch_status("logits_topk (tile statistics)");
    if (st) return st;
    return qg::launch_topk_select(ws, tiles, logits, M, k, sampler, *out, s);
}

}  // extern "C"
