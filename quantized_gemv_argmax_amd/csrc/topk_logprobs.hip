// Top-k, log-softmax and the top-k sampler over a logit vector, for gfx950.
//
// Method (dotLLM README: the news entry on log-probabilities, which returns the
// top_logprobs (0..20) alternatives from the per-token log-softmax taken before
// sampling; Key Features, composable sampling: temperature -> top-k -> top-p ->
// min-p -> categorical draw). Here the whole step runs on the device so that the
// 608 KB logit vector of a 152064-token head never crosses to the host.
//
// Two stages.
//  1. Per 16-row tile: the first maximum (value, row) and the sum of
//     exp(z - tile max). For the LM head this is fused into the projection kernel
//     (q8_0_gemv.hip); for a given logit vector topk_tile_stats_kernel computes it.
//  2. topk_select_kernel, one workgroup of 1024 threads:
//     - log-sum-exp: the global maximum, then sum_t s_t exp(m_t - max) in a
//       fixed order; lse = max + log(sum).
//     - tile selection: every element of the top k is at least as good as the
//       k-th best tile maximum (the k best tile maxima are k distinct elements),
//       and a tile whose maximum ranks below the k best holds no top-k element.
//       So the k best tiles by their (max, row) key contain the answer: at most
//       16k candidates instead of M.
//     - the k best of those candidates, then a 64-lane bitonic sort of the
//       winners by (value, lower row).
//     Both selections find the k-th largest 64-bit key (order-preserving value
//     bits, then the complement of the row) by radix selection over 8-bit digits
//     with an LDS histogram, stopping as soon as the chosen digit's bucket holds
//     exactly the keys still needed. Histogram increments are aggregated per
//     wavefront (one LDS atomic per distinct digit), since the leading digits of
//     similar logits collide.
//     - optionally one draw of the sampler chain over the sorted k (one wavefront).
#include <algorithm>
#include <climits>

#include "qg_device.h"
#include "qg_host.h"

namespace {

constexpr int T = QG_TILE_ROWS;
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

struct SelArgs {
    float4* partials;
    int32_t tiles;
    int32_t M;
    const float* logits;
    int32_t k;
    int32_t sample;  // 1: draw a token
    float temperature, top_p, min_p;
    const float* u;
    qg_topk_out out;
};

QG_DEV uint64_t elem_key(float v, int row) { return ((uint64_t)qg_ord(v) << 32) | (uint32_t)(0xffffffffu - (uint32_t)row); }
QG_DEV float key_value(uint64_t key) { return qg_unord((uint32_t)(key >> 32)); }
QG_DEV int key_row(uint64_t key) { return (int)(0xffffffffu - (uint32_t)key); }

QG_DEV float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
QG_DEV float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// The k-th largest of the workgroup's keys (R per thread; 0 marks an empty slot
// and never ranks among the k as long as at least k keys are nonzero). Returns a
// threshold t such that exactly k keys are >= t when keys are distinct.
template <int R>
QG_DEV uint64_t wg_kth_largest(const uint64_t (&key)[R], uint32_t k, uint32_t* hist, uint32_t* sc) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint64_t prefix = 0, pmask = 0;
    uint32_t kk = k;
    for (int round = 0; round < 8; ++round) {
        const int shift = 56 - 8 * round;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            bool act = (key[r] & pmask) == prefix;
            const uint32_t dg = (uint32_t)(key[r] >> shift) & 255u;
            uint64_t pending = __ballot(act);
            while (pending) {  // wave-uniform: one LDS atomic per distinct digit
                const int leader = __builtin_ctzll(pending);
                const uint32_t ldg = __builtin_amdgcn_readlane(dg, leader);
                const uint64_t same = __ballot(act && dg == ldg);
                if (lane == leader) atomicAdd(&hist[ldg], (uint32_t)__builtin_popcountll(same));
                if (dg == ldg) act = false;
                pending &= ~same;
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds digits 255-4l .. 252-4l; counts accumulate from the top digit down
            const uint32_t c0 = hist[255 - 4 * lane], c1 = hist[254 - 4 * lane];
            const uint32_t c2 = hist[253 - 4 * lane], c3 = hist[252 - 4 * lane];
            const uint32_t tot = c0 + c1 + c2 + c3;
            uint32_t incl = tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off, 64);
                if (lane >= off) incl += o;
            }
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

// Bitonic sort of one key per lane over the 64 lanes, largest first.
QG_DEV uint64_t wave_sort_desc(uint64_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint32_t lo = __shfl_xor((uint32_t)x, stride, 64);
            const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), stride, 64);
            const uint64_t o = ((uint64_t)hi << 32) | lo;
            const bool lower = (lane & stride) == 0;
            const bool desc = (lane & size) == 0;  // block direction; the last block is descending
            x = (lower == desc) ? (x > o ? x : o) : (x < o ? x : o);
        }
    }
    return x;
}

template <int R>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(SelArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sc[4];
    __shared__ float redf[kWaves];
    __shared__ int32_t sel_tiles[QG_TOPK_MAX];
    __shared__ uint64_t winners[QG_TOPK_MAX];
    __shared__ uint32_t counts[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float ninf = -__builtin_huge_valf();

    // per-tile partials: key (max, row), max, exponential sum; cleared after reading
    uint64_t key[R];
    float m[R], s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int t = tid + kThreads * r;
        if (t < a.tiles) {
            const float4 p = a.partials[t];
            m[r] = p.x;
            s[r] = p.z;
            key[r] = elem_key(p.x, __builtin_bit_cast(int, p.y));
        } else {
            m[r] = ninf;
            s[r] = 0.f;
            key[r] = 0;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int t = tid + kThreads * r;
        if (t < a.tiles) a.partials[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < 2) counts[tid] = 0;

    // log-sum-exp: global max, then the rescaled sums in a fixed order
    float mx = m[0];
#pragma unroll
    for (int r = 1; r < R; ++r) mx = fmaxf(mx, m[r]);
    mx = wave_max(mx);
    if (lane == 0) redf[wave] = mx;
    __syncthreads();
    mx = redf[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, redf[w]);
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc += (m[r] == ninf) ? 0.f : s[r] * __expf(m[r] - mx);
    acc = wave_sum(acc);
    __syncthreads();  // every thread has read redf
    if (lane == 0) redf[wave] = acc;
    __syncthreads();
    float total = redf[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) total += redf[w];
    const float lse = (mx == ninf) ? ninf : mx + __logf(total);

    // the k best tiles by their (max, row) key
    const int nsel = min(a.tiles, a.k);
    if (a.tiles <= a.k) {
        if (tid < a.tiles) sel_tiles[tid] = tid;
    } else {
        const uint64_t t = wg_kth_largest<R>(key, (uint32_t)a.k, hist, sc);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (key[r] != 0 && key[r] >= t) {
                const uint32_t pos = atomicAdd(&counts[0], 1u);  // exactly k keys reach t
                if (pos < QG_TOPK_MAX) sel_tiles[pos] = tid + kThreads * r;
            }
    }
    __syncthreads();

    // their rows are the candidates (16 per tile, one per thread)
    uint64_t ck[1] = {0};
    if (tid < T * nsel) {
        const int row = sel_tiles[tid >> 4] * T + (tid & 15);
        if (row < a.M) ck[0] = elem_key(a.logits[row], row);
    }
    const uint64_t t2 = wg_kth_largest<1>(ck, (uint32_t)a.k, hist, sc);
    if (ck[0] != 0 && ck[0] >= t2) {
        const uint32_t pos = atomicAdd(&counts[1], 1u);
        if (pos < QG_TOPK_MAX) winners[pos] = ck[0];
    }
    __syncthreads();
    if (wave != 0) return;

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
    const float z0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
    int pick = 0;
    if (a.temperature > 0.f && a.k > 1 && z0 != ninf) {
        const bool in = lane < a.k;
        const float q = in ? __expf((v - z0) / a.temperature) : 0.f;
        float c = q;  // inclusive prefix sum over lanes, fixed order
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(c, off, 64);
            if (lane >= off) c += o;
        }
        const float ctot = __shfl(c, a.k - 1, 64);
        int n = a.k;
        if (a.top_p < 1.f) {
            const uint64_t reach = __ballot(in && c >= a.top_p * ctot);
            if (reach) n = __builtin_ctzll(reach) + 1;
        }
        const uint64_t keep = __ballot(lane < n && q >= a.min_p);  // q of the first entry is 1
        const int mk = keep ? 64 - __builtin_clzll(keep) : 1;
        const float kept = __shfl(c, mk - 1, 64);
        const float target = a.u[0] * kept;
        const uint64_t past = __ballot(lane < mk && c > target);
        pick = past ? __builtin_ctzll(past) : mk - 1;
    }
    const int tok = __shfl(row, pick, 64);
    if (lane == 0 && a.out.token) a.out.token[0] = tok;
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

}  // namespace

namespace qg {

size_t topk_ws_bytes(int64_t M) {
    if (M < 1 || M > QG_TOPK_MAX_ROWS) return 0;
    return align_up((size_t)ceil_div(M, T) * 16, 256);
}

int validate_topk(int64_t M, int k, const qg_sampler* sampler, const qg_topk_out* out) {
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

int launch_topk_select(float4* partials, int tiles, const float* logits, int64_t M, int k, const qg_sampler* sampler,
                       const qg_topk_out& out, hipStream_t s) {
    SelArgs a{};
    a.partials = partials;
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
    const int per = (int)ceil_div(tiles, kThreads);
    if (per <= 1)
        hipLaunchKernelGGL(topk_select_kernel<1>, dim3(1), dim3(kThreads), 0, s, a);
    else if (per <= 2)
        hipLaunchKernelGGL(topk_select_kernel<2>, dim3(1), dim3(kThreads), 0, s, a);
    else if (per <= 4)
        hipLaunchKernelGGL(topk_select_kernel<4>, dim3(1), dim3(kThreads), 0, s, a);
    else if (per <= 8)
        hipLaunchKernelGGL(topk_select_kernel<8>, dim3(1), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(topk_select_kernel<16>, dim3(1), dim3(kThreads), 0, s, a);
    return launch_status("top-k selection");
}

}  // namespace qg

extern "C" {

size_t logits_topk_workspace_bytes(int64_t M) { return qg::topk_ws_bytes(M); }

int logits_topk(const float* logits, int64_t M, int k, const qg_sampler* sampler, void* ws, size_t ws_bytes,
                const qg_topk_out* out, qg_stream_t stream) {
    qg::clear_error();
    if (!logits) return qg::fail(QG_ERR_NULL, "logits is NULL");
    int st = qg::validate_topk(M, k, sampler, out);
    if (st) return st;
    if (!qg::aligned16(logits)) return qg::fail(QG_ERR_ALIGN, "logits not 16-byte aligned");
    const size_t need = qg::topk_ws_bytes(M);
    if (!ws || ws_bytes < need) return qg::fail(QG_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : 0);
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    st = qg::check_device();
    if (st) return st;
    const int tiles = (int)qg::ceil_div(M, T);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(topk_tile_stats_kernel, dim3((unsigned)qg::ceil_div(tiles, 16)), dim3(256), 0, s, logits,
                       (int)M, tiles, (float4*)ws);
    st = qg::launch_status("logits_topk (tile statistics)");
    if (st) return st;
    return qg::launch_topk_select((float4*)ws, tiles, logits, M, k, sampler, *out, s);
}

}  // extern "C"
