// Device helpers of the top-k router, shared by the routing kernels and by the
// small-batch expert kernels that route their own few tokens.
//
// Page "Nex-N2.5-mini FP8 W8A8 with Calibrated FP8 KV Scales", Artifact summary: 256
// routed experts, 8 active per token.  The chosen experts are weighted by the softmax of
// all logits renormalised over the chosen ones, which equals the softmax of the chosen
// logits alone.
#pragma once
#include "common.h"

namespace w4a16 {
namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;


// Wave-wide maximum / minimum by DPP moves (quad permutes, row mirrors, then row
// broadcasts of lanes 15 and 31): the full result lands in lane 63 and is read back as a
// scalar, so every lane gets it without LDS.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ float fdpp_max(float v, int o) { return fmaxf(v, __int_as_float(o)); }

__device__ __forceinline__ float wave_max_f32(float v) {
    v = fdpp_max(v, dpp_i32<0xb1, 0xf>(__float_as_int(v)));    // quad_perm [1,0,3,2]
    v = fdpp_max(v, dpp_i32<0x4e, 0xf>(__float_as_int(v)));    // quad_perm [2,3,0,1]
    v = fdpp_max(v, dpp_i32<0x141, 0xf>(__float_as_int(v)));   // row_half_mirror
    v = fdpp_max(v, dpp_i32<0x140, 0xf>(__float_as_int(v)));   // row_mirror: every row holds its max
    v = fdpp_max(v, dpp_i32<0x142, 0xa>(__float_as_int(v)));   // row_bcast:15 into rows 1 and 3
    v = fdpp_max(v, dpp_i32<0x143, 0xc>(__float_as_int(v)));   // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_min_i32(int v) {
    v = min(v, dpp_i32<0xb1, 0xf>(v));
    v = min(v, dpp_i32<0x4e, 0xf>(v));
    v = min(v, dpp_i32<0x141, 0xf>(v));
    v = min(v, dpp_i32<0x140, 0xf>(v));
    v = min(v, dpp_i32<0x142, 0xa>(v));
    v = min(v, dpp_i32<0x143, 0xc>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// Top-k of one token by one wave.  Lane l holds the logits of experts l, l + 64, ...
// Each of the k rounds takes the wave-wide maximum of the lanes' best remaining logits;
// when several lanes tie on it, the lowest expert index among them wins (a second,
// rarely taken reduction).  The winner's lane removes it.  -0 and +0 compare equal, so
// they tie; NaN logits rank below every other value.  With NV <= 4 logits per lane the
// lane keeps them sorted (larger first, lower index first on equal values) so its best
// is its first register; with more, the lane scans them each round.
// Lane j < k returns slot j's expert and its softmax weight over the chosen logits.
// This lane's logits of one token (experts lane, lane + 64, ...): unconditional (clamped)
// loads, all in flight together.
template <int NV>
__device__ __forceinline__ void wave_topk_load(const float* __restrict__ row, int E, float (&raw)[NV]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NV; ++i) raw[i] = row[min(lane + 64 * i, E - 1)];
}

// WEIGHTS false: only the experts (my_w untouched), for callers that need just a rank's
// winner; the rounds are the same.
template <int NV, bool WEIGHTS = true>   // logits per lane: E <= 64 * NV
__device__ void wave_topk_from(const float (&raw)[NV], int E, int k, int* my_id, float* my_w) {
    constexpr bool kSorted = NV <= 4;
    const int lane = threadIdx.x & 63;
    float hv[NV];
    int he[kSorted ? NV : 1];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        const float v = raw[i];
        hv[i] = (e < E && !__builtin_isnan(v)) ? v : -__builtin_inff();
        if constexpr (kSorted) he[i] = e < E ? e : 0x7fffffff;
    }
    if constexpr (kSorted) {
#pragma unroll
        for (int i = 1; i < NV; ++i)     // stable insertion sort, larger value first
#pragma unroll
            for (int j = i; j > 0; --j) {
                const bool sw = hv[j] > hv[j - 1];
                const float tv = hv[j];
                const int te = he[j];
                hv[j] = sw ? hv[j - 1] : hv[j];
                he[j] = sw ? he[j - 1] : he[j];
                hv[j - 1] = sw ? tv : hv[j - 1];
                he[j - 1] = sw ? te : he[j - 1];
            }
    }
    float v0 = 0.f, den = 0.f, mine = 0.f;
    int id = -1;
    for (int j = 0; j < k; ++j) {
        float best;
        int best_e;
        if constexpr (kSorted) {
            best = hv[0];
            best_e = he[0];
        } else {   // the lane's largest remaining value, lowest index first on ties
            best = hv[0];
            int bi = 0;
#pragma unroll
            for (int i = 1; i < NV; ++i) {
                const bool gt = hv[i] > best;
                best = gt ? hv[i] : best;
                bi = gt ? i : bi;
            }
            const int e = lane + 64 * bi;
            best_e = e < E ? e : 0x7fffffff;
        }
        const float m = wave_max_f32(best);
        const bool at_max = best == m;
        const uint64_t cand = __ballot(at_max);
        int wl;
        if (__popcll(cand) == 1) {
            wl = (int)__ffsll((long long)cand) - 1;
        } else {   // equal logits: the lowest expert index among the tied lanes
            const int emin = wave_min_i32(at_max ? best_e : 0x7fffffff);
            wl = (int)__ffsll((long long)__ballot(at_max && best_e == emin)) - 1;
        }
        const int widx = __builtin_amdgcn_readlane(best_e, wl);
        const bool pop = lane == wl;
        if constexpr (kSorted) {
#pragma unroll
            for (int i = 0; i + 1 < NV; ++i) {
                hv[i] = pop ? hv[i + 1] : hv[i];
                he[i] = pop ? he[i + 1] : he[i];
            }
            hv[NV - 1] = pop ? -__builtin_inff() : hv[NV - 1];
            he[NV - 1] = pop ? 0x7fffffff : he[NV - 1];
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) hv[i] = (pop && lane + 64 * i == widx) ? -__builtin_inff() : hv[i];
        }
        if constexpr (WEIGHTS) {
            if (j == 0) v0 = m;
            const float ex = __expf(m - v0);
            den += ex;
            if (lane == j) {
                id = widx;
                mine = ex;
            }
        } else {
            if (lane == j) id = widx;
        }
    }
    *my_id = lane < k ? id : -1;
    if constexpr (WEIGHTS) *my_w = lane < k ? mine / den : 0.f;
}

// NT tokens of one wave at once (E <= 256: four logits per lane and token): the same
// rounds, tie rule and weights as wave_topk_from<4>, with the tokens' independent
// reduction chains interleaved so that their latencies overlap.
template <int NT>
__device__ void wave_topk_multi(const float (&raw)[NT][4], int E, int k, int (&my_id)[NT], float (&my_w)[NT]) {
    const int lane = threadIdx.x & 63;
    float hv[NT][4];
    int he[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            hv[t][i] = (e < E && !__builtin_isnan(raw[t][i])) ? raw[t][i] : -__builtin_inff();
            he[t][i] = e < E ? e : 0x7fffffff;
        }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 1; i < 4; ++i)   // stable insertion sort, larger value first
#pragma unroll
            for (int j = i; j > 0; --j) {
                const bool sw = hv[t][j] > hv[t][j - 1];
                const float tv = hv[t][j];
                const int te = he[t][j];
                hv[t][j] = sw ? hv[t][j - 1] : hv[t][j];
                he[t][j] = sw ? he[t][j - 1] : he[t][j];
                hv[t][j - 1] = sw ? tv : hv[t][j - 1];
                he[t][j - 1] = sw ? te : he[t][j - 1];
            }
    float v0[NT], den[NT], mine[NT];
    int id[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        v0[t] = 0.f;
        den[t] = 0.f;
        mine[t] = 0.f;
        id[t] = -1;
    }
    for (int j = 0; j < k; ++j) {
        float v[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = hv[t][0];
        // the wave maxima, one DPP stage at a time over the tokens (as wave_max_f32)
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = fdpp_max(v[t], dpp_i32<0xb1, 0xf>(__float_as_int(v[t])));
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = fdpp_max(v[t], dpp_i32<0x4e, 0xf>(__float_as_int(v[t])));
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = fdpp_max(v[t], dpp_i32<0x141, 0xf>(__float_as_int(v[t])));
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = fdpp_max(v[t], dpp_i32<0x140, 0xf>(__float_as_int(v[t])));
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = fdpp_max(v[t], dpp_i32<0x142, 0xa>(__float_as_int(v[t])));
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = fdpp_max(v[t], dpp_i32<0x143, 0xc>(__float_as_int(v[t])));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[t]), 63));
            const bool at_max = hv[t][0] == m;
            const uint64_t cand = __ballot(at_max);
            int wl;
            if (__popcll(cand) == 1) {
                wl = (int)__ffsll((long long)cand) - 1;
            } else {   // equal logits: the lowest expert index among the tied lanes
                const int emin = wave_min_i32(at_max ? he[t][0] : 0x7fffffff);
                wl = (int)__ffsll((long long)__ballot(at_max && he[t][0] == emin)) - 1;
            }
            const int widx = __builtin_amdgcn_readlane(he[t][0], wl);
            const bool pop = lane == wl;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                hv[t][i] = pop ? hv[t][i + 1] : hv[t][i];
                he[t][i] = pop ? he[t][i + 1] : he[t][i];
            }
            hv[t][3] = pop ? -__builtin_inff() : hv[t][3];
            he[t][3] = pop ? 0x7fffffff : he[t][3];
            if (j == 0) v0[t] = m;
            const float ex = __expf(m - v0[t]);
            den[t] += ex;
            if (lane == j) {
                id[t] = widx;
                mine[t] = ex;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        my_id[t] = lane < k ? id[t] : -1;
        my_w[t] = lane < k ? mine[t] / den[t] : 0.f;
    }
}

template <int NV>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int* my_id, float* my_w) {
    float raw[NV];
    wave_topk_load<NV>(row, E, raw);
    wave_topk_from<NV>(raw, E, k, my_id, my_w);
}

__device__ __forceinline__ void wave_topk_any(const float* __restrict__ row, int E, int k, int* my_id,
                                              float* my_w) {
    if (E <= 256) wave_topk<4>(row, E, k, my_id, my_w);
    else if (E <= 512) wave_topk<8>(row, E, k, my_id, my_w);
    else wave_topk<16>(row, E, k, my_id, my_w);
}

// Checked copy of caller-supplied ids: out of range or repeated within the token -> -1.
__device__ __forceinline__ int checked_id(const int32_t* tok_ids, int j, int E) {
    const int e = tok_ids[j];
    if (e < 0 || e >= E) return -1;
    for (int jj = 0; jj < j; ++jj)
        if (tok_ids[jj] == e) return -1;
    return e;
}

}  // namespace
}  // namespace w4a16
