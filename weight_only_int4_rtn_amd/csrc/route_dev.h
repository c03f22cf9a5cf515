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


// Logits are compared as ordered integer keys: signed comparison of two keys is the
// float comparison of the logits, -0 and +0 get the same key (0) and so tie, and a NaN
// logit takes the key of -inf, below every other value.  kKeyNone, below every logit's
// key, marks a slot with no expert.
constexpr int kKeyNone = (int)0x80000000;
__device__ __forceinline__ int logit_key(float v) {
    const int b = __float_as_int(__builtin_isnan(v) ? -__builtin_inff() : v + 0.0f);
    return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float key_logit(int key) { return __int_as_float(key >= 0 ? key : key ^ 0x7fffffff); }

// One DPP stage of a wave-wide reduction: lanes outside ROW_MASK's rows read IDENT, the
// identity of the reduction, so the move folds into the max / min instruction itself.
template <int CTRL, int ROW_MASK, int IDENT>
__device__ __forceinline__ int dpp_in(int v) {
    return __builtin_amdgcn_update_dpp(IDENT, v, CTRL, ROW_MASK, 0xf, false);
}
// Stage s of the wave-wide maximum / minimum (quad permutes, row mirrors, then row
// broadcasts of lanes 15 and 31): after the sixth, lane 63 holds the result.
template <int S, bool MAX>
__device__ __forceinline__ int wave_stage(int v) {
    constexpr int I = MAX ? (int)0x80000000 : 0x7fffffff;
    constexpr int C = S == 0 ? 0xb1 : S == 1 ? 0x4e : S == 2 ? 0x141 : S == 3 ? 0x140 : S == 4 ? 0x142 : 0x143;
    constexpr int R = S == 4 ? 0xa : S == 5 ? 0xc : 0xf;
    const int o = dpp_in<C, R, I>(v);
    return MAX ? max(v, o) : min(v, o);
}
__device__ __forceinline__ int wave_min_i32(int v) {
    v = wave_stage<0, false>(v);
    v = wave_stage<1, false>(v);
    v = wave_stage<2, false>(v);
    v = wave_stage<3, false>(v);
    v = wave_stage<4, false>(v);
    v = wave_stage<5, false>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

// Top-k of NT tokens by one wave, their rounds interleaved so that the latencies of the
// tokens' reduction chains overlap.  Lane l holds the logits of experts l, l + 64, ... of
// each token.  Each of the k rounds takes the wave-wide maximum of the lanes' best
// remaining keys; when several lanes tie on it, the lowest expert index among them wins (a
// second, rarely taken reduction).  The winner's lane removes it.  With NV <= 4 logits per
// lane the lane keeps its keys sorted (larger first, lower expert first on equal keys, the
// experts' positions packed 2 bits each) so its best is its first register; with more, the
// lane scans them each round.  Lane j < k returns slot j's expert and, with WEIGHTS, its
// softmax weight over the chosen logits.
template <int NT, int NV, bool WEIGHTS>
__device__ void wave_topk_core(const float (&raw)[NT][NV], int E, int k, int (&my_id)[NT], float (&my_w)[NT]) {
    constexpr bool kSorted = NV <= 4;
    const int lane = threadIdx.x & 63;
    int hk[NT][NV];
    uint32_t perm[NT];   // sorted: slot s holds the lane's logit i = (perm >> 2s) & 3
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < NV; ++i) hk[t][i] = lane + 64 * i < E ? logit_key(raw[t][i]) : kKeyNone;
        perm[t] = 0xe4u;   // identity: 0, 1, 2, 3
        if constexpr (kSorted) {
#pragma unroll
            for (int i = 1; i < NV; ++i)     // stable insertion sort, larger key first
#pragma unroll
                for (int j = i; j > 0; --j) {
                    const bool sw = hk[t][j] > hk[t][j - 1];
                    const int tk = hk[t][j];
                    hk[t][j] = sw ? hk[t][j - 1] : hk[t][j];
                    hk[t][j - 1] = sw ? tk : hk[t][j - 1];
                    // swap the 2-bit fields of slots j - 1 and j
                    const uint32_t a = (perm[t] >> (2 * j - 2)) & 3u, b = (perm[t] >> (2 * j)) & 3u;
                    const uint32_t swapped = (perm[t] & ~(0xfu << (2 * j - 2))) | (b << (2 * j - 2)) | (a << (2 * j));
                    perm[t] = sw ? swapped : perm[t];
                }
        }
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
        int best[NT], bi[NT], v[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if constexpr (kSorted) {
                best[t] = hk[t][0];
                bi[t] = (int)(perm[t] & 3u);
            } else {   // the lane's largest remaining key, lowest position first on ties
                best[t] = hk[t][0];
                bi[t] = 0;
#pragma unroll
                for (int i = 1; i < NV; ++i) {
                    const bool gt = hk[t][i] > best[t];
                    best[t] = gt ? hk[t][i] : best[t];
                    bi[t] = gt ? i : bi[t];
                }
            }
            v[t] = best[t];
        }
        // the wave maxima, one DPP stage at a time over the tokens
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = wave_stage<0, true>(v[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = wave_stage<1, true>(v[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = wave_stage<2, true>(v[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = wave_stage<3, true>(v[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = wave_stage<4, true>(v[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = wave_stage<5, true>(v[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int m = __builtin_amdgcn_readlane(v[t], 63);
            const bool at_max = best[t] == m;
            const int be = best[t] == kKeyNone ? 0x7fffffff : lane + 64 * bi[t];
            const uint64_t cand = __ballot(at_max);
            int wl;
            if (__popcll(cand) == 1) {
                wl = (int)__ffsll((long long)cand) - 1;
            } else {   // equal logits: the lowest expert index among the tied lanes
                const int emin = wave_min_i32(at_max ? be : 0x7fffffff);
                wl = (int)__ffsll((long long)__ballot(at_max && be == emin)) - 1;
            }
            const int widx = __builtin_amdgcn_readlane(be, wl);
            const bool pop = lane == wl;
            if constexpr (kSorted) {
#pragma unroll
                for (int i = 0; i + 1 < NV; ++i) hk[t][i] = pop ? hk[t][i + 1] : hk[t][i];
                hk[t][NV - 1] = pop ? kKeyNone : hk[t][NV - 1];
                perm[t] = pop ? perm[t] >> 2 : perm[t];
            } else {
#pragma unroll
                for (int i = 0; i < NV; ++i) hk[t][i] = (pop && i == bi[t]) ? kKeyNone : hk[t][i];
            }
            if constexpr (WEIGHTS) {
                const float mf = key_logit(m);
                if (j == 0) v0[t] = mf;
                const float ex = __expf(mf - v0[t]);
                den[t] += ex;
                if (lane == j) {
                    id[t] = widx;
                    mine[t] = ex;
                }
            } else {
                if (lane == j) id[t] = widx;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        my_id[t] = lane < k ? id[t] : -1;
        if constexpr (WEIGHTS) my_w[t] = lane < k ? mine[t] / den[t] : 0.f;
    }
}

// This lane's logits of one token (experts lane, lane + 64, ...): unconditional (clamped)
// loads, all in flight together.
template <int NV>
__device__ __forceinline__ void wave_topk_load(const float* __restrict__ row, int E, float (&raw)[NV]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NV; ++i) raw[i] = row[min(lane + 64 * i, E - 1)];
}

// One token (WEIGHTS false: only the experts, my_w untouched, for callers that need just a
// rank's winner; the rounds are the same).
template <int NV, bool WEIGHTS = true>   // logits per lane: E <= 64 * NV
__device__ __forceinline__ void wave_topk_from(const float (&raw)[NV], int E, int k, int* my_id, float* my_w) {
    int id[1];
    float w[1];
    wave_topk_core<1, NV, WEIGHTS>(reinterpret_cast<const float(&)[1][NV]>(raw), E, k, id, w);
    *my_id = id[0];
    if constexpr (WEIGHTS) *my_w = w[0];
}

// NT tokens of one wave at once (E <= 256: four logits per lane and token).
template <int NT>
__device__ __forceinline__ void wave_topk_multi(const float (&raw)[NT][4], int E, int k, int (&my_id)[NT],
                                                float (&my_w)[NT]) {
    wave_topk_core<NT, 4, true>(raw, E, k, my_id, my_w);
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

// Expert of pair (token t, top-k rank j), the same in every lane (-1: dropped).  From
// logits the wave runs the top-k only up to round j (the rounds are those of the full
// routing, so the winner is the same), which lets a workgroup that serves one pair start
// loading its weights before the whole batch is routed.
// Rank j's expert of one token (E <= 256, four logits per lane), up to two winners per
// round: one reduction gives the two largest lane-best keys M1 > M2 (a max / second-max
// pair per DPP stage); the lane holding M1 wins first, and the second winner is that lane's
// next key when it is larger than M2, else the lane holding M2.  Any equal keys among these
// candidates (where the lower expert index decides) take a round of one winner with the
// tie rule of wave_topk_core instead.  Same winners, in the same order, as wave_topk_core.
__device__ int wave_rank_expert2(const float (&raw)[4], int E, int j) {
    const int lane = threadIdx.x & 63;
    int hk[4];
    uint32_t perm = 0xe4u;
#pragma unroll
    for (int i = 0; i < 4; ++i) hk[i] = lane + 64 * i < E ? logit_key(raw[i]) : kKeyNone;
#pragma unroll
    for (int i = 1; i < 4; ++i)   // stable insertion sort, larger key first
#pragma unroll
        for (int jj = i; jj > 0; --jj) {
            const bool sw = hk[jj] > hk[jj - 1];
            const int tk = hk[jj];
            hk[jj] = sw ? hk[jj - 1] : hk[jj];
            hk[jj - 1] = sw ? tk : hk[jj - 1];
            const uint32_t a = (perm >> (2 * jj - 2)) & 3u, b = (perm >> (2 * jj)) & 3u;
            const uint32_t swapped = (perm & ~(0xfu << (2 * jj - 2))) | (b << (2 * jj - 2)) | (a << (2 * jj));
            perm = sw ? swapped : perm;
        }
    auto pop = [&](bool me) {
#pragma unroll
        for (int i = 0; i < 3; ++i) hk[i] = me ? hk[i + 1] : hk[i];
        hk[3] = me ? kKeyNone : hk[3];
        perm = me ? perm >> 2 : perm;
    };
    for (int r = 0;;) {
        // the two largest lane-best keys: (first, second) pairs merged stage by stage
        int a1 = hk[0], a2 = kKeyNone;
#pragma unroll
        for (int st = 0; st < 6; ++st) {
            const int b1 = st == 0 ? dpp_in<0xb1, 0xf, (int)0x80000000>(a1)
                         : st == 1 ? dpp_in<0x4e, 0xf, (int)0x80000000>(a1)
                         : st == 2 ? dpp_in<0x141, 0xf, (int)0x80000000>(a1)
                         : st == 3 ? dpp_in<0x140, 0xf, (int)0x80000000>(a1)
                         : st == 4 ? dpp_in<0x142, 0xa, (int)0x80000000>(a1)
                                   : dpp_in<0x143, 0xc, (int)0x80000000>(a1);
            const int b2 = st == 0 ? dpp_in<0xb1, 0xf, (int)0x80000000>(a2)
                         : st == 1 ? dpp_in<0x4e, 0xf, (int)0x80000000>(a2)
                         : st == 2 ? dpp_in<0x141, 0xf, (int)0x80000000>(a2)
                         : st == 3 ? dpp_in<0x140, 0xf, (int)0x80000000>(a2)
                         : st == 4 ? dpp_in<0x142, 0xa, (int)0x80000000>(a2)
                                   : dpp_in<0x143, 0xc, (int)0x80000000>(a2);
            a2 = max(min(a1, b1), max(a2, b2));
            a1 = max(a1, b1);
        }
        const int M1 = __builtin_amdgcn_readlane(a1, 63), M2 = __builtin_amdgcn_readlane(a2, 63);
        const int be = hk[0] == kKeyNone ? 0x7fffffff : lane + 64 * (int)(perm & 3u);
        const uint64_t c1 = __ballot(hk[0] == M1);
        if (__popcll(c1) == 1) {
            const int w1 = (int)__ffsll((long long)c1) - 1;
            if (r == j) return __builtin_amdgcn_readlane(be, w1);
            const int s = __builtin_amdgcn_readlane(hk[1], w1);
            if (s > M2) {   // the winner lane's next key is second
                if (r + 1 == j) return __builtin_amdgcn_readlane(lane + 64 * (int)((perm >> 2) & 3u), w1);
                pop(lane == w1);
                pop(lane == w1);
                r += 2;
                continue;
            }
            const uint64_t c2 = __ballot(hk[0] == M2);
            if (s < M2 && __popcll(c2) == 1) {   // another lane's best is second
                const int w2 = (int)__ffsll((long long)c2) - 1;
                if (r + 1 == j) return __builtin_amdgcn_readlane(be, w2);
                pop(lane == w1 || lane == w2);
                r += 2;
                continue;
            }
            pop(lane == w1);   // equal keys behind the first: one winner this round
            r += 1;
            continue;
        }
        // equal keys on top: the lowest expert index among the tied lanes, one winner
        const int emin = wave_min_i32(hk[0] == M1 ? be : 0x7fffffff);
        const int wl = (int)__ffsll((long long)__ballot(hk[0] == M1 && be == emin)) - 1;
        if (r == j) return emin;
        pop(lane == wl);
        r += 1;
    }
}

// TWO: the two-winner rounds (E <= 256); measured faster in the single-launch kernel and
// slightly slower inside the streaming kernel, whose code around it it changes.
template <bool TWO>
__device__ __forceinline__ int pair_expert(const float* logits, const int32_t* ids, int E, int k, int t, int j) {
    if (!logits) return checked_id(ids + t * k, j, E);
    const float* row = logits + (int64_t)t * E;
    int id;
    float w;
    if (E <= 256) {
        float raw[4];
        wave_topk_load<4>(row, E, raw);
        if constexpr (TWO) return __builtin_amdgcn_readfirstlane(wave_rank_expert2(raw, E, j));
        wave_topk_from<4, false>(raw, E, j + 1, &id, &w);
    } else if (E <= 512) {
        float raw[8];
        wave_topk_load<8>(row, E, raw);
        wave_topk_from<8, false>(raw, E, j + 1, &id, &w);
    } else {
        float raw[16];
        wave_topk_load<16>(row, E, raw);
        wave_topk_from<16, false>(raw, E, j + 1, &id, &w);
    }
    return __builtin_amdgcn_readlane(id, j);
}

}  // namespace
}  // namespace w4a16
