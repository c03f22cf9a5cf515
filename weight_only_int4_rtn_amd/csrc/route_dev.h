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


// Order-preserving unsigned key of a finite float (-0 is taken as +0, so equal logits
// get equal keys); larger logit <=> larger key, and no finite value maps to 0.
__device__ __forceinline__ uint32_t ordered_key(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u << 1) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Lane-wise max of a 64-bit key across the wave, returned in every lane.  DPP moves
// (quad permutes, row mirrors, then row broadcasts of lanes 15 and 31) keep every step
// in registers; the full maximum lands in lane 63 and is read back as a scalar.
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v, uint64_t o) { return o > v ? o : v; }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const uint32_t nlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false);
    const uint32_t nhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false);
    return (uint64_t)nhi << 32 | nlo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_step(v, dpp_u64<0xb1, 0xf>(v));    // quad_perm [1,0,3,2]
    v = dpp_max_step(v, dpp_u64<0x4e, 0xf>(v));    // quad_perm [2,3,0,1]
    v = dpp_max_step(v, dpp_u64<0x141, 0xf>(v));   // row_half_mirror
    v = dpp_max_step(v, dpp_u64<0x140, 0xf>(v));   // row_mirror: each row of 16 holds its max
    v = dpp_max_step(v, dpp_u64<0x142, 0xa>(v));   // row_bcast:15 into rows 1 and 3
    v = dpp_max_step(v, dpp_u64<0x143, 0xc>(v));   // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return (uint64_t)hi << 32 | lo;
}

// Top-k of one token by one wave: k rounds of a wave-wide maximum over 64-bit keys
// (ordered logit in the high half, the inverted expert index in the low half, so equal
// logits resolve to the lower index); the round's winner is marked taken by its lane.
// Lane j < k returns slot j's expert and its softmax weight over the chosen logits.
template <int NV>   // logits per lane: E <= 64 * NV
__device__ void wave_topk(const float* __restrict__ row, int E, int k, int* my_id, float* my_w) {
    const int lane = threadIdx.x & 63;
    uint64_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {   // unconditional (clamped) loads: all in flight together
        const int e = lane + 64 * i;
        const float v = row[min(e, E - 1)];
        key[i] = e < E ? ((uint64_t)ordered_key(v) << 32 | (uint32_t)~e) : 0ull;
    }
    float v0 = 0.f, den = 0.f, mine = 0.f;
    int id = -1;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) best = key[i] > best ? key[i] : best;
        const uint64_t win = wave_max_u64(best);
        const int widx = (int)~(uint32_t)win;
        const float wval = key_value((uint32_t)(win >> 32));
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (key[i] == win) key[i] = 0;   // only the owner lane holds this key
        if (j == 0) v0 = wval;
        const float ex = __expf(wval - v0);
        den += ex;
        if (lane == j) {
            id = widx;
            mine = ex;
        }
    }
    *my_id = lane < k ? id : -1;
    *my_w = lane < k ? mine / den : 0.f;
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
