// Top-k routing with renormalised softmax weights, expert histogram and the canonical
// (expert, token) permutation of (token, slot) pairs.
//
// Page "Nex-N2.5-mini FP8 W8A8 with Calibrated FP8 KV Scales", Artifact summary: 256
// routed experts, 8 active per token.  The chosen experts are weighted by the softmax of
// all logits renormalised over the chosen ones, which equals the softmax of the chosen
// logits alone.
//
// Every result is deterministic: counts come from integer atomics, positions from ranks
// computed with per-expert token bitmasks (a token picks an expert at most once), never
// from the order in which atomics land.
//
// Small batches (T <= 64): one 1024-thread workgroup does everything in one launch; or,
// from logits, route_split_kernel: one token per wave over ceil(T / 8) workgroups, and the
// last workgroup to arrive finishes the routing of the whole batch.
// Large batches: route_block_kernel (top-k, block histogram, in-block ranks, activation
// group sums) -> route_colscan_kernel (per expert: ranks of each block's first pair, total)
// -> route_scan_kernel (offsets, active experts, GEMM tile list) -> route_scatter_kernel
// (sorted pair list).
#include "common.h"
#include "route_dev.h"
#include "route_small.h"

namespace w4a16 {

// ------------------------------------------------------------------ small batch

__global__ __launch_bounds__(1024) void route_small_kernel(RouteArgs a) {
    __shared__ SmallRouteLds lds;
    route_small_wg(a, lds, true);
}

// Wave w of workgroup b runs the top-k of token 8 b + w and writes its experts and weights
// through to memory; the workgroup then counts its arrival (the atomic releases its
// writes), and the last one to arrive reads every pair back past the caches, resets the
// counter for the next call and finishes the routing alone.  A wave's top-k is a chain of
// dependent reductions (about 2 us for k = 8), so spreading the tokens over waves instead
// of queueing several per wave shortens the launch by the difference.
constexpr int kSplitWaves = 8;
__global__ __launch_bounds__(64 * kSplitWaves) void route_split_kernel(RouteArgs a) {
    __shared__ SmallRouteLds lds;
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, k = a.k, P = a.T * k;
    const int t = blockIdx.x * kSplitWaves + wave;
    const __amdgpu_buffer_rsrc_t ir = make_rsrc(a.ids, (uint32_t)(P * 4));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wts, (uint32_t)(P * 4));
    if (t < a.T) {
        int my_id;
        float my_w;
        wave_topk_any(a.logits + (int64_t)t * E, E, k, &my_id, &my_w);
        if (lane < k) {
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)my_id, ir, (uint32_t)((t * k + lane) * 4), 0, kSc1);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(my_w), wr, (uint32_t)((t * k + lane) * 4), 0, kSc1);
        }
    }
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(sync_word(a.sync, kSyncRoute), 1u, __ATOMIC_ACQ_REL,
                                        __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    if (tid == 0) __hip_atomic_store(sync_word(a.sync, kSyncRoute), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int p = tid; p < P; p += blockDim.x) {
        lds.ids[p] = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, (uint32_t)(p * 4), 0, kSc1);
        lds.w[p] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wr, (uint32_t)(p * 4), 0, kSc1));
    }
    route_small_finish(a, lds, true);
}

// ------------------------------------------------------------------ large batch

// One workgroup per block of kRouteBlockT = 32 tokens (16 waves, 2 tokens each).
static_assert(kRouteBlockT == 32, "route_block_kernel: two tokens per wave, 16 waves");
__global__ __launch_bounds__(1024) void route_block_kernel(RouteArgs a) {
    __shared__ int s_ids[kRouteBlockT * kMaxK];
    __shared__ int s_cnt[kMaxE];
    __shared__ uint32_t s_mlo[kMaxE], s_mhi[kMaxE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, k = a.k;
    const int t0 = blockIdx.x * kRouteBlockT;
    const int nt = min(kRouteBlockT, a.T - t0);
    for (int e = tid; e < E; e += blockDim.x) { s_cnt[e] = 0; s_mlo[e] = 0; s_mhi[e] = 0; }

    // Wave w takes tokens w and w + 16 of the block.  Their activations (lane: 32 columns of
    // each 2048) are loaded before anything else, all at once, so that the latency overlaps
    // the top-k; from logits with E <= 256 the two selections run interleaved.
    const int tl0 = wave, tl1 = wave + 16;
    const int ntok = (tl0 < nt) + (tl1 < nt);
    u32x4_t r[2][4];
    auto load_x = [&](int j, int64_t c) {
        const uint16_t* xr = a.x + (int64_t)(t0 + (j ? tl1 : tl0)) * a.H;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[j][i] = *reinterpret_cast<const u32x4_t*>(xr + c + 8 * i);
    };
    if (lane * 32 < a.H) {
        if (ntok > 0) load_x(0, lane * 32);
        if (ntok > 1) load_x(1, lane * 32);
    }
    auto put = [&](int tl, int my_id, float my_w) {
        const int t = t0 + tl;
        if (lane < k) {
            a.ids[(int64_t)t * k + lane] = my_id;
            a.wts[(int64_t)t * k + lane] = my_w;
            s_ids[tl * k + lane] = my_id;
        }
    };
    if (a.logits && E <= 256 && ntok == 2) {
        float raw[2][4];
        wave_topk_load<4>(a.logits + (int64_t)(t0 + tl0) * E, E, raw[0]);
        wave_topk_load<4>(a.logits + (int64_t)(t0 + tl1) * E, E, raw[1]);
        int my_id[2];
        float my_w[2];
        wave_topk_multi<2>(raw, E, k, my_id, my_w);
        put(tl0, my_id[0], my_w[0]);
        put(tl1, my_id[1], my_w[1]);
    } else {
        for (int j = 0; j < ntok; ++j) {
            const int tl = j ? tl1 : tl0, t = t0 + tl;
            if (a.logits) {
                int my_id;
                float my_w;
                wave_topk_any(a.logits + (int64_t)t * E, E, k, &my_id, &my_w);
                put(tl, my_id, my_w);
            } else if (lane < k) {
                s_ids[tl * k + lane] = checked_id(a.ids + (int64_t)t * k, lane, E);
            }
        }
    }
    // sums of the bf16 activations over each group of 128 columns (lane: 32 columns), and
    // the row copied with every 8-column block in the MFMA operand order
    for (int j = 0; j < ntok; ++j) {
        const int t = t0 + (j ? tl1 : tl0);
        uint16_t* xpr = a.xp + (int64_t)t * a.H;
        for (int64_t c0 = 0; c0 < a.H; c0 += 64 * 32) {
            const int64_t c = c0 + lane * 32;
            float sum = 0.0f;
            if (c < a.H) {
                if (c0 > 0) load_x(j, c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    *reinterpret_cast<u32x4_t*>(xpr + c + 8 * i) = perm_act(r[j][i]);
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        sum += __uint_as_float(r[j][i][h] << 16) + __uint_as_float(r[j][i][h] & 0xffff0000u);
                }
            }
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            if ((lane & 3) == 0 && c < a.H) a.xsum[(int64_t)t * (a.H / kGroup) + c / kGroup] = sum;
        }
    }
    __syncthreads();

    for (int p = tid; p < nt * k; p += blockDim.x) {
        const int e = s_ids[p];
        if (e >= 0) {
            const int tl = p / k;
            atomicAdd(&s_cnt[e], 1);
            if (tl < 32) atomicOr(&s_mlo[e], 1u << tl);
            else atomicOr(&s_mhi[e], 1u << (tl - 32));
        }
    }
    __syncthreads();

    for (int p = tid; p < nt * k; p += blockDim.x) {
        const int e = s_ids[p];
        int rank = -1;
        if (e >= 0) {
            const int tl = p / k;
            const uint32_t lo = s_mlo[e], hi = s_mhi[e];
            rank = tl < 32 ? __popc(lo & ((1u << tl) - 1u)) : __popc(lo) + __popc(hi & ((1u << (tl - 32)) - 1u));
        }
        a.lrank[(int64_t)t0 * k + p] = e >= 0 ? (e << 8 | rank) : -1;   // rank < 64 fits 8 bits
    }
    for (int e = tid; e < E; e += blockDim.x) a.hist[(int64_t)e * a.nblk + blockIdx.x] = s_cnt[e];
}

// One 256-thread workgroup per expert: the exclusive prefix of the expert's per-block
// counts (expert-major, in place: each block's first rank within the expert) and the
// expert's total.
__global__ __launch_bounds__(256) void route_colscan_kernel(RouteArgs a) {
    __shared__ int s_tmp[64];
    const int e = blockIdx.x, tid = threadIdx.x, nblk = a.nblk;
    int32_t* h = a.hist + (int64_t)e * nblk;
    int carry = 0;
    for (int b0 = 0; b0 < nblk; b0 += 256) {
        const int b = b0 + tid;
        const int v = b < nblk ? h[b] : 0;
        int tot = 0;
        const int ex = block_exclusive_scan(v, s_tmp, &tot);
        if (b < nblk) h[b] = carry + ex;
        carry += tot;
    }
    if (tid == 0) a.counts[e] = carry;
}

// One 1024-thread workgroup: offsets from the experts' totals, the active list and the
// M-tile list of the grouped GEMM.
__global__ __launch_bounds__(1024) void route_scan_kernel(RouteArgs a) {
    __shared__ int s_tmp[64];
    const int e = threadIdx.x, E = a.E;
    const int c = e < E ? a.counts[e] : 0;
    int total = 0, n_active = 0, n_tiles = 0;
    const int off = block_exclusive_scan(c, s_tmp, &total);
    const int act = block_exclusive_scan(c > 0 ? 1 : 0, s_tmp, &n_active);
    const int nt = (c + kPrefillMT - 1) / kPrefillMT;
    const int toff = block_exclusive_scan(nt, s_tmp, &n_tiles);
    if (e < E) {
        a.offsets[e] = off;
        if (c > 0) a.active[act] = e;
        for (int i = 0; i < nt && toff + i < a.max_tiles; ++i) {
            a.tiles[2 * (toff + i)] = e;
            a.tiles[2 * (toff + i) + 1] = i * kPrefillMT;
        }
    }
    if (e == 0) {
        a.offsets[E] = total;
        a.meta[0] = n_active;
        a.meta[1] = (int)min((int64_t)n_tiles, a.max_tiles);
    }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= (int64_t)a.T * a.k) return;
    const int v = a.lrank[p];
    if (v < 0) {
        a.inv[p] = -1;
        return;
    }
    const int e = v >> 8, rank = v & 255;
    const int t = (int)(p / a.k);
    const int b = t / kRouteBlockT;
    const int pos = a.offsets[e] + a.hist[(int64_t)e * a.nblk + b] + rank;
    a.sorted[pos] = (int)p;
    a.tokw[pos] = int2{t, __float_as_int(a.wts[p])};
    a.inv[p] = pos;
}

hipError_t launch_route_small(const RouteArgs& a, hipStream_t s, StageTimer* t) {
    launch(t, "route_small", route_small_kernel, dim3(1), dim3(1024), s, 0u, a);
    return hipGetLastError();
}

hipError_t launch_route_split(const RouteArgs& a, hipStream_t s, StageTimer* t) {
    launch(t, "route_split", route_split_kernel, dim3((unsigned)((a.T + kSplitWaves - 1) / kSplitWaves)),
           dim3(64 * kSplitWaves), s, 0u, a);
    return hipGetLastError();
}

hipError_t launch_route_large(const RouteArgs& a, hipStream_t s, StageTimer* t) {
    launch(t, "route_block", route_block_kernel, dim3(a.nblk), dim3(1024), s, 0u, a);
    launch(t, "route_colscan", route_colscan_kernel, dim3((unsigned)a.E), dim3(256), s, 0u, a);
    launch(t, "route_scan", route_scan_kernel, dim3(1), dim3(1024), s, 0u, a);
    const int64_t P = (int64_t)a.T * a.k;
    launch(t, "route_scatter", route_scatter_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), s, 0u, a);
    return hipGetLastError();
}

}  // namespace w4a16
