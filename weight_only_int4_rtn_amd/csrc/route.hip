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
// Small batches (T <= 64): one 1024-thread workgroup does everything in one launch.
// Large batches: route_block_kernel (top-k, block histogram, in-block ranks, activation
// group sums) -> route_scan_kernel (offsets, active experts, GEMM tile list) ->
// route_scatter_kernel (sorted pair list).
#include "common.h"

namespace w4a16 {

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

// True when (va, ia) ranks before (vb, ib): larger logit first, lower index on ties.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    if (ia < 0) return false;
    if (ib < 0) return true;
    return va > vb || (va == vb && ia < ib);
}

// Top-k of one token by one wave.  Lane j < k ends holding the j-th chosen expert and
// its logit in (*my_id, *my_val).
__device__ void wave_topk(const float* __restrict__ row, int E, int k, int* my_id, float* my_val) {
    const int lane = threadIdx.x & 63;
    constexpr int NV = kMaxE / 64;
    float v[NV];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? row[e] : 0.0f;
        if (e >= E) taken |= 1u << i;
    }
    *my_id = -1;
    *my_val = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (64 * i < E) {
                const int e = lane + 64 * i;
                if (!(taken >> i & 1u) && ranks_before(v[i], e, bv, bi)) { bv = v[i]; bi = e; }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        bv = __shfl(bv, 0);
        bi = __shfl(bi, 0);
        if (bi >= 0 && (bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) { *my_id = bi; *my_val = bv; }
    }
}

// Softmax weights of the k chosen logits; lanes j < k write slot j to global memory.
__device__ __forceinline__ void wave_weights(int my_id, float my_val, int k, int32_t* ids, float* wts) {
    const int lane = threadIdx.x & 63;
    const float v0 = __shfl(my_val, 0);
    float den = 0.0f;
    for (int j = 0; j < k; ++j) den += __expf(__shfl(my_val, j) - v0);
    if (lane < k) {
        wts[lane] = __expf(my_val - v0) / den;
        ids[lane] = my_id;
    }
}

// Checked copy of caller-supplied ids: out of range or repeated within the token -> -1.
__device__ __forceinline__ int checked_id(const int32_t* tok_ids, int j, int E) {
    const int e = tok_ids[j];
    if (e < 0 || e >= E) return -1;
    for (int jj = 0; jj < j; ++jj)
        if (tok_ids[jj] == e) return -1;
    return e;
}

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024, multiple of 64).
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_tmp[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int t = lane < nw ? s_tmp[lane] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(t, off);
            if (lane >= off) t += o;
        }
        if (lane < nw) s_tmp[32 + lane] = t;   // inclusive wave prefix
    }
    __syncthreads();
    const int base = wave ? s_tmp[32 + wave - 1] : 0;
    *total = s_tmp[32 + nw - 1];
    __syncthreads();
    return base + incl - v;
}

}  // namespace

// ------------------------------------------------------------------ small batch

__global__ __launch_bounds__(1024) void route_small_kernel(RouteArgs a) {
    __shared__ int s_ids[kSmallT * kMaxK];
    __shared__ int s_cnt[kMaxE];
    __shared__ uint32_t s_mlo[kMaxE], s_mhi[kMaxE];
    __shared__ int s_off[kMaxE];
    __shared__ int s_tmp[64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T, E = a.E, k = a.k, P = T * k;
    for (int e = tid; e < E; e += blockDim.x) { s_cnt[e] = 0; s_mlo[e] = 0; s_mhi[e] = 0; }

    if (a.logits) {
        for (int t = wave; t < T; t += blockDim.x >> 6) {
            int my_id;
            float my_val;
            wave_topk(a.logits + (int64_t)t * E, E, k, &my_id, &my_val);
            wave_weights(my_id, my_val, k, a.ids + t * k, a.wts + t * k);
            if (lane < k) s_ids[t * k + lane] = my_id;
        }
    } else {
        for (int p = tid; p < P; p += blockDim.x) s_ids[p] = checked_id(a.ids + (p / k) * k, p % k, E);
    }
    __syncthreads();

    for (int p = tid; p < P; p += blockDim.x) {
        const int e = s_ids[p];
        if (e >= 0) {
            const int t = p / k;
            atomicAdd(&s_cnt[e], 1);
            if (t < 32) atomicOr(&s_mlo[e], 1u << t);
            else atomicOr(&s_mhi[e], 1u << (t - 32));
        }
    }
    __syncthreads();

    // offsets (exclusive scan of counts) and the ascending list of active experts
    int total = 0, n_active = 0;
    const int c = tid < E ? s_cnt[tid] : 0;
    const int off = block_exclusive_scan(c, s_tmp, &total);
    const int act = block_exclusive_scan(c > 0 ? 1 : 0, s_tmp, &n_active);
    if (tid < E) {
        s_off[tid] = off;
        a.offsets[tid] = off;
        a.counts[tid] = c;
        if (c > 0) a.active[act] = tid;
    }
    if (tid == 0) {
        a.offsets[E] = total;
        a.meta[0] = n_active;
        a.meta[1] = 0;
    }
    __syncthreads();

    for (int p = tid; p < P; p += blockDim.x) {
        const int e = s_ids[p];
        if (e >= 0) {
            const int t = p / k;
            const uint32_t lo = s_mlo[e], hi = s_mhi[e];
            const int rank = t < 32 ? __popc(lo & ((1u << t) - 1u))
                                    : __popc(lo) + __popc(hi & ((1u << (t - 32)) - 1u));
            a.sorted[s_off[e] + rank] = p;
        }
    }
}

// ------------------------------------------------------------------ large batch

// One workgroup per block of kRouteBlockT tokens (4 waves, 16 tokens each).
__global__ __launch_bounds__(256) void route_block_kernel(RouteArgs a) {
    __shared__ int s_ids[kRouteBlockT * kMaxK];
    __shared__ int s_cnt[kMaxE];
    __shared__ uint32_t s_mlo[kMaxE], s_mhi[kMaxE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, k = a.k;
    const int t0 = blockIdx.x * kRouteBlockT;
    const int nt = min(kRouteBlockT, a.T - t0);
    for (int e = tid; e < E; e += blockDim.x) { s_cnt[e] = 0; s_mlo[e] = 0; s_mhi[e] = 0; }

    for (int tl = wave; tl < nt; tl += 4) {
        const int t = t0 + tl;
        if (a.logits) {
            int my_id;
            float my_val;
            wave_topk(a.logits + (int64_t)t * E, E, k, &my_id, &my_val);
            wave_weights(my_id, my_val, k, a.ids + (int64_t)t * k, a.wts + (int64_t)t * k);
            if (lane < k) s_ids[tl * k + lane] = my_id;
        } else if (lane < k) {
            s_ids[tl * k + lane] = checked_id(a.ids + (int64_t)t * k, lane, E);
        }
        // sums of the bf16 activations over each group of 128 columns (lane: 32 columns)
        const uint16_t* xr = a.x + (int64_t)t * a.H;
        for (int64_t c0 = 0; c0 < a.H; c0 += 64 * 32) {
            const int64_t c = c0 + lane * 32;
            float sum = 0.0f;
            if (c < a.H) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4_t r = *reinterpret_cast<const u32x4_t*>(xr + c + 8 * i);
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        sum += __uint_as_float(r[h] << 16) + __uint_as_float(r[h] & 0xffff0000u);
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
    for (int e = tid; e < E; e += blockDim.x) a.hist[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

// One 1024-thread workgroup: per-expert totals over blocks, offsets, per-block bases
// (written over the histogram), the active list and the M-tile list of the grouped GEMM.
__global__ __launch_bounds__(1024) void route_scan_kernel(RouteArgs a) {
    __shared__ int s_tmp[64];
    const int tid = threadIdx.x, E = a.E, nblk = a.nblk;
    int c = 0;
    if (tid < E)
        for (int b = 0; b < nblk; ++b) c += a.hist[(int64_t)b * E + tid];
    int total = 0, n_active = 0, n_tiles = 0;
    const int off = block_exclusive_scan(c, s_tmp, &total);
    const int act = block_exclusive_scan(c > 0 ? 1 : 0, s_tmp, &n_active);
    const int nt = (c + kPrefillMT - 1) / kPrefillMT;
    const int toff = block_exclusive_scan(nt, s_tmp, &n_tiles);
    if (tid < E) {
        a.offsets[tid] = off;
        a.counts[tid] = c;
        if (c > 0) a.active[act] = tid;
        int run = off;
        for (int b = 0; b < nblk; ++b) {
            const int64_t i = (int64_t)b * E + tid;
            const int h = a.hist[i];
            a.hist[i] = run;
            run += h;
        }
        for (int i = 0; i < nt && toff + i < a.max_tiles; ++i) {
            a.tiles[2 * (toff + i)] = tid;
            a.tiles[2 * (toff + i) + 1] = i * kPrefillMT;
        }
    }
    if (tid == 0) {
        a.offsets[E] = total;
        a.meta[0] = n_active;
        a.meta[1] = (int)min((int64_t)n_tiles, a.max_tiles);
    }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= (int64_t)a.T * a.k) return;
    const int v = a.lrank[p];
    if (v < 0) return;
    const int e = v >> 8, rank = v & 255;
    const int b = (int)(p / a.k) / kRouteBlockT;
    a.sorted[a.hist[(int64_t)b * a.E + e] + rank] = (int)p;
}

hipError_t launch_route_small(const RouteArgs& a, hipStream_t s) {
    route_small_kernel<<<1, 1024, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_route_large(const RouteArgs& a, hipStream_t s) {
    route_block_kernel<<<a.nblk, 256, 0, s>>>(a);
    route_scan_kernel<<<1, 1024, 0, s>>>(a);
    const int64_t P = (int64_t)a.T * a.k;
    route_scatter_kernel<<<(unsigned)((P + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace w4a16
