// Routing of a small batch (T <= kSmallT tokens) by one workgroup of any multiple of 64
// threads: top-k with renormalised softmax weights (page "Nex-N2.5-mini FP8 W8A8 with
// Calibrated FP8 KV Scales", Artifact summary: 256 routed experts, 8 active per token),
// per-expert counts, the (expert, token) order of the pairs and M-tiles of at most 16 rows.
// Shared by the routing kernel and by the streaming gate/up kernel, whose every workgroup
// routes the batch itself (one of them writes the results out).
#pragma once
#include "common.h"
#include "route_dev.h"

namespace w4a16 {
namespace {

// Block-wide exclusive scan of one value per thread (blockDim.x <= 1024, multiple of 64);
// s_tmp holds 64 values.
template <typename V>
__device__ V block_exclusive_scan(V v, V* s_tmp, V* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    V incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const V o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_tmp[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        V t = lane < nw ? s_tmp[lane] : V(0);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const V o = __shfl_up(t, off);
            if (lane >= off) t += o;
        }
        if (lane < nw) s_tmp[32 + lane] = t;   // inclusive wave prefix
    }
    __syncthreads();
    const V base = wave ? s_tmp[32 + wave - 1] : V(0);
    *total = s_tmp[32 + nw - 1];
    __syncthreads();
    return base + incl - v;
}

struct SmallRouteLds {
    int ids[kSmallT * kMaxK];   // per pair: expert, -1 when dropped
    float w[kSmallT * kMaxK];   // per pair: router weight
    int cnt[kMaxE];             // pairs per expert
    uint32_t mlo[kMaxE], mhi[kMaxE];   // tokens of each expert (bit t)
    int off[kMaxE];             // first sorted position of each expert
    int tstart[kMaxE];          // first M-tile of each expert
    uint64_t tmp[64];
    int n_tiles, n_active;
};

// Record of routed M-tile t (two int4, see RouteArgs::trec) from the workgroup's routing.
// pair_k > 0: each row's pair index t * pair_k + j in place of its token t.
__device__ __forceinline__ void small_tile_record(const SmallRouteLds& s, int E, int t, int4& r0, int4& r1,
                                                  int pair_k = 0) {
    int lo = 0, hi = E - 1;   // the last expert whose first tile is <= t owns tile t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.tstart[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo, j = t - s.tstart[e];
    const int cnt = min(16, s.cnt[e] - 16 * j);
    uint64_t m = (uint64_t)s.mhi[e] << 32 | s.mlo[e];
    for (int i = 0; i < 16 * j; ++i) m &= m - 1;
    unsigned __int128 toks = 0;
    for (int i = 0; i < cnt; ++i) {
        int v = __builtin_ctzll(m);
        if (pair_k > 0) {   // the token's rank of expert e (ids are distinct within a token)
            int j = 0;
            while (j < pair_k - 1 && s.ids[v * pair_k + j] != e) ++j;
            v = v * pair_k + j;
        }
        toks |= (unsigned __int128)v << (kRecTokBits * i);
        m &= m - 1;
    }
    r0 = int4{e, s.off[e] + 16 * j, cnt, 0};
    r1 = int4{(int)(uint32_t)toks, (int)(uint32_t)(toks >> 32), (int)(uint32_t)(toks >> 64), 0};
}

__device__ void route_small_finish(const RouteArgs& a, SmallRouteLds& s, bool writer);

// Routes the batch into `s` (all threads of the workgroup take part; E <= 2 * blockDim.x).
// `writer`: also stores every routing output of RouteArgs.
__device__ void route_small_wg(const RouteArgs& a, SmallRouteLds& s, bool writer) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int T = a.T, E = a.E, k = a.k, P = T * k;

    if (a.logits) {
        auto emit = [&](int t, int my_id, float my_w) {
            if (lane < k) {
                if (writer) {
                    a.ids[t * k + lane] = my_id;
                    a.wts[t * k + lane] = my_w;
                }
                s.ids[t * k + lane] = my_id;
                s.w[t * k + lane] = my_w;
            }
        };
        if (E <= 256 && T <= 2 * nw) {   // at most two tokens per wave: their rounds interleaved
            const int t0 = wave, t1 = wave + nw;
            if (t0 < T) {
                float raw[2][4];
                wave_topk_load<4>(a.logits + (int64_t)t0 * E, E, raw[0]);
                wave_topk_load<4>(a.logits + (int64_t)min(t1, T - 1) * E, E, raw[1]);
                int my_id[2];
                float my_w[2];
                wave_topk_multi<2>(raw, E, k, my_id, my_w);
                emit(t0, my_id[0], my_w[0]);
                if (t1 < T) emit(t1, my_id[1], my_w[1]);
            }
        } else if (E <= 256) {   // up to four tokens of this wave loaded before their top-k, one after another
            for (int t0 = wave; t0 < T; t0 += 4 * nw) {
                float raw[4][4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    wave_topk_load<4>(a.logits + (int64_t)min(t0 + j * nw, T - 1) * E, E, raw[j]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = t0 + j * nw;
                    if (t < T) {
                        int my_id;
                        float my_w;
                        wave_topk_from<4>(raw[j], E, k, &my_id, &my_w);
                        emit(t, my_id, my_w);
                    }
                }
            }
        } else {
            for (int t = wave; t < T; t += nw) {
                int my_id;
                float my_w;
                wave_topk_any(a.logits + (int64_t)t * E, E, k, &my_id, &my_w);
                emit(t, my_id, my_w);
            }
        }
    } else {
        for (int p = tid; p < P; p += blockDim.x) {
            s.ids[p] = checked_id(a.ids + (p / k) * k, p % k, E);
            s.w[p] = a.wts[p];
        }
    }
    route_small_finish(a, s, writer);
}

// The rest of the routing once s.ids and s.w hold every pair (the workgroup's own writes
// to them need no barrier before the call): counts, offsets, tiles, and with `writer` every
// output of RouteArgs but ids and wts.
__device__ void route_small_finish(const RouteArgs& a, SmallRouteLds& s, bool writer) {
    const int tid = threadIdx.x;
    const int T = a.T, E = a.E, k = a.k, P = T * k;
    for (int e = tid; e < E; e += blockDim.x) { s.cnt[e] = 0; s.mlo[e] = 0; s.mhi[e] = 0; }
    __syncthreads();

    for (int p = tid; p < P; p += blockDim.x) {
        const int e = s.ids[p];
        if (e >= 0) {
            const int t = p / k;
            atomicAdd(&s.cnt[e], 1);
            if (t < 32) atomicOr(&s.mlo[e], 1u << t);
            else atomicOr(&s.mhi[e], 1u << (t - 32));
        }
    }
    __syncthreads();

    // offsets (exclusive scan of counts), the ascending list of active experts and the first
    // M-tile of each, from one scan of count << 42 | M-tiles << 21 | (count > 0) (every sum
    // stays below 2^21 for T * k <= 1024).  Thread i owns experts 2i and 2i + 1 when the
    // workgroup has fewer threads than experts, else expert i.
    const int ept = E > (int)blockDim.x ? 2 : 1;
    const int e0 = tid * ept;
    uint64_t mine[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = e0 + j;
        if (j < ept && e < E) {
            const int c = s.cnt[e];
            mine[j] = (uint64_t)c << 42 | (uint64_t)((c + 15) >> 4) << 21 | (uint64_t)(c > 0);
        }
    }
    uint64_t packed_total = 0;
    uint64_t packed = block_exclusive_scan<uint64_t>(mine[0] + mine[1], s.tmp, &packed_total);
    constexpr uint64_t kF = (1u << 21) - 1;
    const int total = (int)(packed_total >> 42);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = e0 + j;
        if (j < ept && e < E) {
            const int c = s.cnt[e];
            const int off = (int)(packed >> 42), t0 = (int)((packed >> 21) & kF), act = (int)(packed & kF);
            s.off[e] = off;
            s.tstart[e] = t0;
            if (writer) {
                a.offsets[e] = off;
                a.counts[e] = c;
                if (c > 0) {
                    // the first kRecTokens tokens of the expert, ascending, kRecTokBits bits each
                    uint64_t m = (uint64_t)s.mhi[e] << 32 | s.mlo[e];
                    int toks = 0;
                    for (int i = 0; i < kRecTokens && m; ++i) {
                        toks |= __builtin_ctzll(m) << (kRecTokBits * i);
                        m &= m - 1;
                    }
                    a.active[act] = e;
                    a.rec[act] = int4{e, off, c, toks};
                    // the expert's M-tiles (tiles t0, t0 + 1, ...): every row's token (or
                    // pair), kRecTokBits bits each, in three words per tile
                    m = (uint64_t)s.mhi[e] << 32 | s.mlo[e];
                    for (int j0 = 0; j0 < c; j0 += 16) {
                        const int cnt = min(16, c - j0);
                        uint32_t w[3] = {0u, 0u, 0u};
                        for (int i = 0; i < cnt; ++i) {
                            int v = __builtin_ctzll(m);
                            m &= m - 1;
                            if (a.pair_rows) {   // the token's rank of expert e (ids are distinct within a token)
                                int jj = 0;
                                while (jj < k - 1 && s.ids[v * k + jj] != e) ++jj;
                                v = v * k + jj;
                            }
                            const int b = kRecTokBits * i;
                            w[b >> 5] |= (uint32_t)v << (b & 31);
                            if ((b & 31) + kRecTokBits > 32) w[(b >> 5) + 1] |= (uint32_t)v >> (32 - (b & 31));
                        }
                        const int tile = t0 + j0 / 16;
                        a.trec[2 * tile] = int4{e, off + j0, cnt, 0};
                        a.trec[2 * tile + 1] = int4{(int)w[0], (int)w[1], (int)w[2], 0};
                    }
                }
            }
            packed += mine[j];
        }
    }
    if (tid == 0) {
        s.n_tiles = (int)((packed_total >> 21) & kF);
        s.n_active = (int)(packed_total & kF);
        if (writer) {
            a.offsets[E] = total;
            a.meta[0] = s.n_active;
            a.meta[1] = s.n_tiles;
        }
    }
    __syncthreads();
    if (!writer) return;
    for (int sl = s.n_active + tid; sl < a.max_slots; sl += blockDim.x) a.rec[sl] = int4{0, 0, 0, 0};
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = s.ids[p];
        if (e >= 0) {
            const int t = p / k;
            const uint32_t lo = s.mlo[e], hi = s.mhi[e];
            const int rank = t < 32 ? __popc(lo & ((1u << t) - 1u))
                                    : __popc(lo) + __popc(hi & ((1u << (t - 32)) - 1u));
            a.sorted[s.off[e] + rank] = p;
            a.tokw[s.off[e] + rank] = int2{t, __float_as_int(s.w[p])};
            a.inv[p] = s.off[e] + rank;
        } else {
            a.inv[p] = -1;
        }
    }
}

}  // namespace
}  // namespace w4a16
