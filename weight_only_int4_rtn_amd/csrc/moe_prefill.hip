// Large-batch W4A16 expert FFN as two grouped GEMMs on bf16 MFMA (gfx950).
//
// gk_prefill_kernel: items are (M-tile of up to 128 tokens of one expert, 64 output
//   columns).  The tile's activation rows are gathered from x through the sorted pair
//   list, K-slice-reordered and staged per 128-column group into LDS (double buffered);
//   each wave (2 x 2 waves, 64 x 32 outputs) loads its 16 gate + 16 up code rows per
//   16-column subtile straight from global memory, dequantises them in registers and
//   runs 16x16x32 MFMAs.  The code offset is cancelled by seeding each group's
//   accumulator with -OFF * sum(x) over that group (precomputed per token by the
//   routing kernel), and the group scale is applied to the fp32 partial.  Epilogue:
//   a = SiLU(g) * u as bf16 rows in sorted-pair order.
// dk_prefill_kernel: items are (M-tile, 128 output rows); A is the contiguous block of
//   a-rows, K = I.  The offset seed comes from an MFMA against the constant -OFF.  The
//   router-weighted result is added into an fp32 [T, H] accumulator with float atomics
//   (each output element receives top_k addends, in arrival order).
// finalize_kernel: y = bf16(acc + residual).
//
// Both GEMMs walk their items with a persistent grid whose size is a multiple of 8;
// item L is remapped so that each of the 8 XCDs (workgroup id mod 8) takes one
// contiguous range of items, keeping a tile's activation rows and an expert's codes in
// that XCD's L2.
#include "common.h"

namespace w4a16 {

namespace {

constexpr int MT = kPrefillMT;       // 128 rows per M-tile
constexpr int kRowPad = kGroup + 8;  // bf16 per staged LDS row (16 B pad: conflict-free reads)
constexpr int kGkCols = 64;          // output columns per gate/up item
constexpr int kDkRows = 128;         // output rows per down item

struct TileRows {
    int count;        // valid rows in the tile
    int tok_base;     // routed: first sorted position; shared: first token
    int orow_base;    // first row of the tile in the gate/up output buffer
    bool shared;
};

__device__ __forceinline__ int tile_token(const PrefillArgs& a, const TileRows& tr, int r) {
    return tr.shared ? tr.tok_base + r : a.sorted[tr.tok_base + r] / a.k;
}

// Item L of the persistent walk; false when beyond the real work.
__device__ __forceinline__ bool item_tile(const PrefillArgs& a, int L, int nb, int SB, int I_shared,
                                          TileRows* tr, int* e, int* nblk) {
    const int routed_items = a.meta[1] * nb;
    *nblk = L % nb;
    if (L < routed_items) {
        const int tile = L / nb;
        *e = a.tiles[2 * tile];
        const int m0 = a.tiles[2 * tile + 1];
        const int pos0 = a.offsets[*e];
        tr->count = min(MT, a.offsets[*e + 1] - pos0 - m0);
        tr->tok_base = pos0 + m0;
        tr->orow_base = pos0 + m0;
        tr->shared = false;
        return true;
    }
    if (SB == 0) return false;
    const int st = (L - routed_items) / nb;
    if (st * MT >= a.T) return false;
    *e = -1;
    tr->count = min(MT, a.T - st * MT);
    tr->tok_base = st * MT;
    tr->orow_base = a.T * a.k + st * MT;
    tr->shared = true;
    (void)I_shared;
    return true;
}

// ---------------------------------------------------------------- gate / up

template <int BITS>
__device__ void gk_item(const PrefillArgs& a, const TileRows& tr, int64_t I_e, const int32_t* __restrict__ w13e,
                        const uint16_t* __restrict__ s13e, int n0, uint16_t* s_a, float* s_xs, int* s_tok) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t H = a.H;
    const int G = (int)(H / kGroup);
    constexpr float kOff = BITS == 4 ? 136.0f : 2304.0f;
    constexpr int kLaneBytes = 32 * BITS / 8, kGroupBytes = kGroup * BITS / 8;
    const int64_t row_bytes = H * BITS / 8;

    if (tid < MT) s_tok[tid] = tid < tr.count ? tile_token(a, tr, tid) : -1;
    __syncthreads();

    // staging assignment: 8 chunks of 16 B per thread, rows (tid>>4) + 16 j, column slice tid & 15
    const int col8 = (tid & 15) * 8;
    const uint16_t* xrow[8];
    uint32_t xok = 0;   // bit j: row (tid >> 4) + 16 j is a real token
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = s_tok[(tid >> 4) + 16 * j];
        xok |= (t >= 0 ? 1u : 0u) << j;
        xrow[j] = a.x + (int64_t)(t >= 0 ? t : s_tok[0]) * H + col8;
    }
    const int xs_tok = tid < MT ? s_tok[tid] : -1;
    const float* xs_row = a.xsum + (int64_t)(xs_tok >= 0 ? xs_tok : s_tok[0]) * G;

    // code rows of the four B subtiles: gate/up x two 16-column halves
    const uint8_t* brow[4];
    const uint16_t* srow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t r = (b >= 2 ? I_e : 0) + n0 + 32 * wn + 16 * (b & 1) + ml;
        brow[b] = reinterpret_cast<const uint8_t*>(w13e) + r * row_bytes + q * kLaneBytes;
        srow[b] = s13e + r * G;
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[mi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t stage[8];
    float xs_stage = 0.f;
    auto load_stage = [&](int g) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            stage[j] = load16_or_zero(xrow[j] + (int64_t)g * kGroup, xok >> j & 1u, xrow[j]);
        const float xs = xs_row[g];
        xs_stage = xs_tok >= 0 ? -kOff * xs : 0.f;
    };
    auto store_stage = [&](int buf) {
        uint16_t* dst = s_a + buf * (MT * kRowPad);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<u32x4_t*>(dst + ((tid >> 4) + 16 * j) * kRowPad + col8) = perm_act<BITS>(stage[j]);
        if (tid < MT) s_xs[buf * MT + tid] = xs_stage;
    };

    u32x4_t braw[4][BITS / 4];
    auto load_b = [&](int g) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c)
                braw[b][c] = *reinterpret_cast<const u32x4_t*>(brow[b] + (int64_t)g * kGroupBytes + 16 * c);
    };

    load_stage(0);
    load_b(0);
    store_stage(0);
    __syncthreads();

    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        float sc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) sc[b] = bf16_to_f32(srow[b][g]);
        u32x4_t bcur[4][BITS / 4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c) bcur[b][c] = braw[b][c];
        if (g + 1 < G) {
            load_stage(g + 1);
            load_b(g + 1);
        }
        const uint16_t* A = s_a + buf * (MT * kRowPad);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r0 = 64 * wm + 16 * mi;
            u32x4_t av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *reinterpret_cast<const u32x4_t*>(A + (r0 + ml) * kRowPad + 32 * q + 8 * i);
            const f32x4_t seed = *reinterpret_cast<const f32x4_t*>(s_xs + buf * MT + r0 + 4 * q);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f32x4_t t = seed;
                if constexpr (BITS == 4) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) t = mfma16(av[i], dq4(bcur[b][0][i]), t);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w0 = bcur[b][i >> 1][(2 * i) & 3], w1 = bcur[b][i >> 1][(2 * i + 1) & 3];
                        t = mfma16(av[i], dq8_lo(w0, w1), t);
                        t = mfma16(av[i], dq8_hi(w0, w1), t);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mi][b][r] += sc[b] * t[r];
            }
        }
        if (g + 1 < G) store_stage(buf ^ 1);
        __syncthreads();
    }

    // epilogue: a = SiLU(gate) * up, bf16, rows in sorted-pair order
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 64 * wm + 16 * mi + 4 * q + r;
                if (m < tr.count) {
                    const float v = silu_mul(acc[mi][ns][r], acc[mi][2 + ns][r]);
                    a.abuf[(int64_t)(tr.orow_base + m) * a.width_a + n0 + 32 * wn + 16 * ns + ml] =
                        (uint16_t)f32_to_bf16(v);
                }
            }
}

// -------------------------------------------------------------------- down

template <int BITS>
__device__ void dk_item(const PrefillArgs& a, const TileRows& tr, int64_t I_e, const int32_t* __restrict__ w2e,
                        const uint16_t* __restrict__ s2e, int h0, uint16_t* s_a, int* s_tok, float* s_wt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    const int G2 = (int)(I_e / kGroup);
    constexpr int kLaneBytes = 32 * BITS / 8, kGroupBytes = kGroup * BITS / 8;
    const int64_t row_bytes = I_e * BITS / 8;

    if (tid < MT) {
        int t = -1;
        float w = 0.f;
        if (tid < tr.count) {
            if (tr.shared) {
                t = tr.tok_base + tid;
                w = 1.f;
            } else {
                const int p = a.sorted[tr.tok_base + tid];
                t = p / a.k;
                w = a.wts[p];
            }
        }
        s_tok[tid] = t;
        s_wt[tid] = w;
    }

    const int col8 = (tid & 15) * 8;
    const uint16_t* arow[8];
    uint32_t aok = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = (tid >> 4) + 16 * j;
        aok |= (r < tr.count ? 1u : 0u) << j;
        arow[j] = a.abuf + (int64_t)(tr.orow_base + (r < tr.count ? r : 0)) * a.width_a + col8;
    }
    const uint8_t* brow[4];
    const uint16_t* srow[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        const int64_t r = h0 + 64 * wn + 16 * ns + ml;
        brow[ns] = reinterpret_cast<const uint8_t*>(w2e) + r * row_bytes + q * kLaneBytes;
        srow[ns] = s2e + r * G2;
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[mi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t stage[8];
    auto load_stage = [&](int g) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            stage[j] = load16_or_zero(arow[j] + (int64_t)g * kGroup, aok >> j & 1u, arow[j]);
    };
    auto store_stage = [&](int buf) {
        uint16_t* dst = s_a + buf * (MT * kRowPad);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<u32x4_t*>(dst + ((tid >> 4) + 16 * j) * kRowPad + col8) = perm_act<BITS>(stage[j]);
    };
    u32x4_t braw[4][BITS / 4];
    auto load_b = [&](int g) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c)
                braw[b][c] = *reinterpret_cast<const u32x4_t*>(brow[b] + (int64_t)g * kGroupBytes + 16 * c);
    };

    load_stage(0);
    load_b(0);
    store_stage(0);
    __syncthreads();
    const u32x4_t neg = neg_offset_operand<BITS>();

    for (int g = 0; g < G2; ++g) {
        const int buf = g & 1;
        float sc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) sc[b] = bf16_to_f32(srow[b][g]);
        u32x4_t bcur[4][BITS / 4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c) bcur[b][c] = braw[b][c];
        if (g + 1 < G2) {
            load_stage(g + 1);
            load_b(g + 1);
        }
        const uint16_t* A = s_a + buf * (MT * kRowPad);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r0 = 64 * wm + 16 * mi;
            u32x4_t av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *reinterpret_cast<const u32x4_t*>(A + (r0 + ml) * kRowPad + 32 * q + 8 * i);
            f32x4_t seed = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) seed = mfma16(av[i], neg, seed);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f32x4_t t = seed;
                if constexpr (BITS == 4) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) t = mfma16(av[i], dq4(bcur[b][0][i]), t);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w0 = bcur[b][i >> 1][(2 * i) & 3], w1 = bcur[b][i >> 1][(2 * i + 1) & 3];
                        t = mfma16(av[i], dq8_lo(w0, w1), t);
                        t = mfma16(av[i], dq8_hi(w0, w1), t);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mi][b][r] += sc[b] * t[r];
            }
        }
        if (g + 1 < G2) store_stage(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * wm + 16 * mi + 4 * q + r;
            if (m < tr.count) {
                const int t = s_tok[m];
                const float w = s_wt[m];
                float* yrow = a.y32 + (int64_t)t * a.H + h0 + 64 * wn + ml;
#pragma unroll
                for (int ns = 0; ns < 4; ++ns) unsafeAtomicAdd(yrow + 16 * ns, w * acc[mi][ns][r]);
            }
        }
}

// Persistent walk over `total` items with the per-XCD contiguous remap.
template <typename F>
__device__ __forceinline__ void for_each_item(int total, F&& f) {
    const int C = (total + 7) / 8;
    for (int w = blockIdx.x; w < 8 * C; w += gridDim.x) {
        const int L = (w & 7) * C + (w >> 3);
        if (L < total) f(L);
    }
}

}  // namespace

template <int BITS, int SBITS>
__global__ __launch_bounds__(256, 2) void gk_prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2 * MT * kRowPad];
    __shared__ __attribute__((aligned(16))) float s_xs[2 * MT];
    __shared__ int s_tok[MT];

    // zero the fp32 output accumulator for the down kernel
    {
        const int64_t n4 = (int64_t)a.T * a.H / 4;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
            reinterpret_cast<float4*>(a.y32)[i] = float4{0.f, 0.f, 0.f, 0.f};
    }
    const int64_t Imax = std::max(a.routed.I, SBITS ? a.shared.I : (int64_t)0);
    const int nb = (int)(Imax / kGkCols);
    const int shared_items = SBITS ? ((a.T + MT - 1) / MT) * nb : 0;
    const int total = a.meta[1] * nb + shared_items;
    for_each_item(total, [&](int L) {
        TileRows tr;
        int e, nblk;
        if (!item_tile(a, L, nb, SBITS, 0, &tr, &e, &nblk)) return;
        const int n0 = nblk * kGkCols;
        if (tr.shared) {
            if constexpr (SBITS != 0)
                if (n0 < a.shared.I) gk_item<SBITS>(a, tr, a.shared.I, a.shared.w13, a.shared.s13, n0, s_a, s_xs, s_tok);
        } else if (n0 < a.routed.I) {
            const int64_t I_e = a.routed.I;
            gk_item<BITS>(a, tr, I_e, a.routed.w13 + (int64_t)e * (2 * I_e * a.H * BITS / 32),
                          a.routed.s13 + (int64_t)e * 2 * I_e * (a.H / kGroup), n0, s_a, s_xs, s_tok);
        }
        __syncthreads();
    });
}

template <int BITS, int SBITS>
__global__ __launch_bounds__(256, 2) void dk_prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2 * MT * kRowPad];
    __shared__ int s_tok[MT];
    __shared__ float s_wt[MT];
    const int nb = (int)(a.H / kDkRows);
    const int shared_items = SBITS ? ((a.T + MT - 1) / MT) * nb : 0;
    const int total = a.meta[1] * nb + shared_items;
    for_each_item(total, [&](int L) {
        TileRows tr;
        int e, nblk;
        if (!item_tile(a, L, nb, SBITS, 0, &tr, &e, &nblk)) return;
        const int h0 = nblk * kDkRows;
        if (tr.shared) {
            if constexpr (SBITS != 0) dk_item<SBITS>(a, tr, a.shared.I, a.shared.w2, a.shared.s2, h0, s_a, s_tok, s_wt);
        } else {
            const int64_t I_e = a.routed.I;
            dk_item<BITS>(a, tr, I_e, a.routed.w2 + (int64_t)e * (a.H * I_e * BITS / 32),
                          a.routed.s2 + (int64_t)e * a.H * (I_e / kGroup), h0, s_a, s_tok, s_wt);
        }
        __syncthreads();
    });
}

__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ acc, int64_t n,
                                                       const uint16_t* residual, uint16_t* y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = acc[i];
    if (residual) s += bf16_to_f32(residual[i]);
    y[i] = (uint16_t)f32_to_bf16(s);
}

namespace {

unsigned persistent_grid(int64_t max_items) {
    int64_t g = std::min<int64_t>(max_items, 512);
    g = std::max<int64_t>(g, 8);
    return (unsigned)((g + 7) / 8 * 8);
}

template <int BITS, int SBITS>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    const int64_t Imax = std::max(a.routed.I, SBITS ? a.shared.I : (int64_t)0);
    const int64_t shared_tiles = SBITS ? (a.T + MT - 1) / MT : 0;
    const int64_t gk_items = (a.max_tiles + shared_tiles) * (Imax / kGkCols);
    const int64_t dk_items = (a.max_tiles + shared_tiles) * (a.H / kDkRows);
    gk_prefill_kernel<BITS, SBITS><<<persistent_grid(gk_items), 256, 0, s>>>(a);
    mark(t, "gk_prefill");
    dk_prefill_kernel<BITS, SBITS><<<persistent_grid(dk_items), 256, 0, s>>>(a);
    mark(t, "dk_prefill");
    const int64_t n = (int64_t)a.T * a.H;
    finalize_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.y32, n, a.residual, a.y);
    mark(t, "finalize");
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (a.routed.bits == 4) {
        if (sb == 0) return launch_prefill_t<4, 0>(a, s, t);
        if (sb == 4) return launch_prefill_t<4, 4>(a, s, t);
        return launch_prefill_t<4, 8>(a, s, t);
    }
    if (sb == 0) return launch_prefill_t<8, 0>(a, s, t);
    if (sb == 4) return launch_prefill_t<8, 4>(a, s, t);
    return launch_prefill_t<8, 8>(a, s, t);
}

}  // namespace w4a16
