// Large-batch W4A16 expert FFN as two grouped GEMMs on bf16 MFMA (gfx950).
//
// gk_prefill_kernel: items are (M-tile of up to 128 tokens of one expert, 64 output
//   columns = 64 gate rows + the 64 matching up rows).  Per 128-column group of K:
//     - the tile's activation rows (already K-slice reordered by the routing kernel) are
//       copied global -> LDS by direct LDS loads (no registers), into an XOR-swizzled
//       double buffer, the next group's copy overlapping this group's MFMAs;
//     - each wave (2 x 2 waves, 64 rows x 64 code rows) loads its code rows straight
//       from global memory, expands them in registers and runs 16x16x32 MFMAs seeded
//       with -OFF * sum(x) of the group (group sums from the routing kernel); the
//       group scale is applied to the fp32 partial.
//   Epilogue: a = SiLU(g) * u as bf16, columns written in the reordered K order the
//   down GEMM consumes, rows in sorted-pair order.
// dk_prefill_kernel: items are (M-tile, 128 output rows); A is the tile's contiguous
//   block of a-rows, K = I, staged the same way.  The offset seed is an MFMA against
//   the constant -OFF.  The router-weighted result is added into an fp32 [T, H]
//   accumulator with float atomics (each element receives top_k addends, in arrival
//   order).
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
constexpr int kChunks = kGroup / 8;  // 16-byte chunks per staged row (one group of K)
constexpr int kTileElems = MT * kGroup;
constexpr int kGkCols = 64;          // output columns per gate/up item
constexpr int kDkRows = 128;         // output rows per down item

struct TileRows {
    int count;        // valid rows in the tile
    int tok_base;     // routed: first sorted position; shared: first token
    int orow_base;    // first row of the tile in the gate/up output buffer
    bool shared;
};

// Item L of the persistent walk; false when beyond the real work.
__device__ __forceinline__ bool item_tile(const PrefillArgs& a, int L, int nb, int SB, TileRows* tr, int* e,
                                          int* nblk) {
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
    return true;
}

// Swizzled LDS position (in 16-byte chunks) of logical chunk c of tile row r.
__device__ __forceinline__ int swz(int r, int c) { return r * kChunks + (c ^ (r & 15)); }

// The tile row and logical chunk that lane copies for direct load j of its wave: lane l
// of load j fills LDS chunk L = (8w + j) * 64 + l, i.e. row L / 16 at logical chunk
// (L % 16) ^ (row % 16).
__device__ __forceinline__ void stage_coords(int j, int* row, int* chunk) {
    const int L = ((threadIdx.x >> 6) * 8 + j) * 64 + (threadIdx.x & 63);
    *row = L / kChunks;
    *chunk = (L % kChunks) ^ (*row & 15);
}

// Direct global -> LDS copy of one 128 x 128 group of a tile: 8 buffer loads of 64 lanes
// x 16 B per wave.  voff[j] is the byte offset of this lane's source (row and chunk) for
// the first group; col_bytes (scalar) selects the group.  The host keeps every staged
// array below 2^32 bytes.
__device__ __forceinline__ void stage_group(__amdgpu_buffer_rsrc_t src, const uint32_t (&voff)[8], uint32_t col_bytes,
                                            uint16_t* lds_tile) {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, lds_tile + (wave * 8 + j) * 64 * 8, 16, voff[j], col_bytes, 0, 0);
}

// Expands one lane's codes for MFMA k-step i into bf16 operand(s).
template <int BITS>
__device__ __forceinline__ void expand(const u32x4_t (&braw)[BITS / 4], int i, u32x4_t& b0, u32x4_t& b1,
                                       uint32_t M) {
    if constexpr (BITS == 4) {
        b0 = dq4(braw[0][i], M);
    } else {
        dq8(braw[i >> 1][(2 * i) & 3], braw[i >> 1][(2 * i + 1) & 3], b0, b1, M);
    }
}

// One wave's 64 x 64 block for one group: 4 M-subtiles x 4 code subtiles of 16x16.
// The group's A fragments (4 M-subtiles x 4 k-steps) are read from LDS once and held;
// code subtiles are expanded one at a time, so the VALU expansion of subtile b + 1 can
// run under the MFMAs of subtile b.  seed(mi, av) gives the offset seed of M-subtile mi.
// With CACHED_SEED the seeds are computed once per group and held; otherwise seed() is
// called again for every code subtile (cheap when it is an LDS broadcast read).
template <int BITS, bool CACHED_SEED, typename Seed>
__device__ __forceinline__ void mfma_group(const uint16_t* A, int wm, const u32x4_t (&braw)[4][BITS / 4],
                                           const uint32_t (&scp)[2], f32x4_t (&acc)[4][4], Seed&& seed) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, ml = lane & 15;
    const uint32_t M = nibble_mask();
    u32x4_t av[4][4];
    f32x4_t s0[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = 64 * wm + 16 * mi + ml;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[mi][i] = *reinterpret_cast<const u32x4_t*>(A + swz(r, 4 * q + i) * 8);
        if constexpr (CACHED_SEED) s0[mi] = seed(mi, av[mi]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4_t t[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) t[mi] = CACHED_SEED ? s0[mi] : seed(mi, av[mi]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4_t lo, hi;
            expand<BITS>(braw[b], i, lo, hi, M);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                t[mi] = mfma16(av[mi][i], lo, t[mi]);
                if constexpr (BITS == 8) t[mi] = mfma16(av[mi][i], hi, t[mi]);
            }
        }
        const float sc = bf16_to_f32((scp[b >> 1] >> (16 * (b & 1))) & 0xffffu);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) acc[mi][b][r2] += sc * t[mi][r2];
    }
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

    if (tid < MT) {
        const int r = min(tid, tr.count - 1);   // padding rows repeat a real row
        s_tok[tid] = tr.shared ? tr.tok_base + r : a.tokw[tr.tok_base + r].x;
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t xp_r = make_rsrc(a.xp, (uint32_t)(a.T * H * 2));
    uint32_t voff[8];   // byte offset of each staged chunk's source row and chunk
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int r, c;
        stage_coords(j, &r, &c);
        voff[j] = ((uint32_t)s_tok[r] * (uint32_t)H + c * 8) * 2;
    }
    auto xs_at = [&](int g) { return a.xsum[(int64_t)s_tok[tid & (MT - 1)] * G + g]; };

    // this wave's 64 code rows: gate rows n0 + 32 wn + 16 b + ml (b = 0, 1), up rows + I_e;
    // one vector offset per lane, the subtile and group go into the scalar offset
    const __amdgpu_buffer_rsrc_t b_r = make_rsrc(w13e, (uint32_t)(2 * I_e * row_bytes));
    const __amdgpu_buffer_rsrc_t s_r = make_rsrc(s13e, (uint32_t)(2 * I_e * G * 2));
    const uint32_t bvoff = (uint32_t)((n0 + 32 * wn + ml) * row_bytes + q * kLaneBytes);
    const uint32_t svoff = (uint32_t)((n0 + 32 * wn + ml) * G * 2);

    f32x4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[mi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t braw[4][BITS / 4];
    uint32_t scp[2];   // the four code subtiles' group scales, bf16 pairs
    auto load_b = [&](int g) {
        uint32_t s16[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t roff = (uint32_t)((b >= 2 ? I_e : 0) + 16 * (b & 1));
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c)
                braw[b][c] = buf_load16(b_r, bvoff, roff * (uint32_t)row_bytes + g * kGroupBytes + 16 * c);
            s16[b] = buf_load_u16(s_r, svoff, (roff * G + g) * 2);
        }
        scp[0] = s16[0] | (s16[1] << 16);
        scp[1] = s16[2] | (s16[3] << 16);
    };

    stage_group(xp_r, voff, 0, s_a);
    if (tid < MT) s_xs[tid] = -kOff * xs_at(0);
    load_b(0);

    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        __syncthreads();   // group g staged (waits for the direct loads), group g-1 reads done
        if (g + 1 < G) {
            stage_group(xp_r, voff, (g + 1) * kGroup * 2, s_a + (buf ^ 1) * kTileElems);
            if (tid < MT) s_xs[(buf ^ 1) * MT + tid] = -kOff * xs_at(g + 1);
        }
        // this group's codes move to bcur; the next group's load into braw
        u32x4_t bcur[4][BITS / 4];
        const uint32_t scg[2] = {scp[0], scp[1]};
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c) bcur[b][c] = braw[b][c];
        if (g + 1 < G) load_b(g + 1);
        const float* xs = s_xs + buf * MT + 64 * wm + 4 * q;
        mfma_group<BITS, false>(s_a + buf * kTileElems, wm, bcur, scg, acc,
                                [&](int mi, const u32x4_t(&)[4]) { return *reinterpret_cast<const f32x4_t*>(xs + 16 * mi); });
    }

    // epilogue: a = SiLU(gate) * up, bf16, columns in the reordered K order of the down GEMM
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 64 * wm + 16 * mi + 4 * q + r;
                if (m < tr.count) {
                    const float v = silu_mul(acc[mi][ns][r], acc[mi][2 + ns][r]);
                    const int col = perm_pos(n0 + 32 * wn + 16 * ns + ml);
                    a.abuf[(int64_t)(tr.orow_base + m) * a.width_a + col] = (uint16_t)f32_to_bf16(v);
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
        int t = 0;
        float w = 0.f;
        if (tid < tr.count) {
            if (tr.shared) {
                t = tr.tok_base + tid;
                w = 1.f;
            } else {
                const int2 tw = a.tokw[tr.tok_base + tid];
                t = tw.x;
                w = __int_as_float(tw.y);
            }
        }
        s_tok[tid] = t;
        s_wt[tid] = w;
    }

    const __amdgpu_buffer_rsrc_t a_r = make_rsrc(a.abuf, (uint32_t)(a.rows_a * a.width_a * 2));
    uint32_t voff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int r, c;
        stage_coords(j, &r, &c);
        voff[j] = ((uint32_t)(tr.orow_base + min(r, tr.count - 1)) * (uint32_t)a.width_a + c * 8) * 2;
    }
    const __amdgpu_buffer_rsrc_t b_r = make_rsrc(w2e, (uint32_t)(a.H * row_bytes));
    const __amdgpu_buffer_rsrc_t s_r = make_rsrc(s2e, (uint32_t)(a.H * G2 * 2));
    const uint32_t bvoff = (uint32_t)((h0 + 64 * wn + ml) * row_bytes + q * kLaneBytes);
    const uint32_t svoff = (uint32_t)((h0 + 64 * wn + ml) * G2 * 2);

    f32x4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[mi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t braw[4][BITS / 4];
    uint32_t scp[2];
    auto load_b = [&](int g) {
        uint32_t s16[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c)
                braw[b][c] = buf_load16(b_r, bvoff, (uint32_t)(16 * b * row_bytes) + g * kGroupBytes + 16 * c);
            s16[b] = buf_load_u16(s_r, svoff, (16 * b * G2 + g) * 2);
        }
        scp[0] = s16[0] | (s16[1] << 16);
        scp[1] = s16[2] | (s16[3] << 16);
    };

    stage_group(a_r, voff, 0, s_a);
    load_b(0);
    const u32x4_t neg = neg_offset_operand<BITS>();

    for (int g = 0; g < G2; ++g) {
        const int buf = g & 1;
        __syncthreads();
        if (g + 1 < G2) stage_group(a_r, voff, (g + 1) * kGroup * 2, s_a + (buf ^ 1) * kTileElems);
        u32x4_t bcur[4][BITS / 4];
        const uint32_t scg[2] = {scp[0], scp[1]};
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c) bcur[b][c] = braw[b][c];
        if (g + 1 < G2) load_b(g + 1);
        mfma_group<BITS, true>(s_a + buf * kTileElems, wm, bcur, scg, acc, [&](int, const u32x4_t(&av)[4]) {
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) s0 = mfma16(av[i], neg, s0);
            return s0;
        });
    }

    // router-weighted rows, stored once each at the row's sorted position (the sum over a
    // token's experts happens in finalize_kernel, in slot order)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * wm + 16 * mi + 4 * q + r;
            if (m < tr.count) {
                const float w = s_wt[m];
                float* yrow = a.ystage + (int64_t)(tr.orow_base + m) * a.H + h0 + 64 * wn + ml;
#pragma unroll
                for (int b = 0; b < 4; ++b) yrow[16 * b] = w * acc[mi][b][r];
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
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2 * kTileElems];   // two staged groups
    __shared__ __attribute__((aligned(16))) float s_xs[2 * MT];
    __shared__ int s_tok[MT];

    const int64_t Imax = std::max(a.routed.I, SBITS ? a.shared.I : (int64_t)0);
    const int nb = (int)(Imax / kGkCols);
    const int shared_items = SBITS ? ((a.T + MT - 1) / MT) * nb : 0;
    const int total = a.meta[1] * nb + shared_items;
    for_each_item(total, [&](int L) {
        TileRows tr;
        int e, nblk;
        if (!item_tile(a, L, nb, SBITS, &tr, &e, &nblk)) return;
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
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2 * kTileElems];
    __shared__ int s_tok[MT];
    __shared__ float s_wt[MT];
    const int nb = (int)(a.H / kDkRows);
    const int shared_items = SBITS ? ((a.T + MT - 1) / MT) * nb : 0;
    const int total = a.meta[1] * nb + shared_items;
    for_each_item(total, [&](int L) {
        TileRows tr;
        int e, nblk;
        if (!item_tile(a, L, nb, SBITS, &tr, &e, &nblk)) return;
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

// y[t] = sum over slots j in order of the staged row of pair (t, j), then the shared
// expert's row, then the residual; rounded once to bf16.  A token's row is split over
// ceil(H / 2048) blocks of 256 threads x 8 columns.  Deterministic: no atomics anywhere.
__global__ __launch_bounds__(256) void finalize_kernel(PrefillArgs a) {
    const int nbx = (int)((a.H / 8 + 255) / 256);
    const int t = (int)(blockIdx.x / nbx);
    const int64_t c = ((int64_t)(blockIdx.x % nbx) * blockDim.x + threadIdx.x) * 8;
    if (c >= a.H) return;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add_row = [&](int64_t row) {
        const float4* p = reinterpret_cast<const float4*>(a.ystage + row * a.H + c);
        const float4 v0 = p[0], v1 = p[1];
        s[0] += v0.x; s[1] += v0.y; s[2] += v0.z; s[3] += v0.w;
        s[4] += v1.x; s[5] += v1.y; s[6] += v1.z; s[7] += v1.w;
    };
    for (int j = 0; j < a.k; ++j) {
        const int pos = a.inv[(int64_t)t * a.k + j];
        if (pos >= 0) add_row(pos);
    }
    if (a.shared.bits) add_row((int64_t)a.T * a.k + t);
    const int64_t o = (int64_t)t * a.H + c;
    if (a.residual) {
        const u32x4_t r = *reinterpret_cast<const u32x4_t*>(a.residual + o);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[2 * e] += bf16_to_f32(r[e] & 0xffffu);
            s[2 * e + 1] += bf16_to_f32(r[e] >> 16);
        }
    }
    u32x4_t out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = f32_to_bf16(s[2 * e]) | (f32_to_bf16(s[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4_t*>(a.y + o) = out;
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
    launch(t, "gk_prefill", gk_prefill_kernel<BITS, SBITS>, dim3(persistent_grid(gk_items)), dim3(256), s, 0u, a);
    launch(t, "dk_prefill", dk_prefill_kernel<BITS, SBITS>, dim3(persistent_grid(dk_items)), dim3(256), s, 0u, a);
    launch(t, "finalize", finalize_kernel, dim3((unsigned)((a.H / 8 + 255) / 256 * a.T)), dim3(256), s, 0u, a);
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
