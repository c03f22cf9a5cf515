// Small-batch (T <= 64) W4A16 expert FFN: gate/up with SiLU(gate)*up, then down with
// the router-weighted sum (page "Nex-N2.5-mini Int4-Int8Mix", Recipe table: gate_proj,
// up_proj, down_proj per routed expert, INT4 group 128).
//
// Decode is a weight stream: every byte of an active expert is read once, 16-byte lane
// loads, dequantised in registers and fed to 16x16x32 bf16 MFMAs whose other operand
// holds the (at most 16) tokens routed to that expert.  The MFMA does the K reduction,
// so no cross-lane sums are needed; zero-padded token rows cost nothing in HBM bytes.
//
// tiny_decode_kernel (T * k <= 16 pairs): routing, gate/up and down in one launch; see
//   the tiny-batch section below.
// gk_decode_kernel: one workgroup per (active expert, 16 gate + 16 matching up rows);
//   its 8 waves split the 128-column groups of K and meet in LDS.  Writes
//   a = SiLU(g) * u as bf16 in sorted-pair order.  Used when the streaming gate/up kernel
//   (decode_stream.hip) does not fit the shape.
// dk_decode_kernel: one 8-wave workgroup per (16 output rows, expert split); each wave walks a
//   strided subset of the active experts in ascending order and accumulates
//   w[t,j] * (W2_e a) per token in LDS.  Waves, then splits, are summed in a fixed
//   order, so the result is bitwise reproducible.  Used when the streaming down kernel
//   does not fit the shape (intermediate size above 512).
#include "common.h"
#include "decode_dev.h"
#include "route_dev.h"

namespace w4a16 {

constexpr int kGkWaves = 8;   // waves per gate/up workgroup (K split 8 ways)
constexpr int kGkPass4 = 2;   // groups per wave per pass (INT4; INT8 codes take twice the registers: 1)
constexpr int kDkWaves = 8;   // waves per down workgroup
constexpr int kDkChunk = 2;   // groups of K per down work unit (group_dot2 assumes 2)

namespace {

// Two groups at once (two independent MFMA chains, interleaved), each started from `t`.
template <int CF>
__device__ __forceinline__ void group_dot2(const u32x4_t (&av)[kDkChunk][4], const u32x4_t (&bw)[kDkChunk][2],
                                           f32x4_t (&t)[kDkChunk], const float (&xs)[kDkChunk]) {
    const uint32_t M = nibble_mask();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j) {
            if constexpr (CF == 4) {
                t[j] = mfma16(av[j][i], dq4(bw[j][0][i], M), t[j]);
            } else if constexpr (CF == 8) {
                u32x4_t lo, hi;
                dq8(bw[j][i >> 1][(2 * i) & 3], bw[j][i >> 1][(2 * i + 1) & 3], lo, hi, M);
                t[j] = mfma16(av[j][i], lo, t[j]);
                t[j] = mfma16(av[j][i], hi, t[j]);
            } else if constexpr (CF == kCfFp8) {
                t[j] = mfma16(av[j][i], dq_fp8(bw[j][i >> 1][(2 * i) & 3], bw[j][i >> 1][(2 * i + 1) & 3]), t[j]);
            } else {
                t[j] = mfma16(av[j][i], dq_mx4(bw[j][0][i], xs[j]), t[j]);
            }
        }
}

// Gate/up of one M-tile (this lane's activation row: token `tok`, zero when !xok) against rows n0..n0+15 of the
// gate half and the same rows of the up half of one expert's [2I, H] bank.  The 8 waves
// split K: wave w takes groups w, w+8, ...; two groups per pass, every load of a pass
// issued before its MFMAs.  (Two groups keep the activation operand, which is K/8
// registers per lane however few tokens there are, at 32 registers.)
// The a row is stored with every 8 columns in MFMA operand order (column j at
// perm_pos(j)), so the down projection reads its A fragments as they lie.  TAGGED: one
// 32-bit word per value, bf16 in the low half and `tag` in the high half, written through
// to memory (sc1) for a reader on another XCD in the same launch; else plain bf16.
template <int CF, bool TAGGED = false>
__device__ void gk_tile(const uint16_t* __restrict__ x, int64_t H, int64_t I_e, const int32_t* __restrict__ w13e,
                        const uint8_t* __restrict__ s13e, int n0, int tok, bool xok, int row_base, int rows,
                        void* __restrict__ abuf, int64_t width_a, float* s_red, uint32_t abuf_bytes = 0,
                        uint32_t tag = 0) {
    constexpr int BITS = cf_bits(CF);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int G = (int)(H / kGroup);
    constexpr int kLaneBytes = 32 * BITS / 8;   // 32 codes per lane per group
    constexpr int kGroupBytes = kGroup * BITS / 8;
    const int64_t row_bytes = H * BITS / 8;
    const uint8_t* wg = reinterpret_cast<const uint8_t*>(w13e) + (int64_t)(n0 + ml) * row_bytes + q * kLaneBytes;
    const uint8_t* wu = reinterpret_cast<const uint8_t*>(w13e) + (int64_t)(I_e + n0 + ml) * row_bytes + q * kLaneBytes;
    const uint16_t* xr = x + (int64_t)tok * H + 32 * q;   // tok is a real token even when !xok

    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    constexpr int kGkPass = BITS == 4 ? kGkPass4 : 1;
    for (int gb = wave; gb < G; gb += kGkWaves * kGkPass) {
        u32x4_t bg[kGkPass][BITS / 4], bu[kGkPass][BITS / 4], av[kGkPass][4];
        float scg[kGkPass], scu[kGkPass], xsg[kGkPass], xsu[kGkPass];
#pragma unroll
        for (int j = 0; j < kGkPass; ++j) {
            const int g = gb + kGkWaves * j;
            if (g < G) {
#pragma unroll
                for (int c = 0; c < BITS / 4; ++c) {
                    bg[j][c] = load_stream16(wg + (int64_t)g * kGroupBytes + 16 * c);
                    bu[j][c] = load_stream16(wu + (int64_t)g * kGroupBytes + 16 * c);
                }
                load_scales<CF>(s13e, scale_at<CF>(n0 + ml, G, g), q, &scg[j], &xsg[j]);
                load_scales<CF>(s13e, scale_at<CF>(I_e + n0 + ml, G, g), q, &scu[j], &xsu[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i) av[j][i] = load_act<CF>(xr, xok, (int64_t)g * kGroup + 8 * i);
            }
        }
#pragma unroll
        for (int j = 0; j < kGkPass; ++j) {
            if (gb + kGkWaves * j < G) {
                const f32x4_t seed = offset_seed<CF>(av[j]);
                const f32x4_t tg = group_dot<CF>(av[j], bg[j], seed, xsg[j]);
                const f32x4_t tu = group_dot<CF>(av[j], bu[j], seed, xsu[j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    accg[r] += scg[j] * tg[r];
                    accu[r] += scu[j] * tu[r];
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        s_red[(wave * 8 + r) * 64 + lane] = accg[r];
        s_red[(wave * 8 + 4 + r) * 64 + lane] = accu[r];
    }
    __syncthreads();
    if (wave < 4) {   // wave r finishes element r of every lane: D row 4q + r, column ml
        const int r = wave;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < kGkWaves; ++w) {
            gs += s_red[(w * 8 + r) * 64 + lane];
            us += s_red[(w * 8 + 4 + r) * 64 + lane];
        }
        const int m = 4 * q + r;
        const int64_t idx = (int64_t)(row_base + m) * width_a + perm_pos(n0 + ml);
        const uint32_t v = cvt_bf16(silu_mul(gs, us));
        if constexpr (TAGGED) {
            if (m < rows)
                __builtin_amdgcn_raw_buffer_store_b32(v | tag, make_rsrc(abuf, abuf_bytes), (uint32_t)(idx * 4), 0,
                                                      kSc1);
        } else {
            if (m < rows) static_cast<uint16_t*>(abuf)[idx] = (uint16_t)v;
        }
    }
    if constexpr (!TAGGED) __syncthreads();   // s_red is reused by the caller's next tile (tagged: one tile)
}

}  // namespace

template <int CF, int SBITS>
__global__ __launch_bounds__(64 * kGkWaves) void gk_decode_kernel(DecodeArgs a) {
    __shared__ float s_red[kGkWaves * 8 * 64];
    const int slot = blockIdx.y;
    const bool shared = SBITS != 0 && slot == (int)gridDim.y - 1;
    const int n0 = blockIdx.x * 16;
    const int ml = threadIdx.x & 15;
    int count, pos0, e = 0, toks = 0;
    int64_t I_e;
    if (shared) {
        I_e = a.shared.I;
        count = a.T;
        pos0 = a.T * a.k;
    } else {
        const int4 r = a.rec[slot];
        e = r.x;
        pos0 = r.y;
        count = r.z;
        toks = r.w;
        I_e = a.routed.I;
    }
    if (count == 0 || n0 >= I_e) return;
    for (int mt = 0; mt < count; mt += 16) {
        const int m = mt + ml;
        const bool ok = m < count;
        const int rows = min(16, count - mt);
        if (shared) {
            if constexpr (SBITS != 0)
                gk_tile<SBITS>(a.x, a.H, I_e, a.shared.w13, reinterpret_cast<const uint8_t*>(a.shared.s13), n0,
                               ok ? m : mt, ok, pos0 + mt, rows, a.abuf, a.width_a, s_red);
        } else {
            const int mm = ok ? m : mt;
            const int tok = mm < kRecTokens ? (toks >> (kRecTokBits * mm)) & ((1 << kRecTokBits) - 1)
                                            : a.tokw[pos0 + mm].x;
            const int64_t w13_words = 2 * I_e * a.H * cf_bits(CF) / 32;
            const uint8_t* s13e = reinterpret_cast<const uint8_t*>(a.routed.s13) +
                                  (int64_t)e * expert_scale_bytes<CF>(2 * I_e, (int)(a.H / kGroup));
            gk_tile<CF>(a.x, a.H, I_e, a.routed.w13 + (int64_t)e * w13_words, s13e, n0, tok, ok, pos0 + mt, rows,
                        a.abuf, a.width_a, s_red);
        }
    }
}

namespace {

// A down-projection work unit: one expert (or the shared expert) and a chunk of
// kDkChunk groups of its K = I columns, for the workgroup's 16 output rows.
struct DkUnit {
    const uint8_t* wrow;    // this lane's code bytes in row h0 + ml at the chunk's first group
    const uint8_t* sbase;   // scales of the unit's expert
    int64_t srow;           // row h0 + ml of those scales
    int G2;                 // groups along the expert's K = I
    int pos0, count, ngroups, col0, g0;
    bool shared;
    float sc[kDkChunk];     // the chunk's partial-sum scales, loaded with the codes (0: no group)
    float xs[kDkChunk];     // the chunk's conversion scales (MXFP4 blocks; else 1)
};

// Issues the unit's code and scale loads (nothing waits for them here).
template <int CF>
__device__ __forceinline__ void dk_load_codes(DkUnit& u, u32x4_t (&bw)[kDkChunk][2]) {
    constexpr int BITS = cf_bits(CF);
    constexpr int kGroupBytes = kGroup * BITS / 8;
    const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int j = 0; j < kDkChunk; ++j)
        if (j < u.ngroups) {
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c)
                bw[j][c] = load_stream16(u.wrow + (int64_t)j * kGroupBytes + 16 * c);
            load_scales<CF>(u.sbase, scale_at<CF>(u.srow, u.G2, u.g0 + j), q, &u.sc[j], &u.xs[j]);
        } else {
#pragma unroll
            for (int c = 0; c < 2; ++c) bw[j][c] = u32x4_t{0u, 0u, 0u, 0u};
            u.sc[j] = 0.f;
            u.xs[j] = 1.f;
        }
}

// Down projection of one unit for every M-tile of its tokens, accumulated with the
// router weights into this wave's LDS accumulator yacc[T][16].
// Without group sums (XSUM false) every group's accumulator starts from the MFMA offset
// seed -OFF * sum(a); with them (xsum(pos, g) = sum of a row's group g, fp32) the MFMA
// chains start at zero and the offset term is removed with one FMA per element, which
// halves the MFMAs of a unit.
template <int CF, bool XSUM, typename TokW, typename AFetch, typename XSum>
__device__ void dk_unit(const DkUnit& u, const u32x4_t (&bw)[kDkChunk][2], TokW tokw, AFetch afetch, XSum xsum,
                        float* yacc, const float* sgate) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, ml = lane & 15;
    const int g0 = u.col0 / kGroup;
    for (int mt = 0; mt < u.count; mt += 16) {
        int tk[4], pr[4];
        float wk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {   // token, router weight and a row of D rows 4q + r
            const int m = min(mt + 4 * q + r, u.count - 1);
            pr[r] = u.pos0 + m;
            if (u.shared) {
                tk[r] = m;
                wk[r] = sgate ? sgate[m] : 1.0f;
            } else {
                const int2 tw = tokw(u.pos0 + m);
                tk[r] = tw.x;
                wk[r] = __int_as_float(tw.y);
            }
        }
        const int mload = mt + ml;
        const bool aok = mload < u.count;
        const int pos = u.pos0 + (aok ? mload : mt);   // a valid row even for padding lanes
        const int col = u.col0 + 32 * q;
        // every load unconditional (a missing second group re-reads the first, masked to
        // zero), so they all issue before the first wait
        u32x4_t av[kDkChunk][4];
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j) {
            const bool okj = aok && j < u.ngroups;
            const int cj = col + (j < u.ngroups ? j : 0) * kGroup;
#pragma unroll
            for (int i = 0; i < 4; ++i) av[j][i] = afetch(okj, pos, cj + 8 * i);
        }
        f32x4_t t[kDkChunk];
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j) t[j] = XSUM ? f32x4_t{0.f, 0.f, 0.f, 0.f} : offset_seed<CF>(av[j]);
        group_dot2<CF>(av, bw, t, u.xs);   // a missing second group has zero a and scale 0
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = t[j][r];
                if constexpr (XSUM && cf_int(CF)) v -= code_offset<CF>() * xsum(pr[r], g0 + (j < u.ngroups ? j : 0));
                acc[r] += u.sc[j] * v;   // sc is 0 for a missing group
            }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (mt + 4 * q + r < u.count) yacc[tk[r] * 16 + ml] += wk[r] * acc[r];
    }
}

// Unit `u` of the down kernel (routed units first, then the shared expert's); `rec`
// gives the (expert, first sorted row, count) of an active-expert slot.
template <typename Rec>
__device__ __forceinline__ DkUnit dk_make_unit(const ExpertSet& routed, const ExpertSet& shared, int64_t H, int T,
                                               int k, Rec rec, int u, int n_routed_units, int nch, int nch_s, int h0,
                                               int* bits) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, ml = lane & 15;
    DkUnit r;
    const ExpertSet* es;
    int64_t ebase = 0;
    int chunk;
    if (u < n_routed_units) {
        const int4 rr = rec(u / nch);
        chunk = u % nch;
        es = &routed;
        ebase = rr.x;
        r.pos0 = rr.y;
        r.count = rr.z;
        r.shared = false;
    } else {
        chunk = (u - n_routed_units) % nch_s;
        es = &shared;
        r.pos0 = T * k;
        r.count = T;
        r.shared = true;
    }
    *bits = es->bits;
    const int64_t I_e = es->I;
    const int G2 = (int)(I_e / kGroup);
    const int g0 = chunk * kDkChunk;
    r.ngroups = min(kDkChunk, G2 - g0);
    r.col0 = g0 * kGroup;
    r.g0 = g0;
    r.G2 = G2;
    const int64_t row_bytes = I_e * es->bits / 8;
    const uint8_t* w2e = reinterpret_cast<const uint8_t*>(es->w2) + ebase * H * row_bytes;
    r.wrow = w2e + (int64_t)(h0 + ml) * row_bytes + (int64_t)g0 * (kGroup * es->bits / 8) + q * (32 * es->bits / 8);
    // scales: INT bf16 [H, G2]; FP8 fp32 [H]; MXFP4 E8M0 [H, 4 G2]  (per expert)
    const int64_t es_bytes = es->fmt == 1 ? H * 4 : es->fmt == 2 ? H * G2 * 4 : H * G2 * 2;
    r.sbase = reinterpret_cast<const uint8_t*>(es->s2) + ebase * es_bytes;
    r.srow = h0 + ml;
    return r;
}

}  // namespace

template <int CF, int SBITS>
__global__ __launch_bounds__(64 * kDkWaves) void dk_decode_kernel(DecodeArgs a) {
    __shared__ float s_y[kDkWaves][kSmallT * 16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h0 = blockIdx.x * 16;
    const int T = a.T;
    float* yacc = s_y[wave];
    for (int i = lane; i < T * 16; i += 64) yacc[i] = 0.f;

    const int nch = (int)((a.routed.I / kGroup + kDkChunk - 1) / kDkChunk);
    const int nch_s = SBITS != 0 ? (int)((a.shared.I / kGroup + kDkChunk - 1) / kDkChunk) : 0;
    const int n_routed_units = a.meta[0] * nch;
    const int n_units = n_routed_units + nch_s;
    const int V = gridDim.y * kDkWaves;
    int u = blockIdx.y * kDkWaves + wave;
    const int4* rec = a.rec;
    auto recf = [rec](int slot) { return rec[slot]; };
    // software pipeline: the next unit's codes are in flight while this one computes
    u32x4_t cur[kDkChunk][2], nxt[kDkChunk][2];
    // a unit uses the routed code format unless it is a shared-expert unit of another one
    int bits = 0;
    bool rt = true;
    DkUnit cu;
    if (u < n_units) {
        cu = dk_make_unit(a.routed, a.shared, a.H, a.T, a.k, recf, u, n_routed_units, nch, nch_s, h0, &bits);
        rt = !cu.shared || SBITS == CF;
        if (rt) dk_load_codes<CF>(cu, cur);
        else if constexpr (SBITS != 0 && SBITS != CF) dk_load_codes<SBITS>(cu, cur);
    }
    while (u < n_units) {
        const int un = u + V;
        bool nrt = true;
        DkUnit nu;
        if (un < n_units) {
            nu = dk_make_unit(a.routed, a.shared, a.H, a.T, a.k, recf, un, n_routed_units, nch, nch_s, h0, &bits);
            nrt = !nu.shared || SBITS == CF;
            if (nrt) dk_load_codes<CF>(nu, nxt);
            else if constexpr (SBITS != 0 && SBITS != CF) dk_load_codes<SBITS>(nu, nxt);
        }
        const int2* tokw = a.tokw;
        auto tw = [tokw](int pos) { return tokw[pos]; };
        const uint16_t* abuf = a.abuf;
        const int64_t width_a = a.width_a;
        auto af = [abuf, width_a](bool ok, int pos, int col) {
            const uint16_t* p = abuf + (int64_t)pos * width_a + col;
            return load16_or_zero(p, ok, p);
        };
        auto nox = [](int, int) { return 0.f; };
        if (rt) dk_unit<CF, false>(cu, cur, tw, af, nox, yacc, a.shared_gate);
        else if constexpr (SBITS != 0 && SBITS != CF) dk_unit<SBITS, false>(cu, cur, tw, af, nox, yacc, a.shared_gate);
        if (un >= n_units) break;
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j) {
            cur[j][0] = nxt[j][0];
            cur[j][1] = nxt[j][1];
        }
        cu = nu;
        rt = nrt;
        u = un;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * 16; i += blockDim.x) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kDkWaves; ++w) s += s_y[w][i];
        const int t = i >> 4, n = i & 15;
        const int64_t o = (int64_t)t * a.H + h0 + n;
        if (gridDim.y == 1) {
            const float r = a.residual ? bf16_to_f32(a.residual[o]) : 0.f;
            a.y[o] = (uint16_t)cvt_bf16(s + r);
        } else {
            a.part[(int64_t)blockIdx.y * T * a.H + o] = s;
        }
    }
}

__global__ __launch_bounds__(256) void dk_combine_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                         const uint16_t* residual, uint16_t* y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part[(int64_t)sp * n + i];
    if (residual) s += bf16_to_f32(residual[i]);
    y[i] = (uint16_t)cvt_bf16(s);
}

// ------------------------------------------------------------------ tiny batches
//
// T * k <= kTinyP pairs (one or two tokens at top-8): one launch.  Every workgroup routes
// the batch itself from the logits (a few KB), so no workgroup waits on a routing kernel.
// Workgroups [0, H / 16) own 16 output rows each: they route the whole batch, issue the
// loads of their first down-projection codes, then read every a word this launch
// produces, past the caches, until each carries the current epoch; the values go to LDS
// and the workgroup finishes the down projection of all active experts for its rows (the
// sum over experts stays in one workgroup and in a fixed order).  The workgroups after
// them each own one 16-row block of the gate/up bank of one (token, rank) pair: they run
// the top-k of that token only up to that rank, so the first ranks start streaming their
// weights while later ones are still being chosen, and the shared expert's row blocks
// start at once.  They write their a values through to memory, row p of the tag area in
// the workspace head for pair p: one 32-bit word per value, the bf16 value in the low half
// and this launch's epoch in the high half.  A value carries its own readiness: no counter
// is raised between the two halves.  The down workgroups come first so that they are
// resident, with their codes in flight, while gate/up runs.
//
// Epochs run 1..65535 (the epoch word holds epoch - 1).  Down workgroups count their
// exits in groups of 16; the last one to leave resets those counters and advances the
// epoch word, and when the epoch wraps to 1 it also clears the tag area, so a word left by
// an earlier launch never carries the current epoch.
//
// Progress: gate/up workgroups never wait, and the host takes this path only when the
// down workgroups fill at most half of the workgroups the GPU holds at once
// (tiny_max_down_workgroups), so gate/up workgroups always find room, in whatever order
// workgroups are dispatched.  A wait is still bounded: on time-out the workgroup raises
// the sticky error word and continues.

namespace {

constexpr int kTinySpinLimit = 1 << 22;
constexpr uint32_t kTinyEpochs = 65535;
constexpr int kTinyPoll = 4;   // 16-byte chunks of a words each thread keeps in flight

struct TinyRoute {
    int ids[kTinyP];          // per pair (token * k + slot): expert, -1 when dropped
    float w[kTinyP];          // per pair: router weight
    int pair_at[kTinyP];      // per sorted position: pair
    int2 tw[kTinyP];          // per sorted position: (token, weight bits)
    float sg[kTinyP];         // per token: weight of its shared-expert row (the gate, or 1)
    int4 slot[kTinyP];        // per active expert, ascending: (expert, first position, count, 0)
    int n_active, n_valid;
};

// Routing of the whole batch into LDS (all threads of the workgroup take part).
// `writer` also stores the routing outputs.
__device__ void tiny_route(const TinyArgs& a, TinyRoute& r, bool writer) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int T = a.T, E = a.E, k = a.k, P = T * k;
    for (int t = wave; t < T; t += nw) {
        int id;
        float w;
        if (a.logits) {
            wave_topk_any(a.logits + (int64_t)t * E, E, k, &id, &w);
            if (writer && lane < k) {
                a.ids[t * k + lane] = id;
                a.wts[t * k + lane] = w;
            }
        } else {
            id = lane < k ? checked_id(a.ids + t * k, lane, E) : -1;
            w = lane < k ? a.wts[t * k + lane] : 0.f;
        }
        if (lane < k) {
            r.ids[t * k + lane] = id;
            r.w[t * k + lane] = w;
        }
    }
    if ((int)threadIdx.x < T) r.sg[threadIdx.x] = a.shared_gate ? a.shared_gate[threadIdx.x] : 1.0f;
    __syncthreads();
    if (wave == 0) {   // stable order by (expert, pair): rank of each key among the P keys
        const int e = lane < P ? r.ids[lane] : -1;
        const int key = e >= 0 ? (e << 6 | lane) : 0x7fffffff;
        int rank = 0;
        for (int q = 0; q < P; ++q) rank += __builtin_amdgcn_readlane(key, q) < key;
        if (e >= 0) r.pair_at[rank] = lane;
        const uint64_t vm = __ballot(e >= 0);
        if (lane == 0) r.n_valid = __popcll(vm);
    }
    __syncthreads();
    if (wave == 0) {   // active experts: the first sorted position of each
        const int nv = r.n_valid;
        const bool in = lane < nv;
        const int p = in ? r.pair_at[lane] : 0;
        const int e = in ? r.ids[p] : -1;
        const int pe = (in && lane > 0) ? r.ids[r.pair_at[lane - 1]] : -1;
        const bool first = in && e != pe;
        const uint64_t fm = __ballot(first);
        const uint64_t upto = (2ull << lane) - 1ull;   // lanes 0..lane (all lanes at 63)
        if (in) r.tw[lane] = int2{p / k, __float_as_int(r.w[p])};
        if (first) {
            const uint64_t above = fm & ~upto;
            const int next = above ? (int)__ffsll((long long)above) - 1 : nv;
            r.slot[__popcll(fm & upto) - 1] = int4{e, lane, next - lane, 0};
        }
        if (lane == 0) r.n_active = __popcll(fm);
        if (writer && in) a.sorted[lane] = p;
    }
    __syncthreads();
    if (writer) {   // counts and offsets of every expert (binary search of the slot list)
        const int na = r.n_active;
        for (int e = threadIdx.x; e <= E; e += blockDim.x) {
            int lo = 0, hi = na;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (r.slot[mid].x < e) lo = mid + 1;
                else hi = mid;
            }
            a.offsets[e] = lo < na ? r.slot[lo].y : r.n_valid;
            if (e < E) a.counts[e] = (lo < na && r.slot[lo].x == e) ? r.slot[lo].z : 0;
        }
    }
}

// Gate/up workgroup b: pair p = b / n_rb (token p / k, rank p % k) and its 16-row block
// b % n_rb, writing row p of the tag area; or, after the pairs, a row block of the shared
// expert for every token (rows T * k + t).  CF: the routed experts' code format.
template <int CF, int SBITS>
__device__ void tiny_gate_up(const TinyArgs& a, float* s_red, uint32_t tag) {
    constexpr int BITS = cf_bits(CF);
    const int b = blockIdx.x - (int)(a.H / 16);   // down workgroups come first in the grid
    const int Tk = a.T * a.k;
    const int p = b / a.n_rb, rb = b % a.n_rb;
    const int n0 = rb * 16;
    const int ml = threadIdx.x & 15;
    if (p < Tk) {
        const int64_t I_e = a.routed.I;
        if (n0 >= I_e) return;
        const int t = p / a.k;
        const int e = pair_expert<true>(a.logits, a.ids, a.E, a.k, t, p % a.k);
        if (e < 0) return;   // dropped pair: the down workgroups skip its row
        const int64_t w13_words = 2 * I_e * a.H * BITS / 32;
        gk_tile<CF, true>(a.x, a.H, I_e, a.routed.w13 + (int64_t)e * w13_words,
                          reinterpret_cast<const uint8_t*>(a.routed.s13) +
                              (int64_t)e * expert_scale_bytes<CF>(2 * I_e, (int)(a.H / kGroup)),
                          n0, t, ml == 0, p, 1, a.tags, a.width_a, s_red, a.tag_bytes, tag);
    } else if constexpr (SBITS != 0) {
        const int64_t I_e = a.shared.I;
        if (p > Tk || n0 >= I_e) return;
        const bool ok = ml < a.T;
        gk_tile<SBITS, true>(a.x, a.H, I_e, a.shared.w13, reinterpret_cast<const uint8_t*>(a.shared.s13), n0,
                             ok ? ml : 0, ok, Tk, a.T, a.tags, a.width_a, s_red, a.tag_bytes, tag);
    }
}

// A unit of the single-launch down projection: kTinyCh<BITS> groups of one slot's a rows
// (a slot holds at most 16 rows here: T <= 16) against the workgroup's 16 output rows.
// Groups beyond the expert's last re-read its last group with scale 0.
template <int BITS>
constexpr int kTinyCh = BITS == 4 ? 4 : 2;

struct TinyUnit {
    const uint8_t* wrow;    // this lane's code bytes: row h0 + ml, the unit's first group, quarter q
    const uint8_t* sexp;    // the expert's scale buffer (bytes; layout of its code format)
    int64_t srow;           // row h0 + ml of it
    int G;                  // groups of K = I
    int pos0, count;        // a rows pos0 .. pos0 + count - 1
    int g0, ngroups;        // first group, groups present
    int shared;
};

template <int CF>
struct TinyCodes {
    u32x4_t w[kTinyCh<cf_bits(CF)>][cf_bits(CF) / 4];
    uint32_t s[kTinyCh<cf_bits(CF)>];   // raw scales: INT bf16, FP8 fp32 bits, MXFP4 the lane's E8M0 byte
};

// Unit `u` of this workgroup: routed slots (kTinyCh-group chunks) first, then the shared
// expert's chunks.  CF: the routed experts' code format (the shared expert's is INT).
// Returns the unit's code width.
template <int CF>
__device__ __forceinline__ int tiny_make_unit(const TinyArgs& a, const TinyRoute& r, int u, int nch, int h0,
                                              TinyUnit& t) {
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const int n_routed = r.n_active * nch;
    const ExpertSet& es = u < n_routed ? a.routed : a.shared;
    int64_t e = 0;
    int chunk;
    if (u < n_routed) {
        const int4 sl = r.slot[u / nch];
        e = sl.x;
        t.pos0 = sl.y;
        t.count = sl.z;
        t.shared = 0;
        chunk = u % nch;
    } else {
        t.pos0 = a.T * a.k;
        t.count = a.T;
        t.shared = 1;
        chunk = u - n_routed;
    }
    const int ch = es.bits == 4 ? kTinyCh<4> : kTinyCh<8>;
    const int G = (int)(es.I / kGroup);
    t.g0 = chunk * ch;
    t.ngroups = min(ch, G - t.g0);
    const int64_t row_bytes = es.I * es.bits / 8;
    t.wrow = reinterpret_cast<const uint8_t*>(es.w2) + e * a.H * row_bytes + (int64_t)(h0 + ml) * row_bytes +
             (int64_t)t.g0 * (kGroup * es.bits / 8) + q * (32 * es.bits / 8);
    t.G = G;
    t.srow = h0 + ml;
    t.sexp = reinterpret_cast<const uint8_t*>(es.s2) +
             e * (t.shared ? expert_scale_bytes<4>(a.H, G) : expert_scale_bytes<CF>(a.H, G));
    return es.bits;
}

// Issues the unit's code and scale loads; nothing waits for them here.
template <int CF>
__device__ __forceinline__ void tiny_load_unit(const TinyUnit& t, TinyCodes<CF>& c) {
    constexpr int BITS = cf_bits(CF);
    constexpr int kGroupBytes = kGroup * BITS / 8;
    const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int j = 0; j < kTinyCh<BITS>; ++j) {
        const int jj = min(j, t.ngroups - 1);
#pragma unroll
        for (int v = 0; v < BITS / 4; ++v) c.w[j][v] = load_stream16(t.wrow + (int64_t)jj * kGroupBytes + 16 * v);
        const uint8_t* sp = t.sexp + scale_at<CF>(t.srow, t.G, t.g0 + jj);
        if constexpr (CF == kCfFp8) c.s[j] = *reinterpret_cast<const uint32_t*>(sp);
        else if constexpr (CF == kCfMx4) c.s[j] = sp[q];
        else c.s[j] = *reinterpret_cast<const uint16_t*>(sp);
    }
}

// y[token][h0 + ml] += router weight * sum over the unit's groups of
// scale * (sum_k a_k (q_k + OFF) - OFF * sum_k a_k), added into this wave's yacc with LDS
// adds (one wave owns its yacc, so the additions keep program order: deterministic).
// A fragments come from the staged rows (stride Ws, padded so that the 16 rows of an
// M-tile fall in different LDS banks); a padding lane reads its own 16 bytes of the zero
// block `zb` instead, so no two lanes of a read share an address.
template <int CF>
__device__ __forceinline__ void tiny_unit(const TinyUnit& t, const TinyCodes<CF>& c, const uint16_t* stage,
                                          const float* xs, int Ws, int G, const uint16_t* zb, const TinyRoute& r,
                                          float* yacc) {
    constexpr int BITS = cf_bits(CF);
    constexpr int CH = kTinyCh<BITS>;
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const bool real = ml < t.count;
    // stage rows: routed a rows sit at their pair index, shared rows at T * k + token
    const int srow = t.shared ? t.pos0 + ml : r.pair_at[t.pos0 + min(ml, t.count - 1)];
    const uint16_t* arow = stage + (int64_t)srow * Ws + 32 * q;
    const uint16_t* zl = zb + 8 * lane;
    // two groups at a time: both groups' A fragments first, then their MFMA chains side by side
    const uint32_t M = nibble_mask();
    f32x4_t d[CH];
#pragma unroll
    for (int j0 = 0; j0 < CH; j0 += 2) {
        u32x4_t av[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int g = t.g0 + min(j0 + jj, t.ngroups - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[jj][i] = *reinterpret_cast<const u32x4_t*>(real ? arow + g * kGroup + 8 * i : zl);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = j0 + jj;
                const f32x4_t c0 = i == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : d[j];
                if constexpr (CF == 4) {
                    d[j] = mfma16(av[jj][i], dq4(c.w[j][0][i], M), c0);
                } else if constexpr (CF == 8) {
                    u32x4_t lo, hi;
                    dq8(c.w[j][i >> 1][(2 * i) & 3], c.w[j][i >> 1][(2 * i + 1) & 3], lo, hi, M);
                    d[j] = mfma16(av[jj][i], hi, mfma16(av[jj][i], lo, c0));
                } else if constexpr (CF == kCfFp8) {
                    d[j] = mfma16(av[jj][i], dq_fp8(c.w[j][i >> 1][(2 * i) & 3], c.w[j][i >> 1][(2 * i + 1) & 3]), c0);
                } else {
                    d[j] = mfma16(av[jj][i], dq_mx4(c.w[j][0][i], e8m0_scale(c.s[j])), c0);
                }
            }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int m = 4 * q + rr;
        const int p = t.pos0 + min(m, t.count - 1);
        const int xr = t.shared ? p : r.pair_at[p];   // stage row of D row m
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int g = t.g0 + min(j, t.ngroups - 1);
            // INT: the group's scale, offset seed from the row's group sum; FP8: the row's
            // scale; MXFP4: 1 (the block scale is inside the conversion)
            float sc = CF == kCfFp8 ? __uint_as_float(c.s[j]) : CF == kCfMx4 ? 1.f : bf16_to_f32(c.s[j]);
            sc = j < t.ngroups ? sc : 0.f;
            if constexpr (cf_int(CF)) acc += sc * (d[j][rr] - code_offset<CF>() * xs[xr * G + g]);
            else acc += sc * d[j][rr];
        }
        if (m < t.count) {
            const int2 tw = t.shared ? int2{m, __float_as_int(r.sg[m])} : r.tw[p];
            atomicAdd(&yacc[tw.x * 16 + ml], __int_as_float(tw.y) * acc);
        }
    }
}

// One wave gathers the a values its unit reads from the tag area ([rows_a, W] words): the
// unit's groups of each of its rows (routed rows at their pair index, shared rows at
// T * k + token), waiting for every 16-byte chunk until all four of its words carry `tag`,
// and stages them in `stage` ([rows_a, Ws] bf16); then the sum of each (row, group) into
// xs.  Units cover disjoint (row, group) ranges, so no other wave touches them.
__device__ bool tiny_collect_unit(const TinyArgs& a, const TinyRoute& r, const TinyUnit& t, uint32_t tag,
                                  uint16_t* stage, int Ws, float* xs, int G, int spin_limit) {
    const int lane = threadIdx.x & 63;
    const int W = (int)a.width_a;
    const int cg = t.ngroups * (kGroup / 4);   // chunks of 4 values per row in the unit's groups
    const int n_c = t.count * cg;
    const __amdgpu_buffer_rsrc_t tr = make_rsrc(a.tags, a.tag_bytes);
    auto row_of = [&](int m) { return t.shared ? t.pos0 + m : r.pair_at[t.pos0 + m]; };
    bool timed_out = false;
    for (int c0 = lane; c0 < n_c; c0 += kTinyPoll * 64) {
        uint32_t off[kTinyPoll];
        int soff[kTinyPoll];
        uint32_t pending = 0;
#pragma unroll
        for (int i = 0; i < kTinyPoll; ++i) {
            const int c = c0 + i * 64;
            const int row = c < n_c ? row_of(c / cg) : 0;
            const int col = t.g0 * kGroup + 4 * (c % cg);
            off[i] = c < n_c ? (uint32_t)(row * W + col) * 4 : 0xfffffff0u;   // beyond the buffer: reads zeros
            soff[i] = row * Ws + col;
            if (c < n_c) pending |= 1u << i;
        }
        for (int spins = 0; pending; ++spins) {
            u32x4_t v[kTinyPoll];
#pragma unroll
            for (int i = 0; i < kTinyPoll; ++i)
                v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(tr, off[i], 0, kSc1));
#pragma unroll
            for (int i = 0; i < kTinyPoll; ++i) {
                const uint32_t diff = (v[i][0] ^ tag) | (v[i][1] ^ tag) | (v[i][2] ^ tag) | (v[i][3] ^ tag);
                if ((pending >> i & 1u) && diff < 0x10000u) {
                    const uint32_t lo = (v[i][0] & 0xffffu) | (v[i][1] << 16);
                    const uint32_t hi = (v[i][2] & 0xffffu) | (v[i][3] << 16);
                    *reinterpret_cast<uint2*>(stage + soff[i]) = make_uint2(lo, hi);
                    pending &= ~(1u << i);
                }
            }
            if (!pending) break;
            if (spins >= spin_limit) {
                timed_out = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (timed_out) __hip_atomic_store(sync_word(a.sync, kSyncError), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // (row, group) sums: 16 lanes per pair, 8 values each (this wave's own LDS writes above
    // are complete before its reads: one wave's LDS accesses stay in order)
    const int n_pairs = t.count * t.ngroups;
    for (int p = lane >> 4; p < n_pairs; p += 4) {
        const int row = row_of(p / t.ngroups);
        const int g = t.g0 + p % t.ngroups;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + (int64_t)row * Ws + g * kGroup + (lane & 15) * 8);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += bf16_to_f32(v[e] & 0xffffu) + bf16_to_f32(v[e] >> 16);
        sum += __shfl_xor(sum, 8, 16);
        sum += __shfl_xor(sum, 4, 16);
        sum += __shfl_xor(sum, 2, 16);
        sum += __shfl_xor(sum, 1, 16);
        if ((lane & 15) == 0) xs[row * G + g] = sum;
    }
    return timed_out;
}

template <int CF, int SBITS>
__device__ void tiny_down(const TinyArgs& a, const TinyRoute& r, float* s_dyn, uint32_t epoch_word) {
    __shared__ int s_last;
    __shared__ int s_bad;   // a wait of this workgroup timed out, or an earlier call's did
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = blockIdx.x, n_dk = (int)(a.H / 16);
    const int h0 = d * 16;
    const int T = a.T;
    const int W = (int)a.width_a, G = W / kGroup, Ws = W + kTinyPad;
    float* yacc = s_dyn + wave * T * 16;                                       // [waves][T][16]
    uint16_t* stage = reinterpret_cast<uint16_t*>(s_dyn + kDkWaves * T * 16);   // [rows_a][Ws] a rows
    uint16_t* zb = stage + (int64_t)a.rows_a * Ws;                              // 1 KiB of zeros
    float* xs = reinterpret_cast<float*>(zb + 512);                            // [rows_a][G] group sums
    for (int i = lane; i < T * 16; i += 64) yacc[i] = 0.f;
    if (threadIdx.x < 64) *reinterpret_cast<u32x4_t*>(zb + 8 * threadIdx.x) = u32x4_t{0u, 0u, 0u, 0u};
    // a set time-out word (this workspace's earlier call): no waiting, NaN rows out
    if (threadIdx.x == 0)
        s_bad = __hip_atomic_load(sync_word(a.sync, kSyncError), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    // the residual of this thread's output (T * 16 <= blockDim.x), loaded now, off the tail
    float res_pre = 0.f;
    if (a.residual && (int)threadIdx.x < T * 16)
        res_pre = bf16_to_f32(a.residual[(int64_t)(threadIdx.x >> 4) * a.H + h0 + (threadIdx.x & 15)]);
    __syncthreads();   // the zero block is read by every wave

    // units: kTinyCh-group chunks of every active slot, then of the shared expert
    constexpr int BITS = cf_bits(CF);
    // shared-expert units use their own code type when their format differs from the routed one
    constexpr bool kSep = SBITS != 0 && SBITS != CF;
    const int nch = (int)((a.routed.I / kGroup + kTinyCh<BITS> - 1) / kTinyCh<BITS>);
    const int nch_s = SBITS != 0 ? (int)((a.shared.I / kGroup + kTinyCh<SBITS> - 1) / kTinyCh<SBITS>) : 0;
    const int n_units = r.n_active * nch + nch_s;
    const int V = kDkWaves;
    int u = wave;
    TinyUnit cu, nu;
    TinyCodes<CF> cc, nc;
    TinyCodes<SBITS ? SBITS : 4> cs, ns;   // shared-expert codes when their format differs
    // the first two units' codes go out before the wait for the a rows
    if (u < n_units) {
        tiny_make_unit<CF>(a, r, u, nch, h0, cu);
        if (!kSep || !cu.shared) tiny_load_unit<CF>(cu, cc);
        else if constexpr (kSep) tiny_load_unit<SBITS>(cu, cs);
    }
    if (u + V < n_units) {
        tiny_make_unit<CF>(a, r, u + V, nch, h0, nu);
        if (!kSep || !nu.shared) tiny_load_unit<CF>(nu, nc);
        else if constexpr (kSep) tiny_load_unit<SBITS>(nu, ns);
    }

    // each wave waits for the a values of its own units only, unit by unit, so a wave whose
    // experts are done early computes while later ranks are still in flight
    const uint32_t tag = (epoch_word + 1) << 16;
    const int spin_limit = s_bad ? 0 : kTinySpinLimit;   // (s_bad is read after the barrier above)
    bool bad = false;
    while (u < n_units) {
        bad |= tiny_collect_unit(a, r, cu, tag, stage, Ws, xs, G, spin_limit);
        if (!kSep || !cu.shared) tiny_unit<CF>(cu, cc, stage, xs, Ws, G, zb, r, yacc);
        else if constexpr (kSep) tiny_unit<SBITS>(cu, cs, stage, xs, Ws, G, zb, r, yacc);
        u += V;
        if (u >= n_units) break;
        cu = nu;
        cc = nc;
        if constexpr (kSep) cs = ns;
        if (u + V < n_units) {
            tiny_make_unit<CF>(a, r, u + V, nch, h0, nu);
            if (!kSep || !nu.shared) tiny_load_unit<CF>(nu, nc);
            else if constexpr (kSep) tiny_load_unit<SBITS>(nu, ns);
        }
    }
    if (bad) s_bad = 1;   // (benign race: every writer stores 1)
    __syncthreads();
    // every wave is done with the tag area: count this workgroup's exit now, so that the
    // atomic's round trip overlaps the sum below (groups of 16; the last workgroup resets
    // the counters and advances the epoch, clearing the tag area when it wraps)
    const int ng = (n_dk + 15) >> 4;
    if (threadIdx.x == 0) {
        const int g = d >> 4, gsz = min(16, n_dk - (g << 4));
        s_last = __hip_atomic_fetch_add(sync_word(a.sync, kSyncGroup + g), 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)gsz - 1 &&
                 __hip_atomic_fetch_add(sync_word(a.sync, kSyncTop), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)ng - 1;
    }
    const bool poison = s_bad != 0;
    for (int i = threadIdx.x; i < T * 16; i += blockDim.x) {
        float s = res_pre;
#pragma unroll
        for (int w = 0; w < kDkWaves; ++w) s += s_dyn[w * T * 16 + i];
        const int t = i >> 4, n = i & 15;
        a.y[(int64_t)t * a.H + h0 + n] = poison ? (uint16_t)0x7fc0u : (uint16_t)cvt_bf16(s);
    }
    __syncthreads();
    if (s_last) {
        const uint32_t next = (epoch_word + 1) % kTinyEpochs;
        if (next == 0) {   // the whole area: earlier calls may have used more rows than this one
            const __amdgpu_buffer_rsrc_t tr = make_rsrc(a.tags, (uint32_t)kTagBytes);
            for (uint32_t o = threadIdx.x * 16; o < (uint32_t)kTagBytes; o += blockDim.x * 16)
                __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, tr, o, 0, kSc1);
        }
        if (threadIdx.x == 0) {
            for (int i = 0; i < ng; ++i)
                __hip_atomic_store(sync_word(a.sync, kSyncGroup + i), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync_word(a.sync, kSyncTop), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync_word(a.sync, kSyncEpoch), next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int CF, int SBITS>
__device__ __forceinline__ void tiny_decode_body(const TinyArgs& a) {
    __shared__ TinyRoute route;
    // 16-byte aligned: the static route table before it would leave it at a 4-byte boundary
    extern __shared__ __attribute__((aligned(16))) float s_dyn[];   // gate/up: partial sums; down: y, a rows, group sums
    // epoch - 1 of this launch (written by the previous launch's last workgroup)
    const uint32_t epoch_word =
        __hip_atomic_load(sync_word(a.sync, kSyncEpoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int)blockIdx.x >= (int)(a.H / 16)) {
        tiny_gate_up<CF, SBITS>(a, s_dyn, (epoch_word + 1) << 16);
    } else {
        tiny_route(a, route, blockIdx.x == 0);
        tiny_down<CF, SBITS>(a, route, s_dyn, epoch_word);
    }
}

// Two workgroups per CU where the registers allow it without spilling (4-bit codes with
// no 8-bit expert), one otherwise.
template <int CF, int SBITS>
__global__ __launch_bounds__(64 * kDkWaves) __attribute__((amdgpu_waves_per_eu(4))) void tiny_decode_kernel(
    TinyArgs a) {
    tiny_decode_body<CF, SBITS>(a);
}
template <int CF, int SBITS>
__global__ __launch_bounds__(64 * kDkWaves) void tiny_decode_wide_kernel(TinyArgs a) {
    tiny_decode_body<CF, SBITS>(a);
}
template <int CF, int SBITS>
constexpr bool tiny_narrow() { return (CF == 4 && SBITS != 8) || (CF == kCfMx4 && SBITS == 0); }

__global__ __launch_bounds__(256) void head_init_kernel(uint32_t* head) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < (int)(kHeadBytes / 16); i += gridDim.x * blockDim.x)
        reinterpret_cast<u32x4_t*>(head)[i] = u32x4_t{0u, 0u, 0u, 0u};
}

}  // namespace

namespace {

template <int CF, int SBITS>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    const int max_active = (int)std::min<int64_t>((int64_t)a.E, (int64_t)a.T * a.k);
    if (a.gk_stream) {   // stream_fits (or pair_fits) holds
        if (hipError_t st = launch_gk_stream(a, s, t)) return st;
    } else {
        const int64_t Imax = std::max(a.routed.I, SBITS ? a.shared.I : (int64_t)0);
        const dim3 gk_grid((unsigned)(Imax / 16), (unsigned)(max_active + (SBITS ? 1 : 0)));
        launch(t, "gk_decode", gk_decode_kernel<CF, SBITS>, gk_grid, dim3(64 * kGkWaves), s, 0u, a);
    }
    if (dk_stream_fits(a)) return launch_dk_stream(a, s, t);
    const dim3 dk_grid((unsigned)(a.H / 16), (unsigned)a.splits);
    launch(t, "dk_decode", dk_decode_kernel<CF, SBITS>, dk_grid, dim3(64 * kDkWaves), s, 0u, a);
    if (a.splits > 1) {
        const int64_t n = (int64_t)a.T * a.H;
        launch(t, "dk_combine", dk_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u,
               (const float*)a.part, a.splits, n, a.residual, a.y);
    }
    return hipGetLastError();
}

template <int CF>
hipError_t launch_decode_cf(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (sb == 0) return launch_decode_t<CF, 0>(a, s, t);
    if (sb == 4) return launch_decode_t<CF, 4>(a, s, t);
    return launch_decode_t<CF, 8>(a, s, t);
}

}  // namespace

namespace {
template <int CF>
hipError_t launch_down_decode_t(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    const dim3 dk_grid((unsigned)(a.H / 16), (unsigned)a.splits);
    launch(t, "dk_decode", dk_decode_kernel<CF, 0>, dk_grid, dim3(64 * kDkWaves), s, 0u, a);
    if (a.splits > 1) {
        const int64_t n = (int64_t)a.T * a.H;
        launch(t, "dk_combine", dk_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u,
               (const float*)a.part, a.splits, n, a.residual, a.y);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_down_decode(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    switch (cf_of(a.routed.fmt, a.routed.bits)) {
        case 4: return launch_down_decode_t<4>(a, s, t);
        case 8: return launch_down_decode_t<8>(a, s, t);
        case kCfFp8: return launch_down_decode_t<kCfFp8>(a, s, t);
        default: return launch_down_decode_t<kCfMx4>(a, s, t);
    }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    switch (cf_of(a.routed.fmt, a.routed.bits)) {
        case 4: return launch_decode_cf<4>(a, s, t);
        case 8: return launch_decode_cf<8>(a, s, t);
        case kCfFp8: return launch_decode_cf<kCfFp8>(a, s, t);
        default: return launch_decode_cf<kCfMx4>(a, s, t);
    }
}

}  // namespace w4a16

namespace w4a16 {

namespace {
template <int CF, int SBITS>
hipError_t launch_tiny_t(const TinyArgs& a, hipStream_t s, StageTimer* t) {
    const int n_dk = (int)(a.H / 16);
    if constexpr (tiny_narrow<CF, SBITS>())
        launch(t, "tiny_decode", tiny_decode_kernel<CF, SBITS>, dim3((unsigned)(a.n_gk + n_dk)),
               dim3(64 * kDkWaves), s, a.lds_bytes, a);
    else
        launch(t, "tiny_decode", tiny_decode_wide_kernel<CF, SBITS>, dim3((unsigned)(a.n_gk + n_dk)),
               dim3(64 * kDkWaves), s, a.lds_bytes, a);
    return hipGetLastError();
}
}  // namespace

namespace {
// Workgroups of the single-launch kernel that the current device holds at once (CUs times
// the occupancy at the largest dynamic LDS the path allows), cached per device.
template <int CF, int SBITS>
int tiny_capacity_t() {
    static int cache[64];   // 0: not yet known, -1: query failed
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int cus = 0, nb = 0;
        hipError_t st = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (st == hipSuccess) {
            if constexpr (tiny_narrow<CF, SBITS>())
                st = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &nb, reinterpret_cast<const void*>(tiny_decode_kernel<CF, SBITS>), 64 * kDkWaves, kTinyMaxLds);
            else
                st = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &nb, reinterpret_cast<const void*>(tiny_decode_wide_kernel<CF, SBITS>), 64 * kDkWaves,
                    kTinyMaxLds);
        }
        cache[dev] = (st == hipSuccess && cus > 0 && nb > 0) ? cus * nb : -1;
    }
    return cache[dev] > 0 ? cache[dev] : 0;
}

template <int CF>
int tiny_capacity_cf(int sbits) {
    return sbits == 0 ? tiny_capacity_t<CF, 0>() : sbits == 4 ? tiny_capacity_t<CF, 4>() : tiny_capacity_t<CF, 8>();
}

template <int CF>
hipError_t launch_tiny_cf(const TinyArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (sb == 0) return launch_tiny_t<CF, 0>(a, s, t);
    if (sb == 4) return launch_tiny_t<CF, 4>(a, s, t);
    return launch_tiny_t<CF, 8>(a, s, t);
}
}  // namespace

int tiny_max_down_workgroups(int fmt, int bits, int sbits) {
    int cap;
    switch (cf_of(fmt, bits)) {
        case 4: cap = tiny_capacity_cf<4>(sbits); break;
        case 8: cap = tiny_capacity_cf<8>(sbits); break;
        case kCfFp8: cap = tiny_capacity_cf<kCfFp8>(sbits); break;
        default: cap = tiny_capacity_cf<kCfMx4>(sbits); break;
    }
    return cap / 2;
}

hipError_t launch_tiny(const TinyArgs& a, hipStream_t s, StageTimer* t) {
    switch (cf_of(a.routed.fmt, a.routed.bits)) {
        case 4: return launch_tiny_cf<4>(a, s, t);
        case 8: return launch_tiny_cf<8>(a, s, t);
        case kCfFp8: return launch_tiny_cf<kCfFp8>(a, s, t);
        default: return launch_tiny_cf<kCfMx4>(a, s, t);
    }
}

hipError_t launch_head_init(uint32_t* head, hipStream_t s) {
    hipLaunchKernelGGL(head_init_kernel, dim3(16), dim3(256), 0, s, head);
    return hipGetLastError();
}

}  // namespace w4a16
