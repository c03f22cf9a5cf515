// Small-batch (T <= 64) W4A16 expert FFN: gate/up with SiLU(gate)*up, then down with
// the router-weighted sum (page "Nex-N2.5-mini Int4-Int8Mix", Recipe table: gate_proj,
// up_proj, down_proj per routed expert, INT4 group 128).
//
// Decode is a weight stream: every byte of an active expert is read once, 16-byte lane
// loads, dequantised in registers and fed to 16x16x32 bf16 MFMAs whose other operand
// holds the (at most 16) tokens routed to that expert.  The MFMA does the K reduction,
// so no cross-lane sums are needed; zero-padded token rows cost nothing in HBM bytes.
//
// gk_decode_kernel: one workgroup per (active expert, 16 gate + 16 matching up rows);
//   its 4 waves split the 128-column groups of K and meet in LDS.  Writes
//   a = SiLU(g) * u as bf16 in sorted-pair order.
// dk_decode_kernel: one 8-wave workgroup per (16 output rows, expert split); each wave walks a
//   strided subset of the active experts in ascending order and accumulates
//   w[t,j] * (W2_e a) per token in LDS.  Waves, then splits, are summed in a fixed
//   order, so the result is bitwise reproducible.
#include "common.h"

namespace w4a16 {

constexpr int kGkWaves = 8;   // waves per gate/up workgroup (K split 8 ways)
constexpr int kGkPass = 2;    // groups per wave per pass
constexpr int kDkWaves = 8;   // waves per down workgroup
constexpr int kDkChunk = 2;   // groups of K per down work unit

namespace {

// 16 bytes of one activation row (8 bf16) at column c, reordered for a BITS-wide code;
// zero when the row is padding (`ok` false; `row` then points at any valid row).
template <int BITS>
__device__ __forceinline__ u32x4_t load_act(const uint16_t* row, bool ok, int64_t c) {
    return perm_act(load16_or_zero(row + c, ok, row));
}

// One 128-column group: seed with -OFF * sum(x), then add sum_k x_k * (q_k + OFF) for the
// lane's four 8-column slices.  bw holds the lane's 32 codes (16 B for INT4, 32 B INT8).
template <int BITS>
__device__ __forceinline__ f32x4_t group_dot(const u32x4_t (&av)[4], const u32x4_t (&bw)[BITS / 4],
                                             f32x4_t seed) {
    f32x4_t t = seed;
    const uint32_t M = nibble_mask();
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma16(av[i], dq4(bw[0][i], M), t);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4_t lo, hi;
            dq8(bw[i >> 1][(2 * i) & 3], bw[i >> 1][(2 * i + 1) & 3], lo, hi, M);
            t = mfma16(av[i], lo, t);
            t = mfma16(av[i], hi, t);
        }
    }
    return t;
}

template <int BITS>
__device__ __forceinline__ f32x4_t offset_seed(const u32x4_t (&av)[4]) {
    const u32x4_t neg = neg_offset_operand<BITS>();
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) c = mfma16(av[i], neg, c);
    return c;
}

// Gate/up of one M-tile (this lane's activation row: token `tok`, zero when !xok) against rows n0..n0+15 of the
// gate half and the same rows of the up half of one expert's [2I, H] bank.  The 8 waves
// split K: wave w takes groups w, w+8, ...; two groups per pass, every load of a pass
// issued before its MFMAs.  (Two groups keep the activation operand, which is K/8
// registers per lane however few tokens there are, at 32 registers.)
template <int BITS>
__device__ void gk_tile(const uint16_t* __restrict__ x, int64_t H, int64_t I_e, const int32_t* __restrict__ w13e,
                        const uint16_t* __restrict__ s13e, int n0, int tok, bool xok, int row_base, int rows,
                        uint16_t* __restrict__ abuf, int64_t width_a, float* s_red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int G = (int)(H / kGroup);
    constexpr int kLaneBytes = 32 * BITS / 8;   // 32 codes per lane per group
    constexpr int kGroupBytes = kGroup * BITS / 8;
    const int64_t row_bytes = H * BITS / 8;
    const uint8_t* wg = reinterpret_cast<const uint8_t*>(w13e) + (int64_t)(n0 + ml) * row_bytes + q * kLaneBytes;
    const uint8_t* wu = reinterpret_cast<const uint8_t*>(w13e) + (int64_t)(I_e + n0 + ml) * row_bytes + q * kLaneBytes;
    const uint16_t* sg = s13e + (int64_t)(n0 + ml) * G;
    const uint16_t* su = s13e + (int64_t)(I_e + n0 + ml) * G;
    const uint16_t* xr = x + (int64_t)tok * H + 32 * q;   // tok is a real token even when !xok

    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    for (int gb = wave; gb < G; gb += kGkWaves * kGkPass) {
        u32x4_t bg[kGkPass][BITS / 4], bu[kGkPass][BITS / 4], av[kGkPass][4];
        float scg[kGkPass], scu[kGkPass];
#pragma unroll
        for (int j = 0; j < kGkPass; ++j) {
            const int g = gb + kGkWaves * j;
            if (g < G) {
#pragma unroll
                for (int c = 0; c < BITS / 4; ++c) {
                    bg[j][c] = *reinterpret_cast<const u32x4_t*>(wg + (int64_t)g * kGroupBytes + 16 * c);
                    bu[j][c] = *reinterpret_cast<const u32x4_t*>(wu + (int64_t)g * kGroupBytes + 16 * c);
                }
                scg[j] = bf16_to_f32(sg[g]);
                scu[j] = bf16_to_f32(su[g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) av[j][i] = load_act<BITS>(xr, xok, (int64_t)g * kGroup + 8 * i);
            }
        }
#pragma unroll
        for (int j = 0; j < kGkPass; ++j) {
            if (gb + kGkWaves * j < G) {
                const f32x4_t seed = offset_seed<BITS>(av[j]);
                const f32x4_t tg = group_dot<BITS>(av[j], bg[j], seed);
                const f32x4_t tu = group_dot<BITS>(av[j], bu[j], seed);
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
        if (m < rows) abuf[(int64_t)(row_base + m) * width_a + n0 + ml] = (uint16_t)f32_to_bf16(silu_mul(gs, us));
    }
    __syncthreads();
}

}  // namespace

template <int BITS, int SBITS>
__global__ __launch_bounds__(64 * kGkWaves) void gk_decode_kernel(DecodeArgs a) {
    __shared__ float s_red[kGkWaves * 8 * 64];
    const int slot = blockIdx.y;
    const bool shared = SBITS != 0 && slot == (int)gridDim.y - 1;
    const int n0 = blockIdx.x * 16;
    const int ml = threadIdx.x & 15;
    int count, pos0, e = 0;
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
        I_e = a.routed.I;
    }
    if (count == 0 || n0 >= I_e) return;
    for (int mt = 0; mt < count; mt += 16) {
        const int m = mt + ml;
        const bool ok = m < count;
        const int rows = min(16, count - mt);
        if (shared) {
            if constexpr (SBITS != 0)
                gk_tile<SBITS>(a.x, a.H, I_e, a.shared.w13, a.shared.s13, n0, ok ? m : mt, ok, pos0 + mt, rows,
                               a.abuf, a.width_a, s_red);
        } else {
            const int tok = a.tokw[pos0 + (ok ? m : mt)].x;
            const int64_t w13_words = 2 * I_e * a.H * BITS / 32;
            gk_tile<BITS>(a.x, a.H, I_e, a.routed.w13 + (int64_t)e * w13_words,
                          a.routed.s13 + (int64_t)e * 2 * I_e * (a.H / kGroup), n0, tok, ok, pos0 + mt, rows,
                          a.abuf, a.width_a, s_red);
        }
    }
}

namespace {

// A down-projection work unit: one expert (or the shared expert) and a chunk of
// kDkChunk groups of its K = I columns, for the workgroup's 16 output rows.
struct DkUnit {
    const uint8_t* wrow;    // this lane's code bytes in row h0 + ml at the chunk's first group
    const uint16_t* srow;   // scales of row h0 + ml at the chunk's first group
    int pos0, count, ngroups, col0;
    bool shared;
};

template <int BITS>
__device__ __forceinline__ void dk_load_codes(const DkUnit& u, u32x4_t (&bw)[kDkChunk][2]) {
    constexpr int kGroupBytes = kGroup * BITS / 8;
#pragma unroll
    for (int j = 0; j < kDkChunk; ++j)
        if (j < u.ngroups)
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c)
                bw[j][c] = *reinterpret_cast<const u32x4_t*>(u.wrow + (int64_t)j * kGroupBytes + 16 * c);
}

// Down projection of one unit for every M-tile of its tokens, accumulated with the
// router weights into this wave's LDS accumulator yacc[T][16].
template <int BITS>
__device__ void dk_unit(const DkUnit& u, const u32x4_t (&bw)[kDkChunk][2], const uint16_t* __restrict__ abuf,
                        int64_t width_a, const int2* __restrict__ tokw, float* yacc) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, ml = lane & 15;
    float sc[kDkChunk];
#pragma unroll
    for (int j = 0; j < kDkChunk; ++j) sc[j] = j < u.ngroups ? bf16_to_f32(u.srow[j]) : 0.f;
    for (int mt = 0; mt < u.count; mt += 16) {
        int tk[4];
        float wk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {   // token and router weight of D rows 4q + r
            const int m = min(mt + 4 * q + r, u.count - 1);
            if (u.shared) {
                tk[r] = m;
                wk[r] = 1.0f;
            } else {
                const int2 tw = tokw[u.pos0 + m];
                tk[r] = tw.x;
                wk[r] = __int_as_float(tw.y);
            }
        }
        const int mload = mt + ml;
        const bool aok = mload < u.count;
        const uint16_t* arow = abuf + (int64_t)(u.pos0 + (aok ? mload : mt)) * width_a + u.col0 + 32 * q;
        u32x4_t av[kDkChunk][4];
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j)
            if (j < u.ngroups)
#pragma unroll
                for (int i = 0; i < 4; ++i) av[j][i] = load_act<BITS>(arow, aok, (int64_t)j * kGroup + 8 * i);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j) {
            if (j < u.ngroups) {
                u32x4_t b[BITS / 4];
#pragma unroll
                for (int c = 0; c < BITS / 4; ++c) b[c] = bw[j][c];
                const f32x4_t t = group_dot<BITS>(av[j], b, offset_seed<BITS>(av[j]));
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += sc[j] * t[r];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (mt + 4 * q + r < u.count) yacc[tk[r] * 16 + ml] += wk[r] * acc[r];
    }
}

// Unit `u` of the down kernel (routed units first, then the shared expert's).
__device__ __forceinline__ DkUnit dk_make_unit(const DecodeArgs& a, int u, int n_routed_units, int nch, int nch_s,
                                               int h0, int* bits) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, ml = lane & 15;
    DkUnit r;
    const ExpertSet* es;
    int64_t ebase = 0;
    int chunk;
    if (u < n_routed_units) {
        const int4 rr = a.rec[u / nch];
        chunk = u % nch;
        es = &a.routed;
        ebase = rr.x;
        r.pos0 = rr.y;
        r.count = rr.z;
        r.shared = false;
    } else {
        chunk = (u - n_routed_units) % nch_s;
        es = &a.shared;
        r.pos0 = a.T * a.k;
        r.count = a.T;
        r.shared = true;
    }
    *bits = es->bits;
    const int64_t I_e = es->I;
    const int G2 = (int)(I_e / kGroup);
    const int g0 = chunk * kDkChunk;
    r.ngroups = min(kDkChunk, G2 - g0);
    r.col0 = g0 * kGroup;
    const int64_t row_bytes = I_e * es->bits / 8;
    const uint8_t* w2e = reinterpret_cast<const uint8_t*>(es->w2) + ebase * a.H * row_bytes;
    r.wrow = w2e + (int64_t)(h0 + ml) * row_bytes + (int64_t)g0 * (kGroup * es->bits / 8) + q * (32 * es->bits / 8);
    r.srow = es->s2 + ebase * a.H * G2 + (int64_t)(h0 + ml) * G2 + g0;
    return r;
}

}  // namespace

template <int BITS, int SBITS>
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
    // software pipeline: the next unit's codes are in flight while this one computes
    u32x4_t cur[kDkChunk][2], nxt[kDkChunk][2];
    int bits = BITS;
    DkUnit cu;
    if (u < n_units) {
        cu = dk_make_unit(a, u, n_routed_units, nch, nch_s, h0, &bits);
        if (bits == BITS) dk_load_codes<BITS>(cu, cur);
        else if constexpr (SBITS != 0) dk_load_codes<SBITS>(cu, cur);
    }
    while (u < n_units) {
        const int un = u + V;
        int nbits = BITS;
        DkUnit nu;
        if (un < n_units) {
            nu = dk_make_unit(a, un, n_routed_units, nch, nch_s, h0, &nbits);
            if (nbits == BITS) dk_load_codes<BITS>(nu, nxt);
            else if constexpr (SBITS != 0) dk_load_codes<SBITS>(nu, nxt);
        }
        if (bits == BITS) dk_unit<BITS>(cu, cur, a.abuf, a.width_a, a.tokw, yacc);
        else if constexpr (SBITS != 0) dk_unit<SBITS>(cu, cur, a.abuf, a.width_a, a.tokw, yacc);
        if (un >= n_units) break;
#pragma unroll
        for (int j = 0; j < kDkChunk; ++j) {
            cur[j][0] = nxt[j][0];
            cur[j][1] = nxt[j][1];
        }
        cu = nu;
        bits = nbits;
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
            a.y[o] = (uint16_t)f32_to_bf16(s + r);
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
    y[i] = (uint16_t)f32_to_bf16(s);
}

namespace {

template <int BITS, int SBITS>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    const int max_active = (int)std::min<int64_t>((int64_t)a.E, (int64_t)a.T * a.k);
    const int64_t Imax = std::max(a.routed.I, SBITS ? a.shared.I : (int64_t)0);
    const dim3 gk_grid((unsigned)(Imax / 16), (unsigned)(max_active + (SBITS ? 1 : 0)));
    launch(t, "gk_decode", gk_decode_kernel<BITS, SBITS>, gk_grid, dim3(64 * kGkWaves), s, a);
    const dim3 dk_grid((unsigned)(a.H / 16), (unsigned)a.splits);
    launch(t, "dk_decode", dk_decode_kernel<BITS, SBITS>, dk_grid, dim3(64 * kDkWaves), s, a);
    if (a.splits > 1) {
        const int64_t n = (int64_t)a.T * a.H;
        launch(t, "dk_combine", dk_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s,
               (const float*)a.part, a.splits, n, a.residual, a.y);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (a.routed.bits == 4) {
        if (sb == 0) return launch_decode_t<4, 0>(a, s, t);
        if (sb == 4) return launch_decode_t<4, 4>(a, s, t);
        return launch_decode_t<4, 8>(a, s, t);
    }
    if (sb == 0) return launch_decode_t<8, 0>(a, s, t);
    if (sb == 4) return launch_decode_t<8, 4>(a, s, t);
    return launch_decode_t<8, 8>(a, s, t);
}

}  // namespace w4a16
