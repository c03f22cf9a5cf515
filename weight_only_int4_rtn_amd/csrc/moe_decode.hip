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
// dk_decode_kernel: one workgroup per (16 output rows, expert split); each wave walks a
//   strided subset of the active experts in ascending order and accumulates
//   w[t,j] * (W2_e a) per token in LDS.  Waves, then splits, are summed in a fixed
//   order, so the result is bitwise reproducible.
#include "common.h"

namespace w4a16 {

namespace {

// 16 bytes of one activation row (8 bf16) at column c, reordered for a BITS-wide code;
// zero when the row is padding.
template <int BITS>
__device__ __forceinline__ u32x4_t load_act(const uint16_t* row, int64_t c) {
    if (!row) return u32x4_t{0u, 0u, 0u, 0u};
    return perm_act<BITS>(*reinterpret_cast<const u32x4_t*>(row + c));
}

// One 128-column group: seed with -OFF * sum(x), then add sum_k x_k * (q_k + OFF) for the
// lane's four 8-column slices.  bw holds the lane's 32 codes (16 B for INT4, 32 B INT8).
template <int BITS>
__device__ __forceinline__ f32x4_t group_dot(const u32x4_t (&av)[4], const u32x4_t (&bw)[BITS / 4],
                                             f32x4_t seed) {
    f32x4_t t = seed;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma16(av[i], dq4(bw[0][i]), t);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w0 = bw[i >> 1][(2 * i) & 3], w1 = bw[i >> 1][(2 * i + 1) & 3];
            t = mfma16(av[i], dq8_lo(w0, w1), t);
            t = mfma16(av[i], dq8_hi(w0, w1), t);
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

// Gate/up of one M-tile (tokens in s_tok, -1 = padding) against rows n0..n0+15 of the
// gate half and the same rows of the up half of one expert's [2I, H] bank.
template <int BITS>
__device__ void gk_tile(const uint16_t* __restrict__ x, int64_t H, int64_t I_e, const int32_t* __restrict__ w13e,
                        const uint16_t* __restrict__ s13e, int n0, const int* s_tok, const int* s_row,
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
    const int tok = s_tok[ml];
    const uint16_t* xr = tok >= 0 ? x + (int64_t)tok * H + 32 * q : nullptr;

    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    for (int g = wave; g < G; g += 4) {
        u32x4_t bg[BITS / 4], bu[BITS / 4];
#pragma unroll
        for (int c = 0; c < BITS / 4; ++c) {
            bg[c] = *reinterpret_cast<const u32x4_t*>(wg + (int64_t)g * kGroupBytes + 16 * c);
            bu[c] = *reinterpret_cast<const u32x4_t*>(wu + (int64_t)g * kGroupBytes + 16 * c);
        }
        u32x4_t av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = load_act<BITS>(xr, (int64_t)g * kGroup + 8 * i);
        const float scg = bf16_to_f32(sg[g]), scu = bf16_to_f32(su[g]);
        const f32x4_t seed = offset_seed<BITS>(av);
        const f32x4_t tg = group_dot<BITS>(av, bg, seed);
        const f32x4_t tu = group_dot<BITS>(av, bu, seed);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            accg[r] += scg * tg[r];
            accu[r] += scu * tu[r];
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        s_red[(wave * 8 + r) * 64 + lane] = accg[r];
        s_red[(wave * 8 + 4 + r) * 64 + lane] = accu[r];
    }
    __syncthreads();
    {   // wave w finishes element r = w of every lane: D row 4q + w, column ml
        const int r = wave;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            gs += s_red[(w * 8 + r) * 64 + lane];
            us += s_red[(w * 8 + 4 + r) * 64 + lane];
        }
        const int row = s_row[4 * q + r];
        if (row >= 0) abuf[(int64_t)row * width_a + n0 + ml] = (uint16_t)f32_to_bf16(silu_mul(gs, us));
    }
    __syncthreads();
}

}  // namespace

template <int BITS, int SBITS>
__global__ __launch_bounds__(256) void gk_decode_kernel(DecodeArgs a) {
    __shared__ int s_tok[16], s_row[16];
    __shared__ float s_red[4 * 8 * 64];
    const int slot = blockIdx.y;
    const bool shared = SBITS != 0 && slot == (int)gridDim.y - 1;
    const int n0 = blockIdx.x * 16;
    int count, pos0, e = 0;
    int64_t I_e;
    if (shared) {
        I_e = a.shared.I;
        count = a.T;
        pos0 = a.T * a.k;
    } else {
        if (slot >= a.meta[0]) return;
        e = a.active[slot];
        I_e = a.routed.I;
        pos0 = a.offsets[e];
        count = a.offsets[e + 1] - pos0;
    }
    if (n0 >= I_e) return;
    for (int mt = 0; mt < count; mt += 16) {
        if (threadIdx.x < 16) {
            const int m = mt + threadIdx.x;
            const bool valid = m < count;
            s_tok[threadIdx.x] = valid ? (shared ? m : a.sorted[pos0 + m] / a.k) : -1;
            s_row[threadIdx.x] = valid ? pos0 + m : -1;
        }
        __syncthreads();
        if (shared) {
            if constexpr (SBITS != 0)
                gk_tile<SBITS>(a.x, a.H, I_e, a.shared.w13, a.shared.s13, n0, s_tok, s_row, a.abuf, a.width_a, s_red);
        } else {
            const int64_t w13_words = 2 * I_e * a.H * BITS / 32;
            gk_tile<BITS>(a.x, a.H, I_e, a.routed.w13 + (int64_t)e * w13_words,
                          a.routed.s13 + (int64_t)e * 2 * I_e * (a.H / kGroup), n0, s_tok, s_row, a.abuf,
                          a.width_a, s_red);
        }
    }
}

namespace {

// Down projection of one expert's tokens for output rows h0..h0+15, accumulated with the
// router weights into this wave's LDS accumulator yacc[T][16].
template <int BITS>
__device__ void dk_expert(const int32_t* __restrict__ w2e, const uint16_t* __restrict__ s2e, int64_t I_e,
                          int h0, const uint16_t* __restrict__ abuf, int64_t width_a, int pos0, int count,
                          bool shared, const int32_t* __restrict__ sorted, const float* __restrict__ wts, int k,
                          float* yacc) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, ml = lane & 15;
    const int G2 = (int)(I_e / kGroup);
    constexpr int kLaneBytes = 32 * BITS / 8;
    constexpr int kGroupBytes = kGroup * BITS / 8;
    const uint8_t* wrow = reinterpret_cast<const uint8_t*>(w2e) + (int64_t)(h0 + ml) * (I_e * BITS / 8) + q * kLaneBytes;
    const uint16_t* srow = s2e + (int64_t)(h0 + ml) * G2;
    for (int mt = 0; mt < count; mt += 16) {
        const int mload = mt + ml;
        const uint16_t* arow = mload < count ? abuf + (int64_t)(pos0 + mload) * width_a + 32 * q : nullptr;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int g = 0; g < G2; ++g) {
            u32x4_t bw[BITS / 4];
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c)
                bw[c] = *reinterpret_cast<const u32x4_t*>(wrow + (int64_t)g * kGroupBytes + 16 * c);
            u32x4_t av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = load_act<BITS>(arow, (int64_t)g * kGroup + 8 * i);
            const float sc = bf16_to_f32(srow[g]);
            const f32x4_t t = group_dot<BITS>(av, bw, offset_seed<BITS>(av));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += sc * t[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mt + 4 * q + r;
            if (m < count) {
                int t;
                float w;
                if (shared) {
                    t = m;
                    w = 1.0f;
                } else {
                    const int p = sorted[pos0 + m];
                    t = p / k;
                    w = wts[p];
                }
                yacc[t * 16 + ml] += w * acc[r];
            }
        }
    }
}

}  // namespace

template <int BITS, int SBITS>
__global__ __launch_bounds__(256) void dk_decode_kernel(DecodeArgs a) {
    __shared__ float s_y[4][kSmallT * 16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h0 = blockIdx.x * 16;
    const int T = a.T;
    float* yacc = s_y[wave];
    for (int i = lane; i < T * 16; i += 64) yacc[i] = 0.f;

    const int n_active = a.meta[0];
    const int n_units = n_active + (SBITS != 0 ? 1 : 0);
    const int V = gridDim.y * 4;
    for (int u = blockIdx.y * 4 + wave; u < n_units; u += V) {
        if (SBITS != 0 && u == n_active) {
            if constexpr (SBITS != 0)
                dk_expert<SBITS>(a.shared.w2, a.shared.s2, a.shared.I, h0, a.abuf, a.width_a, T * a.k, T, true,
                                 a.sorted, a.wts, a.k, yacc);
        } else {
            const int e = a.active[u];
            const int pos0 = a.offsets[e];
            const int64_t I_e = a.routed.I;
            dk_expert<BITS>(a.routed.w2 + (int64_t)e * (a.H * I_e * BITS / 32),
                            a.routed.s2 + (int64_t)e * a.H * (I_e / kGroup), I_e, h0, a.abuf, a.width_a, pos0,
                            a.offsets[e + 1] - pos0, false, a.sorted, a.wts, a.k, yacc);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * 16; i += blockDim.x) {
        const float s = ((s_y[0][i] + s_y[1][i]) + s_y[2][i]) + s_y[3][i];
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
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    const int max_active = (int)std::min<int64_t>((int64_t)a.E, (int64_t)a.T * a.k);
    const int64_t Imax = std::max(a.routed.I, SBITS ? a.shared.I : (int64_t)0);
    const dim3 gk_grid((unsigned)(Imax / 16), (unsigned)(max_active + (SBITS ? 1 : 0)));
    gk_decode_kernel<BITS, SBITS><<<gk_grid, 256, 0, s>>>(a);
    const dim3 dk_grid((unsigned)(a.H / 16), (unsigned)a.splits);
    dk_decode_kernel<BITS, SBITS><<<dk_grid, 256, 0, s>>>(a);
    if (a.splits > 1) {
        const int64_t n = (int64_t)a.T * a.H;
        dk_combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.part, a.splits, n, a.residual, a.y);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int sb = a.shared.bits;
    if (a.routed.bits == 4) {
        if (sb == 0) return launch_decode_t<4, 0>(a, s);
        if (sb == 4) return launch_decode_t<4, 4>(a, s);
        return launch_decode_t<4, 8>(a, s);
    }
    if (sb == 0) return launch_decode_t<8, 0>(a, s);
    if (sb == 4) return launch_decode_t<8, 4>(a, s);
    return launch_decode_t<8, 8>(a, s);
}

}  // namespace w4a16
