// Set-up of a dense projection y = x . W^T on the expert down-projection kernels (page
// "Nex-N2.5-mini Int4-Int8Mix", Recipe table: the attention and Gated DeltaNet projections
// at INT8 group 128).  A dense projection is one expert that every token uses with
// weight 1: its input rows are x itself, so this kernel writes x in the K order of the
// codes' MFMA operands (each 8-column block reordered, as the gate/up epilogue writes a;
// not for 8-bit codes, whose GEMM reads x unpermuted: abuf NULL), each row's fp32 sums
// over 128-column groups (the INT codes' offset seeds, large batches), and the routing
// records of that one expert.
#include "common.h"
#include "decode_dev.h"

namespace w4a16 {

namespace {

// One thread per 8 columns of a row: 16 threads cover one 128-column group.
__global__ __launch_bounds__(256) void linear_prep_kernel(LinearPrep p) {
    const int64_t cols8 = p.K / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool ok = i < (int64_t)p.T * cols8;
    const int64_t t = ok ? i / cols8 : 0, c8 = ok ? i % cols8 : 0;
    float sum = 0.f;
    if (ok) {
        const u32x4_t X = *reinterpret_cast<const u32x4_t*>(p.x + t * p.K + 8 * c8);
        if (p.abuf) *reinterpret_cast<u32x4_t*>(p.abuf + t * p.K + 8 * c8) = perm_act(X);
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += bf16_to_f32(X[e] & 0xffffu) + bf16_to_f32(X[e] >> 16);
    }
    // group sums: the 16 threads of a group are 16 consecutive lanes (K % 128 == 0)
    sum += __shfl_xor(sum, 1, 16);
    sum += __shfl_xor(sum, 2, 16);
    sum += __shfl_xor(sum, 4, 16);
    sum += __shfl_xor(sum, 8, 16);
    if (ok && p.asum && (c8 & 15) == 0) p.asum[t * (p.K / kGroup) + c8 / 16] = sum;
    // the one expert's records: every token in order, weight 1
    if (i < p.T) {
        p.tokw[i] = int2{(int)i, __float_as_int(1.0f)};
        p.wts[i] = 1.0f;
        p.inv[i] = (int)i;
    }
    const int n_tiles = (p.T + kPrefillMT - 1) / kPrefillMT;
    if (i < n_tiles) {
        p.tiles[2 * i] = 0;
        p.tiles[2 * i + 1] = (int)i * kPrefillMT;
    }
    if (i == 0) {
        p.rec[0] = int4{0, 0, p.T, 0};
        p.meta[0] = 1;
        p.meta[1] = n_tiles;
        p.offsets[0] = 0;
        p.offsets[1] = p.T;
    }
}

// ------------------------------------------------------------------ small batches
//
// T <= 64 tokens: a weight stream with no set-up launch.  Workgroup b owns output rows
// 16 RB b .. 16 RB (b + 1) - 1 (RB row blocks of 16) and all of K; wave w takes the GW
// groups w GW .. w GW + GW - 1 of every row block and issues every code and scale load of
// them before its first MFMA (16x16x32 bf16: tokens on the M side, codes as exact bf16
// values, the lane's activations read straight from x and reordered into the codes' K
// order in registers; one activation fragment serves the RB row blocks, so two row blocks
// per workgroup halve the reads of x).  Each wave leaves its partial sums of every token
// in LDS; the workgroup adds them in wave order (bitwise reproducible), adds the residual
// and rounds once to bf16.  The launch makes GW * waves == K / 128.
template <int CF, int GW, int RB>
__global__ __launch_bounds__(1024) void linear_small_kernel(LinearSmall p) {
    constexpr int BITS = cf_bits(CF);
    constexpr int kGroupBytes = kGroup * BITS / 8;
    constexpr int NW = 16 * RB;         // output rows of the workgroup
    extern __shared__ float s_part[];   // [waves][T][NW]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, S = (int)(blockDim.x >> 6);
    const int q = lane >> 4, ml = lane & 15;
    const int T = p.T, G = (int)(p.K / kGroup);
    const int64_t h0 = (int64_t)blockIdx.x * NW;
    const int g0 = wave * GW;
    u32x4_t bw[RB][GW][BITS / 4];
    float sc[RB][GW], xs[RB][GW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int64_t n = h0 + 16 * rb + ml;   // this lane's code row of row block rb
        const uint8_t* wrow = reinterpret_cast<const uint8_t*>(p.w) + n * (p.K * BITS / 8) +
                              (int64_t)g0 * kGroupBytes + q * (32 * BITS / 8);
#pragma unroll
        for (int j = 0; j < GW; ++j) {
#pragma unroll
            for (int c = 0; c < BITS / 4; ++c) bw[rb][j][c] = load_stream16(wrow + j * kGroupBytes + 16 * c);
            load_scales<CF>(p.s, scale_at<CF>(n, G, g0 + j), q, &sc[rb][j], &xs[rb][j]);
        }
    }
    float* part = s_part + (int64_t)wave * T * NW;
    for (int mt = 0; mt < T; mt += 16) {
        const int tok = mt + ml;
        const bool ok = tok < T;
        const uint16_t* xr = p.x + (int64_t)(ok ? tok : 0) * p.K;
        u32x4_t av[GW][4];
#pragma unroll
        for (int j = 0; j < GW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) av[j][i] = load_act<CF>(xr, ok, (int64_t)(g0 + j) * kGroup + 32 * q + 8 * i);
        f32x4_t acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < GW; ++j) {
            const f32x4_t seed = offset_seed<CF>(av[j]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const f32x4_t t = group_dot<CF>(av[j], bw[rb][j], seed, xs[rb][j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rb][r] += sc[rb][j] * t[r];
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r)   // D row 4q + r of the tile is token mt + 4q + r
                if (mt + 4 * q + r < T) part[(mt + 4 * q + r) * NW + 16 * rb + ml] = acc[rb][r];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * NW; i += blockDim.x) {
        float sum = 0.f;
        for (int w = 0; w < S; ++w) sum += s_part[w * T * NW + i];
        const int64_t o = (int64_t)(i / NW) * p.N + h0 + (i % NW);
        if (p.residual) sum += bf16_to_f32(p.residual[o]);
        p.y[o] = (uint16_t)cvt_bf16(sum);
    }
}

constexpr int kLinearMaxLds = 128 * 1024;   // partial sums of 16 waves x 64 tokens x 32 rows

template <int CF, int GW, int RB>
hipError_t launch_linear_small_k(const LinearSmall& p, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                                 StageTimer* t) {
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(linear_small_kernel<CF, GW, RB>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kLinearMaxLds);
        return true;
    }();
    (void)attr;
    launch(t, "linear_small", linear_small_kernel<CF, GW, RB>, grid, block, s, lds, p);
    return hipGetLastError();
}

template <int CF>
hipError_t launch_linear_small_cf(const LinearSmall& p, int cfg, hipStream_t s, StageTimer* t) {
    const int gw = cfg & 15, rb = cfg >> 4;
    const int waves = (int)(p.K / kGroup) / gw;
    const dim3 grid((unsigned)(p.N / (16 * rb))), block((unsigned)(64 * waves));
    const uint32_t lds = (uint32_t)(waves * p.T * 16 * rb * 4);
    if constexpr (cf_bits(CF) == 4) {
        if (cfg == (4 | 1 << 4)) return launch_linear_small_k<CF, 4, 1>(p, grid, block, lds, s, t);
        if (cfg == (2 | 2 << 4)) return launch_linear_small_k<CF, 2, 2>(p, grid, block, lds, s, t);
    }
    if (cfg == (2 | 1 << 4)) return launch_linear_small_k<CF, 2, 1>(p, grid, block, lds, s, t);
    if (cfg == (1 | 2 << 4)) return launch_linear_small_k<CF, 1, 2>(p, grid, block, lds, s, t);
    if (cfg == (1 | 1 << 4)) return launch_linear_small_k<CF, 1, 1>(p, grid, block, lds, s, t);
    return hipErrorInvalidValue;   // a configuration linear_small_cfg does not produce
}

}  // namespace

// Configuration of the small-batch dense kernel: gw | rb << 4, or 0 when the shape does not
// fit it.  gw groups per wave (4, 2, 1; rb * gw * bits <= 16: at most 2 KiB of codes per
// wave and 16 rows), at most 16 waves per workgroup, gw dividing the group count.  Above 16
// tokens two row blocks per workgroup (rb = 2) when that launch still has 2048 waves (8
// per SIMD); otherwise one, with the largest gw that still launches 2048 waves, else the
// smallest gw.
int linear_small_cfg(int64_t T, int64_t K, int64_t N, int bits) {
    if (T < 1 || T > kSmallT) return 0;
    const int64_t G = K / kGroup, R = N / 16;
    auto fits = [&](int gw, int rb) { return gw * rb * bits <= 16 && G % gw == 0 && G / gw <= 16 && R % rb == 0; };
    if (T > 16)
        for (int gw : {4, 2, 1})
            if (fits(gw, 2) && (R / 2) * (G / gw) >= 2048) return gw | 2 << 4;
    int best = 0;
    for (int gw : {4, 2, 1}) {
        if (!fits(gw, 1)) continue;
        best = gw | 1 << 4;
        if (R * (G / gw) >= 2048) return best;
    }
    return best;
}

hipError_t launch_linear_small(const LinearSmall& p, int cf, int cfg, hipStream_t s, StageTimer* t) {
    switch (cf) {
        case 4: return launch_linear_small_cf<4>(p, cfg, s, t);
        case 8: return launch_linear_small_cf<8>(p, cfg, s, t);
        case kCfFp8: return launch_linear_small_cf<kCfFp8>(p, cfg, s, t);
        default: return launch_linear_small_cf<kCfMx4>(p, cfg, s, t);
    }
}

hipError_t launch_linear_prep(const LinearPrep& p, hipStream_t s, StageTimer* t) {
    const int64_t n = std::max<int64_t>((int64_t)p.T * (p.K / 8), (int64_t)p.T);
    launch(t, "linear_prep", linear_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u, p);
    return hipGetLastError();
}

}  // namespace w4a16
