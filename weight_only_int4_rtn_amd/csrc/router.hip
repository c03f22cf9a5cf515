// Router logits and the shared-expert gate from the token activations (gfx950).
//
// Both stay in bf16 on the pages (page "Nex-N2.5-mini Int4-Int8Mix", Recipe table: the
// routers and shared_expert_gate are left untouched in BF16), so this is a plain bf16
// product x[T, H] . [Wr; wg]^T on v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
// rows [0, E) of the right operand are the router, row E (when given) the gate, whose
// value goes through the logistic sigmoid.  Every sum is formed in a fixed order, so the
// logits (and the top-k decided on them) are bitwise reproducible.
//
// Two launch shapes:
//   router_small_kernel (T <= kRouterSmallT): one workgroup per (16 tokens, 16 rows); its
//     8 waves split K round-robin by 32-column steps and meet in LDS, so a single token's
//     256 logits are spread over 17 workgroups of short, fully overlapped load streams.
//   router_large_kernel: one workgroup per 32 tokens and all rows; the tokens' activations
//     go through LDS once per 128-column chunk and each wave streams the rows of its own
//     16-row tiles from L2 (the router is 1 MiB, read by every workgroup).
#include "common.h"

namespace w4a16 {

namespace {

constexpr int kRWaves = 8;
constexpr int kRThreads = 64 * kRWaves;
constexpr int kLT = 32;               // tokens per large-kernel workgroup
constexpr int kKC = 128;              // K columns per LDS chunk
constexpr int kLdsRow = kKC + 8;      // bf16 per staged row (16 B of padding against bank conflicts)
constexpr int kMaxTilesPerWave = 9;   // ceil((E + 1) / 16) tiles over 8 waves: E <= 1135

// 16 bytes (8 bf16) of row n of the right operand at column k: router row, gate row, or
// zeros past the rows.
__device__ __forceinline__ u32x4_t rhs16(const RouterArgs& a, int n, int64_t k) {
    const uint16_t* p = n < a.n_router ? a.wr + (int64_t)n * a.H + k
                                       : (n == a.n_router && a.wg ? a.wg + k : nullptr);
    return p ? *reinterpret_cast<const u32x4_t*>(p) : u32x4_t{0u, 0u, 0u, 0u};
}

// Logit or gate value of (token t, row n) out.
__device__ __forceinline__ void store_out(const RouterArgs& a, int t, int n, float v) {
    if (t >= a.T) return;
    if (n < a.n_router) a.logits[(int64_t)t * a.n_router + n] = v;
    else if (n == a.n_router && a.wg) a.gate[t] = 1.0f / (1.0f + __expf(-v));
}

__global__ __launch_bounds__(kRThreads) void router_small_kernel(RouterArgs a) {
    __shared__ f32x4_t red[kRWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
    const int q = lane >> 4, ml = lane & 15;
    const int t = t0 + ml, n = n0 + ml;
    const int steps = (int)(a.H / 32);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xrow = a.x + (int64_t)min(t, a.T - 1) * a.H;
    const bool tok_ok = t < a.T;
    // A: token t's 8 columns; B: row n's 8 columns (D[token][row] in lane (row, token group)).
    // Eight steps of this wave per pass, all loads issued before the first MFMA.
    constexpr int kPass = 8;
    for (int s0 = wave; s0 < steps; s0 += kPass * kRWaves) {
        u32x4_t av[kPass], bv[kPass];
#pragma unroll
        for (int i = 0; i < kPass; ++i) {
            const int st = s0 + i * kRWaves;
            const bool ok = st < steps;
            const int64_t k = (int64_t)min(st, steps - 1) * 32 + 8 * q;
            const u32x4_t xa = *reinterpret_cast<const u32x4_t*>(xrow + k);
            av[i] = tok_ok && ok ? xa : u32x4_t{0u, 0u, 0u, 0u};
            bv[i] = ok ? rhs16(a, n, k) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kPass; ++i) acc = mfma16(av[i], bv[i], acc);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f32x4_t s = red[0][lane];
#pragma unroll
        for (int w = 1; w < kRWaves; ++w) {
            const f32x4_t v = red[w][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] += v[r];
        }
        // D row 4q + r is token t0 + 4q + r, column ml is row n0 + ml
#pragma unroll
        for (int r = 0; r < 4; ++r) store_out(a, t0 + 4 * q + r, n0 + ml, s[r]);
    }
}

__global__ __launch_bounds__(kRThreads) void router_large_kernel(RouterArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kLT * kLdsRow];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int t0 = blockIdx.x * kLT;
    const int n_tiles = (a.n_router + (a.wg ? 1 : 0) + 15) / 16;
    const int chunks = (int)(a.H / kKC);
    // each thread stages 16 bytes of the chunk: row r, columns c .. c + 7
    const int sr = threadIdx.x >> 4, sc = (threadIdx.x & 15) * 8;
    const bool s_ok = t0 + sr < a.T;
    const uint16_t* srow = a.x + (int64_t)min(t0 + sr, a.T - 1) * a.H + sc;
    f32x4_t acc[kMaxTilesPerWave][2];
#pragma unroll
    for (int j = 0; j < kMaxTilesPerWave; ++j) acc[j][0] = acc[j][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t nxt = s_ok ? *reinterpret_cast<const u32x4_t*>(srow) : u32x4_t{0u, 0u, 0u, 0u};
    for (int c = 0; c < chunks; ++c) {
        uint16_t* buf = xs[c & 1];
        *reinterpret_cast<u32x4_t*>(buf + sr * kLdsRow + sc) = nxt;
        __syncthreads();   // chunk c staged; chunk c - 2's buffer no longer read
        if (c + 1 < chunks)
            nxt = s_ok ? *reinterpret_cast<const u32x4_t*>(srow + (int64_t)(c + 1) * kKC) : u32x4_t{0u, 0u, 0u, 0u};
        const int64_t k0 = (int64_t)c * kKC;
        u32x4_t av[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[s][i] = *reinterpret_cast<const u32x4_t*>(buf + (16 * i + ml) * kLdsRow + 32 * s + 8 * q);
#pragma unroll
        for (int j = 0; j < kMaxTilesPerWave; ++j) {
            const int tile = wave + kRWaves * j;
            if (tile >= n_tiles) break;
            const int n = 16 * tile + ml;
            u32x4_t bv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) bv[s] = rhs16(a, n, k0 + 32 * s + 8 * q);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[j][i] = mfma16(av[s][i], bv[s], acc[j][i]);
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxTilesPerWave; ++j) {
        const int tile = wave + kRWaves * j;
        if (tile >= n_tiles) break;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) store_out(a, t0 + 16 * i + 4 * q + r, 16 * tile + ml, acc[j][i][r]);
    }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t s, StageTimer* t) {
    const int rows = a.n_router + (a.wg ? 1 : 0);
    if (a.T <= 0 || rows == 0) return hipSuccess;
    const int n_tiles = (rows + 15) / 16;
    if (a.T <= kRouterSmallT) {
        launch(t, "router", router_small_kernel, dim3((unsigned)n_tiles, (unsigned)((a.T + 15) / 16)),
               dim3(kRThreads), s, 0u, a);
    } else {
        launch(t, "router", router_large_kernel, dim3((unsigned)((a.T + kLT - 1) / kLT)), dim3(kRThreads), s, 0u, a);
    }
    return hipGetLastError();
}

}  // namespace w4a16
