// Quantizers of the two other expert formats the pages evaluate.
//
// FP8 E4M3, one scale per output channel (page "Nex-N2.5-mini-mixed-NVFP4-FP8", What's
// quantized to what; weights-only round-to-nearest): per row s = absmax / 448 (fp32,
// IEEE division), codes = E4M3(w / s) rounded to nearest even by the hardware conversion
// (v_cvt_pk_fp8_f32).  One workgroup per row: a max pass, then a code pass.
//
// MXFP4 (page "Nex-N2.5-mini-MXFP4-MxWave", Model summary and Quantization method): E2M1
// codes with one E8M0 scale per block of 32 columns.  One 32-lane half-wave per block,
// one value per lane.  Round-to-nearest exponent: floor(log2 amax) - 2.  Search: the
// candidates floor(log2(p99.5 / 6)) - 4 .. + 1 and the smallest exponent that does not
// clip, the lowest squared weight error winning (equal errors: the smaller exponent).
// Every decision is exact: exponents from frexp, p99.5 = a + (b - a) * 0.845 from the two
// largest |w| of the block, the error of a candidate summed in fp64 by a fixed butterfly
// over the 32 lanes (lane i with i ^ 16, then ^ 8, ^ 4, ^ 2, ^ 1), with no fused multiply-add.
#include "common.h"

namespace w4a16 {

namespace {

template <bool BF16_IN>
__device__ __forceinline__ float load_w(const void* w, int64_t i) {
    if constexpr (BF16_IN) return bf16_to_f32(static_cast<const uint16_t*>(w)[i]);
    else return static_cast<const float*>(w)[i];
}

template <bool BF16_IN>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const void* __restrict__ w, int64_t cols,
                                                           int32_t* __restrict__ packed, float* __restrict__ scales) {
    __shared__ float s_max[4];
    const int64_t row = blockIdx.x;
    const int64_t base = row * cols;
    const int n4 = (int)(cols / 4);
    float amax = 0.f;
    for (int c4 = threadIdx.x; c4 < n4; c4 += blockDim.x)
#pragma unroll
        for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(load_w<BF16_IN>(w, base + 4 * c4 + j)));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float s = amax / 448.0f;   // IEEE fp32 division
    for (int c4 = threadIdx.x; c4 < n4; c4 += blockDim.x) {
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = s != 0.f ? load_w<BF16_IN>(w, base + 4 * c4 + j) / s : 0.f;
        uint32_t word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
        word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], (int)word, true);
        packed[row * n4 + c4] = (int32_t)word;
    }
    if (threadIdx.x == 0) scales[row] = s;
}

// E2M1 code of r (round to nearest, ties to the even code, saturating at 6; sign bit of r):
// the number of decision points |r| has passed, a tie passing only into an even code.
__device__ __forceinline__ uint32_t e2m1_code(double r) {
    const double a = fabs(r);
    uint32_t c = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
    return c | (signbit(r) ? 8u : 0u);
}

__device__ __forceinline__ double e2m1_value(uint32_t code) {
    const uint32_t m = code & 7u;
    const double mag = m < 4 ? 0.5 * m : (m == 4 ? 2.0 : m == 5 ? 3.0 : m == 6 ? 4.0 : 6.0);
    return (code & 8u) ? -mag : mag;
}

// floor(log2 y) of a positive finite value, from its binary exponent.
__device__ __forceinline__ int floor_log2(double y) {
    int e;
    (void)frexp(y, &e);
    return e - 1;
}

// Squared error of the block (this lane's value v) at exponent e, summed over the 32 lanes
// by the fixed butterfly; every lane returns the same bits.
__device__ double block_sse(float v, int e) {
#pragma clang fp contract(off)
    const double vd = (double)v;
    const double sc = ldexp(1.0, e);
    const double rec = e2m1_value(e2m1_code(vd / sc)) * sc;
    const double d = vd - rec;
    double s = d * d;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
        const double o = __shfl_xor(s, off, 32);
        s = s + o;
    }
    return s;
}

template <bool BF16_IN, bool MSE>
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const void* __restrict__ w, int64_t n_blocks,
                                                             int32_t* __restrict__ packed,
                                                             uint8_t* __restrict__ scales) {
#pragma clang fp contract(off)
    const int64_t blk = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    if (blk >= n_blocks) return;   // the 32 lanes of a block leave together
    const float v = load_w<BF16_IN>(w, blk * 32 + lane);
    const float av = fabsf(v);
    float amax = av;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
    int e;
    if (amax == 0.f) {
        e = -127;
    } else {
        int ex;
        const float m = frexpf(amax, &ex);   // amax = m * 2^ex, m in [0.5, 1)
        const int E = ex - 1;                // floor(log2 amax)
        if constexpr (!MSE) {
            e = E - 2;
        } else {
            // the second largest |w|: the largest itself when it occurs twice
            const unsigned long long at_max = __ballot(av == amax);
            const uint32_t half = (uint32_t)(at_max >> ((threadIdx.x & 32) ? 32 : 0));
            float second = av == amax ? -1.f : av;
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) second = fmaxf(second, __shfl_xor(second, off, 32));
            if (__popc(half) >= 2) second = amax;
            const double a = (double)second, b = (double)amax;
            const double p = a + (b - a) * 0.845;
            const int e0 = floor_log2(p / 6.0);
            const int e_nc = m <= 0.75f ? E - 2 : E - 1;   // smallest e with amax <= 6 * 2^e
            int best_e = max(-127, min(127, e_nc));
            double best = block_sse(v, best_e);
            for (int d = -4; d <= 1; ++d) {
                const int c = max(-127, min(127, e0 + d));
                const double err = block_sse(v, c);
                if (err < best || (err == best && c < best_e)) {
                    best = err;
                    best_e = c;
                }
            }
            e = best_e;
        }
        e = max(-127, min(127, e));
    }
    const uint32_t code = e2m1_code((double)v / ldexp(1.0, e));
    // eight lanes form one word: lane 8j + i holds nibble i
    uint32_t word = code << (4 * (lane & 7));
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) word |= __shfl_xor(word, off, 32);
    if ((lane & 7) == 0) packed[blk * 4 + (lane >> 3)] = (int32_t)word;
    if (lane == 0) scales[blk] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_fp8_quantize(const void* w, bool bf16_in, int64_t total_rows, int64_t cols, int32_t* packed,
                               float* scales, hipStream_t s) {
    if (total_rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)total_rows), block(256);
    if (bf16_in) fp8_quantize_kernel<true><<<grid, block, 0, s>>>(w, cols, packed, scales);
    else fp8_quantize_kernel<false><<<grid, block, 0, s>>>(w, cols, packed, scales);
    return hipGetLastError();
}

hipError_t launch_mxfp4_quantize(const void* w, bool bf16_in, int64_t total_rows, int64_t cols, bool mse,
                                 int32_t* packed, uint8_t* scales, hipStream_t s) {
    const int64_t n_blocks = total_rows * (cols / 32);
    if (n_blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_blocks + 7) / 8)), block(256);
    if (bf16_in) {
        if (mse) mxfp4_quantize_kernel<true, true><<<grid, block, 0, s>>>(w, n_blocks, packed, scales);
        else mxfp4_quantize_kernel<true, false><<<grid, block, 0, s>>>(w, n_blocks, packed, scales);
    } else {
        if (mse) mxfp4_quantize_kernel<false, true><<<grid, block, 0, s>>>(w, n_blocks, packed, scales);
        else mxfp4_quantize_kernel<false, false><<<grid, block, 0, s>>>(w, n_blocks, packed, scales);
    }
    return hipGetLastError();
}

}  // namespace w4a16
