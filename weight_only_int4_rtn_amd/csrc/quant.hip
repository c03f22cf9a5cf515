// RTN group quantizer and packer (page "Nex-N2.5-mini Int4-Int8Mix", section Recipe:
// symmetric round-to-nearest, one min-max scale per 128 input columns, no calibration).
//
// One group of 128 consecutive columns is handled by 16 lanes, 8 values per lane, so a
// wave covers four consecutive groups: 2 KB of fp32 (or 1 KB of bf16) read as 32-byte
// (16-byte) lane slices, fully coalesced.  Lane i of a group writes packed word i
// (INT4) or words 2i, 2i+1 (INT8); lane 0 writes the bf16 scale.  HBM-bound: about
// 4.5 bytes move per fp32 weight.
#include "common.h"

namespace w4a16 {

template <int BITS, bool BF16_IN>
__global__ __launch_bounds__(256) void quantize_pack_kernel(const void* __restrict__ w, int64_t n_groups,
                                                            int32_t* __restrict__ packed,
                                                            uint16_t* __restrict__ scales) {
    const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    if (gid >= n_groups) return;  // all 16 lanes of a group leave together

    const int64_t e0 = gid * kGroup + sub * 8;
    float v[8];
    if constexpr (BF16_IN) {
        const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(w) + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(raw[i] << 16);
            v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
        }
    } else {
        const float* src = static_cast<const float*>(w) + e0;
        const float4 lo = *reinterpret_cast<const float4*>(src);
        const float4 hi = *reinterpret_cast<const float4*>(src + 4);
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    }

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));

    constexpr float qmax = BITS == 4 ? 7.0f : 127.0f;
    constexpr int offset = 1 << (BITS - 1);
    const uint32_t sbits = f32_to_bf16(amax / qmax);   // IEEE fp32 division, then RNE to bf16
    const float s = bf16_to_f32(sbits);

    uint32_t u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float q = 0.0f;
        if (s != 0.0f) q = fminf(fmaxf(rintf(v[i] / s), -qmax - 1.0f), qmax);   // IEEE division, ties to even
        u[i] = (uint32_t)((int)q + offset);
    }

    if constexpr (BITS == 4) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= u[i] << (4 * i);
        packed[gid * 16 + sub] = (int32_t)word;
    } else {
        u32x2_t words;
        words[0] = u[0] | (u[1] << 8) | (u[2] << 16) | (u[3] << 24);
        words[1] = u[4] | (u[5] << 8) | (u[6] << 16) | (u[7] << 24);
        *reinterpret_cast<u32x2_t*>(packed + gid * 32 + sub * 2) = words;
    }
    if (sub == 0) scales[gid] = (uint16_t)sbits;
}

hipError_t launch_quantize(const void* w, bool bf16_in, int64_t total_rows, int64_t cols, int bits,
                           int32_t* packed, uint16_t* scales, hipStream_t s) {
    const int64_t n_groups = total_rows * (cols / kGroup);
    if (n_groups == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_groups + 15) / 16)), block(256);
    if (bits == 4) {
        if (bf16_in) quantize_pack_kernel<4, true><<<grid, block, 0, s>>>(w, n_groups, packed, scales);
        else quantize_pack_kernel<4, false><<<grid, block, 0, s>>>(w, n_groups, packed, scales);
    } else {
        if (bf16_in) quantize_pack_kernel<8, true><<<grid, block, 0, s>>>(w, n_groups, packed, scales);
        else quantize_pack_kernel<8, false><<<grid, block, 0, s>>>(w, n_groups, packed, scales);
    }
    return hipGetLastError();
}

}  // namespace w4a16
