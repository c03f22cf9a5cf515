// Device helpers of the decode (GEMV-shaped) kernels: activation fragments and one
// 128-column group of a 16x16 MFMA tile with codes as exact bf16 integers.
#pragma once
#include "common.h"

namespace w4a16 {
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

// The code offset OFF of a BITS-wide code (see neg_offset_operand).
template <int BITS>
constexpr float code_offset() { return BITS == 4 ? 136.f : 2304.f; }

}  // namespace
}  // namespace w4a16
