// Device helpers of the decode (GEMV-shaped) kernels: activation fragments and one
// 128-column group of a 16x16 MFMA tile with codes as exact bf16 integers.
#pragma once
#include "common.h"

namespace w4a16 {
namespace {

// 16 bytes of one activation row (8 bf16) at column c, reordered into the codes' K order;
// zero when the row is padding (`ok` false; `row` then points at any valid row).
template <int CF>
__device__ __forceinline__ u32x4_t load_act(const uint16_t* row, bool ok, int64_t c) {
    return perm_act(load16_or_zero(row + c, ok, row));
}

// One 128-column group: seed with -OFF * sum(x), then add sum_k x_k * (q_k + OFF) for the
// lane's four 8-column slices.  bw holds the lane's 32 codes (16 B for 4-bit codes, 32 B for
// 8-bit ones; columns 32q .. 32q + 31 of the group for lane group q).  FP8 / MXFP4 codes are
// converted to their exact bf16 values (MXFP4 times xs, the lane's block scale) and need
// no seed.
template <int CF>
__device__ __forceinline__ f32x4_t group_dot(const u32x4_t (&av)[4], const u32x4_t (&bw)[cf_bits(CF) / 4],
                                             f32x4_t seed, float xs = 1.f) {
    f32x4_t t = seed;
    const uint32_t M = nibble_mask();
    if constexpr (CF == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma16(av[i], dq4(bw[0][i], M), t);
    } else if constexpr (CF == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4_t lo, hi;
            dq8(bw[i >> 1][(2 * i) & 3], bw[i >> 1][(2 * i + 1) & 3], lo, hi, M);
            t = mfma16(av[i], lo, t);
            t = mfma16(av[i], hi, t);
        }
    } else if constexpr (CF == kCfFp8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma16(av[i], dq_fp8(bw[i >> 1][(2 * i) & 3], bw[i >> 1][(2 * i + 1) & 3]), t);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma16(av[i], dq_mx4(bw[0][i], xs), t);
    }
    return t;
}

template <int CF>
__device__ __forceinline__ f32x4_t offset_seed(const u32x4_t (&av)[4]) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
    if constexpr (cf_int(CF)) {
        const u32x4_t neg = neg_offset_operand<CF>();
#pragma unroll
        for (int i = 0; i < 4; ++i) c = mfma16(av[i], neg, c);
    }
    return c;
}

// The code offset OFF of an INT code (see neg_offset_operand); 0 for the float formats.
template <int CF>
constexpr float code_offset() { return CF == 4 ? 136.f : CF == 8 ? 2304.f : 0.f; }

// Scale storage of a code format, for an expert whose rows hold K = G * 128 columns:
// INT bf16 [rows, G]; FP8 fp32 [rows]; MXFP4 E8M0 bytes [rows, 4 G].  Byte offset of row
// `row`'s scale at group g (FP8: the row's one scale), and of expert e's scales.
template <int CF>
__device__ __forceinline__ int64_t scale_at(int64_t row, int G, int g) {
    if constexpr (CF == kCfFp8) return row * 4;
    else if constexpr (CF == kCfMx4) return (row * G + g) * 4;
    else return (row * G + g) * 2;
}
template <int CF>
__device__ __forceinline__ int64_t expert_scale_bytes(int64_t rows, int G) {
    return CF == kCfFp8 ? rows * 4 : CF == kCfMx4 ? rows * G * 4 : rows * G * 2;
}

// The partial-sum scale (INT: the group's bf16 scale; FP8: the row's fp32 scale; MXFP4: 1)
// and the conversion scale (MXFP4: the block of lane group q; else 1) at byte offset `off`.
template <int CF>
__device__ __forceinline__ void load_scales(const uint8_t* base, int64_t off, int q, float* sc, float* xs) {
    if constexpr (CF == kCfFp8) {
        *sc = *reinterpret_cast<const float*>(base + off);
        *xs = 1.f;
    } else if constexpr (CF == kCfMx4) {
        *sc = 1.f;
        *xs = e8m0_scale(base[off + q]);
    } else {
        *sc = bf16_to_f32(*reinterpret_cast<const uint16_t*>(base + off));
        *xs = 1.f;
    }
}

}  // namespace
}  // namespace w4a16
