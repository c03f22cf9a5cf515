// Set-up of a dense projection y = x . W^T on the expert down-projection kernels (page
// "Nex-N2.5-mini Int4-Int8Mix", Recipe table: the attention and Gated DeltaNet projections
// at INT8 group 128).  A dense projection is one expert that every token uses with
// weight 1: its input rows are x itself, so this kernel writes x in the K order of the
// codes' MFMA operands (each 8-column block reordered, as the gate/up epilogue writes a),
// each row's fp32 sums over 128-column groups (the INT codes' offset seeds, large batches),
// and the routing records of that one expert.
#include "common.h"

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
        *reinterpret_cast<u32x4_t*>(p.abuf + t * p.K + 8 * c8) = perm_act(X);
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

}  // namespace

hipError_t launch_linear_prep(const LinearPrep& p, hipStream_t s, StageTimer* t) {
    const int64_t n = std::max<int64_t>((int64_t)p.T * (p.K / 8), (int64_t)p.T);
    launch(t, "linear_prep", linear_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u, p);
    return hipGetLastError();
}

}  // namespace w4a16
