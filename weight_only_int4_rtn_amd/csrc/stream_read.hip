// A plain streaming read of a byte range: the reference against which the decode
// kernels' time for the same bytes is judged (the achievable read time of that many bytes
// in one launch).  Every lane reads 16-byte vectors in a grid-stride loop, four in flight,
// and the XOR of all 32-bit words is folded into one output word, so no load can be dropped.
#include "common.h"

namespace w4a16 {

namespace {

constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t* __restrict__ v, int64_t n16,
                                                                   uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = v[i], b = v[i + stride], c = v[i + 2 * stride], d = v[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= v[i];
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x ^= __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0 && x != 0u) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    // enough workgroups to keep every CU's loads in flight, at most one pass of four vectors
    // per lane when the range is small
    const int64_t want = (n16 + 4 * kReadThreads - 1) / (4 * kReadThreads);
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 256 * 16));
    stream_read_kernel<<<grid, kReadThreads, 0, s>>>(static_cast<const u32x4_t*>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace w4a16
