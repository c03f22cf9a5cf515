// Internal device helpers and kernel-launch declarations of the W4A16 MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include "w4a16.h"
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

namespace w4a16 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The same rounding for activations and outputs by the hardware conversion
// (v_cvt_pk_bf16_f32, round to nearest even; a NaN stays a NaN with its own payload).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------------- MFMA

// D = A * B + C with A 16x32, B 32x16 bf16 and C/D 16x16 fp32 (gfx950).
// Lane l supplies A[l % 16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l % 16] and holds
// D[4*(l/16) + r][l % 16] in element r.  The K order inside each lane's 8-element
// slice is free as long as A and B use the same one.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ------------------------------------------------- code -> bf16 operand packing
//
// A packed code u (offset binary) becomes an exact bf16 integer by OR-ing it into the
// mantissa of a power of two: bits 0x4300|n are 128 + n, bits 0x4500|n are 2048 + 16n
// (n < 16).  The MFMA then forms sum_k x_k (q_k + OFF) and the offset term
// OFF * sum_k x_k is cancelled by seeding the accumulator with an MFMA against the
// constant -OFF.  INT4: OFF = 136 (q = u - 8 = (128 + u) - 136).
// INT8: the byte splits into nibbles lo + 16 hi, two MFMAs with (128 + lo) and
// (2048 + 16 hi) give u + 2176, so q = u - 128 has OFF = 2304.
//
// INT4 word w holds k0..k7 (k0 lowest).  dq4 returns the bf16 pairs
// (k0,k4) (k1,k5) (k2,k6) (k3,k7); the activation slice must use that order.
// A VOP3 instruction can read only one scalar or literal operand on gfx9, so the nibble
// mask is kept in a vector register (nibble_mask()) to let (w & mask) | C fuse into a
// single v_and_or_b32.
__device__ __forceinline__ uint32_t nibble_mask() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m));
    return m;
}
__device__ __forceinline__ u32x4_t dq4(uint32_t w, uint32_t M) {
    const uint32_t C = 0x43004300u;
    u32x4_t r;
    r[0] = (w & M) | C;
    r[1] = ((w >> 4) & M) | C;
    r[2] = ((w >> 8) & M) | C;
    r[3] = ((w >> 12) & M) | C;
    return r;
}
__device__ __forceinline__ u32x4_t dq4(uint32_t w) { return dq4(w, 0x000f000fu); }

// INT8 words w0 = k0..k3, w1 = k4..k7 (one byte each).  Each byte splits into its low
// and high nibble; v_perm gathers bytes j and j+4 into one word so the pairs come out
// in the same K order as dq4: (k0,k4) (k1,k5) (k2,k6) (k3,k7).
__device__ __forceinline__ void dq8(uint32_t w0, uint32_t w1, u32x4_t& lo, u32x4_t& hi, uint32_t M = 0x000f000fu) {
    const uint32_t CL = 0x43004300u, CH = 0x45004500u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // bytes: [w0.byte j, 0, w1.byte j, 0]   (selector 0x0c yields a zero byte)
        const uint32_t sel = (uint32_t)j | 0x0c00u | ((uint32_t)(4 + j) << 16) | 0x0c000000u;
        const uint32_t t = __builtin_amdgcn_perm(w1, w0, sel);
        lo[j] = (t & M) | CL;
        hi[j] = ((t >> 4) & M) | CH;
    }
}

// The same INT8 words as one operand: each byte u (0..255) converted to fp32 and packed
// to bf16, exact (bf16 holds every integer up to 256), pairs in the K order of dq4.  One
// MFMA per 8 codes with OFF = 128 (q = u - 128), at 12 VALU instructions.
__device__ __forceinline__ u32x4_t dq8_cvt(uint32_t w0, uint32_t w1) {
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        r[j] = cvt_bf16x2((float)((w0 >> (8 * j)) & 0xffu), (float)((w1 >> (8 * j)) & 0xffu));
    return r;
}

// ------------------------------------------------- other code formats
//
// A code format CF is a template constant: 4 and 8 are the INT4 / INT8 group-128 RTN
// codes above; kCfFp8 is FP8 E4M3 with one fp32 scale per output row; kCfMx4 is MXFP4,
// E2M1 codes with one E8M0 (power-of-two) scale per 32 columns.  Both dequantise to
// exact bf16 through the gfx950 conversions, so they need no offset seed; FP8's row scale
// multiplies the fp32 partials like a group scale, MXFP4's block scale is applied inside
// the conversion (a power of two: exact).
constexpr int kCfFp8 = 0x18, kCfMx4 = 0x24;
constexpr int cf_bits(int cf) { return cf & 0xF; }
constexpr bool cf_int(int cf) { return cf == 4 || cf == 8; }
// w4a16 weight_format values (0 INT, 1 FP8, 2 MXFP4) and the code format of each
constexpr int cf_of(int fmt, int bits) { return fmt == 1 ? kCfFp8 : fmt == 2 ? kCfMx4 : bits; }

// FP8 words w0 = k0..k3, w1 = k4..k7 (one E4M3 byte each) -> bf16 pairs in the K order
// of dq4: (k0,k4) (k1,k5) (k2,k6) (k3,k7).  Exact (E4M3 is a subset of bf16).
__device__ __forceinline__ u32x4_t dq_fp8(uint32_t w0, uint32_t w1) {
    const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);   // w0.b0 w1.b0 w0.b1 w1.b1
    const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);   // w0.b2 w1.b2 w0.b3 w1.b3
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t0, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t0, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t1, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t1, 1.0f, true));
    return r;
}

// MXFP4 word w = k0..k7 (one E2M1 nibble each, k0 lowest) -> bf16 pairs (k0,k4) (k1,k5)
// (k2,k6) (k3,k7), each value times `scale` (a power of two: exact).  Byte j of w holds
// k_2j (low nibble) and k_2j+1, which one conversion turns into the bf16 pair
// (k_2j, k_2j+1); byte permutes then regroup the halves.
__device__ __forceinline__ u32x4_t dq_mx4(uint32_t w, float scale) {
    const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    const uint32_t p45 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    const uint32_t p67 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    u32x4_t r;
    r[0] = __builtin_amdgcn_perm(p45, p01, 0x05040100u);   // k0 k4: low halves
    r[1] = __builtin_amdgcn_perm(p45, p01, 0x07060302u);   // k1 k5: high halves
    r[2] = __builtin_amdgcn_perm(p67, p23, 0x05040100u);   // k2 k6
    r[3] = __builtin_amdgcn_perm(p67, p23, 0x07060302u);   // k3 k7
    return r;
}

// The power of two 2^(code - 127) of an E8M0 scale code (code 0: 0, outside the range the
// quantizer produces for nonzero blocks).
__device__ __forceinline__ float e8m0_scale(uint32_t code) { return __uint_as_float((code & 0xffu) << 23); }

// Reorder eight natural-order bf16 activations X = (x0,x1)(x2,x3)(x4,x5)(x6,x7) to the
// K order of the weight operands: (x0,x4) (x1,x5) (x2,x6) (x3,x7).  Within each block
// of 8 columns, logical column j sits at position 2*(j % 4) + j / 4.
__device__ __forceinline__ u32x4_t perm_act(u32x4_t X) {
    u32x4_t a;
    a[0] = (X[0] & 0xffffu) | (X[2] << 16);
    a[1] = (X[0] >> 16) | (X[2] & 0xffff0000u);
    a[2] = (X[1] & 0xffffu) | (X[3] << 16);
    a[3] = (X[1] >> 16) | (X[3] & 0xffff0000u);
    return a;
}
__device__ __forceinline__ int perm_pos(int j) { return (j & ~7) | ((j & 3) << 1) | ((j >> 2) & 1); }

// Guarded 16-byte load without a branch: reads `p` when `ok`, otherwise reads `fallback`
// (any valid address) and returns zeros.  A load inside a divergent branch makes the
// compiler wait for every outstanding load at that point, which serialises independent
// HBM requests; this form keeps all loads of a pass in flight together.
__device__ __forceinline__ u32x4_t load16_or_zero(const void* p, bool ok, const void* fallback) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ok ? p : fallback);
    const uint32_t m = ok ? 0xffffffffu : 0u;
    return u32x4_t{v[0] & m, v[1] & m, v[2] & m, v[3] & m};
}

// 16 bytes of a weight stream that is read once: a non-temporal load, so the streamed
// codes do not push reusable lines (activations, routing data, kernel code) out of L2.
__device__ __forceinline__ u32x4_t load_stream16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Raw buffer resource over `bytes` bytes at p (gfx9-family descriptor word 3).  Buffer
// loads take a per-lane 32-bit offset plus a scalar offset, so loop-varying parts of an
// address cost no vector instructions; reads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}

// Cache-policy operand of buffer loads and stores: sc1 = device-coherent access (a store
// writes through to memory, a load reads past the XCD's L2), for data exchanged between
// workgroups of one launch.
constexpr int kSc1 = 16;

// bf16 pair of -OFF (see above): -136 = 0xC308, -2304 = 0xC510.
template <int BITS>
__device__ __forceinline__ u32x4_t neg_offset_operand() {
    const uint32_t v = BITS == 4 ? 0xC308C308u : 0xC510C510u;
    u32x4_t r = {v, v, v, v};
    return r;
}

// SiLU(g) * u = g / (1 + e^-g) * u, with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// ------------------------------------------------------------ workspace layout

// Head of every workspace: the state of the single-launch tiny-batch path, kept across
// calls.  It must be zero before a workspace's first use (moe_w4a16_workspace_init).
// kSyncBytes of counters, one per 128-byte line (index * 32 words): [80, 96) exit counts
// of down-workgroup groups and 100 their total (zero between calls), 101 a sticky error
// word (a wait that timed out), 102 the epoch word (epoch - 1 of the next call), 103 the
// arrivals of the split routing kernel's workgroups (zero between calls).  Then
// kTagBytes of tagged a words (bf16 value | epoch << 16), rows of width max(I, shared I).
constexpr size_t kSyncBytes = 16384;
constexpr size_t kTagBytes = 131072;
constexpr size_t kHeadBytes = kSyncBytes + kTagBytes;
static_assert(kHeadBytes == W4A16_WORKSPACE_HEAD_BYTES, "workspace head size");
constexpr int kSyncGroup = 80, kSyncTop = 100, kSyncError = 101, kSyncEpoch = 102, kSyncRoute = 103;
static_assert(kSyncError * 32 * 4 == W4A16_WORKSPACE_ERROR_OFFSET, "time-out word offset");
__device__ __forceinline__ uint32_t* sync_word(uint32_t* sync, int i) { return sync + i * 32; }

struct WsLayout {
    size_t sync, ids, wts, counts, offsets, sorted, active, meta, hist, lrank, tiles, xsum, abuf, part,
        ystage, inv, asum, tokw, rec, trec, xp, logits, gate, total;
    int64_t rows_a;     // rows of the gate/up output buffer (routed pairs + shared tokens)
    int64_t width_a;    // columns of that buffer: max(I, shared_I)
    int nblk;           // routing blocks of the large-batch path
    int splits;         // expert splits of the small-batch down kernel
    int64_t max_tiles;  // M-tiles of the large-batch grouped GEMM
};

constexpr int kSmallT = 64;      // batches up to this size take the small-batch path
constexpr int kSplitRouteT = 24;  // above this many tokens (from logits, not pair mode) routing takes its own launch
constexpr int kPairP = 64;       // T * k up to this may take the pair-mapped gate/up (pair < 2^kRecTokBits)
// A small-path slot record carries its expert's first kRecTokens tokens (ascending,
// kRecTokBits bits each) so gate/up can fetch activations without reading the row list.
constexpr int kRecTokBits = 6;
constexpr int kRecTokens = 5;
static_assert(kSmallT <= (1 << kRecTokBits) && kPairP <= (1 << kRecTokBits) && kRecTokens * kRecTokBits <= 31 && 16 * kRecTokBits <= 96,
              "record token packing");
constexpr int kTinyP = 16;       // T * k up to this (and H <= kTinyMaxH) take the single-launch path
constexpr int kTinyMaxH = 4096;
constexpr size_t kTinyMaxLds = 64 * 1024;   // LDS of a single-launch down workgroup at most
constexpr int kTinyPad = 8;   // bf16 padding of an a row staged in LDS: 16 rows start in 16 different bank quads
constexpr int kRouteBlockT = 32; // tokens per routing block on the large-batch path
constexpr int kPrefillMT = 128;  // tokens per M-tile of the large-batch grouped GEMM

// ------------------------------------------------------------- stage timer

// Optional per-kernel timing.  Launchers enqueue every kernel through launch(); with a
// timer, the kernel goes out by hipExtLaunchKernelGGL with a start and a stop event bound
// to its own dispatch, so the elapsed time between them is the kernel's execution (no
// marker packets between kernels, no dispatch gap counted).
constexpr int kMaxStages = 16;
struct StageTimer {
    hipEvent_t beg[kMaxStages], end[kMaxStages];
    const char* name[kMaxStages];
    int n;
};

template <typename... KArgs, typename... Args>
inline void launch(StageTimer* t, const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                   hipStream_t s, uint32_t shmem, Args... args) {
    if (t && t->n < kMaxStages) {
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, t->beg[t->n], t->end[t->n], 0, args...);
        t->name[t->n++] = name;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
    }
}

// ----------------------------------------------------------- kernel launchers
// Each returns hipGetLastError() after the launch.

hipError_t launch_quantize(const void* w, bool bf16_in, int64_t total_rows, int64_t cols, int bits,
                           int32_t* packed, uint16_t* scales, hipStream_t s);
// FP8 E4M3 with one fp32 scale per row; MXFP4 with one E8M0 scale per 32 columns (mse:
// the scale-exponent search, else round-to-nearest exponents).
hipError_t launch_fp8_quantize(const void* w, bool bf16_in, int64_t total_rows, int64_t cols, int32_t* packed,
                               float* scales, hipStream_t s);
hipError_t launch_mxfp4_quantize(const void* w, bool bf16_in, int64_t total_rows, int64_t cols, bool mse,
                                 int32_t* packed, uint8_t* scales, hipStream_t s);

struct RouteArgs {
    const float* logits;  // NULL: ids/wts are inputs
    int T, E, k;
    int32_t* ids;
    float* wts;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* active;
    int32_t* meta;        // [0] active experts, [1] M-tiles (routed)
    int32_t* hist;        // large path: [E, nblk] per-block counts, then first ranks
    int32_t* lrank;       // large path: [T*k]
    int32_t* tiles;       // large path: [max_tiles, 2] (expert, first row)
    const uint16_t* x;    // large path: activations for the group sums
    float* xsum;          // large path: [T, H/128] sums of bf16 activations per group
    uint16_t* xp;         // large path: [T, H] activations with each 8-column block reordered
    int2* tokw;           // [T*k] (token, weight bits) of each pair, in sorted order
    int32_t* inv;         // [T*k] sorted position of each pair, -1 when dropped
    int4* rec;            // small path: [max_slots] (expert, first sorted row, count, first tokens);
                          // count 0 marks a slot beyond the active experts
    int4* trec;           // small path: [max_slots + T*k/16][2] M-tiles of <= 16 rows: (expert,
                          // first sorted row, count, 0), (96 bits of tokens: m at bit 6m, 0)
    int pair_rows;        // 1 (T*k <= kPairP): trec's 96 bits hold each row's pair t*k + j, not its token
    uint32_t* sync;       // workspace head counters (route_split_kernel's arrivals)
    int max_slots;
    int64_t H;
    int nblk;
    int64_t max_tiles;
};
hipError_t launch_route_small(const RouteArgs& a, hipStream_t s, StageTimer* t = nullptr);
// Small batch from logits over ceil(T / 8) workgroups, one token per wave (see route.hip).
hipError_t launch_route_split(const RouteArgs& a, hipStream_t s, StageTimer* t = nullptr);
hipError_t launch_route_large(const RouteArgs& a, hipStream_t s, StageTimer* t = nullptr);

// Router logits (rows [0, n_router) of the right operand) and the shared-expert gate (row
// n_router when wg is given, through the sigmoid) of every token: a bf16 product on MFMA.
struct RouterArgs {
    const uint16_t* x;    // bf16 [T, H]
    const uint16_t* wr;   // bf16 [n_router, H] (n_router 0: none)
    const uint16_t* wg;   // bf16 [H] or NULL
    int T, n_router;
    int64_t H;
    float* logits;        // [T, n_router]
    float* gate;          // [T]
};
constexpr int kRouterSmallT = 256;   // up to this many tokens: split-K workgroups per (16 tokens, 16 rows)
hipError_t launch_router(const RouterArgs& a, hipStream_t s, StageTimer* t = nullptr);

struct ExpertSet {       // one family of experts sharing a code format
    const int32_t* w13;
    const uint16_t* s13;     // scales: bf16 [.., G] (INT), fp32 [..] (FP8) or E8M0 bytes [.., K/32] (MXFP4)
    const int32_t* w2;
    const uint16_t* s2;
    int64_t I;
    int bits;                // code width: 4 or 8 (FP8: 8, MXFP4: 4)
    int fmt;                 // 0 INT (RTN group 128), 1 FP8 E4M3 per row, 2 MXFP4
};

struct DecodeArgs {
    const uint16_t* x;
    int T, E, k;
    int64_t H;
    ExpertSet routed, shared;   // shared.bits == 0: none
    const int32_t* ids;
    const float* wts;
    const int32_t* offsets;
    const int32_t* sorted;
    const int32_t* active;
    const int32_t* meta;
    const int4* rec;            // per active-expert slot: (expert, first sorted row, count, first tokens)
    const int4* trec;           // per routed M-tile: two int4 (see RouteArgs::trec)
    const int2* tokw;           // per sorted row: (token, weight bits)
    uint16_t* abuf;             // [rows_a, width_a]
    int64_t width_a;
    float* part;                // [splits, T, H]
    int splits;
    const int32_t* inv;         // [T*k] sorted position of each pair (-1: dropped)
    float* ystage;              // [rows_a, H] unweighted down-projection rows (streaming path)
    int64_t rows_a;             // rows of abuf and ystage: T * k routed, then T shared
    const uint16_t* residual;
    const float* shared_gate;   // [T] weight of each token's shared-expert row, or NULL: 1
    uint16_t* y;
    int gk_stream;              // 1: gate/up by the streaming kernel (stream_fits), else one workgroup per tile
    int fused_route;            // 1: the streaming gate/up kernel routes the batch itself
    int a_by_pair;              // 1: pair mode (pair_fits); routed a rows lie in pair order (row t*k + j)
    RouteArgs route;            // ... with these outputs (workgroup 0 of either kernel writes them)
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, StageTimer* t = nullptr);
// Workgroups of the streaming gate/up kernel (one per CU of the current device, 0 when
// unknown) and whether it can take a batch of these shapes (H <= 2048 and a bounded
// number of M-tiles per workgroup); otherwise launch_decode uses one workgroup per tile.
int stream_workgroups();
bool stream_fits(const DecodeArgs& a, int max_tiles);
hipError_t launch_gk_stream(const DecodeArgs& a, hipStream_t s, StageTimer* t = nullptr);
// The streaming down projection (intermediate sizes up to 512) and the kernel that sums
// each token's rows in slot order; otherwise launch_decode splits experts over workgroups.
bool dk_stream_fits(const DecodeArgs& a);
// Pair mode of the streaming gate/up (T * k <= kPairP, at least twice as many experts as
// pairs): its routed tiles are the pairs themselves, each workgroup finds the experts of
// its own pairs with a top-k that stops at their ranks, and workgroup 0 routes the batch.
bool pair_fits(const DecodeArgs& a);
hipError_t launch_dk_stream(const DecodeArgs& a, hipStream_t s, StageTimer* t = nullptr);

// Single-launch path for tiny batches (T * k <= kTinyP): every workgroup routes the batch
// itself; workgroups [0, H / 16) compute 16 output rows of the down projection each, from
// a values they read back as soon as every word carries this launch's epoch; the n_gk
// workgroups after them compute gate/up row blocks of one (token, rank) pair each, or of
// the shared expert, and write those tagged words.
struct TinyArgs {
    const uint16_t* x;
    int T, E, k;
    int64_t H;
    ExpertSet routed, shared;
    const float* logits;        // NULL: ids / wts are inputs
    int32_t* ids;               // [T, k]
    float* wts;                 // [T, k]
    int32_t* counts;            // [E] out
    int32_t* offsets;           // [E + 1] out
    int32_t* sorted;            // [T * k] out
    uint32_t* sync;             // workspace head: counters (kSyncBytes) ...
    uint32_t* tags;             // ... then tagged a words [rows_a, width_a] (tag_bytes <= kTagBytes)
    int64_t width_a;
    int rows_a;                 // T * k routed rows, then T shared rows
    uint32_t tag_bytes;
    const uint16_t* residual;
    const float* shared_gate;   // [T] weight of each token's shared-expert row, or NULL: 1
    uint16_t* y;
    int n_gk;                   // gate/up workgroups: (T * k pairs + shared) * n_rb
    int n_rb;                   // 16-row blocks per slot: max(I, shared I) / 16
    uint32_t lds_bytes;         // dynamic LDS per workgroup
};
hipError_t launch_tiny(const TinyArgs& a, hipStream_t s, StageTimer* t = nullptr);
// Down workgroups the single-launch path may use on the current device: half of the
// workgroups of its kernel that the device holds at once (0 when unknown).
int tiny_max_down_workgroups(int fmt, int bits, int sbits);
hipError_t launch_head_init(uint32_t* head, hipStream_t s);

struct PrefillArgs {
    const uint16_t* x;
    int T, E, k;
    int64_t H;
    ExpertSet routed, shared;
    const int32_t* ids;
    const float* wts;
    const int32_t* offsets;
    const int32_t* sorted;
    const int32_t* meta;
    const int32_t* tiles;
    const int2* tokw;
    int64_t max_tiles;
    const float* xsum;
    const uint16_t* xp;
    uint16_t* abuf;
    int64_t rows_a;
    int64_t width_a;
    float* asum;                // [rows_a, width_a / 128] fp32: sum of each a row over each group
    uint16_t* ystage;           // [rows_a, H] bf16: down output of each sorted row (unweighted)
    const int32_t* inv;         // [T*k] sorted position of each pair (-1: dropped)
    const uint16_t* residual;
    const float* shared_gate;   // [T] weight of each token's shared-expert row, or NULL: 1
    uint16_t* y;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, StageTimer* t = nullptr);

// The down-projection kernels alone, for a dense projection run as one expert of weight 1
// over all tokens: the small-batch kernel (dk_decode, + dk_combine) or the grouped GEMM,
// whose epilogue then writes y = bf16(row + residual) itself (rows are tokens).
hipError_t launch_down_decode(const DecodeArgs& a, hipStream_t s, StageTimer* t = nullptr);
hipError_t launch_down_prefill(const PrefillArgs& a, hipStream_t s, StageTimer* t = nullptr);

// Set-up of a dense projection on those kernels: x in the codes' K order (abuf), each
// row's fp32 group sums (asum; large batches), and the routing records of one expert that
// every token uses with weight 1 (rec, meta, tokw, offsets, tiles, wts, inv).
struct LinearPrep {
    const uint16_t* x;   // bf16 [T, K]
    int T;
    int64_t K;
    uint16_t* abuf;      // [T, K], or NULL: not written (8-bit codes, whose GEMM reads x itself)
    float* asum;         // [T, K / 128] or NULL
    int4* rec;           // [1]
    int32_t* meta;       // [2]: active experts, M-tiles
    int2* tokw;          // [T]
    int32_t* offsets;    // [2]
    int32_t* tiles;      // [ceil(T / 128), 2]
    float* wts;          // [T]
    int32_t* inv;        // [T]
};
hipError_t launch_linear_prep(const LinearPrep& p, hipStream_t s, StageTimer* t = nullptr);

// Small-batch dense projection y[T, N] = x[T, K] . W^T (+ residual), T <= kSmallT, in one
// launch with no workspace: N / (16 rb) workgroups of K / (128 gw) waves, each wave a range
// of gw 128-column groups of rb 16-row blocks (configuration cfg = gw | rb << 4, from
// linear_small_cfg).
struct LinearSmall {
    const uint16_t* x;          // bf16 [T, K]
    const int32_t* w;           // codes [N, K * bits / 32]
    const uint8_t* s;           // scales (INT bf16 [N, K/128]; FP8 fp32 [N]; MXFP4 E8M0 [N, K/32])
    const uint16_t* residual;   // bf16 [T, N] or NULL (may alias y)
    uint16_t* y;                // bf16 [T, N]
    int T;
    int64_t K, N;
};
// Configuration of the small-batch dense kernel, 0 when the shape does not fit it.
int linear_small_cfg(int64_t T, int64_t K, int64_t N, int bits);
hipError_t launch_linear_small(const LinearSmall& p, int cf, int cfg, hipStream_t s, StageTimer* t = nullptr);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace w4a16
