// Gate/up projection of the small-batch path (2 < T <= 64 tokens) as one persistent
// stream per CU.
//
// Work is a flat list of items: (M-tile of <= 16 rows of one expert, 16-row block of its
// gate/up bank, 8-group K chunk) for the routed tiles, then the shared expert's tiles of 16
// tokens.  The routed tiles come from the routing kernel's tile records, or from the batch
// routed again by every workgroup (fused_route), or, in pair mode, are the (token, rank)
// pairs themselves: one row each, whose experts each workgroup finds for its own range
// with a top-k that stops at the pair's rank (workgroup 0 then only routes the batch for
// the down kernels).  A 4-bit item carries the 16 gate rows and the 16 up rows of its K
// chunk, an 8-bit item one of the two halves; either way 16 KiB of codes.  Each workgroup
// (one per CU) walks a contiguous range of the list, so an M-tile's activations are
// fetched once and serve every row block of its expert.
//
// Every item's codes and scales reach LDS by direct-to-LDS buffer loads into a ring of
// kSStages stages: while item s computes, items s+1 .. s+kSStages-2 are in flight, which
// keeps about 85 KiB of weights in flight per CU without spending registers on them.  A
// tile's activation rows (at most kSARows of them) are copied the same way, together with
// the tile's first item, into one of two LDS buffers, and moved into registers when that
// item computes; larger tiles (rare at decode) load their rows straight into registers.
//
// Within an item, wave w computes K group 8 * kh + w of the item's rows with 16x16x32 bf16
// MFMAs (INT codes as exact bf16 integers, offset removed by the seed, see dq4 / dq8 in
// common.h; FP8 and MXFP4 codes as their exact bf16 values, see dq_fp8 / dq_mx4); the
// fp32 partial sums of the 8 waves meet in LDS after the row block's last K chunk, and
// the epilogue stores a = SiLU(g) * u as bf16 in MFMA operand order.  The code bytes of
// an item are laid out alike for every format of one width; only the scale copies differ.
#include "common.h"
#include "decode_dev.h"
#include "dma.h"
#include "route_small.h"

namespace w4a16 {

namespace {

constexpr int kSWaves = 8;                         // compute waves
constexpr int kSIssuers = 2;                       // producer waves: they only issue the copies
constexpr int kSThreads = 64 * (kSWaves + kSIssuers);
constexpr int kSStages = 6;
constexpr int kSCodeBytes = 16384;                 // one item: 16 blocks of 64 lanes x 16 B
constexpr int kSStageBytes = kSCodeBytes + 1024;   // + one block of scales
constexpr int kSARows = 4;                         // activation rows an A buffer holds
constexpr int kSARowBytes = 4096 + 16;             // one row (H <= 2048), padded against bank conflicts
constexpr int kSABytes = kSARows * kSARowBytes;
constexpr int kSMaxTiles = 8;                      // routed M-tiles one workgroup's range may touch
constexpr int kSMaxH = 2048;
constexpr int kSKH = kSMaxH / kGroup / 8;          // 8-group K chunks at the largest H: 2
// dynamic LDS: stages | two A buffers | zero block | partial sums | tile records
constexpr int kSOffA = kSStages * kSStageBytes;
constexpr int kSOffZero = kSOffA + 2 * kSABytes;
constexpr int kSOffRed = kSOffZero + 1024;
constexpr int kSOffTiles = kSOffRed + kSWaves * 8 * 64 * 4;
constexpr int kSLdsBytes = kSOffTiles + kSMaxTiles * 32;
static_assert(kSLdsBytes <= 160 * 1024, "streaming gate/up LDS");

// One M-tile: expert, first row of the a buffer, rows, and how to find each row's token.
struct STile {
    int e;          // expert (routed)
    int row0;       // first row in the a buffer
    int count;      // rows (1..16)
    int shared;     // 1: the shared expert, token of row m is tbase + m
    int tbase;
    uint32_t tk0, tk1, tk2;   // routed: token m in bits [6m, 6m + 6) of tk2:tk1:tk0
};

__device__ __forceinline__ int stile_token(const STile& t, int m) {
    if (t.shared) return t.tbase + m;
    // one 96-bit shift (no indexed array: that would live in scratch memory, and a scratch
    // load makes the compiler wait for every copy in flight)
    const unsigned __int128 v = (unsigned __int128)t.tk0 | ((unsigned __int128)t.tk1 << 32) |
                                ((unsigned __int128)t.tk2 << 64);
    return (int)(uint32_t)(v >> (kRecTokBits * m)) & ((1 << kRecTokBits) - 1);
}

struct SLayout {    // per-launch constants, wave-uniform
    int G, T, Tk;
    int n_rb_r, n_rb_s, sub_r, sub_s, n_tiles_r;
    int t_lo;       // first routed tile of this workgroup's range
};

// A position in the item list: tile, row block, K chunk.  Advanced one item at a time
// with compares only (the scalar unit is the scarce resource of this loop: one per CU,
// shared by its eight waves), and the current tile's record kept at hand.
struct SCursor {
    int tile;       // global tile id: routed tiles first, then shared tiles
    int rb, sub;    // row block; K chunk (4-bit) or K chunk * 2 + half (8-bit)
    int n_rb, n_sub, bits;
    STile tl;
};

template <int BITS, int SBITS>
__device__ __forceinline__ void s_set_tile(SCursor& c, const SLayout& L, const int* s_tiles) {
    const bool shared = c.tile >= L.n_tiles_r;
    c.n_rb = shared ? L.n_rb_s : L.n_rb_r;
    c.n_sub = shared ? L.sub_s : L.sub_r;
    c.bits = shared ? SBITS : BITS;
    if (!shared) {
        // (a cursor stepping past the range end lands on a record it never uses)
        const int* r = s_tiles + 8 * min(c.tile - L.t_lo, kSMaxTiles - 1);
        c.tl.e = __builtin_amdgcn_readfirstlane(r[0]);   // wave-uniform: keep it in scalar registers
        c.tl.row0 = __builtin_amdgcn_readfirstlane(r[1]);
        c.tl.count = __builtin_amdgcn_readfirstlane(r[2]);
        c.tl.tk0 = __builtin_amdgcn_readfirstlane(r[4]);
        c.tl.tk1 = __builtin_amdgcn_readfirstlane(r[5]);
        c.tl.tk2 = __builtin_amdgcn_readfirstlane(r[6]);
        c.tl.shared = 0;
        c.tl.tbase = 0;
    } else {
        const int ts = c.tile - L.n_tiles_r;
        c.tl.e = 0;
        c.tl.tbase = 16 * ts;
        c.tl.row0 = L.Tk + 16 * ts;
        c.tl.count = min(16, L.T - 16 * ts);
        c.tl.shared = 1;
        c.tl.tk0 = c.tl.tk1 = c.tl.tk2 = 0u;
    }
}

// Every field is wave-uniform; saying so keeps the cursor in scalar registers and its
// tests as scalar branches (the compiler cannot prove it through the loop).
__device__ __forceinline__ void s_uniform(SCursor& c) {
    c.tile = __builtin_amdgcn_readfirstlane(c.tile);
    c.rb = __builtin_amdgcn_readfirstlane(c.rb);
    c.sub = __builtin_amdgcn_readfirstlane(c.sub);
    c.n_rb = __builtin_amdgcn_readfirstlane(c.n_rb);
    c.n_sub = __builtin_amdgcn_readfirstlane(c.n_sub);
    c.bits = __builtin_amdgcn_readfirstlane(c.bits);
    c.tl.e = __builtin_amdgcn_readfirstlane(c.tl.e);
    c.tl.row0 = __builtin_amdgcn_readfirstlane(c.tl.row0);
    c.tl.count = __builtin_amdgcn_readfirstlane(c.tl.count);
    c.tl.shared = __builtin_amdgcn_readfirstlane(c.tl.shared);
    c.tl.tbase = __builtin_amdgcn_readfirstlane(c.tl.tbase);
    c.tl.tk0 = __builtin_amdgcn_readfirstlane(c.tl.tk0);
    c.tl.tk1 = __builtin_amdgcn_readfirstlane(c.tl.tk1);
    c.tl.tk2 = __builtin_amdgcn_readfirstlane(c.tl.tk2);
}

// Moves to the next item; true when it starts a new tile.
template <int BITS, int SBITS>
__device__ __forceinline__ bool s_advance(SCursor& c, const SLayout& L, const int* s_tiles) {
    bool start = false;
    if (++c.sub >= c.n_sub) {
        c.sub = 0;
        if (++c.rb >= c.n_rb) {
            c.rb = 0;
            ++c.tile;
            s_set_tile<BITS, SBITS>(c, L, s_tiles);
            start = true;
        }
    }
    s_uniform(c);
    return start;
}

// What the issuing side keeps per tile: buffer descriptors and this lane's offsets.
struct SIssueTile {
    i32x4_t wr, sr;        // codes and scales of the tile's expert
    int64_t I_e, row_bytes;
    int fmt;               // the expert's code format (0 INT, 1 FP8, 2 MXFP4): its scale layout
    uint32_t v_code;       // lane part of a code copy offset
    uint32_t v_scale;      // lane part of the scale copy offset (kOob: idle lane)
};

__device__ __forceinline__ void s_issue_tile(const DecodeArgs& a, const SLayout& L, const SCursor& c,
                                             SIssueTile& st) {
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const ExpertSet& es = c.tl.shared ? a.shared : a.routed;
    st.I_e = es.I;
    st.row_bytes = a.H * c.bits / 8;
    const int64_t e = c.tl.e;
    st.wr = uniform_rsrc(dma_rsrc(reinterpret_cast<const uint8_t*>(es.w13) + e * 2 * st.I_e * st.row_bytes,
                                  (uint32_t)(2 * st.I_e * st.row_bytes)));
    st.fmt = es.fmt;
    // scale bytes of one gate/up row: INT bf16 per group, FP8 one fp32, MXFP4 one E8M0 byte
    // per 32 columns
    const int64_t srow = es.fmt == 1 ? 4 : es.fmt == 2 ? 4 * L.G : 2 * L.G;
    st.sr = uniform_rsrc(dma_rsrc(reinterpret_cast<const uint8_t*>(es.s13) + e * 2 * st.I_e * srow,
                                  (uint32_t)(2 * st.I_e * srow)));
    st.v_code = (uint32_t)(ml * st.row_bytes + q * (c.bits == 4 ? 16 : 32));
    if (es.fmt == 1)        // the 16 rows' fp32 scales: 64 contiguous bytes
        st.v_scale = lane < 4 ? (uint32_t)(lane * 16) : kOob;
    else if (es.fmt == 2)   // 32 bytes (8 groups x 4 blocks) of each of the 32 gate and up rows
        st.v_scale = (uint32_t)((((lane >> 5) * st.I_e + ((lane >> 1) & 15)) * L.G) * 4 + (lane & 1) * 16);
    else if (c.bits == 4)   // 16 bytes (8 groups) of each of the 32 gate and up rows
        st.v_scale = lane < 32 ? (uint32_t)((((lane >> 4) * st.I_e + ml) * L.G) * 2) : kOob;
    else
        st.v_scale = lane < 16 ? (uint32_t)(lane * L.G * 2) : kOob;
}

// Issues producer wave w's copies of the cursor's item into `stage`: code blocks
// 8w .. 8w + 7 (producer 0 also the scales) and, at a tile start whose rows fit an A
// buffer, its share of the tile's activation rows into `abuf_lds`.  Returns the copies
// issued.  The producers do nothing else: an issue stalls while the memory system is
// saturated, and that stall must not hold up the MFMAs (nor should all waves repeat the
// per-item scalar work on the CU's one scalar unit).
__device__ __forceinline__ int s_issue(const DecodeArgs& a, const SLayout& L, const SCursor& c,
                                       const SIssueTile& st, uint32_t stage, bool tile_start, uint32_t abuf_lds) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) - kSWaves);   // producer index
    const int n0 = c.rb * 16;
    const int kh = c.bits == 4 ? c.sub : c.sub >> 1, half = c.bits == 4 ? 0 : c.sub & 1;
    const i32x4_t wr = uniform_rsrc(st.wr);   // in scalar registers whatever the compiler kept
    // groups past the last (a hidden size that is not a multiple of 1024) read other rows
    // or past the buffer (zeros); no wave computes them
    uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + wave * 8 * 1024);
    if (c.bits == 4) {   // blocks 8w + j: half w (gate, up), group 8 kh + j
        int soff = __builtin_amdgcn_readfirstlane((int)((wave * st.I_e + n0) * st.row_bytes) + 8 * kh * 64);
#pragma unroll
        for (int j = 0; j < 8; ++j, soff += 64, m0 += 1024) dma16(wr, m0, st.v_code, soff);
    } else {             // blocks 8w + i: group 8 kh + 4w + i / 2, 16-byte half i % 2
        const int soff =
            __builtin_amdgcn_readfirstlane((int)((half * st.I_e + n0) * st.row_bytes) + (8 * kh + 4 * wave) * 128);
#pragma unroll
        for (int i = 0; i < 8; ++i, m0 += 1024) dma16(wr, m0, st.v_code, soff + (i >> 1) * 128 + (i & 1) * 16);
    }
    int n = 8;
    if (wave == 0) {   // scales of the item's rows and groups
        const int soff = st.fmt == 1   ? (int)((half * st.I_e + n0) * 4)
                         : st.fmt == 2 ? (n0 * L.G + 8 * kh) * 4
                         : c.bits == 4 ? (n0 * L.G + 8 * kh) * 2
                                       : (int)(((half * st.I_e + n0) * L.G + 8 * kh) * 2);
        dma16(uniform_rsrc(st.sr), __builtin_amdgcn_readfirstlane(stage + kSCodeBytes), st.v_scale,
              __builtin_amdgcn_readfirstlane(soff));
        ++n;
    }
    if (tile_start && c.tl.count <= kSARows) {   // the tile's activation rows, 1 KiB per copy
        const int row_b = (int)(a.H * 2);
        const int cpr = (row_b + 1023) / 1024;
        const int n_dma = c.tl.count * cpr;
        const i32x4_t xr = uniform_rsrc(dma_rsrc(a.x, (uint32_t)((int64_t)a.T * row_b)));
        for (int d = wave; d < n_dma; d += kSIssuers) {
            const int r = d / cpr, cc = d - r * cpr;
            const int b = cc * 1024 + lane * 16;
            const uint32_t off = b < row_b ? (uint32_t)(stile_token(c.tl, r) * row_b + b) : kOob;
            dma16(xr, __builtin_amdgcn_readfirstlane(abuf_lds + r * kSARowBytes + cc * 1024), off, 0);
            ++n;
        }
    }
    return n;
}

// This wave's activation fragments of K groups w and w + 8 for the tile's 16 rows
// (padding rows zero), and their MFMA offset seeds.  Each branch computes the seeds
// itself: the register path's loads are then complete before the branches join, so the
// compiler puts no wait for them (a wait for every copy in flight) on the LDS path.
// The seed of an item's MFMA chains: the INT offset seed; for the float formats (no
// offset) zero, computed by the same four MFMAs on a zero operand so that, as with the INT
// codes, the fragments' loads are read inside the branch that issued them (the compiler
// then puts no wait for every memory access in flight into each item's MFMAs).
template <int CF>
__device__ __forceinline__ f32x4_t s_seed(const u32x4_t (&A)[4]) {
    if constexpr (cf_int(CF)) {
        return offset_seed<CF>(A);
    } else {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) c = mfma16(A[i], u32x4_t{0u, 0u, 0u, 0u}, c);
        return c;
    }
}

template <int CF>
__device__ __forceinline__ void s_load_a(const DecodeArgs& a, const SLayout& L, const STile& tl, const uint8_t* smem,
                                         const uint8_t* abuf, u32x4_t (&A)[kSKH][4], f32x4_t (&seed)[kSKH]) {
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool real = ml < tl.count;
    if (tl.count <= kSARows) {
        const uint8_t* row = abuf + ml * kSARowBytes + 64 * q;
        const uint8_t* zl = smem + kSOffZero + 16 * lane;
#pragma unroll
        for (int kh = 0; kh < kSKH; ++kh) {
            const int g = 8 * kh + wave;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint8_t* p = (real && g < L.G) ? row + g * 256 + 16 * i : zl;
                A[kh][i] = perm_act(*reinterpret_cast<const u32x4_t*>(p));
            }
        }
#pragma unroll
        for (int kh = 0; kh < kSKH; ++kh) seed[kh] = s_seed<CF>(A[kh]);
    } else {   // more rows than an A buffer holds: straight from memory into registers
        const uint16_t* xr = a.x + (int64_t)stile_token(tl, real ? ml : 0) * a.H + 32 * q;
#pragma unroll
        for (int kh = 0; kh < kSKH; ++kh) {
            const int g = min(8 * kh + wave, L.G - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) A[kh][i] = load_act<CF>(xr, real && 8 * kh + wave < L.G, g * kGroup + 8 * i);
        }
#pragma unroll
        for (int kh = 0; kh < kSKH; ++kh) seed[kh] = s_seed<CF>(A[kh]);
    }
}

// One item's MFMAs for this wave: K group 8 * kh + wave of the item's rows.  Scales in the
// stage: INT 8 bf16 per row (gate rows, then up rows); FP8 the 16 rows' fp32; MXFP4 32
// E8M0 bytes per row (group j's four blocks at 4 j), applied inside the conversion.
template <int CF>
__device__ __forceinline__ void s_compute(const SLayout& L, int kh, int half, const uint8_t* stage,
                                          const u32x4_t (&A)[4], f32x4_t seed, f32x4_t& accg, f32x4_t& accu) {
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (8 * kh + wave >= L.G) return;
    const uint8_t* sb = stage + kSCodeBytes;
    if constexpr (cf_bits(CF) == 4) {
        const u32x4_t bg[1] = {*reinterpret_cast<const u32x4_t*>(stage + wave * 1024 + lane * 16)};
        const u32x4_t bu[1] = {*reinterpret_cast<const u32x4_t*>(stage + (8 + wave) * 1024 + lane * 16)};
        if constexpr (CF == kCfMx4) {
            const float xg = e8m0_scale(sb[ml * 32 + 4 * wave + q]), xu = e8m0_scale(sb[(16 + ml) * 32 + 4 * wave + q]);
            const f32x4_t tg = group_dot<CF>(A, bg, seed, xg);
            const f32x4_t tu = group_dot<CF>(A, bu, seed, xu);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                accg[r] += tg[r];
                accu[r] += tu[r];
            }
        } else {
            const uint16_t* sc = reinterpret_cast<const uint16_t*>(sb);
            const float sg = bf16_to_f32(sc[ml * 8 + wave]), su = bf16_to_f32(sc[(16 + ml) * 8 + wave]);
            const f32x4_t tg = group_dot<CF>(A, bg, seed);
            const f32x4_t tu = group_dot<CF>(A, bu, seed);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                accg[r] += sg * tg[r];
                accu[r] += su * tu[r];
            }
        }
    } else {
        const u32x4_t bw[2] = {*reinterpret_cast<const u32x4_t*>(stage + (2 * wave) * 1024 + lane * 16),
                               *reinterpret_cast<const u32x4_t*>(stage + (2 * wave + 1) * 1024 + lane * 16)};
        const float s = CF == kCfFp8 ? reinterpret_cast<const float*>(sb)[ml]
                                     : bf16_to_f32(reinterpret_cast<const uint16_t*>(sb)[ml * 8 + wave]);
        const float sg = half == 0 ? s : 0.f, su = half == 0 ? 0.f : s;   // selects, no branch
        const f32x4_t t = group_dot<CF>(A, bw, seed);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            accg[r] += sg * t[r];
            accu[r] += su * t[r];
        }
    }
}

// The first unit (row block) of range b of n when ranges are cut by items, rounded up to a
// unit boundary: units [0, U_r) hold sub_r items each, units [U_r, U) sub_s.
__device__ __forceinline__ int s_unit_at(int N_items, int b, int n, int U_r, int U, int sub_r, int sub_s) {
    const int i = (int)((int64_t)N_items * b / n);
    if (i <= U_r * sub_r) return (i + sub_r - 1) / sub_r;
    return min(U, U_r + (i - U_r * sub_r + sub_s - 1) / sub_s);
}

template <int CF, int SBITS>
// One workgroup of ten waves per CU (its LDS ring takes the CU): three waves share a SIMD at most.
__global__ __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(3))) void gk_stream_kernel(
    DecodeArgs a) {
    constexpr int BITS = cf_bits(CF);
    // an INT shared expert beside routed experts of another code format takes its own code
    // path, chosen by the tile; else by the code width
    constexpr bool kSep = SBITS != 0 && SBITS != CF;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, ml = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    SLayout L;
    L.G = (int)(a.H / kGroup);
    const int KH = (L.G + 7) / 8;
    L.T = a.T;
    L.Tk = a.T * a.k;
    L.n_rb_r = (int)(a.routed.I / 16);
    L.n_rb_s = SBITS != 0 ? (int)(a.shared.I / 16) : 0;
    L.sub_r = BITS == 4 ? KH : 2 * KH;
    L.sub_s = SBITS == 4 ? KH : 2 * KH;
    // the batch's routing: done here by every workgroup (in the LDS the ring will reuse,
    // workgroup 0 also writing it out), or read from the routing kernel's outputs
    SmallRouteLds& rl = *reinterpret_cast<SmallRouteLds*>(smem);
    static_assert(sizeof(SmallRouteLds) <= kSOffA, "routing scratch inside the stage ring");
    int wg = blockIdx.x, n_wg = gridDim.x;
    if (a.a_by_pair) {   // workgroup 0 routes the batch for the down kernels; routed tiles are the pairs
        if (blockIdx.x == 0) {
            route_small_wg(a.route, rl, true);
            return;
        }
        --wg;
        --n_wg;
        L.n_tiles_r = L.Tk;
    } else if (a.fused_route) {
        route_small_wg(a.route, rl, blockIdx.x == 0);
        L.n_tiles_r = __builtin_amdgcn_readfirstlane(rl.n_tiles);
    } else {
        L.n_tiles_r = __builtin_amdgcn_readfirstlane(a.meta[1]);
    }
    // ranges are cut between row blocks (units), never inside one: a row block's K chunks
    // are summed in one workgroup's registers
    const int U_r = L.n_tiles_r * L.n_rb_r;
    const int U = U_r + (SBITS != 0 ? ((a.T + 15) / 16) * L.n_rb_s : 0);
    const int N_items = U_r * L.sub_r + (U - U_r) * L.sub_s;
    const int u0 = s_unit_at(N_items, wg, n_wg, U_r, U, L.sub_r, L.sub_s);
    const int u1 = s_unit_at(N_items, wg + 1, n_wg, U_r, U, L.sub_r, L.sub_s);
    const int nI = (min(u1, U_r) - min(u0, U_r)) * L.sub_r + (max(u1, U_r) - max(u0, U_r)) * L.sub_s;
    if (nI <= 0) return;

    // routed tile records of this range into LDS
    int* s_tiles = reinterpret_cast<int*>(smem + kSOffTiles);
    L.t_lo = u0 < U_r ? u0 / L.n_rb_r : L.n_tiles_r;
    const int t_hi = u0 < U_r ? (min(u1, U_r) - 1) / L.n_rb_r : L.n_tiles_r - 1;
    if (t_hi - L.t_lo + 1 > kSMaxTiles) return;   // excluded on the host (stream_fits)
    if (a.a_by_pair) {
        // wave w finds the expert of pair t_lo + w (token p / k, rank p % k) with a top-k that
        // stops at that rank; a dropped pair keeps its items (expert 0's rows, no row written)
        static_assert(kSMaxTiles <= kSWaves + kSIssuers, "one wave per routed tile of a range");
        if (wave <= t_hi - L.t_lo) {
            const int p = L.t_lo + wave, t = p / a.k;
            const int e = pair_expert<false>(a.route.logits, a.route.ids, a.E, a.k, t, p - t * a.k);
            if (lane < 8)
                s_tiles[8 * wave + lane] = lane == 0 ? max(e, 0) : lane == 1 ? p : lane == 2 ? (e >= 0 ? 1 : 0)
                                                                                 : lane == 4 ? t : 0;
        }
    } else if (a.fused_route) {
        if (tid < t_hi - L.t_lo + 1) {
            int4 r0, r1;
            small_tile_record(rl, a.E, L.t_lo + tid, r0, r1);
            reinterpret_cast<int4*>(s_tiles)[2 * tid] = r0;
            reinterpret_cast<int4*>(s_tiles)[2 * tid + 1] = r1;
        }
    } else if (tid < 2 * (t_hi - L.t_lo + 1)) {
        reinterpret_cast<int4*>(s_tiles)[tid] = a.trec[2 * L.t_lo + tid];
    }
    if (tid < 64) *reinterpret_cast<u32x4_t*>(smem + kSOffZero + 16 * tid) = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();

    // two cursors over the range: copies run kSStages - 1 items ahead of the MFMAs
    SCursor ic;
    ic.tile = u0 < U_r ? u0 / L.n_rb_r : L.n_tiles_r + (u0 - U_r) / L.n_rb_s;
    ic.rb = u0 < U_r ? u0 % L.n_rb_r : (u0 - U_r) % L.n_rb_s;
    ic.sub = 0;
    s_set_tile<BITS, SBITS>(ic, L, s_tiles);
    s_uniform(ic);
    SCursor cc = ic;
    const int first_tile = ic.tile;

    const uint32_t lds0 = lds_offset(smem);
    const bool issuer = wave >= kSWaves;
    const int base_ops = wave == kSWaves ? 9 : 8;   // copies per item of a producer wave
    // copies of the two most recent tile starts (by A buffer): relative item, this wave's count
    int a_rel0 = -1, a_cnt0 = 0, a_rel1 = -1, a_cnt1 = 0;
    SIssueTile st;
    s_issue_tile(a, L, ic, st);
    int i_stage = 0;
    bool i_start = true;

    auto issue = [&](int rel) {
        const int b = (ic.tile - first_tile) & 1;
        const int n = __builtin_amdgcn_readfirstlane(
            s_issue(a, L, ic, st, lds0 + i_stage * kSStageBytes, i_start, lds0 + kSOffA + b * kSABytes));
        if (i_start) {
            if (b == 0) { a_rel0 = rel; a_cnt0 = n - base_ops; }
            else { a_rel1 = rel; a_cnt1 = n - base_ops; }
        }
        i_stage = i_stage + 1 == kSStages ? 0 : i_stage + 1;
        i_start = s_advance<BITS, SBITS>(ic, L, s_tiles);
        if (i_start && rel + 1 < nI) s_issue_tile(a, L, ic, st);
    };

    if (issuer) {   // ---- producer waves: copies only, kSStages - 1 items ahead
        for (int rel = 0; rel < kSStages - 1 && rel < nI; ++rel) issue(rel);
        for (int rel = 0; rel < nI; ++rel) {
            // this wave's copies of item rel have landed once only the later items' remain
            const int later = min(nI - 1 - rel, kSStages - 2);
            int n = later * base_ops;
            if (a_rel0 > rel && a_rel0 <= rel + later) n += a_cnt0;
            if (a_rel1 > rel && a_rel1 <= rel + later) n += a_cnt1;
            n = __builtin_amdgcn_readfirstlane(n);
            if (n == (kSStages - 2) * 8) wait_vmcnt<(kSStages - 2) * 8>();
            else if (n == (kSStages - 2) * 9) wait_vmcnt<(kSStages - 2) * 9>();
            else wait_vmcnt_dyn(n);
            bar();   // item rel is in LDS; every compute wave is done with item rel - 1's stage
            if (rel + kSStages - 1 < nI) issue(rel + kSStages - 1);
        }
        bar();   // matches the compute waves' final barrier
        return;
    }

    // ---- compute waves
    u32x4_t A[kSKH][4];
    f32x4_t seed[kSKH];
    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    bool c_start = true;
    int c_stage = 0;
    int ep_row0 = 0, ep_count = 0, ep_n0 = 0, ep_pending = 0;
    float* s_red = reinterpret_cast<float*>(smem + kSOffRed);

    // FP8 / MXFP4 routed codes: the previous row block's epilogue runs after the item's
    // MFMAs rather than before them.  Their items' MFMA blocks carry a wait for all of the
    // wave's memory accesses (vmcnt, which counts the epilogue's stores too), so stores
    // issued right after the barrier held up that item; issued after the MFMAs they are
    // done by the next item.  (Same-box A/B at 32 tokens: FP8 gate/up 76 -> 72.6 us, MXFP4
    // 53.5 -> 50.5 us; INT codes, without that wait, keep the early epilogue.)  A row block
    // spans at least two items (stream_fits), so the epilogue never meets the rewrite of
    // the partial sums it reads.
    constexpr bool kLateEpilogue = !cf_int(CF);
    // waves 4..7: element r = wave - 4 of every lane (D row 4q + r, column ml)
    auto epilogue = [&]() {
        if (wave >= 4) {
            const int r = wave - 4;
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int w = 0; w < kSWaves; ++w) {
                gs += s_red[(w * 8 + r) * 64 + lane];
                us += s_red[(w * 8 + 4 + r) * 64 + lane];
            }
            const int m = 4 * q + r;
            if (m < ep_count)
                a.abuf[(int64_t)(ep_row0 + m) * a.width_a + perm_pos(ep_n0 + ml)] = (uint16_t)cvt_bf16(silu_mul(gs, us));
        }
    };

    for (int rel = 0; rel < nI; ++rel) {
        wait_lgkm0();   // this wave's partial sums are in LDS before the barrier
        bar();          // item rel is in LDS (the producers waited); the partial sums are complete
        if (!kLateEpilogue && ep_pending) {
            epilogue();
            ep_pending = 0;
        }
        const bool sep = kSep && cc.tl.shared;
        if (c_start) {
            const uint8_t* abuf = smem + kSOffA + ((cc.tile - first_tile) & 1) * kSABytes;
            if (!sep) s_load_a<CF>(a, L, cc.tl, smem, abuf, A, seed);
            else if constexpr (kSep) s_load_a<SBITS>(a, L, cc.tl, smem, abuf, A, seed);
        }
        const uint8_t* stage = smem + c_stage * kSStageBytes;
        const int kh = cc.bits == 4 ? cc.sub : cc.sub >> 1, half = cc.bits == 4 ? 0 : cc.sub & 1;
        if (!sep) {
            if (kh == 0) s_compute<CF>(L, kh, half, stage, A[0], seed[0], accg, accu);
            else s_compute<CF>(L, kh, half, stage, A[1], seed[1], accg, accu);
        } else if constexpr (kSep) {
            if (kh == 0) s_compute<SBITS>(L, kh, half, stage, A[0], seed[0], accg, accu);
            else s_compute<SBITS>(L, kh, half, stage, A[1], seed[1], accg, accu);
        }
        if (kLateEpilogue && ep_pending) {
            epilogue();
            ep_pending = 0;
        }
        if (cc.sub == cc.n_sub - 1) {   // the row block's last K chunk
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s_red[(wave * 8 + r) * 64 + lane] = accg[r];
                s_red[(wave * 8 + 4 + r) * 64 + lane] = accu[r];
                accg[r] = 0.f;
                accu[r] = 0.f;
            }
            ep_row0 = cc.tl.row0;
            ep_count = cc.tl.count;
            ep_n0 = cc.rb * 16;
            ep_pending = 1;
        }
        c_stage = c_stage + 1 == kSStages ? 0 : c_stage + 1;
        c_start = s_advance<BITS, SBITS>(cc, L, s_tiles);
    }
    wait_lgkm0();
    bar();
    if (ep_pending) epilogue();
}

// ------------------------------------------------------------ down projection
//
// Items: (M-tile, 16-row block of the output, K half for 8-bit codes).  Every wave streams
// its own contiguous range of items through a private ring of kDStages LDS stages (no
// barriers): per item 4 code blocks of 1 KiB (all K <= 512 of 16 rows for 4-bit codes,
// half of it for 8-bit codes) and the 16 rows' scales.  The M-tile's a rows, stored by
// gate/up in MFMA operand order, stay in registers while the range stays on that tile.
// Each finished row block is written unweighted in fp32 to its sorted rows of ystage;
// dk_finalize_kernel applies the router weights and sums each token's rows in slot order.

// Twelve waves with three stages each (two items in flight per wave, 153 KiB of LDS): the
// same bytes in flight as eight waves of four stages, and more waves to hide the latency
// of each one's chain.  Same-box A/B at 32 tokens: down stream 24.6 -> 23.9 us; fewer,
// deeper rings were slower (6 x 5: 28 us, 4 x 8: 34 us).
constexpr int kDWaves = 12;                        // waves per workgroup, one ring each
constexpr int kDStages = 3;
constexpr int kDCodeBytes = 4096;                  // 4 blocks of 64 lanes x 16 B
constexpr int kDStageBytes = kDCodeBytes + 256;    // + scales (64 lanes x 4 B)
constexpr int kDWaveBytes = kDStages * kDStageBytes;
constexpr int kDLdsBytes = kDWaves * kDWaveBytes;
constexpr int kDMaxI = 512;
constexpr int kDOps = 5;                           // copies per item
constexpr uint32_t kDSkip = 0x40000000u;           // scalar offset that puts a copy past its buffer

struct DCursor {
    int tile, hb, kh;
    int n_kh, bits, fmt, G2;   // fmt: the tile's code format (0 INT, 1 FP8, 2 MXFP4)
    STile tl;
};

__device__ __forceinline__ void d_uniform(DCursor& c) {
    c.tile = __builtin_amdgcn_readfirstlane(c.tile);
    c.hb = __builtin_amdgcn_readfirstlane(c.hb);
    c.kh = __builtin_amdgcn_readfirstlane(c.kh);
    c.n_kh = __builtin_amdgcn_readfirstlane(c.n_kh);
    c.bits = __builtin_amdgcn_readfirstlane(c.bits);
    c.fmt = __builtin_amdgcn_readfirstlane(c.fmt);
    c.G2 = __builtin_amdgcn_readfirstlane(c.G2);
    c.tl.e = __builtin_amdgcn_readfirstlane(c.tl.e);
    c.tl.row0 = __builtin_amdgcn_readfirstlane(c.tl.row0);
    c.tl.count = __builtin_amdgcn_readfirstlane(c.tl.count);
    c.tl.shared = __builtin_amdgcn_readfirstlane(c.tl.shared);
}

template <int BITS, int SBITS>
__device__ __forceinline__ void d_set_tile(const DecodeArgs& a, DCursor& c, int n_tiles_r) {
    const bool shared = c.tile >= n_tiles_r;
    const ExpertSet& es = shared ? a.shared : a.routed;
    c.bits = shared ? SBITS : BITS;
    c.fmt = es.fmt;
    c.G2 = (int)(es.I / kGroup);
    c.n_kh = c.bits == 4 ? 1 : (c.G2 + 1) / 2;
    if (!shared) {
        const int4 r = a.trec[2 * c.tile];
        c.tl.e = r.x;
        c.tl.row0 = r.y;
        c.tl.count = r.z;
        c.tl.shared = 0;
        if (a.a_by_pair) {   // the rows' pair indices (their a rows), 6 bits each
            const int4 r1 = a.trec[2 * c.tile + 1];
            c.tl.tk0 = __builtin_amdgcn_readfirstlane((uint32_t)r1.x);
            c.tl.tk1 = __builtin_amdgcn_readfirstlane((uint32_t)r1.y);
            c.tl.tk2 = __builtin_amdgcn_readfirstlane((uint32_t)r1.z);
        }
    } else {
        const int ts = c.tile - n_tiles_r;
        c.tl.e = 0;
        c.tl.row0 = a.T * a.k + 16 * ts;
        c.tl.count = min(16, a.T - 16 * ts);
        c.tl.shared = 1;
    }
    d_uniform(c);
}

// This wave's copies of the cursor's item into `stage` (kDOps of them).
__device__ __forceinline__ void d_issue(const DecodeArgs& a, const DCursor& c, uint32_t stage) {
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const ExpertSet& es = c.tl.shared ? a.shared : a.routed;
    const int64_t row_bytes = es.I * c.bits / 8;
    const int64_t e = c.tl.e;
    const i32x4_t wr = uniform_rsrc(dma_rsrc(reinterpret_cast<const uint8_t*>(es.w2) + e * a.H * row_bytes,
                                             (uint32_t)(a.H * row_bytes)));
    // scale bytes of one down row: INT bf16 per group, FP8 one fp32, MXFP4 one E8M0 byte per
    // 32 columns; the 16 rows' scales are contiguous (at most 256 bytes, 4 per lane)
    const int srow = c.fmt == 1 ? 4 : c.fmt == 2 ? 4 * c.G2 : 2 * c.G2;
    const i32x4_t sr = uniform_rsrc(dma_rsrc(reinterpret_cast<const uint8_t*>(es.s2) + e * a.H * srow,
                                             (uint32_t)(a.H * srow)));
    const int h0 = c.hb * 16;
    const uint32_t v = (uint32_t)(ml * row_bytes + q * (c.bits == 4 ? 16 : 32));
    const int base = __builtin_amdgcn_readfirstlane((int)(h0 * row_bytes));
#pragma unroll
    for (int b = 0; b < 4; ++b) {   // 4-bit: block b = group b; 8-bit: group 2 kh + b / 2, 16-byte half b % 2
        const int g = c.bits == 4 ? b : 2 * c.kh + (b >> 1);
        const int off = c.bits == 4 ? g * 64 : g * 128 + (b & 1) * 16;
        dma16(wr, stage + b * 1024, v, g < c.G2 ? base + off : (int)kDSkip);
    }
    dma4(sr, stage + kDCodeBytes, lane < 4 * srow ? (uint32_t)(lane * 4) : kOob,
         __builtin_amdgcn_readfirstlane(h0 * srow));
}

// The tile's a rows as MFMA A fragments (groups 0..3, padding rows zero); d_seed gives
// their seeds once they have landed.
__device__ __forceinline__ void d_load_a(const DecodeArgs& a, const DCursor& c, u32x4_t (&A)[4][4]) {
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const bool real = ml < c.tl.count;
    // a rows in sorted order, or (pair-mapped gate/up) routed rows at their pair index
    const int r = !real ? c.tl.row0 : (a.a_by_pair && !c.tl.shared) ? stile_token(c.tl, ml) : c.tl.row0 + ml;
    const uint16_t* row = a.abuf + (int64_t)r * a.width_a + 32 * q;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int gg = min(g, c.G2 - 1);
            A[g][i] = load16_or_zero(row + gg * kGroup + 8 * i, real && g < c.G2, row);
        }
}
template <int CF>
__device__ __forceinline__ void d_seed(const u32x4_t (&A)[4][4], f32x4_t (&seed)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) seed[g] = offset_seed<CF>(A[g]);
}

// One item's MFMAs: groups of this K part, partial sums (rows 4q + r, column ml) into acc.
// Row ml's scales in the stage: INT G2 bf16; FP8 one fp32; MXFP4 4 G2 E8M0 bytes (group
// g's four blocks at 4 g), applied inside the conversion.
template <int CF>
__device__ __forceinline__ void d_compute(const DCursor& c, const uint8_t* stage, const u32x4_t (&A)[4][4],
                                          const f32x4_t (&seed)[4], f32x4_t& acc) {
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const uint8_t* sb = stage + kDCodeBytes;
    if constexpr (cf_bits(CF) == 4) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (g < c.G2) {
                const u32x4_t bw[1] = {*reinterpret_cast<const u32x4_t*>(stage + g * 1024 + lane * 16)};
                if constexpr (CF == kCfMx4) {
                    const f32x4_t t = group_dot<CF>(A[g], bw, seed[g], e8m0_scale(sb[ml * 4 * c.G2 + 4 * g + q]));
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += t[r];
                } else {
                    const float s = bf16_to_f32(reinterpret_cast<const uint16_t*>(sb)[ml * c.G2 + g]);
                    const f32x4_t t = group_dot<CF>(A[g], bw, seed[g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += s * t[r];
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int g = 2 * c.kh + j;
            if (g < c.G2) {
                const u32x4_t bw[2] = {*reinterpret_cast<const u32x4_t*>(stage + (2 * j) * 1024 + lane * 16),
                                       *reinterpret_cast<const u32x4_t*>(stage + (2 * j + 1) * 1024 + lane * 16)};
                const float s = CF == kCfFp8 ? reinterpret_cast<const float*>(sb)[ml]
                                             : bf16_to_f32(reinterpret_cast<const uint16_t*>(sb)[ml * c.G2 + g]);
                const f32x4_t t = c.kh == 0 ? group_dot<CF>(A[j], bw, seed[j]) : group_dot<CF>(A[2 + j], bw, seed[2 + j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += s * t[r];
            }
        }
    }
}

template <int CF, int SBITS>
__global__ __launch_bounds__(64 * kDWaves) void dk_stream_kernel(DecodeArgs a) {
    constexpr int BITS = cf_bits(CF);
    constexpr bool kSep = SBITS != 0 && SBITS != CF;   // as in gk_stream_kernel
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, q = lane >> 4, ml = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_hb = (int)(a.H / 16);
    const int n_tiles_r = __builtin_amdgcn_readfirstlane(a.meta[1]);
    const int n_tiles_s = SBITS != 0 ? (a.T + 15) / 16 : 0;
    const int kh_r = BITS == 4 ? 1 : (int)(a.routed.I / kGroup + 1) / 2;
    const int kh_s = SBITS == 0 ? 0 : SBITS == 4 ? 1 : (int)(a.shared.I / kGroup + 1) / 2;
    // ranges are cut between row blocks, never inside one (8-bit codes take two items per
    // row block, summed in one wave's registers)
    const int U_r = n_tiles_r * n_hb, U = U_r + n_tiles_s * n_hb;
    const int nw = gridDim.x * kDWaves, gw = blockIdx.x * kDWaves + wave;
    const int N_items = U_r * kh_r + (U - U_r) * kh_s;
    const int u0 = s_unit_at(N_items, gw, nw, U_r, U, kh_r, max(kh_s, 1));
    const int u1 = s_unit_at(N_items, gw + 1, nw, U_r, U, kh_r, max(kh_s, 1));
    const int nI = (min(u1, U_r) - min(u0, U_r)) * kh_r + (max(u1, U_r) - max(u0, U_r)) * kh_s;
    if (nI <= 0) return;

    DCursor ic;
    ic.tile = u0 / n_hb;   // routed and shared tiles have n_hb row blocks alike
    ic.hb = u0 - ic.tile * n_hb;
    ic.kh = 0;
    d_set_tile<BITS, SBITS>(a, ic, n_tiles_r);
    DCursor cc = ic;
    auto advance = [&](DCursor& c) {   // true when a new tile starts
        bool start = false;
        if (++c.kh >= c.n_kh) {
            c.kh = 0;
            if (++c.hb >= n_hb) {
                c.hb = 0;
                ++c.tile;
                if (c.tile < n_tiles_r + n_tiles_s) d_set_tile<BITS, SBITS>(a, c, n_tiles_r);
                start = true;
            }
        }
        d_uniform(c);
        return start;
    };

    const uint32_t ring = lds_offset(smem) + wave * kDWaveBytes;
    const uint8_t* ring_p = smem + wave * kDWaveBytes;
    // the first tile's a rows go out before the ring's copies: the wait for the first item
    // then covers them (a later tile's rows are loaded when the tile starts)
    u32x4_t A[4][4];
    f32x4_t seed[4];
    d_load_a(a, cc, A);
    for (int rel = 0; rel < kDStages - 1 && rel < nI; ++rel) {
        d_issue(a, ic, ring + rel * kDStageBytes);
        advance(ic);
    }
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.ystage, (uint32_t)((int64_t)a.rows_a * a.H * 4));
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    bool c_start = true;
    // store instructions of the last kDStages - 1 items (those issued after item rel's
    // copies), 3 bits each
    constexpr int kHist = kDStages - 1;
    static_assert(3 * kHist <= 30, "store history fits one int");
    int st_hist = 0;
    for (int rel = 0; rel < nI; ++rel) {
        // copies after item rel's: the later items' (at most kDStages - 2 of them) and the
        // stores of the kDStages - 1 items before it
        const int later = min(nI - 1 - rel, kDStages - 2);
        int n_st = 0;
#pragma unroll
        for (int e = 0; e < kHist; ++e) n_st += (st_hist >> (3 * e)) & 7;
        const int n = __builtin_amdgcn_readfirstlane(later * kDOps + n_st);
        wait_vmcnt_dyn(n);
        asm volatile("" ::: "memory");
        if (rel + kDStages - 1 < nI) {
            d_issue(a, ic, ring + ((rel + kDStages - 1) % kDStages) * kDStageBytes);
            advance(ic);
        }
        const bool sep = kSep && cc.tl.shared;
        if (c_start) {
            if (rel > 0) d_load_a(a, cc, A);
            if (!sep) d_seed<CF>(A, seed);
            else if constexpr (kSep) d_seed<SBITS>(A, seed);
        }
        const uint8_t* stage = ring_p + (rel % kDStages) * kDStageBytes;
        if (!sep) d_compute<CF>(cc, stage, A, seed, acc);
        else if constexpr (kSep) d_compute<SBITS>(cc, stage, A, seed, acc);
        int nst = 0;
        if (cc.kh == cc.n_kh - 1) {   // the row block is complete: rows 4q + r, column ml
            const int h = cc.hb * 16 + ml;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * q + r;
                const uint32_t off = m < cc.tl.count ? (uint32_t)(((int64_t)(cc.tl.row0 + m) * a.H + h) * 4) : kOob;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r]), yr, off, 0, 0);
                acc[r] = 0.f;
            }
            nst = 4;
        }
        st_hist = ((st_hist << 3) | nst) & ((1 << (3 * kHist)) - 1);
        c_start = advance(cc);
    }
}

// y[t] = residual[t] + sum over slots j of w[t, j] * ystage[position of (t, j)] (+ the
// shared expert's row), in slot order.  Workgroup (t, c) covers 512 columns of token t, so
// the token's positions and weights are wave-uniform loads and every row read is issued
// at once.
constexpr int kFinCols = 512;
template <int KMAX>   // KMAX == 8 == k, or KMAX = 16 >= k: every load is issued before the first use
__global__ __launch_bounds__(256) void dk_finalize_kernel(DecodeArgs a) {
    const int nc = (int)((a.H + kFinCols - 1) / kFinCols);
    const int t = blockIdx.x / nc;
    const int64_t h = (int64_t)(blockIdx.x - t * nc) * kFinCols + 2 * threadIdx.x;
    if (h >= a.H) return;
    const int k = a.k;
    int pos[KMAX];
    float w[KMAX];
    if constexpr (KMAX == 8) {   // k == 8: two 16-byte loads of each (the token's row starts 32-byte aligned)
        const int4 p0 = *reinterpret_cast<const int4*>(a.inv + t * 8), p1 = *reinterpret_cast<const int4*>(a.inv + t * 8 + 4);
        const float4 w0 = *reinterpret_cast<const float4*>(a.wts + t * 8), w1 = *reinterpret_cast<const float4*>(a.wts + t * 8 + 4);
        const int pp[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pos[j] = max(pp[j], 0);
            w[j] = pp[j] >= 0 ? ww[j] : 0.f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {   // slots past k repeat slot k - 1 with weight 0
            const int idx = t * k + min(j, k - 1);
            const int p = a.inv[idx];
            pos[j] = max(p, 0);
            w[j] = (j < k && p >= 0) ? a.wts[idx] : 0.f;
        }
    }
    float2 v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) v[j] = *reinterpret_cast<const float2*>(a.ystage + (int64_t)pos[j] * a.H + h);
    float2 sh = {0.f, 0.f};
    if (a.shared.bits) sh = *reinterpret_cast<const float2*>(a.ystage + (int64_t)(a.T * k + t) * a.H + h);
    const int64_t o = (int64_t)t * a.H + h;
    const uint32_t res = a.residual ? *reinterpret_cast<const uint32_t*>(a.residual + o) : 0u;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        s0 += w[j] * v[j].x;
        s1 += w[j] * v[j].y;
    }
    const float g = a.shared_gate ? a.shared_gate[t] : 1.0f;
    s0 += g * sh.x;
    s1 += g * sh.y;
    if (a.residual) {
        s0 += bf16_to_f32(res & 0xffffu);
        s1 += bf16_to_f32(res >> 16);
    }
    *reinterpret_cast<uint32_t*>(a.y + o) = cvt_bf16x2(s0, s1);
}

template <int CF, int SBITS>
hipError_t launch_dk_stream_t(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(dk_stream_kernel<CF, SBITS>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, kDLdsBytes);
        if (st != hipSuccess) return st;
        attr_set = true;
    }
    launch(t, "dk_stream", dk_stream_kernel<CF, SBITS>, dim3((unsigned)stream_workgroups()),
           dim3(64 * kDWaves), s, (uint32_t)kDLdsBytes, a);
    const int64_t nb = (int64_t)a.T * ((a.H + kFinCols - 1) / kFinCols);
    if (a.k == 8) launch(t, "dk_finalize", dk_finalize_kernel<8>, dim3((unsigned)nb), dim3(256), s, 0u, a);
    else launch(t, "dk_finalize", dk_finalize_kernel<16>, dim3((unsigned)nb), dim3(256), s, 0u, a);
    return hipGetLastError();
}

int g_stream_wgs[64];   // per device: CUs (0: not yet known, -1: query failed)

template <int CF, int SBITS>
hipError_t launch_stream_t(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(gk_stream_kernel<CF, SBITS>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, kSLdsBytes);
        if (st != hipSuccess) return st;
        attr_set = true;
    }
    launch(t, a.a_by_pair ? "gk_pair_stream" : "gk_stream", gk_stream_kernel<CF, SBITS>,
           dim3((unsigned)stream_workgroups()), dim3(kSThreads), s, (uint32_t)kSLdsBytes, a);
    return hipGetLastError();
}

}  // namespace

int stream_workgroups() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (g_stream_wgs[dev] == 0) {
        int cus = 0;
        g_stream_wgs[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                                    cus > 0
                                ? cus
                                : -1;
    }
    return g_stream_wgs[dev] > 0 ? g_stream_wgs[dev] : 0;
}

bool stream_fits(const DecodeArgs& a, int max_tiles) {
    const int nwg = stream_workgroups() - (a.a_by_pair ? 1 : 0);   // pair mode: workgroup 0 only routes
    if (nwg <= 0 || a.H > kSMaxH || a.T > kSmallT) return false;
    const int64_t G = a.H / kGroup, KH = (G + 7) / 8;
    // the INT scale copies read 16 bytes from each row's first bf16 group of a K chunk:
    // with an even group count every such address is 4-byte aligned (FP8 and MXFP4 scale
    // addresses are multiples of 4 at any group count)
    if (G % 2 != 0 && (a.routed.fmt == 0 || a.shared.bits)) return false;
    // a 4-bit row block must span two K chunks: its partial sums are read back one item
    // after they are written and rewritten no sooner than two items later
    if (KH < 2 && (a.routed.bits == 4 || a.shared.bits == 4)) return false;
    const int64_t n_rb_r = a.routed.I / 16;
    if (n_rb_r <= 0) return false;
    const int U_s = a.shared.bits ? (int)(((a.T + 15) / 16) * (a.shared.I / 16)) : 0;
    // routed units of a range at most: a cut by items, each end rounded up to a unit,
    // whatever the device-side tile count
    const int64_t sub_r = a.routed.bits == 4 ? KH : 2 * KH, sub_s = a.shared.bits == 4 ? KH : 2 * KH;
    const int64_t N = max_tiles * n_rb_r * sub_r + U_s * sub_s;
    const int64_t cap_r = ((N + nwg - 1) / nwg + 2 * sub_r) / sub_r;
    // routed tiles a range can touch
    return (cap_r + n_rb_r - 1) / n_rb_r + 1 <= kSMaxTiles;
}

namespace {
template <int CF>
hipError_t launch_gk_stream_cf(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (sb == 0) return launch_stream_t<CF, 0>(a, s, t);
    if (sb == 4) return launch_stream_t<CF, 4>(a, s, t);
    return launch_stream_t<CF, 8>(a, s, t);
}
template <int CF>
hipError_t launch_dk_stream_cf(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (sb == 0) return launch_dk_stream_t<CF, 0>(a, s, t);
    if (sb == 4) return launch_dk_stream_t<CF, 4>(a, s, t);
    return launch_dk_stream_t<CF, 8>(a, s, t);
}
}  // namespace

hipError_t launch_gk_stream(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    switch (cf_of(a.routed.fmt, a.routed.bits)) {
        case 4: return launch_gk_stream_cf<4>(a, s, t);
        case 8: return launch_gk_stream_cf<8>(a, s, t);
        case kCfFp8: return launch_gk_stream_cf<kCfFp8>(a, s, t);
        default: return launch_gk_stream_cf<kCfMx4>(a, s, t);
    }
}

bool pair_fits(const DecodeArgs& a) {
    const int64_t Tk = (int64_t)a.T * a.k;
    // every pair reads its own expert's rows: only for batches whose pairs rarely share one
    if (Tk > kPairP || 2 * Tk > a.E || a.E > kMaxE || a.k > kMaxK || !dk_stream_fits(a)) return false;
    DecodeArgs p = a;
    p.a_by_pair = 1;
    return stream_fits(p, (int)Tk);
}

bool dk_stream_fits(const DecodeArgs& a) {
    if (stream_workgroups() <= 0) return false;
    if (a.routed.I > kDMaxI || (a.shared.bits && a.shared.I > kDMaxI)) return false;
    return a.H % 32 == 0 && a.rows_a * a.H * 4 < (int64_t)kDSkip;
}

hipError_t launch_dk_stream(const DecodeArgs& a, hipStream_t s, StageTimer* t) {
    switch (cf_of(a.routed.fmt, a.routed.bits)) {
        case 4: return launch_dk_stream_cf<4>(a, s, t);
        case 8: return launch_dk_stream_cf<8>(a, s, t);
        case kCfFp8: return launch_dk_stream_cf<kCfFp8>(a, s, t);
        default: return launch_dk_stream_cf<kCfMx4>(a, s, t);
    }
}

}  // namespace w4a16
