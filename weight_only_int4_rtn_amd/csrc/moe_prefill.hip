// Large-batch W4A16 expert FFN as two grouped GEMMs on bf16 MFMA (gfx950).
//
// Both GEMMs run as persistent workgroups of 8 waves (2 along M x 4 along N, each wave a
// 64 x 64 block of 16x16x32 MFMAs) over items of 128 rows of one expert's sorted tokens
// by 256 code rows:
//   gk_prefill_kernel: 128 gate rows + the matching 128 up rows (one 128-column group of
//     the intermediate output), K = H.  Epilogue: a = SiLU(g) * u as bf16 in the K order
//     the down GEMM consumes, plus the fp32 sum of each a row over that group (the down
//     GEMM's offset seeds).
//   dk_prefill_kernel: 256 output rows, K = I.  Epilogue: the unweighted rows, rounded to
//     bf16, at their sorted positions; finalize_kernel applies the router weights and sums
//     each token's rows in fp32 in slot order (no atomics anywhere).
//
// The K loop is a flat stream of steps (item, 128-column group of K), so the pipeline
// runs on across item boundaries.  Every operand of a step reaches LDS by direct-to-LDS
// buffer loads (no registers): the activation tile (XOR-swizzled), the code rows
// (swizzled so the 16 rows one MFMA fragment reads sit in distinct banks), the code
// rows' group scales and the activation rows' group sums.  With 4-bit codes steps s+1
// and s+2 are in flight while step s computes (three LDS stages; 8-bit codes, whose
// code tile is twice as large, keep two).  Each wave waits for its own step-s loads with
// s_waitcnt vmcnt and a plain s_barrier covers the other waves; a __syncthreads() there
// would also wait for the later steps' loads.
//
// INT codes enter the MFMA as exact bf16 integers (see dq4 / dq8 in common.h): the
// accumulator of a group starts from -OFF * (sum of the group's activations) and the
// group scale multiplies the fp32 partial.  FP8 E4M3 codes (one fp32 scale per code row)
// and MXFP4 codes (an E8M0 scale per 32 columns) become exact bf16 values through the
// hardware conversions (dq_fp8 / dq_mx4): no seed; the FP8 row scale multiplies the
// partial like a group scale, the MXFP4 block scale is applied by the conversion.  The
// per-step scale copy brings one 4-byte word per code row in every format: the word
// holding the bf16 group scale, the fp32 row scale, or the group's four E8M0 bytes.
//
// Routed items (code format CF) and the shared expert's items (SCF, INT) are walked as two
// separate streams by every workgroup.
#include "common.h"
#include "dma.h"

namespace w4a16 {

namespace {

constexpr int MT = kPrefillMT;                // 128 rows per item
constexpr int NT = 256;                       // code rows per item
constexpr int kPWaves = 8;                    // 2 (M) x 4 (N)
constexpr int kPThreads = 64 * kPWaves;
constexpr int kAStageBytes = MT * kGroup * 2;   // 32 KB of activations per step
constexpr int kSeedSlots = 64 * kPWaves;        // 16 real row sums per wave, 4 B each
constexpr int kScaleSlots = 64 * kPWaves;       // 32 real code-row scale words per wave, 4 B each
constexpr int kMaxItems = 32;                   // items one workgroup walks (the grid grows if needed)

template <int BITS>
struct Pipe {
    static constexpr int kStages = BITS == 4 ? 3 : 2;
    static constexpr int kRowBytes = kGroup * BITS / 8;     // one code row's group: 64 / 128 B
    static constexpr int kChunksPerRow = kRowBytes / 16;    // 4 / 8
    static constexpr int kBStageBytes = NT * kRowBytes;     // 16 / 32 KB
    static constexpr int kBLoads = kBStageBytes / (kPThreads * 16);   // per wave per step: 2 / 4
    static constexpr int kStageBytes = kAStageBytes + kBStageBytes + kSeedSlots * 4 + kScaleSlots * 4;
    // vector-memory instructions per wave per step: A (4) + B + row sums (1) + scales (1)
    static constexpr int kLoadsPerStep = 4 + kBLoads + 2;
};

struct Item {        // one work item, resolved into LDS at kernel start
    int e;           // expert (-1: the shared expert)
    int row0;        // first row of the tile: sorted position (routed) or token (shared)
    int orow0;       // first row of the tile in the a / staging buffers
    int count;       // valid rows
    int nblk;        // N block
};

// Item L of a walk with nb N blocks per tile: routed tiles, or (SHARED) the shared
// expert's tiles of 128 consecutive tokens.  count 0: no work.
template <bool SHARED>
__device__ Item make_item(const PrefillArgs& a, int L, int nb) {
    Item it{};
    it.nblk = L % nb;
    const int tile = L / nb;
    if constexpr (!SHARED) {
        it.e = a.tiles[2 * tile];
        const int m0 = a.tiles[2 * tile + 1];
        const int pos0 = a.offsets[it.e];
        it.count = min(MT, a.offsets[it.e + 1] - pos0 - m0);
        it.row0 = pos0 + m0;
        it.orow0 = pos0 + m0;
    } else {
        it.e = -1;
        it.count = min(MT, a.T - tile * MT);
        it.row0 = tile * MT;
        it.orow0 = a.T * a.k + tile * MT;
    }
    return it;
}


// ------------------------------------------------------------- operand layouts
//
// A stage: 128 rows x 16 chunks of 16 B; chunk c of row r sits at r * 16 + (c ^ (r & 15)).
// A-load j (0..3) of wave w, lane l, fills chunk C = (4w + j) * 64 + l.
__device__ __forceinline__ int a_swz(int r, int c) { return r * 16 + (c ^ (r & 15)); }
__device__ __forceinline__ void a_coords(int j, int* r, int* c) {
    const int C = ((threadIdx.x >> 6) * 4 + j) * 64 + (threadIdx.x & 63);
    *r = C >> 4;
    *c = (C & 15) ^ (*r & 15);
}

// B stage: 256 code rows x kChunksPerRow chunks.  Row R = 64 wn + 16 b + ml holds wave
// wn's code subtile b, row ml.  Physical chunk p of row R holds logical chunk
// p ^ swizzle(R), which puts the 16 rows one fragment read touches in distinct banks.
template <int BITS>
__device__ __forceinline__ int b_swizzle(int R) {
    return BITS == 4 ? ((R >> 2) & 3) : ((R >> 1) & 7);
}
template <int BITS>
__device__ __forceinline__ void b_coords(int j, int* R, int* c) {
    using P = Pipe<BITS>;
    const int C = ((threadIdx.x >> 6) * P::kBLoads + j) * 64 + (threadIdx.x & 63);
    *R = C / P::kChunksPerRow;
    *c = (C % P::kChunksPerRow) ^ b_swizzle<BITS>(*R);
}

// Row sums: wave w's load covers rows 16 w .. 16 w + 15 in lanes 0..15; row r at slot
// (r / 16) * 64 + r % 16.  Scales: wave w's load covers code rows 32 w .. 32 w + 31 in
// lanes 0..31; code row R at slot (R / 32) * 64 + R % 32, as the aligned 4-byte word
// holding its bf16 scale (the low half when the scale's index is even).
__device__ __forceinline__ int seed_slot(int r) { return (r >> 4) * 64 + (r & 15); }
__device__ __forceinline__ int scale_slot(int R) { return (R >> 5) * 64 + (R & 31); }

// Gate/up code row of stage row R for N block nblk (one group of I): wave wn's subtiles
// 0, 1 are gate rows, 2, 3 the matching up rows.  Lane ml of subtile b & 1 = ns takes
// column 8 (ml / 4) + ml % 4 + 4 ns of the wave's 32, so that a lane's two output columns
// j and j + 4 of one block of 8 sit next to each other in the down GEMM's K order.
__device__ __forceinline__ int gk_code_row(int R, int nblk, int64_t I_e) {
    const int wn = R >> 6, b = (R >> 4) & 3, ml = R & 15;
    return (b >= 2 ? (int)I_e : 0) + nblk * kGroup + 32 * wn + 8 * (ml >> 2) + (ml & 3) + 4 * (b & 1);
}
// Down code row (output column) of stage row R for N block nblk: lane ml of subtile b
// takes column 4 ml + b of the wave's 64, so that a lane's four outputs of one row are
// adjacent columns.
__device__ __forceinline__ int dk_code_row(int R, int nblk) {
    return nblk * NT + 64 * (R >> 6) + 4 * (R & 15) + ((R >> 4) & 3);
}

// --------------------------------------------------------------- per-item issue state

// What a wave needs to issue the loads of any step of one item.
struct IssueState {
    i32x4_t a_r, b_r, seed_r, s_r;
    uint32_t a_off[4];    // per A-load: the lane's source byte offset at group 0
    uint32_t b_off[4];    // per B-load (kBLoads used)
    uint32_t seed_off;    // the lane's row-sum offset at group 0 (kOob: lanes 16..63)
    uint32_t s_off;       // byte offset of the lane's scale at group 0 (kOob: lanes 32..63)
};

// Byte offset of code row `row`'s scale word at group 0, and the scale buffer's bytes, of
// an expert whose rows hold K columns (INT: bf16 [rows, K/128]; FP8: fp32 [rows];
// MXFP4: E8M0 bytes [rows, K/32]).
template <int CF>
__device__ __forceinline__ uint32_t scale_off(int row, int G) {
    if constexpr (CF == kCfFp8) return (uint32_t)row * 4;
    else if constexpr (CF == kCfMx4) return (uint32_t)row * G * 4;
    else return (uint32_t)row * G * 2;
}
template <int CF>
__device__ __forceinline__ int64_t scale_bytes(int64_t rows, int G) {
    return CF == kCfFp8 ? rows * 4 : CF == kCfMx4 ? rows * G * 4 : rows * G * 2;
}
// The scale buffer of expert eb (its rows x K/128 groups).
template <int CF>
__device__ __forceinline__ const uint8_t* scale_base(const uint16_t* s, int64_t eb, int64_t rows, int G) {
    return reinterpret_cast<const uint8_t*>(s) + eb * scale_bytes<CF>(rows, G);
}

template <int CF, bool GATE_UP>
__device__ void prepare_issue(const PrefillArgs& a, const Item& it, const ExpertSet& es, const int (&tok)[5],
                              IssueState& st) {
    constexpr int BITS = cf_bits(CF);
    using P = Pipe<BITS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t I_e = es.I;
    const int64_t eb = it.e < 0 ? 0 : it.e;
    if constexpr (GATE_UP) {
        const int64_t H = a.H;
        const int G = (int)(H / kGroup);
        const int64_t row_bytes = H * BITS / 8;
        st.a_r = dma_rsrc(a.xp, (uint32_t)(a.T * H * 2));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int r, c;
            a_coords(j, &r, &c);
            st.a_off[j] = ((uint32_t)tok[j] * (uint32_t)H + c * 8) * 2;
        }
        st.b_r = dma_rsrc(es.w13 + eb * (2 * I_e * H * BITS / 32), (uint32_t)(2 * I_e * row_bytes));
#pragma unroll
        for (int j = 0; j < P::kBLoads; ++j) {
            int R, c;
            b_coords<BITS>(j, &R, &c);
            st.b_off[j] = (uint32_t)gk_code_row(R, it.nblk, I_e) * (uint32_t)row_bytes + c * 16;
        }
        st.seed_r = dma_rsrc(a.xsum, (uint32_t)(a.T * G * 4));
        st.seed_off = lane < 16 ? (uint32_t)tok[4] * G * 4 : kOob;
        st.s_r = dma_rsrc(scale_base<CF>(es.s13, eb, 2 * I_e, G), (uint32_t)scale_bytes<CF>(2 * I_e, G));
        st.s_off = lane < 32 ? scale_off<CF>(gk_code_row(32 * wave + lane, it.nblk, I_e), G) : kOob;
    } else {
        const int G2 = (int)(I_e / kGroup);
        const int GW = (int)(a.width_a / kGroup);
        const int64_t row_bytes = I_e * BITS / 8;
        st.a_r = dma_rsrc(a.abuf, (uint32_t)(a.rows_a * a.width_a * 2));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int r, c;
            a_coords(j, &r, &c);
            st.a_off[j] = ((uint32_t)(it.orow0 + min(r, it.count - 1)) * (uint32_t)a.width_a + c * 8) * 2;
        }
        // rows past H read zeros (the buffer ends at H)
        st.b_r = dma_rsrc(es.w2 + eb * (a.H * I_e * BITS / 32), (uint32_t)(a.H * row_bytes));
#pragma unroll
        for (int j = 0; j < P::kBLoads; ++j) {
            int R, c;
            b_coords<BITS>(j, &R, &c);
            st.b_off[j] = (uint32_t)dk_code_row(R, it.nblk) * (uint32_t)row_bytes + c * 16;
        }
        st.seed_r = dma_rsrc(a.asum, (uint32_t)(a.rows_a * GW * 4));
        st.seed_off = lane < 16 ? (uint32_t)(it.orow0 + min(16 * wave + lane, it.count - 1)) * GW * 4 : kOob;
        st.s_r = dma_rsrc(scale_base<CF>(es.s2, eb, a.H, G2), (uint32_t)scale_bytes<CF>(a.H, G2));
        st.s_off = lane < 32 ? scale_off<CF>(dk_code_row(32 * wave + lane, it.nblk), G2) : kOob;
    }
}

// The tokens of a routed gate/up item's MT rows (the token half of tokw), copied into an
// LDS buffer by wave 0 one item ahead: two direct copies of 64 words.  A load the compiler
// sees would make it wait, where the tokens are used, for every copy in flight.
__device__ __forceinline__ void copy_item_tokens(const PrefillArgs& a, const Item& it, uint32_t lds_buf) {
    const int lane = threadIdx.x & 63;
    const i32x4_t tr = uniform_rsrc(dma_rsrc(a.tokw, (uint32_t)((int64_t)a.T * a.k * 8)));
#pragma unroll
    for (int h = 0; h < MT / 64; ++h) {
        const int row = it.row0 + 64 * h + lane;
        dma4(tr, __builtin_amdgcn_readfirstlane(lds_buf + 256 * h),
             it.e >= 0 && 64 * h + lane < it.count ? (uint32_t)(row * 8) : kOob, 0);
    }
}

// The tokens of the rows a lane's A and row-sum loads read for a gate/up item (padding
// rows repeat the last real row), from the item's token buffer.
__device__ __forceinline__ void item_tokens(const Item& it, const int* s_tok, int (&tok)[5]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        int r;
        if (j < 4) {
            int c;
            a_coords(j, &r, &c);
        } else {
            r = 16 * wave + (lane & 15);
        }
        r = min(r, it.count - 1);
        tok[j] = it.e < 0 ? it.row0 + r : s_tok[r];
    }
}

// stage: LDS byte address of the stage the step goes to.  The copies go out in four
// parts (0: activation chunks 0-1, 1: chunks 2-3, 2: code rows, 3: row sums and scales),
// so that a step's copies can be spread over the previous step's MFMAs; part -1: all.
template <int CF>
__device__ __forceinline__ void issue_step(const IssueState& st, int g, uint32_t stage, int part = -1) {
    constexpr int BITS = cf_bits(CF);
    using P = Pipe<BITS>;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t A = stage, B = stage + kAStageBytes, S = B + P::kBStageBytes, SC = S + kSeedSlots * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (part < 0 || part == j / 2)
            dma16_free(st.a_r, A + (wave * 4 + j) * 1024, st.a_off[j], (uint32_t)g * kGroup * 2);
    if (part < 0 || part == 2) {
#pragma unroll
        for (int j = 0; j < P::kBLoads; ++j)
            dma16_free(st.b_r, B + (wave * P::kBLoads + j) * 1024, st.b_off[j], (uint32_t)g * P::kRowBytes);
    }
    if (part < 0 || part == 3) {
        dma4_free(st.seed_r, S + wave * 256, st.seed_off, (uint32_t)g * 4);
        if constexpr (CF == kCfFp8) dma4_free(st.s_r, SC + wave * 256, st.s_off, 0);   // the row's one scale
        else if constexpr (CF == kCfMx4) dma4_free(st.s_r, SC + wave * 256, st.s_off + (uint32_t)g * 4, 0);
        else dma4_free(st.s_r, SC + wave * 256, (st.s_off + (uint32_t)g * 2) & ~3u, 0);
    }
}

// ------------------------------------------------------------------- compute

// One step of one wave: its 64 x 64 block (4 M-subtiles x 4 code subtiles) for one
// group, accumulated into acc with the group scales (D column ml is code row R's).
// sodd: bit b set when code subtile b's scale sits in the high half of its word.
// The K slice (32 columns) is the outer loop: the lane's code chunks of all four code
// subtiles and their scales are read at the start (8-bit codes: the second chunk half-way),
// the four activation fragments once per slice, and each dequantised code fragment feeds
// the four M-subtiles' MFMAs.  The 16 tiles' group partials start from the offset seeds
// (MXFP4: from the accumulators themselves, its block scale being inside the conversion).
// hook(i) runs before slice i's MFMAs with EARLY_FOLD, else after them (the next step's
// copies go out there).  EARLY_FOLD: each code subtile's group scaling runs inside the last
// slice, right after the next subtile's MFMAs go out, so that it overlaps them; the copy
// issue then comes first in each slice, which keeps the compiler from sinking that scaling
// past the issue branch to the end of the step.
// 8-bit codes w0 = k0..k3, w1 = k4..k7 (one byte each) as bf16 pairs in natural column
// order, (k0,k1) (k2,k3) (k4,k5) (k6,k7), for activation tiles read unpermuted: INT8 codes
// as exact bf16 integers (OFF = 128, as dq8_cvt), FP8 E4M3 bytes through the hardware
// conversion (exact, as dq_fp8, without its byte permutes).
template <int CF>
__device__ __forceinline__ u32x4_t dq8_natural(uint32_t w0, uint32_t w1) {
    u32x4_t r;
    if constexpr (CF == kCfFp8) {
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = j < 2 ? w0 : w1;
            const int b = 16 * (j & 1);
            r[j] = cvt_bf16x2((float)((w >> b) & 0xffu), (float)((w >> (b + 8)) & 0xffu));
        }
    }
    return r;
}

// NATURAL: the activation tile holds unpermuted rows (a dense projection reading x itself);
// only 8-bit codes take it.
template <int CF, bool EARLY_FOLD, bool NATURAL, typename Hook>
__device__ __forceinline__ void compute_step(const uint8_t* stage, uint32_t sodd, f32x4_t (&acc)[4][4], Hook&& hook) {
    constexpr int BITS = cf_bits(CF);
    using P = Pipe<BITS>;
    constexpr float kOff = CF == 4 ? 136.0f : CF == 8 ? 128.0f : 0.0f;   // INT8 through dq8_cvt
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(stage);
    const uint8_t* B = stage + kAStageBytes;
    const float* S = reinterpret_cast<const float*>(B + P::kBStageBytes);
    const uint32_t* SC = reinterpret_cast<const uint32_t*>(S + kSeedSlots);
    const uint32_t M = nibble_mask();

    // 4-bit codes: the lane's 16-byte chunk (its 32 columns of the group) of code subtile b,
    // word i for slice i.  8-bit codes: the two words of slice i (chunk i / 2, words 2i % 4
    // and 2i % 4 + 1), read per slice.
    auto code_addr = [&](int b, int c) {
        const int R = 64 * wn + 16 * b + ml;
        const int lc = (BITS / 4) * q + c;
        return B + R * P::kRowBytes + ((lc ^ b_swizzle<BITS>(R)) * 16);
    };
    u32x4_t bw[4];
    if constexpr (BITS == 4) {
#pragma unroll
        for (int b = 0; b < 4; ++b) bw[b] = *reinterpret_cast<const u32x4_t*>(code_addr(b, 0));
    }
    float sc[4], xs[4];   // partial's scale; MXFP4: the conversion's block scale
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t sw = SC[scale_slot(64 * wn + 16 * b + ml)];
        sc[b] = 1.f;
        xs[b] = 1.f;
        if constexpr (CF == kCfFp8) sc[b] = __uint_as_float(sw);
        else if constexpr (CF == kCfMx4) xs[b] = e8m0_scale(sw >> (8 * q));   // this lane's block: columns 32q..
        else sc[b] = bf16_to_f32(((sodd >> b) & 1) ? (sw >> 16) : (sw & 0xffffu));
    }
    f32x4_t seed[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if constexpr (cf_int(CF)) {
            const f32x4_t xsum = *reinterpret_cast<const f32x4_t*>(S + seed_slot(64 * wm + 16 * mi + 4 * q));
#pragma unroll
            for (int e = 0; e < 4; ++e) seed[mi][e] = -kOff * xsum[e];
        } else {
            seed[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    // 8-bit codes take the code subtiles in two passes of two (half the partials live at a
    // time, the activation fragments read once per pass)
    constexpr int NB = BITS == 8 ? 2 : 4;
#pragma unroll
    for (int b0 = 0; b0 < 4; b0 += NB) {
        f32x4_t t[4][NB];
        // the group partials of code subtile b0 + bb (complete after slice 3) into acc
        auto fold = [&](int bb) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                if constexpr (CF == kCfMx4) {
                    acc[mi][b0 + bb] = t[mi][bb];
                } else {
#pragma unroll
                    for (int r2 = 0; r2 < 4; ++r2) acc[mi][b0 + bb][r2] += sc[b0 + bb] * t[mi][bb][r2];
                }
            }
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (EARLY_FOLD && b0 == 0) hook(i);
            if constexpr (BITS == 8) {
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    const uint2 w = *reinterpret_cast<const uint2*>(code_addr(b0 + bb, i >> 1) + (2 * i & 3) * 4);
                    bw[b0 + bb][0] = w.x;
                    bw[b0 + bb][1] = w.y;
                }
            }
            u32x4_t av[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                av[mi] = *reinterpret_cast<const u32x4_t*>(A + a_swz(64 * wm + 16 * mi + ml, 4 * q + i) * 8);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const int b = b0 + bb;
                u32x4_t lo;
                if constexpr (CF == 4) {
                    lo = dq4(bw[b][i], M);
                } else if constexpr (CF == 8) {
                    lo = NATURAL ? dq8_natural<CF>(bw[b][0], bw[b][1]) : dq8_cvt(bw[b][0], bw[b][1]);
                } else if constexpr (CF == kCfFp8) {
                    lo = NATURAL ? dq8_natural<CF>(bw[b][0], bw[b][1]) : dq_fp8(bw[b][0], bw[b][1]);
                } else {
                    lo = dq_mx4(bw[b][i], xs[b]);
                }
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const f32x4_t c0 = i > 0 ? t[mi][bb] : CF == kCfMx4 ? acc[mi][b] : seed[mi];
                    t[mi][bb] = mfma16(av[mi], lo, c0);
                }
                // last slice: the previous subtile's partials are complete (their MFMAs went
                // out four MFMAs ago), so their scaling FMAs issue while these MFMAs run
                if (EARLY_FOLD && i == 3 && bb > 0) fold(bb - 1);
            }
            if (EARLY_FOLD && i == 3) fold(NB - 1);
            if (!EARLY_FOLD && b0 == 0) hook(i);
        }
        if constexpr (!EARLY_FOLD) {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) fold(bb);
        }
    }
}

// ------------------------------------------------------------------- epilogues

// a = SiLU(gate) * up for the item's 128 x 128 block, bf16, columns in the reordered K
// order of the down GEMM; and each row's fp32 sum of those bf16 values (one group of I).
// The lane's 16 row partials (mi, r) are summed over the 16 lanes of its row group by a
// reduce-scatter (halves exchanged with lane ^ 8, ^ 4, ^ 2, ^ 1: 15 exchanges), after
// which lane ml holds the sum of row partial ml.
__device__ void gk_epilogue(const PrefillArgs& a, const Item& it, const f32x4_t (&acc)[4][4], float* s_asum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const int GW = (int)(a.width_a / kGroup);
    float v[16];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * wm + 16 * mi + 4 * q + r;
            const uint32_t v0 = cvt_bf16(silu_mul(acc[mi][0][r], acc[mi][2][r]));
            const uint32_t v1 = cvt_bf16(silu_mul(acc[mi][1][r], acc[mi][3][r]));
            v[4 * mi + r] = bf16_to_f32(v0) + bf16_to_f32(v1);
            if (m < it.count) {   // columns j and j + 4 of a block of 8: adjacent in K order
                const int col = perm_pos(it.nblk * kGroup + 32 * wn + 8 * (ml >> 2) + (ml & 3));
                *reinterpret_cast<uint32_t*>(a.abuf + (int64_t)(it.orow0 + m) * a.width_a + col) = v0 | (v1 << 16);
            }
        }
#pragma unroll
    for (int h = 8; h >= 1; h >>= 1) {
        const bool up = (ml & h) != 0;
#pragma unroll
        for (int j = 0; j < h; ++j) {
            const float send = up ? v[j] : v[j + h];
            const float keep = up ? v[j + h] : v[j];
            v[j] = keep + __shfl_xor(send, h, 16);
        }
    }
    s_asum[wn * MT + 64 * wm + 16 * (ml >> 2) + 4 * q + (ml & 3)] = v[0];
    wait_lgkm0();
    bar();
    if ((int)threadIdx.x < it.count) {
        const int m = threadIdx.x;
        const float s = s_asum[m] + s_asum[MT + m] + s_asum[2 * MT + m] + s_asum[3 * MT + m];
        a.asum[(int64_t)(it.orow0 + m) * GW + it.nblk] = s;
    }
    wait_lgkm0();
    bar();   // s_asum is reused by the next item
}

// The unweighted output rows of a down item, rounded to bf16, at their sorted positions:
// a lane's four columns of a row are adjacent (see dk_code_row) and go out as 8 bytes.
template <bool DIRECT>
__device__ void dk_epilogue(const PrefillArgs& a, const Item& it, const f32x4_t (&acc)[4][4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const int h = it.nblk * NT + 64 * wn + 4 * ml;   // H is a multiple of 128: h < H covers h + 3
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * wm + 16 * mi + 4 * q + r;
            if (m < it.count && h < a.H) {
                const int64_t o = (int64_t)(it.orow0 + m) * a.H + h;
                float f[4] = {acc[mi][0][r], acc[mi][1][r], acc[mi][2][r], acc[mi][3][r]};
                if (DIRECT && a.residual) {   // row orow0 + m is the token's
                    const uint2 rv = *reinterpret_cast<const uint2*>(a.residual + o);
                    f[0] += bf16_to_f32(rv.x & 0xffffu);
                    f[1] += bf16_to_f32(rv.x >> 16);
                    f[2] += bf16_to_f32(rv.y & 0xffffu);
                    f[3] += bf16_to_f32(rv.y >> 16);
                }
                uint2 v;
                v.x = cvt_bf16(f[0]) | (cvt_bf16(f[1]) << 16);
                v.y = cvt_bf16(f[2]) | (cvt_bf16(f[3]) << 16);
                *reinterpret_cast<uint2*>((DIRECT ? a.y : a.ystage) + o) = v;
            }
        }
}

// --------------------------------------------------------------------- driver

// One walk: workgroup b takes items w = b, b + grid, ... of `total` (item index L is
// remapped so that each XCD, w mod 8, takes one contiguous range: an expert's tiles share
// that XCD's L2).  The items are resolved once into LDS; the steps of all of them form
// one pipelined stream.
// EARLY_FOLD: the group scaling of each step inside its last K slice (see compute_step);
// DIRECT: the down epilogue writes y (dense projections).
template <int CF, bool GATE_UP, bool SHARED, bool EARLY_FOLD = true, bool DIRECT = false>
__device__ void run_items(const PrefillArgs& a, const ExpertSet& es, int nb, int total, uint8_t* smem,
                          Item* s_items, float* s_asum, int* s_cnt, int* s_tok) {
    using P = Pipe<cf_bits(CF)>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = (total + 7) / 8;
    __syncthreads();   // the previous walk's LDS use is over
    {
        const int w = blockIdx.x + tid * (int)gridDim.x;
        Item it{};
        bool ok = false;
        if (tid < kMaxItems && w < 8 * C) {
            const int L = (w & 7) * C + (w >> 3);
            if (L < total) {
                it = make_item<SHARED>(a, L, nb);
                ok = it.count > 0 && it.nblk * (GATE_UP ? kGroup : NT) < (GATE_UP ? es.I : a.H);
            }
        }
        const uint64_t vm = __ballot(ok);   // compact, keeping the walk order
        if (lane == 0) s_cnt[wave] = __popcll(vm);
        __syncthreads();
        int base = 0;
        for (int i = 0; i < wave; ++i) base += s_cnt[i];
        if (ok) s_items[base + __popcll(vm & ((1ull << lane) - 1ull))] = it;
        __syncthreads();
    }
    int n_items = 0;
    for (int i = 0; i < kPWaves; ++i) n_items += s_cnt[i];
    if (n_items == 0) return;
    const int G = (int)((GATE_UP ? a.H : es.I) / kGroup);   // groups of K per item
    const int total_steps = n_items * G;

    // issue side: item ii, group gi.  Gate/up: item i's tokens sit in token buffer i & 1,
    // copied when item i - 1 starts issuing; the copy is older than every step wait from
    // then on, and a barrier follows wave 0's next wait before any wave reads it.
    int ii = 0, gi = 0, issued = 0;
    int tok[5] = {0, 0, 0, 0, 0};
    const uint32_t lds_tok = lds_offset(s_tok);
    if constexpr (GATE_UP) {
        if (__builtin_amdgcn_readfirstlane(wave) == 0) {   // (wave-uniform branch)
            copy_item_tokens(a, s_items[0], lds_tok);
            if (n_items > 1) copy_item_tokens(a, s_items[1], lds_tok + MT * 4);
            wait_vmcnt<0>();
        }
        __syncthreads();
        item_tokens(s_items[0], s_tok, tok);
    }
    IssueState st;
    prepare_issue<CF, GATE_UP>(a, s_items[0], es, tok, st);
    const uint32_t lds0 = lds_offset(smem);
    // part p of the next step's copies (p = -1: all of them) ...
    auto issue_next = [&](int p) {
        issue_step<CF>(st, gi, lds0 + (uint32_t)(issued % P::kStages) * P::kStageBytes, p);
    };
    // ... and, once they are all out, the issue side moves on to the following step
    auto advance = [&]() {
        ++issued;
        if (++gi == G && ii + 1 < n_items) {
            ++ii;
            gi = 0;
            if constexpr (GATE_UP) {
                item_tokens(s_items[ii], s_tok + (ii & 1) * MT, tok);
                if (__builtin_amdgcn_readfirstlane(wave) == 0 && ii + 1 < n_items)
                    copy_item_tokens(a, s_items[ii + 1], lds_tok + ((ii + 1) & 1) * MT * 4);
            }
            prepare_issue<CF, GATE_UP>(a, s_items[ii], es, tok, st);
        }
    };
    for (int p = 0; p < P::kStages - 1 && issued < total_steps; ++p) {
        issue_next(-1);
        advance();
    }

    // compute side
    int ci = 0, gc = 0;
    f32x4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[mi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // parity of each of this lane's four code rows' first scale index (row * G) for the
    // compute item; a step's scale sits in the high half of its word when row * G + g is odd
    auto row_parity = [&](const Item& it) {
        const int wn = wave & 3, ml = lane & 15;
        uint32_t p = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int R = 64 * wn + 16 * b + ml;
            const int crow = GATE_UP ? gk_code_row(R, it.nblk, es.I) : dk_code_row(R, it.nblk);
            p |= (uint32_t)((crow * G) & 1) << b;
        }
        return p;
    };
    uint32_t cpar = row_parity(s_items[0]);
    int ccount = s_items[0].count;   // valid rows of the compute item
    // An item's epilogue runs after the next step's wait and barrier, before that step's
    // copies go out: its stores are then older than every copy batch still awaited, so
    // the in-order vmcnt waits never hold a batch back behind them.
    bool epi = false;
    auto finish_item = [&]() {   // the item before ci (its record stays in LDS)
        const Item eit = s_items[ci - 1];
        if constexpr (GATE_UP) gk_epilogue(a, eit, acc, s_asum);
        else dk_epilogue<DIRECT>(a, eit, acc);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[mi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        epi = false;
    };
    for (int s = 0; s < total_steps; ++s) {
        // step s's loads are this wave's oldest outstanding ones; at most the later steps'
        // (kLoadsPerStep each) may still be out
        if (issued - s - 1 >= 1) wait_vmcnt<P::kLoadsPerStep>();
        else wait_vmcnt<0>();
        bar();   // every wave's step-s data is in LDS, and stage (s - 1) is no longer read
        if (epi) finish_item();
        // step s + kStages - 1's copies go out at one of this step's four K slices: waves
        // 2j and 2j + 1 (on two different SIMDs) at slice j (before its MFMAs with the early
        // fold, else after them), so that at any time only two waves wait for the load path
        // while the others keep the matrix units busy
        const bool more = issued < total_steps;
        const int slot = __builtin_amdgcn_readfirstlane(wave >> 1);
        if (64 * (slot >> 1) < ccount) {
            compute_step<CF, EARLY_FOLD, DIRECT && cf_bits(CF) == 8>(smem + (s % P::kStages) * P::kStageBytes, (gc & 1) ? (cpar ^ 0xfu) : cpar, acc,
                             [&](int i) {
                                 if (more && i == slot) issue_next(-1);
                             });
        } else if (more) {
            issue_next(-1);   // the wave's 64 rows of a ragged last tile are all padding
        }
        if (more) advance();
        if (++gc == G) {
            epi = true;
            gc = 0;
            if (++ci < n_items) {
                cpar = row_parity(s_items[ci]);
                ccount = s_items[ci].count;
            }
        }
    }
    if (epi) finish_item();
}

template <int CF>
constexpr uint32_t pipe_lds_bytes() {
    return Pipe<cf_bits(CF)>::kStages * Pipe<cf_bits(CF)>::kStageBytes;
}

}  // namespace

// Dynamic LDS: the stages of the larger pipeline, then the item list and the row-sum
// scratch.
template <int CF, int SBITS>
__global__ __launch_bounds__(kPThreads) void gk_prefill_kernel(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr uint32_t kPipe = std::max(pipe_lds_bytes<CF>(), SBITS ? pipe_lds_bytes<SBITS>() : 0u);
    Item* s_items = reinterpret_cast<Item*>(smem + kPipe);
    float* s_asum = reinterpret_cast<float*>(s_items + kMaxItems);
    int* s_tok = reinterpret_cast<int*>(s_asum + 4 * MT);   // two items' tokens
    __shared__ int s_cnt[kPWaves];
    const int nb = (int)(a.routed.I / kGroup);
    run_items<CF, true, false>(a, a.routed, nb, a.meta[1] * nb, smem, s_items, s_asum, s_cnt, s_tok);
    if constexpr (SBITS != 0) {
        const int nbs = (int)(a.shared.I / kGroup);
        run_items<SBITS, true, true>(a, a.shared, nbs, ((a.T + MT - 1) / MT) * nbs, smem, s_items, s_asum, s_cnt,
                                     s_tok);
    }
}

// DIRECT: a dense projection (one expert of weight 1, rows in token order): the epilogue
// writes y itself, and with 8-bit codes the activation rows are x itself, unpermuted.  With a shared stream the step keeps its scaling after the last K slice
// (the early fold would spill there).
template <int CF, int SBITS, bool DIRECT = false>
__global__ __launch_bounds__(kPThreads) void dk_prefill_kernel(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr uint32_t kPipe = std::max(pipe_lds_bytes<CF>(), SBITS ? pipe_lds_bytes<SBITS>() : 0u);
    Item* s_items = reinterpret_cast<Item*>(smem + kPipe);
    float* s_asum = reinterpret_cast<float*>(s_items + kMaxItems);
    __shared__ int s_cnt[kPWaves];
    const int nb = (int)((a.H + NT - 1) / NT);
    run_items<CF, false, false, SBITS == 0, DIRECT>(a, a.routed, nb, a.meta[1] * nb, smem, s_items, s_asum, s_cnt,
                                                    nullptr);
    if constexpr (SBITS != 0)
        run_items<SBITS, false, true, false>(a, a.shared, nb, ((a.T + MT - 1) / MT) * nb, smem, s_items, s_asum,
                                             s_cnt, nullptr);
}

// y[t] = sum over slots j in order of w[t, j] times the staged row of pair (t, j), then
// the shared expert's row (times its gate value when there is one), then the residual;
// rounded once to bf16.  A token's row is
// split over ceil(H / 2048) blocks of 256 threads x 8 columns.  No atomics anywhere.
template <int KMAX>   // KMAX >= k: every position, weight and row load is issued before the first use
__global__ __launch_bounds__(256) void finalize_kernel(PrefillArgs a) {
    const int nbx = (int)((a.H / 8 + 255) / 256);
    const int t = (int)(blockIdx.x / nbx);
    const int64_t c = ((int64_t)(blockIdx.x % nbx) * blockDim.x + threadIdx.x) * 8;
    if (c >= a.H) return;
    const int k = a.k;
    int pos[KMAX];
    float w[KMAX];
    bool kept[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {   // slots past k repeat slot k - 1, not kept
        const int64_t idx = (int64_t)t * k + min(j, k - 1);
        const int p = a.inv[idx];
        kept[j] = j < k && p >= 0;
        pos[j] = max(p, 0);
        w[j] = a.wts[idx];
    }
    u32x4_t v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) v[j] = *reinterpret_cast<const u32x4_t*>(a.ystage + pos[j] * a.H + c);
    u32x4_t vs = {0u, 0u, 0u, 0u};
    if (a.shared.bits) vs = *reinterpret_cast<const u32x4_t*>(a.ystage + ((int64_t)a.T * k + t) * a.H + c);
    const int64_t o = (int64_t)t * a.H + c;
    u32x4_t r = {0u, 0u, 0u, 0u};
    if (a.residual) r = *reinterpret_cast<const u32x4_t*>(a.residual + o);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add_row = [&](const u32x4_t& x, float wt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[2 * e] += wt * bf16_to_f32(x[e] & 0xffffu);
            s[2 * e + 1] += wt * bf16_to_f32(x[e] >> 16);
        }
    };
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (kept[j]) add_row(v[j], w[j]);   // slot order; a dropped slot adds nothing
    if (a.shared.bits) add_row(vs, a.shared_gate ? a.shared_gate[t] : 1.0f);
    if (a.residual) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[2 * e] += bf16_to_f32(r[e] & 0xffffu);
            s[2 * e + 1] += bf16_to_f32(r[e] >> 16);
        }
    }
    u32x4_t out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = cvt_bf16x2(s[2 * e], s[2 * e + 1]);
    *reinterpret_cast<u32x4_t*>(a.y + o) = out;
}

namespace {

unsigned prefill_grid(int64_t max_items) {
    // one workgroup per CU; more when a workgroup would walk more than kMaxItems items
    int64_t g = std::max<int64_t>(256, (max_items + 8 + kMaxItems - 1) / kMaxItems);
    g = std::min<int64_t>(g, std::max<int64_t>(max_items, 8));
    return (unsigned)((g + 7) / 8 * 8);
}

template <int CF, int SBITS>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    constexpr uint32_t kPipe = std::max(pipe_lds_bytes<CF>(), SBITS ? pipe_lds_bytes<SBITS>() : 0u);
    constexpr uint32_t lds = kPipe + kMaxItems * sizeof(Item) + 4 * MT * 4 + 2 * MT * 4;
    static_assert(lds + 64 <= 160 * 1024, "LDS budget of one workgroup");
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gk_prefill_kernel<CF, SBITS>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dk_prefill_kernel<CF, SBITS>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        return true;
    }();
    (void)attr;
    const int64_t shared_tiles = SBITS ? (a.T + MT - 1) / MT : 0;
    const int64_t gk_items = std::max(a.max_tiles * (a.routed.I / kGroup), shared_tiles * (a.shared.I / kGroup));
    const int64_t dk_items = std::max(a.max_tiles, shared_tiles) * ((a.H + NT - 1) / NT);
    launch(t, "gk_prefill", gk_prefill_kernel<CF, SBITS>, dim3(prefill_grid(gk_items)), dim3(kPThreads), s, lds, a);
    launch(t, "dk_prefill", dk_prefill_kernel<CF, SBITS>, dim3(prefill_grid(dk_items)), dim3(kPThreads), s, lds, a);
    const dim3 fin_grid((unsigned)((a.H / 8 + 255) / 256 * a.T));
    if (a.k <= 8) launch(t, "finalize", finalize_kernel<8>, fin_grid, dim3(256), s, 0u, a);
    else launch(t, "finalize", finalize_kernel<16>, fin_grid, dim3(256), s, 0u, a);
    return hipGetLastError();
}

template <int CF>
hipError_t launch_down_prefill_t(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    constexpr uint32_t lds = pipe_lds_bytes<CF>() + kMaxItems * sizeof(Item) + 4 * MT * 4 + 2 * MT * 4;
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dk_prefill_kernel<CF, 0, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        return true;
    }();
    (void)attr;
    const int64_t dk_items = a.max_tiles * ((a.H + NT - 1) / NT);
    launch(t, "dk_prefill", dk_prefill_kernel<CF, 0, true>, dim3(prefill_grid(dk_items)), dim3(kPThreads), s, lds,
           a);
    return hipGetLastError();   // the epilogue wrote y
}

template <int CF>
hipError_t launch_prefill_cf(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (sb == 0) return launch_prefill_t<CF, 0>(a, s, t);
    if (sb == 4) return launch_prefill_t<CF, 4>(a, s, t);
    return launch_prefill_t<CF, 8>(a, s, t);
}

}  // namespace

hipError_t launch_down_prefill(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    switch (cf_of(a.routed.fmt, a.routed.bits)) {
        case 4: return launch_down_prefill_t<4>(a, s, t);
        case 8: return launch_down_prefill_t<8>(a, s, t);
        case kCfFp8: return launch_down_prefill_t<kCfFp8>(a, s, t);
        default: return launch_down_prefill_t<kCfMx4>(a, s, t);
    }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    switch (cf_of(a.routed.fmt, a.routed.bits)) {
        case 4: return launch_prefill_cf<4>(a, s, t);
        case 8: return launch_prefill_cf<8>(a, s, t);
        case kCfFp8: return launch_prefill_cf<kCfFp8>(a, s, t);
        default: return launch_prefill_cf<kCfMx4>(a, s, t);
    }
}

}  // namespace w4a16
