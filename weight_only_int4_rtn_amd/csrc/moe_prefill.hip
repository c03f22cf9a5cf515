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
// Codes enter the MFMA as exact bf16 integers (see dq4 / dq8 in common.h): the
// accumulator of a group starts from -OFF * (sum of the group's activations) and the
// group scale multiplies the fp32 partial.
//
// Routed items (code width BITS) and the shared expert's items (SBITS) are walked as two
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
// 0, 1 are gate rows, 2, 3 the matching up rows.
__device__ __forceinline__ int gk_code_row(int R, int nblk, int64_t I_e) {
    const int wn = R >> 6, b = (R >> 4) & 3, ml = R & 15;
    return (b >= 2 ? (int)I_e : 0) + nblk * kGroup + 32 * wn + 16 * (b & 1) + ml;
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

template <int BITS, bool GATE_UP>
__device__ void prepare_issue(const PrefillArgs& a, const Item& it, const ExpertSet& es, const int (&tok)[5],
                              IssueState& st) {
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
            st.b_off[j] = (uint32_t)(gk_code_row(R, it.nblk, I_e) * row_bytes) + c * 16;
        }
        st.seed_r = dma_rsrc(a.xsum, (uint32_t)(a.T * G * 4));
        st.seed_off = lane < 16 ? (uint32_t)tok[4] * G * 4 : kOob;
        st.s_r = dma_rsrc(es.s13 + eb * 2 * I_e * G, (uint32_t)(2 * I_e * G * 2));
        st.s_off = lane < 32 ? (uint32_t)(gk_code_row(32 * wave + lane, it.nblk, I_e) * G * 2) : kOob;
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
        const int h0 = it.nblk * NT;   // rows past H read zeros (the buffer ends at H)
        st.b_r = dma_rsrc(es.w2 + eb * (a.H * I_e * BITS / 32), (uint32_t)(a.H * row_bytes));
#pragma unroll
        for (int j = 0; j < P::kBLoads; ++j) {
            int R, c;
            b_coords<BITS>(j, &R, &c);
            st.b_off[j] = (uint32_t)((h0 + R) * row_bytes) + c * 16;
        }
        st.seed_r = dma_rsrc(a.asum, (uint32_t)(a.rows_a * GW * 4));
        st.seed_off = lane < 16 ? (uint32_t)(it.orow0 + min(16 * wave + lane, it.count - 1)) * GW * 4 : kOob;
        st.s_r = dma_rsrc(es.s2 + eb * a.H * G2, (uint32_t)(a.H * G2 * 2));
        st.s_off = lane < 32 ? (uint32_t)((h0 + 32 * wave + lane) * G2 * 2) : kOob;
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

// stage: LDS byte address of the stage the step goes to.
template <int BITS>
__device__ __forceinline__ void issue_step(const IssueState& st, int g, uint32_t stage) {
    using P = Pipe<BITS>;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t A = stage, B = stage + kAStageBytes, S = B + P::kBStageBytes, SC = S + kSeedSlots * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(st.a_r, A + (wave * 4 + j) * 1024, st.a_off[j], (uint32_t)g * kGroup * 2);
#pragma unroll
    for (int j = 0; j < P::kBLoads; ++j)
        dma16(st.b_r, B + (wave * P::kBLoads + j) * 1024, st.b_off[j], (uint32_t)g * P::kRowBytes);
    dma4(st.seed_r, S + wave * 256, st.seed_off, (uint32_t)g * 4);
    dma4(st.s_r, SC + wave * 256, (st.s_off + (uint32_t)g * 2) & ~3u, 0);
}

// ------------------------------------------------------------------- compute

// One step of one wave: its 64 x 64 block (4 M-subtiles x 4 code subtiles) for one
// group, accumulated into acc with the group scales (D column ml is code row R's).
// sodd: bit b set when code subtile b's scale sits in the high half of its word.
template <int BITS>
__device__ __forceinline__ void compute_step(const uint8_t* stage, uint32_t sodd, f32x4_t (&acc)[4][4]) {
    using P = Pipe<BITS>;
    constexpr float kOff = BITS == 4 ? 136.0f : 2304.0f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(stage);
    const uint8_t* B = stage + kAStageBytes;
    const float* S = reinterpret_cast<const float*>(B + P::kBStageBytes);
    const uint32_t* SC = reinterpret_cast<const uint32_t*>(S + kSeedSlots);
    const uint32_t M = nibble_mask();

    u32x4_t av[4][4];
    f32x4_t seed[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = 64 * wm + 16 * mi + ml;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[mi][i] = *reinterpret_cast<const u32x4_t*>(A + a_swz(r, 4 * q + i) * 8);
        const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(S + seed_slot(64 * wm + 16 * mi + 4 * q));
#pragma unroll
        for (int e = 0; e < 4; ++e) seed[mi][e] = -kOff * xs[e];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int R = 64 * wn + 16 * b + ml;
        u32x4_t braw[BITS / 4];
#pragma unroll
        for (int c = 0; c < BITS / 4; ++c) {
            const int lc = (BITS / 4) * q + c;   // logical chunk: this lane's K slice
            braw[c] = *reinterpret_cast<const u32x4_t*>(B + R * P::kRowBytes + ((lc ^ b_swizzle<BITS>(R)) * 16));
        }
        const uint32_t sw = SC[scale_slot(R)];
        const float sc = bf16_to_f32(((sodd >> b) & 1) ? (sw >> 16) : (sw & 0xffffu));
        f32x4_t t[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) t[mi] = seed[mi];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4_t lo, hi;
            if constexpr (BITS == 4) {
                lo = dq4(braw[0][i], M);
            } else {
                dq8(braw[i >> 1][(2 * i) & 3], braw[i >> 1][(2 * i + 1) & 3], lo, hi, M);
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                t[mi] = mfma16(av[mi][i], lo, t[mi]);
                if constexpr (BITS == 8) t[mi] = mfma16(av[mi][i], hi, t[mi]);
            }
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) acc[mi][b][r2] += sc * t[mi][r2];
    }
}

// ------------------------------------------------------------------- epilogues

// a = SiLU(gate) * up for the item's 128 x 128 block, bf16, columns in the reordered K
// order of the down GEMM; and each row's fp32 sum of those bf16 values (one group of I).
__device__ void gk_epilogue(const PrefillArgs& a, const Item& it, const f32x4_t (&acc)[4][4], float* s_asum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const int GW = (int)(a.width_a / kGroup);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * wm + 16 * mi + 4 * q + r;
            float rs = 0.f;
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const uint32_t v = cvt_bf16(silu_mul(acc[mi][ns][r], acc[mi][2 + ns][r]));
                rs += bf16_to_f32(v);
                if (m < it.count) {
                    const int col = perm_pos(it.nblk * kGroup + 32 * wn + 16 * ns + ml);
                    a.abuf[(int64_t)(it.orow0 + m) * a.width_a + col] = (uint16_t)v;
                }
            }
            rs += __shfl_xor(rs, 1, 16);   // sum over the row's 16 lanes (columns ml)
            rs += __shfl_xor(rs, 2, 16);
            rs += __shfl_xor(rs, 4, 16);
            rs += __shfl_xor(rs, 8, 16);
            if (ml == 0) s_asum[wn * MT + m] = rs;
        }
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

// The unweighted output rows of a down item, rounded to bf16, at their sorted positions
// (pairs of adjacent columns, exchanged between neighbouring lanes, go out as 4 bytes).
__device__ void dk_epilogue(const PrefillArgs& a, const Item& it, const f32x4_t (&acc)[4][4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, ml = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const int h = it.nblk * NT + 64 * wn + ml;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * wm + 16 * mi + 4 * q + r;
            uint16_t* yrow = a.ystage + (int64_t)(it.orow0 + m) * a.H;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t v = cvt_bf16(acc[mi][b][r]);
                // the neighbouring column: DPP quad_perm [1,0,3,2] swaps adjacent lanes
                const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xb1, 0xf, 0xf, false);
                // even lanes store (col, col + 1); the row and columns are in range for both lanes
                if (m < it.count && (ml & 1) == 0 && h + 16 * b < a.H)
                    *reinterpret_cast<uint32_t*>(yrow + h + 16 * b) = v | (nb << 16);
            }
        }
}

// --------------------------------------------------------------------- driver

// One walk: workgroup b takes items w = b, b + grid, ... of `total` (item index L is
// remapped so that each XCD, w mod 8, takes one contiguous range: an expert's tiles share
// that XCD's L2).  The items are resolved once into LDS; the steps of all of them form
// one pipelined stream.
template <int BITS, bool GATE_UP, bool SHARED>
__device__ void run_items(const PrefillArgs& a, const ExpertSet& es, int nb, int total, uint8_t* smem,
                          Item* s_items, float* s_asum, int* s_cnt, int* s_tok) {
    using P = Pipe<BITS>;
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
    prepare_issue<BITS, GATE_UP>(a, s_items[0], es, tok, st);
    const uint32_t lds0 = lds_offset(smem);
    auto issue_next = [&]() {
        issue_step<BITS>(st, gi, lds0 + (uint32_t)(issued % P::kStages) * P::kStageBytes);
        ++issued;
        if (++gi == G && ii + 1 < n_items) {
            ++ii;
            gi = 0;
            if constexpr (GATE_UP) {
                item_tokens(s_items[ii], s_tok + (ii & 1) * MT, tok);
                if (__builtin_amdgcn_readfirstlane(wave) == 0 && ii + 1 < n_items)
                    copy_item_tokens(a, s_items[ii + 1], lds_tok + ((ii + 1) & 1) * MT * 4);
            }
            prepare_issue<BITS, GATE_UP>(a, s_items[ii], es, tok, st);
        }
    };
    for (int p = 0; p < P::kStages - 1 && issued < total_steps; ++p) issue_next();

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
            const int crow = GATE_UP ? gk_code_row(R, it.nblk, es.I) : it.nblk * NT + R;
            p |= (uint32_t)((crow * G) & 1) << b;
        }
        return p;
    };
    uint32_t cpar = row_parity(s_items[0]);
    // An item's epilogue runs after the next step's wait and barrier, before that step's
    // copies go out: its stores are then older than every copy batch still awaited, so
    // the in-order vmcnt waits never hold a batch back behind them.
    bool epi = false;
    auto finish_item = [&]() {   // the item before ci (its record stays in LDS)
        const Item eit = s_items[ci - 1];
        if constexpr (GATE_UP) gk_epilogue(a, eit, acc, s_asum);
        else dk_epilogue(a, eit, acc);
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
        if (issued < total_steps) issue_next();
        compute_step<BITS>(smem + (s % P::kStages) * P::kStageBytes, (gc & 1) ? (cpar ^ 0xfu) : cpar, acc);
        if (++gc == G) {
            epi = true;
            gc = 0;
            if (++ci < n_items) cpar = row_parity(s_items[ci]);
        }
    }
    if (epi) finish_item();
}

template <int BITS>
constexpr uint32_t pipe_lds_bytes() {
    return Pipe<BITS>::kStages * Pipe<BITS>::kStageBytes;
}

}  // namespace

// Dynamic LDS: the stages of the larger pipeline, then the item list and the row-sum
// scratch.
template <int BITS, int SBITS>
__global__ __launch_bounds__(kPThreads) void gk_prefill_kernel(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr uint32_t kPipe = std::max(pipe_lds_bytes<BITS>(), SBITS ? pipe_lds_bytes<SBITS>() : 0u);
    Item* s_items = reinterpret_cast<Item*>(smem + kPipe);
    float* s_asum = reinterpret_cast<float*>(s_items + kMaxItems);
    int* s_tok = reinterpret_cast<int*>(s_asum + 4 * MT);   // two items' tokens
    __shared__ int s_cnt[kPWaves];
    const int nb = (int)(a.routed.I / kGroup);
    run_items<BITS, true, false>(a, a.routed, nb, a.meta[1] * nb, smem, s_items, s_asum, s_cnt, s_tok);
    if constexpr (SBITS != 0) {
        const int nbs = (int)(a.shared.I / kGroup);
        run_items<SBITS, true, true>(a, a.shared, nbs, ((a.T + MT - 1) / MT) * nbs, smem, s_items, s_asum, s_cnt,
                                     s_tok);
    }
}

template <int BITS, int SBITS>
__global__ __launch_bounds__(kPThreads) void dk_prefill_kernel(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr uint32_t kPipe = std::max(pipe_lds_bytes<BITS>(), SBITS ? pipe_lds_bytes<SBITS>() : 0u);
    Item* s_items = reinterpret_cast<Item*>(smem + kPipe);
    float* s_asum = reinterpret_cast<float*>(s_items + kMaxItems);
    __shared__ int s_cnt[kPWaves];
    const int nb = (int)((a.H + NT - 1) / NT);
    run_items<BITS, false, false>(a, a.routed, nb, a.meta[1] * nb, smem, s_items, s_asum, s_cnt, nullptr);
    if constexpr (SBITS != 0)
        run_items<SBITS, false, true>(a, a.shared, nb, ((a.T + MT - 1) / MT) * nb, smem, s_items, s_asum, s_cnt,
                                      nullptr);
}

// y[t] = sum over slots j in order of w[t, j] times the staged row of pair (t, j), then
// the shared expert's row, then the residual; rounded once to bf16.  A token's row is
// split over ceil(H / 2048) blocks of 256 threads x 8 columns.  No atomics anywhere.
__global__ __launch_bounds__(256) void finalize_kernel(PrefillArgs a) {
    const int nbx = (int)((a.H / 8 + 255) / 256);
    const int t = (int)(blockIdx.x / nbx);
    const int64_t c = ((int64_t)(blockIdx.x % nbx) * blockDim.x + threadIdx.x) * 8;
    if (c >= a.H) return;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add_row = [&](int64_t row, float w) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.ystage + row * a.H + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[2 * e] += w * bf16_to_f32(v[e] & 0xffffu);
            s[2 * e + 1] += w * bf16_to_f32(v[e] >> 16);
        }
    };
    for (int j = 0; j < a.k; ++j) {
        const int pos = a.inv[(int64_t)t * a.k + j];
        if (pos >= 0) add_row(pos, a.wts[(int64_t)t * a.k + j]);
    }
    if (a.shared.bits) add_row((int64_t)a.T * a.k + t, 1.0f);
    const int64_t o = (int64_t)t * a.H + c;
    if (a.residual) {
        const u32x4_t r = *reinterpret_cast<const u32x4_t*>(a.residual + o);
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

template <int BITS, int SBITS>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    constexpr uint32_t kPipe = std::max(pipe_lds_bytes<BITS>(), SBITS ? pipe_lds_bytes<SBITS>() : 0u);
    constexpr uint32_t lds = kPipe + kMaxItems * sizeof(Item) + 4 * MT * 4 + 2 * MT * 4;
    static_assert(lds + 64 <= 160 * 1024, "LDS budget of one workgroup");
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gk_prefill_kernel<BITS, SBITS>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dk_prefill_kernel<BITS, SBITS>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        return true;
    }();
    (void)attr;
    const int64_t shared_tiles = SBITS ? (a.T + MT - 1) / MT : 0;
    const int64_t gk_items = std::max(a.max_tiles * (a.routed.I / kGroup), shared_tiles * (a.shared.I / kGroup));
    const int64_t dk_items = std::max(a.max_tiles, shared_tiles) * ((a.H + NT - 1) / NT);
    launch(t, "gk_prefill", gk_prefill_kernel<BITS, SBITS>, dim3(prefill_grid(gk_items)), dim3(kPThreads), s, lds, a);
    launch(t, "dk_prefill", dk_prefill_kernel<BITS, SBITS>, dim3(prefill_grid(dk_items)), dim3(kPThreads), s, lds, a);
    launch(t, "finalize", finalize_kernel, dim3((unsigned)((a.H / 8 + 255) / 256 * a.T)), dim3(256), s, 0u, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, StageTimer* t) {
    const int sb = a.shared.bits;
    if (a.routed.bits == 4) {
        if (sb == 0) return launch_prefill_t<4, 0>(a, s, t);
        if (sb == 4) return launch_prefill_t<4, 4>(a, s, t);
        return launch_prefill_t<4, 8>(a, s, t);
    }
    if (sb == 0) return launch_prefill_t<8, 0>(a, s, t);
    if (sb == 4) return launch_prefill_t<8, 4>(a, s, t);
    return launch_prefill_t<8, 8>(a, s, t);
}

}  // namespace w4a16
