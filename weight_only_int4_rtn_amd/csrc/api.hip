// Host side of the C ABI declared in include/w4a16.h: argument validation, workspace
// layout and kernel dispatch.  Nothing here allocates device memory; only the timed forward
// and the workspace check synchronise (both documented as doing so).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "common.h"
#include "w4a16.h"

using namespace w4a16;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_status(hipError_t err, const char* what) {
    if (err == hipSuccess) return W4A16_OK;
    return fail(W4A16_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Shape checks shared by the workspace query and the forward call.
int check_shapes(const moe_w4a16_args* a) {
    if (!a) return fail(W4A16_ERR_INVALID_ARG, "args is NULL");
    if (a->T < 0) return fail(W4A16_ERR_INVALID_ARG, "T = %lld < 0", (long long)a->T);
    if (a->group != kGroup) return fail(W4A16_ERR_INVALID_ARG, "group = %d, only 128 is supported", a->group);
    if (a->bits != 4 && a->bits != 8) return fail(W4A16_ERR_INVALID_ARG, "bits = %d, must be 4 or 8", a->bits);
    if (a->H <= 0 || a->H % kGroup) return fail(W4A16_ERR_INVALID_ARG, "H = %lld is not a positive multiple of 128", (long long)a->H);
    if (a->I <= 0 || a->I % kGroup) return fail(W4A16_ERR_INVALID_ARG, "I = %lld is not a positive multiple of 128", (long long)a->I);
    if (a->E < 1) return fail(W4A16_ERR_INVALID_ARG, "E = %lld < 1", (long long)a->E);
    if (a->top_k < 1 || a->top_k > a->E) return fail(W4A16_ERR_INVALID_ARG, "top_k = %lld not in [1, E]", (long long)a->top_k);
    if (a->H > 16384) return fail(W4A16_ERR_UNSUPPORTED, "H = %lld > 16384", (long long)a->H);
    if (a->I > 8192) return fail(W4A16_ERR_UNSUPPORTED, "I = %lld > 8192", (long long)a->I);
    if (a->E > 1024) return fail(W4A16_ERR_UNSUPPORTED, "E = %lld > 1024", (long long)a->E);
    if (a->top_k > 16) return fail(W4A16_ERR_UNSUPPORTED, "top_k = %lld > 16", (long long)a->top_k);
    if (a->T * a->top_k >= (int64_t(1) << 31) || a->T >= (int64_t(1) << 24))
        return fail(W4A16_ERR_UNSUPPORTED, "T = %lld too large", (long long)a->T);
    // staged activation arrays and one expert's codes are addressed with 32-bit byte offsets
    if (a->T * a->H * 2 >= (int64_t(1) << 32) ||
        (a->T + a->T * a->top_k) * std::max(a->I, a->shared_bits ? a->shared_I : (int64_t)0) * 2 >= (int64_t(1) << 32))
        return fail(W4A16_ERR_UNSUPPORTED, "T = %lld too large for these shapes", (long long)a->T);
    if (a->weight_format < W4A16_FORMAT_INT || a->weight_format > W4A16_FORMAT_MXFP4)
        return fail(W4A16_ERR_INVALID_ARG, "weight_format = %d", a->weight_format);
    if (a->weight_format == W4A16_FORMAT_FP8_E4M3 && a->bits != 8)
        return fail(W4A16_ERR_INVALID_ARG, "FP8 E4M3 experts have 8-bit codes: bits = %d", a->bits);
    if (a->weight_format == W4A16_FORMAT_MXFP4 && a->bits != 4)
        return fail(W4A16_ERR_INVALID_ARG, "MXFP4 experts have 4-bit codes: bits = %d", a->bits);
    if (a->shared_bits != 0) {
        if (a->shared_bits != 4 && a->shared_bits != 8)
            return fail(W4A16_ERR_INVALID_ARG, "shared_bits = %d, must be 0, 4 or 8", a->shared_bits);
        if (a->shared_I <= 0 || a->shared_I % kGroup)
            return fail(W4A16_ERR_INVALID_ARG, "shared_I = %lld is not a positive multiple of 128", (long long)a->shared_I);
        if (a->shared_I > 8192) return fail(W4A16_ERR_UNSUPPORTED, "shared_I = %lld > 8192", (long long)a->shared_I);
    }
    return W4A16_OK;
}

// Offsets of every scratch buffer inside the caller's workspace.
WsLayout layout(const moe_w4a16_args* a) {
    WsLayout L{};
    const int64_t T = a->T, H = a->H, E = a->E, k = a->top_k, P = T * k;
    const bool shared = a->shared_bits != 0;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L.sync = take(kHeadBytes);
    L.ids = take(P * 4);
    L.wts = take(P * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.sorted = take(P * 4);
    L.active = take(E * 4);
    L.meta = take(64);
    L.tokw = take(P * 8);
    L.rec = take(std::min(E, P) * 16);
    L.trec = take((std::min(E, P) + P / 16 + 1) * 32);
    L.rows_a = P + (shared ? T : 0);
    L.width_a = std::max(a->I, shared ? a->shared_I : (int64_t)0);
    L.abuf = take((size_t)L.rows_a * L.width_a * 2);
    L.logits = take((size_t)T * E * 4);   // router logits computed from x
    L.gate = take((size_t)T * 4);         // shared-expert gate values
    if (T <= kSmallT) {
        // down-kernel work units: 2-group K chunks of every expert that can be active
        auto chunks = [](int64_t I_e) { return (I_e / kGroup + 1) / 2; };
        const int64_t units = std::min(E, P) * chunks(a->I) + (shared ? chunks(a->shared_I) : 0);
        L.splits = (int)std::min<int64_t>(16, std::max<int64_t>(1, (units + 15) / 16));
        if (L.splits > 1) L.part = take((size_t)L.splits * T * H * 4);
        L.ystage = take((size_t)L.rows_a * H * 4);   // streaming down projection: fp32 rows
        L.inv = take(P * 4);
    } else {
        L.splits = 1;
        L.nblk = (int)((T + kRouteBlockT - 1) / kRouteBlockT);
        L.hist = take((size_t)L.nblk * E * 4);
        L.lrank = take(P * 4);
        L.max_tiles = (P + kPrefillMT - 1) / kPrefillMT + std::min(E, P);
        L.tiles = take((size_t)L.max_tiles * 8);
        L.xsum = take((size_t)T * (H / kGroup) * 4);
        L.xp = take((size_t)T * H * 2);
        L.ystage = take((size_t)L.rows_a * H * 2);
        L.asum = take((size_t)L.rows_a * (L.width_a / kGroup) * 4);
        L.inv = take(P * 4);
    }
    L.total = off;
    return L;
}

int forward_impl(const moe_w4a16_args* a, void* stream, StageTimer* timer, bool allow_coop = true) {
    if (int st = check_shapes(a)) return st;
    if (a->flags & ~W4A16_FLAG_NO_COOPERATIVE) return fail(W4A16_ERR_INVALID_ARG, "unknown flags 0x%x", a->flags);
    if (a->flags & W4A16_FLAG_NO_COOPERATIVE) allow_coop = false;
    if (a->T == 0) return W4A16_OK;
    if (!a->x || !a->w13 || !a->s13 || !a->w2 || !a->s2 || !a->y)
        return fail(W4A16_ERR_INVALID_ARG, "NULL x, w13, s13, w2, s2 or y");
    if (a->router_w && a->router_logits)
        return fail(W4A16_ERR_INVALID_ARG, "router_w and router_logits are exclusive");
    if (!a->router_logits && !a->router_w && (!a->topk_ids || !a->topk_w))
        return fail(W4A16_ERR_INVALID_ARG, "no router_logits or router_w, so topk_ids and topk_w must be given");
    if (a->shared_gate_w && !a->shared_bits)
        return fail(W4A16_ERR_INVALID_ARG, "shared_gate_w needs a shared expert");
    if (a->shared_bits && (!a->shared_w13 || !a->shared_s13 || !a->shared_w2 || !a->shared_s2))
        return fail(W4A16_ERR_INVALID_ARG, "NULL shared expert pointer");
    const void* ptrs[] = {a->x, a->router_logits, a->w13, a->s13, a->w2, a->s2, a->shared_w13, a->shared_s13,
                          a->shared_w2, a->shared_s2, a->residual, a->y, a->topk_ids, a->topk_w,
                          a->expert_counts, a->expert_offsets, a->sorted_pairs, a->workspace,
                          a->router_w, a->shared_gate_w, a->logits_out, a->shared_gate_out};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(W4A16_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (a->y == a->x) return fail(W4A16_ERR_INVALID_ARG, "y must not alias x");

    const WsLayout L = layout(a);
    if (!a->workspace || a->workspace_bytes < L.total)
        return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    char* ws = static_cast<char*>(a->workspace);
    auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
    hipStream_t s = static_cast<hipStream_t>(stream);

    // router logits and the shared expert's gate from x, ahead of everything else
    const float* logits_in = a->router_logits;
    const float* shared_gate = nullptr;
    if (a->router_w || a->shared_gate_w) {
        RouterArgs ra{};
        ra.x = a->x;
        ra.wr = a->router_w;
        ra.wg = a->shared_gate_w;
        ra.T = (int)a->T;
        ra.n_router = a->router_w ? (int)a->E : 0;
        ra.H = a->H;
        ra.logits = a->logits_out ? a->logits_out : static_cast<float*>(at(L.logits));
        ra.gate = a->shared_gate_out ? a->shared_gate_out : static_cast<float*>(at(L.gate));
        if (int st = hip_status(launch_router(ra, s, timer), "router launch")) return st;
        if (a->router_w) logits_in = ra.logits;
        if (a->shared_gate_w) shared_gate = ra.gate;
    }

    RouteArgs r{};
    r.logits = logits_in;
    r.T = (int)a->T;
    r.E = (int)a->E;
    r.k = (int)a->top_k;
    r.ids = a->topk_ids ? a->topk_ids : static_cast<int32_t*>(at(L.ids));
    r.wts = a->topk_w ? a->topk_w : static_cast<float*>(at(L.wts));
    r.counts = a->expert_counts ? a->expert_counts : static_cast<int32_t*>(at(L.counts));
    r.offsets = a->expert_offsets ? a->expert_offsets : static_cast<int32_t*>(at(L.offsets));
    r.sorted = a->sorted_pairs ? a->sorted_pairs : static_cast<int32_t*>(at(L.sorted));
    r.active = static_cast<int32_t*>(at(L.active));
    r.meta = static_cast<int32_t*>(at(L.meta));
    r.x = a->x;
    r.H = a->H;
    r.tokw = static_cast<int2*>(at(L.tokw));
    r.inv = L.inv ? static_cast<int32_t*>(at(L.inv)) : nullptr;
    r.rec = static_cast<int4*>(at(L.rec));
    r.trec = static_cast<int4*>(at(L.trec));
    r.max_slots = (int)std::min(a->E, a->T * a->top_k);

    ExpertSet routed{a->w13, a->s13, a->w2, a->s2, a->I, a->bits, a->weight_format};
    ExpertSet shared{a->shared_w13, a->shared_s13, a->shared_w2, a->shared_s2, a->shared_I, a->shared_bits, 0};
    uint16_t* abuf = static_cast<uint16_t*>(at(L.abuf));

    // single launch for tiny batches when the tagged a words fit the workspace head, the
    // down workgroups' LDS (y accumulators, every a row padded, a zero block, group sums) stays
    // small enough for two workgroups per CU, and the spinning down workgroups leave room
    const size_t tag_bytes = (size_t)L.rows_a * L.width_a * 4;
    const size_t tiny_lds = 8 * (size_t)a->T * 16 * 4 + (size_t)L.rows_a * (L.width_a + kTinyPad) * 2 + 1024 +
                            (size_t)L.rows_a * (L.width_a / kGroup) * 4;
    if (allow_coop && a->T * a->top_k <= kTinyP && a->H <= kTinyMaxH && tag_bytes <= kTagBytes &&
        tiny_lds <= kTinyMaxLds &&
        a->H / 16 <= tiny_max_down_workgroups(a->weight_format, a->bits, a->shared_bits)) {
        TinyArgs d{};
        d.x = a->x;
        d.T = (int)a->T;
        d.E = (int)a->E;
        d.k = (int)a->top_k;
        d.H = a->H;
        d.routed = routed;
        d.shared = shared;
        d.logits = logits_in;
        d.ids = r.ids;
        d.wts = r.wts;
        d.counts = r.counts;
        d.offsets = r.offsets;
        d.sorted = r.sorted;
        d.sync = static_cast<uint32_t*>(at(L.sync));
        d.tags = d.sync + kSyncBytes / 4;
        d.width_a = L.width_a;
        d.rows_a = (int)L.rows_a;
        d.tag_bytes = (uint32_t)tag_bytes;
        d.residual = a->residual;
        d.shared_gate = shared_gate;
        d.y = a->y;
        const int64_t slots = a->T * a->top_k + (a->shared_bits ? 1 : 0);   // one per pair, + the shared expert
        d.n_rb = (int)(L.width_a / 16);
        d.n_gk = (int)(slots * d.n_rb);
        d.lds_bytes = (uint32_t)std::max<size_t>(8 * 8 * 64 * 4, tiny_lds);   // gate/up: partial sums
        return hip_status(launch_tiny(d, s, timer), "decode launch");
    }
    if (a->T <= kSmallT) {
        DecodeArgs d{};
        d.x = a->x;
        d.T = (int)a->T;
        d.E = (int)a->E;
        d.k = (int)a->top_k;
        d.H = a->H;
        d.routed = routed;
        d.shared = shared;
        d.ids = r.ids;
        d.wts = r.wts;
        d.offsets = r.offsets;
        d.sorted = r.sorted;
        d.active = r.active;
        d.meta = r.meta;
        d.rec = r.rec;
        d.trec = r.trec;
        d.tokw = r.tokw;
        d.abuf = abuf;
        d.width_a = L.width_a;
        d.part = L.splits > 1 ? static_cast<float*>(at(L.part)) : nullptr;
        d.splits = L.splits;
        d.inv = r.inv;
        d.ystage = static_cast<float*>(at(L.ystage));
        d.rows_a = L.rows_a;
        d.route = r;
        if (pair_fits(d)) {   // the gate/up kernel's workgroup 0 routes; a rows in pair order
            d.a_by_pair = 1;
            d.gk_stream = 1;
            d.route.pair_rows = 1;
        } else if (logits_in && a->T > kSplitRouteT) {
            // routing spread over waves (one token each) in its own launch; the streaming
            // gate/up kernel, if it takes the shapes, then reads the tile records
            r.sync = static_cast<uint32_t*>(at(L.sync));
            d.route = r;
            d.gk_stream = stream_fits(d, (int)(std::min(a->E, a->T * a->top_k) + a->T * a->top_k / 16)) ? 1 : 0;
            if (int st = hip_status(launch_route_split(r, s, timer), "routing launch")) return st;
        } else {
            d.fused_route = stream_fits(d, (int)(std::min(a->E, a->T * a->top_k) + a->T * a->top_k / 16)) ? 1 : 0;
            d.gk_stream = d.fused_route;
            if (!d.fused_route)
                if (int st = hip_status(launch_route_small(r, s, timer), "routing launch")) return st;
        }
        d.residual = a->residual;
        d.shared_gate = shared_gate;
        d.y = a->y;
        return hip_status(launch_decode(d, s, timer), "decode launch");
    }

    r.hist = static_cast<int32_t*>(at(L.hist));
    r.lrank = static_cast<int32_t*>(at(L.lrank));
    r.tiles = static_cast<int32_t*>(at(L.tiles));
    r.xsum = static_cast<float*>(at(L.xsum));
    r.xp = static_cast<uint16_t*>(at(L.xp));
    r.nblk = L.nblk;
    r.max_tiles = L.max_tiles;
    if (int st = hip_status(launch_route_large(r, s, timer), "routing launch")) return st;
    PrefillArgs p{};
    p.x = a->x;
    p.T = (int)a->T;
    p.E = (int)a->E;
    p.k = (int)a->top_k;
    p.H = a->H;
    p.routed = routed;
    p.shared = shared;
    p.ids = r.ids;
    p.wts = r.wts;
    p.offsets = r.offsets;
    p.sorted = r.sorted;
    p.meta = r.meta;
    p.tiles = r.tiles;
    p.tokw = r.tokw;
    p.max_tiles = L.max_tiles;
    p.xsum = r.xsum;
    p.xp = r.xp;
    p.abuf = abuf;
    p.rows_a = L.rows_a;
    p.width_a = L.width_a;
    p.ystage = static_cast<uint16_t*>(at(L.ystage));
    p.asum = static_cast<float*>(at(L.asum));
    p.inv = r.inv;
    p.residual = a->residual;
    p.shared_gate = shared_gate;
    p.y = a->y;
    return hip_status(launch_prefill(p, s, timer), "prefill launch");
}

// ------------------------------------------------------------ allocation-free entry point
//
// The scratch of moe_w4a16_forward_noalloc: one array per GPU, in the code object, held
// until the process ends.  Host code never passes `scratch` itself (on the host it names a
// stand-in, not device memory): each device's address comes from hipGetSymbolAddress,
// taken once with that device current, and only that address reaches kernels.
static __device__ __align__(256) char scratch[W4A16_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's scratch address; on first use per device also zeroes its workspace
// head on `s` (a fill kernel, so a captured first call stays valid on replay).
int scratch_for_current_device(hipStream_t s, void** out) {
    int dev = -1;
    if (int st = hip_status(hipGetDevice(&dev), "hipGetDevice")) return st;
    if (dev < 0 || dev >= kMaxDevices) return fail(W4A16_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    std::call_once(g_scratch_once[dev], [&] {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e == hipSuccess) e = launch_head_init(static_cast<uint32_t*>(p), s);
        g_scratch_err[dev] = e;
        g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess)
        return hip_status(g_scratch_err[dev], "setting up the static scratch");
    *out = g_scratch_ptr[dev];
    return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char* w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "W4A16_OK";
        case W4A16_ERR_INVALID_ARG: return "W4A16_ERR_INVALID_ARG";
        case W4A16_ERR_UNSUPPORTED: return "W4A16_ERR_UNSUPPORTED";
        case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE";
        case W4A16_ERR_HIP: return "W4A16_ERR_HIP";
        case W4A16_ERR_TIMEOUT: return "W4A16_ERR_TIMEOUT";
        default: return "W4A16_UNKNOWN_STATUS";
    }
}

const char* w4a16_last_error(void) { return g_last_error.c_str(); }

int rtn_quantize_pack(const void* w, int w_dtype, int64_t n_mats, int64_t rows, int64_t cols, int bits, int group,
                      int32_t* packed, uint16_t* scales, void* stream) {
    g_last_error.clear();
    if (w_dtype != W4A16_F32 && w_dtype != W4A16_BF16) return fail(W4A16_ERR_INVALID_ARG, "w_dtype = %d", w_dtype);
    if (bits != 4 && bits != 8) return fail(W4A16_ERR_INVALID_ARG, "bits = %d, must be 4 or 8", bits);
    if (group != kGroup) return fail(W4A16_ERR_INVALID_ARG, "group = %d, only 128 is supported", group);
    if (n_mats < 0 || rows < 0 || cols < 0) return fail(W4A16_ERR_INVALID_ARG, "negative size");
    if (cols % kGroup) return fail(W4A16_ERR_INVALID_ARG, "cols = %lld is not a multiple of 128", (long long)cols);
    if (n_mats != 0 && rows > INT64_MAX / n_mats) return fail(W4A16_ERR_INVALID_ARG, "size overflow");
    const int64_t total_rows = n_mats * rows;
    if (total_rows == 0 || cols == 0) return W4A16_OK;
    if (cols > (int64_t(1) << 40) / total_rows) return fail(W4A16_ERR_UNSUPPORTED, "matrix too large");
    if (!w || !packed || !scales) return fail(W4A16_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(w) || !aligned16(packed) || !aligned16(scales))
        return fail(W4A16_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    return hip_status(launch_quantize(w, w_dtype == W4A16_BF16, total_rows, cols, bits, packed, scales,
                                      static_cast<hipStream_t>(stream)),
                      "rtn_quantize_pack launch");
}

// Shared host checks of the format quantizers; 0 when the call may go ahead (or is empty).
static int check_quant_args(const void* w, int w_dtype, int64_t n_mats, int64_t rows, int64_t cols, int col_mult,
                            const void* packed, const void* scales, bool* empty) {
    *empty = false;
    if (w_dtype != W4A16_F32 && w_dtype != W4A16_BF16) return fail(W4A16_ERR_INVALID_ARG, "w_dtype = %d", w_dtype);
    if (n_mats < 0 || rows < 0 || cols < 0) return fail(W4A16_ERR_INVALID_ARG, "negative size");
    if (cols % col_mult) return fail(W4A16_ERR_INVALID_ARG, "cols = %lld is not a multiple of %d", (long long)cols, col_mult);
    if (n_mats != 0 && rows > INT64_MAX / n_mats) return fail(W4A16_ERR_INVALID_ARG, "size overflow");
    const int64_t total_rows = n_mats * rows;
    if (total_rows == 0 || cols == 0) {
        *empty = true;
        return W4A16_OK;
    }
    if (cols > (int64_t(1) << 40) / total_rows || total_rows >= (int64_t(1) << 31))
        return fail(W4A16_ERR_UNSUPPORTED, "matrix too large");
    if (!w || !packed || !scales) return fail(W4A16_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(w) || !aligned16(packed) || !aligned16(scales))
        return fail(W4A16_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    return W4A16_OK;
}

int fp8_quantize_pack(const void* w, int w_dtype, int64_t n_mats, int64_t rows, int64_t cols, int32_t* packed,
                      float* scales, void* stream) {
    g_last_error.clear();
    bool empty;
    if (int st = check_quant_args(w, w_dtype, n_mats, rows, cols, 4, packed, scales, &empty)) return st;
    if (empty) return W4A16_OK;
    return hip_status(launch_fp8_quantize(w, w_dtype == W4A16_BF16, n_mats * rows, cols, packed, scales,
                                          static_cast<hipStream_t>(stream)),
                      "fp8_quantize_pack launch");
}

int mxfp4_quantize_pack(const void* w, int w_dtype, int64_t n_mats, int64_t rows, int64_t cols, int method,
                        int32_t* packed, uint8_t* scales, void* stream) {
    g_last_error.clear();
    if (method != W4A16_MXFP4_RTN && method != W4A16_MXFP4_MSE)
        return fail(W4A16_ERR_INVALID_ARG, "method = %d", method);
    bool empty;
    if (int st = check_quant_args(w, w_dtype, n_mats, rows, cols, 32, packed, scales, &empty)) return st;
    if (empty) return W4A16_OK;
    return hip_status(launch_mxfp4_quantize(w, w_dtype == W4A16_BF16, n_mats * rows, cols,
                                            method == W4A16_MXFP4_MSE, packed, scales,
                                            static_cast<hipStream_t>(stream)),
                      "mxfp4_quantize_pack launch");
}

// ------------------------------------------------------------------ dense projection

static int check_linear_shapes(int64_t T, int64_t K, int64_t N) {
    if (T < 0) return fail(W4A16_ERR_INVALID_ARG, "T = %lld < 0", (long long)T);
    if (K <= 0 || K % kGroup) return fail(W4A16_ERR_INVALID_ARG, "K = %lld is not a positive multiple of 128", (long long)K);
    if (N <= 0 || N % kGroup) return fail(W4A16_ERR_INVALID_ARG, "N = %lld is not a positive multiple of 128", (long long)N);
    if (K > 8192) return fail(W4A16_ERR_UNSUPPORTED, "K = %lld > 8192", (long long)K);
    if (N > 16384) return fail(W4A16_ERR_UNSUPPORTED, "N = %lld > 16384", (long long)N);
    if (T >= (int64_t(1) << 24) || T * K * 2 >= (int64_t(1) << 32) || T * N * 2 >= (int64_t(1) << 32))
        return fail(W4A16_ERR_UNSUPPORTED, "T = %lld too large for these shapes", (long long)T);
    return W4A16_OK;
}

struct LinearLayout {
    size_t abuf, asum, rec, meta, tokw, offsets, tiles, wts, inv, ystage, part, total;
    int splits;
};

static LinearLayout linear_layout(int64_t T, int64_t K, int64_t N) {
    LinearLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L.abuf = take((size_t)T * K * 2);
    L.rec = take(16);
    L.meta = take(64);
    L.tokw = take((size_t)T * 8);
    L.offsets = take(8);
    L.tiles = take((size_t)((T + kPrefillMT - 1) / kPrefillMT) * 8);
    L.wts = take((size_t)T * 4);
    L.inv = take((size_t)T * 4);
    if (T <= kSmallT) {
        const int64_t units = (K / kGroup + 1) / 2;   // the down kernel's 2-group K chunks
        L.splits = (int)std::min<int64_t>(16, std::max<int64_t>(1, (units + 15) / 16));
        if (L.splits > 1) L.part = take((size_t)L.splits * T * N * 4);
    } else {
        L.splits = 1;
        L.asum = take((size_t)T * (K / kGroup) * 4);
        L.ystage = take((size_t)T * N * 2);
    }
    L.total = off;
    return L;
}

size_t w4a16_linear_workspace_size(int64_t T, int64_t K, int64_t N) {
    g_last_error.clear();
    if (check_linear_shapes(T, K, N)) return 0;
    return std::max<size_t>(linear_layout(T, K, N).total, 256);
}

int w4a16_linear(const w4a16_linear_args* a, void* stream) {
    g_last_error.clear();
    if (!a) return fail(W4A16_ERR_INVALID_ARG, "args is NULL");
    if (int st = check_linear_shapes(a->T, a->K, a->N)) return st;
    if (a->group != kGroup) return fail(W4A16_ERR_INVALID_ARG, "group = %d, only 128 is supported", a->group);
    if (a->weight_format < W4A16_FORMAT_INT || a->weight_format > W4A16_FORMAT_MXFP4)
        return fail(W4A16_ERR_INVALID_ARG, "weight_format = %d", a->weight_format);
    const int want_bits = a->weight_format == W4A16_FORMAT_FP8_E4M3 ? 8 : a->weight_format == W4A16_FORMAT_MXFP4 ? 4 : 0;
    if ((a->bits != 4 && a->bits != 8) || (want_bits && a->bits != want_bits))
        return fail(W4A16_ERR_INVALID_ARG, "bits = %d for weight_format %d", a->bits, a->weight_format);
    if (a->T == 0) return W4A16_OK;
    if (!a->x || !a->w || !a->s || !a->y) return fail(W4A16_ERR_INVALID_ARG, "NULL x, w, s or y");
    const void* ptrs[] = {a->x, a->w, a->s, a->residual, a->y, a->workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(W4A16_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (a->y == a->x) return fail(W4A16_ERR_INVALID_ARG, "y must not alias x");
    const LinearLayout L = linear_layout(a->T, a->K, a->N);
    if (!a->workspace || a->workspace_bytes < L.total)
        return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    char* ws = static_cast<char*>(a->workspace);
    auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
    hipStream_t s = static_cast<hipStream_t>(stream);
    // small batches: one weight-streaming launch that reads x itself (the workspace is unused)
    if (const int cfg = linear_small_cfg(a->T, a->K, a->N, a->bits)) {
        const LinearSmall ls{a->x, a->w, static_cast<const uint8_t*>(a->s), a->residual, a->y, (int)a->T, a->K, a->N};
        return hip_status(launch_linear_small(ls, cf_of(a->weight_format, a->bits), cfg, s), "linear launch");
    }
    const bool small = a->T <= kSmallT;
    // 8-bit codes dequantise in natural column order in the grouped GEMM, which then reads x
    // itself; the other widths read x reordered into the codes' K order by the set-up kernel
    const bool natural = !small && a->bits == 8;

    LinearPrep p{};
    p.x = a->x;
    p.T = (int)a->T;
    p.K = a->K;
    p.abuf = natural ? nullptr : static_cast<uint16_t*>(at(L.abuf));
    p.asum = small ? nullptr : static_cast<float*>(at(L.asum));
    p.rec = static_cast<int4*>(at(L.rec));
    p.meta = static_cast<int32_t*>(at(L.meta));
    p.tokw = static_cast<int2*>(at(L.tokw));
    p.offsets = static_cast<int32_t*>(at(L.offsets));
    p.tiles = static_cast<int32_t*>(at(L.tiles));
    p.wts = static_cast<float*>(at(L.wts));
    p.inv = static_cast<int32_t*>(at(L.inv));
    if (int st = hip_status(launch_linear_prep(p, s), "linear set-up launch")) return st;

    // the projection as the down matrix of one expert: K = its intermediate size, N = hidden
    const ExpertSet w{nullptr, nullptr, a->w, static_cast<const uint16_t*>(a->s), a->K, a->bits, a->weight_format};
    const ExpertSet none{nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
    if (small) {
        DecodeArgs d{};
        d.x = a->x;
        d.T = (int)a->T;
        d.E = 1;
        d.k = 1;
        d.H = a->N;
        d.routed = w;
        d.shared = none;
        d.meta = p.meta;
        d.rec = p.rec;
        d.tokw = p.tokw;
        d.abuf = p.abuf;
        d.width_a = a->K;
        d.splits = L.splits;
        d.part = L.splits > 1 ? static_cast<float*>(at(L.part)) : nullptr;
        d.rows_a = a->T;
        d.residual = a->residual;
        d.y = a->y;
        return hip_status(launch_down_decode(d, s), "linear launch");
    }
    PrefillArgs q{};
    q.x = a->x;
    q.T = (int)a->T;
    q.E = 1;
    q.k = 1;
    q.H = a->N;
    q.routed = w;
    q.shared = none;
    q.offsets = p.offsets;
    q.meta = p.meta;
    q.tiles = p.tiles;
    q.tokw = p.tokw;
    q.max_tiles = (a->T + kPrefillMT - 1) / kPrefillMT;
    q.abuf = natural ? const_cast<uint16_t*>(a->x) : p.abuf;   // only read
    q.rows_a = a->T;
    q.width_a = a->K;
    q.asum = p.asum;
    q.ystage = static_cast<uint16_t*>(at(L.ystage));
    q.wts = p.wts;
    q.inv = p.inv;
    q.residual = a->residual;
    q.y = a->y;
    return hip_status(launch_down_prefill(q, s), "linear launch");
}

size_t moe_w4a16_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, int64_t shared_I) {
    g_last_error.clear();
    if (shared_I < 0) {
        fail(W4A16_ERR_INVALID_ARG, "shared_I = %lld < 0", (long long)shared_I);
        return 0;
    }
    moe_w4a16_args a{};
    a.T = T, a.H = H, a.I = I, a.E = E, a.top_k = top_k;
    a.bits = 4, a.group = kGroup;
    a.shared_bits = shared_I ? 8 : 0, a.shared_I = shared_I;
    if (check_shapes(&a) != W4A16_OK) return 0;
    return layout(&a).total;
}

int moe_w4a16_workspace_check(void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (!workspace) return fail(W4A16_ERR_INVALID_ARG, "NULL workspace");
    if (!aligned16(workspace)) return fail(W4A16_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (workspace_bytes < kHeadBytes)
        return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes is smaller than its head (%zu)", workspace_bytes,
                    kHeadBytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize")) return st;
    uint32_t word = 0;
    const char* p = static_cast<const char*>(workspace) + W4A16_WORKSPACE_ERROR_OFFSET;
    if (int st = hip_status(hipMemcpy(&word, p, sizeof(word), hipMemcpyDeviceToHost), "reading the time-out word"))
        return st;
    if (word == 0) return W4A16_OK;
    if (int st = hip_status(launch_head_init(static_cast<uint32_t*>(workspace), s), "workspace head reset")) return st;
    if (int st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize")) return st;
    return fail(W4A16_ERR_TIMEOUT, "a single-launch wait timed out on this workspace; its head has been reset");
}

int moe_w4a16_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (!workspace) return fail(W4A16_ERR_INVALID_ARG, "NULL workspace");
    if (!aligned16(workspace)) return fail(W4A16_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (workspace_bytes < kHeadBytes)
        return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the smallest layout (%zu)",
                    workspace_bytes, kHeadBytes);
    return hip_status(launch_head_init(static_cast<uint32_t*>(workspace), static_cast<hipStream_t>(stream)),
                      "workspace init launch");
}

int moe_w4a16_forward(const moe_w4a16_args* a, void* stream) {
    g_last_error.clear();
    return forward_impl(a, stream, nullptr);
}

int moe_w4a16_forward_noalloc(const moe_w4a16_args* a, void* stream) {
    g_last_error.clear();
    if (int st = check_shapes(a)) return st;
    if (a->T == 0) return W4A16_OK;
    const size_t need = layout(a).total;
    if (need > (size_t)W4A16_NOALLOC_SCRATCH_BYTES)
        return fail(W4A16_ERR_UNSUPPORTED, "these shapes need %zu bytes of scratch, the static scratch holds %zu", need,
                    (size_t)W4A16_NOALLOC_SCRATCH_BYTES);
    void* ptr = nullptr;
    if (int st = scratch_for_current_device(static_cast<hipStream_t>(stream), &ptr)) return st;
    moe_w4a16_args b = *a;
    b.workspace = ptr;
    b.workspace_bytes = W4A16_NOALLOC_SCRATCH_BYTES;
    return forward_impl(&b, stream, nullptr, /*allow_coop=*/false);
}

int w4a16_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    g_last_error.clear();
    if (!buf || !sink) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer or sink");
    if (bytes < 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return fail(W4A16_ERR_INVALID_ARG, "stream_read needs a 16-byte aligned buffer and a multiple of 16 bytes");
    return hip_status(launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)), "stream_read");
}

int moe_w4a16_forward_timed(const moe_w4a16_args* a, void* stream, int max_kernels, float* kernel_ms,
                            const char** kernel_names, int* n_kernels) {
    g_last_error.clear();
    if (!kernel_ms || !kernel_names || !n_kernels || max_kernels < 0)
        return fail(W4A16_ERR_INVALID_ARG, "NULL timing output or negative max_kernels");
    *n_kernels = 0;
    StageTimer t{};
    int created = 0, st = W4A16_OK;
    for (; created < kMaxStages; ++created) {
        if ((st = hip_status(hipEventCreate(&t.beg[created]), "hipEventCreate"))) break;
        if ((st = hip_status(hipEventCreate(&t.end[created]), "hipEventCreate"))) {
            (void)hipEventDestroy(t.beg[created]);
            break;
        }
    }
    if (!st) st = forward_impl(a, stream, &t);
    if (!st && t.n > 0) st = hip_status(hipEventSynchronize(t.end[t.n - 1]), "hipEventSynchronize");
    if (!st) {
        const int n = std::min(t.n, max_kernels);
        for (int i = 0; i < n && !st; ++i) {
            kernel_names[i] = t.name[i];
            st = hip_status(hipEventSynchronize(t.end[i]), "hipEventSynchronize");
            if (!st) st = hip_status(hipEventElapsedTime(&kernel_ms[i], t.beg[i], t.end[i]), "hipEventElapsedTime");
        }
        if (!st) *n_kernels = n;
    }
    for (int i = 0; i < created; ++i) {
        (void)hipEventDestroy(t.beg[i]);
        (void)hipEventDestroy(t.end[i]);
    }
    return st;
}

}  // extern "C"
