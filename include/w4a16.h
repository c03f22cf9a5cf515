/*
 * w4a16.h - C ABI of the weight-only INT4/INT8 round-to-nearest (RTN) routed-expert
 * MoE library for AMD Instinct MI355X (gfx950).
 *
 * Two operations, both from the model-card pages this library follows:
 *
 *   rtn_quantize_pack   data-free symmetric RTN quantization with one bf16 scale per
 *                       group of 128 input columns, codes packed into int32 words
 *                       (page "Nex-N2.5-mini Int4-Int8Mix", section Recipe).
 *   moe_w4a16_forward   one routed-expert MoE FFN with packed INT4 (or INT8) weights
 *                       and bf16 activations: top-k routing with renormalised softmax
 *                       weights, gate/up projection with SiLU(gate)*up, down projection,
 *                       router-weighted sum (Int4-Int8Mix Recipe table: gate_proj /
 *                       up_proj / down_proj per routed expert; page "Nex-N2.5-mini FP8
 *                       W8A8 with Calibrated FP8 KV Scales", Artifact summary: 256
 *                       routed experts, 8 active per token).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, contiguous.  Device pointers must be 16-byte
 *     aligned.  bf16 values travel as uint16_t bit patterns.
 *   - The caller owns every buffer.  The library allocates no device memory.  Host-side it
 *     keeps a per-thread error message and a few per-device launch facts (CU count,
 *     occupancy) read once from the runtime.  Device-side state lives only in the head of
 *     a caller's workspace (W4A16_WORKSPACE_HEAD_BYTES): a launch epoch, counters that
 *     are zero between calls, a sticky time-out word and epoch-tagged hand-off values,
 *     carried from one forward to the next on that workspace (see
 *     moe_w4a16_workspace_init and moe_w4a16_workspace_check).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream) and
 *     runs asynchronously; no entry point synchronises.  A fault inside a kernel shows
 *     up at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; on a non-zero
 *     return nothing was enqueued (except W4A16_ERR_HIP, which reports a failed launch).
 *   - Every entry point returns a w4a16_status.  Nothing throws across the ABI.
 *     w4a16_last_error() gives a message for the calling thread's last failure.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 7

typedef enum w4a16_status {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misaligned pointer, k > E, ...    */
    W4A16_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement          */
    W4A16_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than moe_w4a16_workspace_size() */
    W4A16_ERR_HIP = 4,         /* a HIP launch reported an error                            */
    W4A16_ERR_TIMEOUT = 5      /* a bounded in-kernel wait timed out (workspace_check)      */
} w4a16_status;

typedef enum w4a16_dtype {
    W4A16_F32 = 0,
    W4A16_BF16 = 1
} w4a16_dtype;

/* W4A16_ABI_VERSION of the built library. */
int w4a16_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* w4a16_status_string(int status);

/* Message describing the calling thread's most recent failure ("" if none). */
const char* w4a16_last_error(void);

/*
 * rtn_quantize_pack - data-free symmetric round-to-nearest group quantization.
 *
 * Page "Nex-N2.5-mini Int4-Int8Mix", section Recipe: routed experts INT4 and the other
 * projections INT8, symmetric, group 128, round-to-nearest with min-max scales and no
 * calibration data; each quantized matrix is a packed tensor plus a scale tensor.
 *
 * For each of n_mats matrices [rows, cols] (row = output channel, col = input channel),
 * each row and each group of `group` consecutive columns:
 *     a = max |w|                          (over the group)
 *     s = bf16_rne( a / QMAX )             (QMAX = 7 for bits 4, 127 for bits 8;
 *                                           IEEE fp32 division)
 *     q = clamp( rint( w / s ), -QMAX-1, QMAX )   (division by the stored bf16 scale,
 *                                           IEEE fp32; rint rounds half to even;
 *                                           s == 0 gives q == 0)
 * Codes are stored offset-binary u = q + 2^(bits-1); column c sits in int32 word
 * c*bits/32 of its row at bit offset bits*(c mod 32/bits) (lowest column lowest).
 *
 *   w        device, [n_mats, rows, cols], fp32 or bf16 (w_dtype); finite values
 *   w_dtype  W4A16_F32 or W4A16_BF16
 *   bits     4 or 8;   group must be 128;   cols % 128 == 0;   n_mats, rows >= 0
 *   packed   device out, int32 [n_mats, rows, cols*bits/32]
 *   scales   device out, bf16 bits [n_mats, rows, cols/128]
 * Results are bit-identical to the definition above for finite inputs.
 */
int rtn_quantize_pack(const void* w, int w_dtype, int64_t n_mats, int64_t rows, int64_t cols,
                      int bits, int group, int32_t* packed, uint16_t* scales, void* stream);

/* Formats of the routed experts' weights (moe_w4a16_args.weight_format). */
typedef enum w4a16_format {
    W4A16_FORMAT_INT = 0,       /* rtn_quantize_pack codes: INT4 / INT8, bf16 scale per 128 columns    */
    W4A16_FORMAT_FP8_E4M3 = 1,  /* fp8_quantize_pack codes: E4M3 bytes, one fp32 scale per row (bits 8) */
    W4A16_FORMAT_MXFP4 = 2      /* mxfp4_quantize_pack codes: E2M1 nibbles, E8M0 per 32 columns (bits 4) */
} w4a16_format;

/* Launch flags (moe_w4a16_args.flags). */
typedef enum w4a16_flags {
    /* Run no kernel whose workgroups wait for each other.  The single-launch path of tiny
     * batches (T * top_k <= 16) needs its gate/up and down workgroups resident on the device
     * together, that is, no other work on the GPU while it runs (see
     * moe_w4a16_workspace_check for what a failed wait does).  With this flag those batches
     * take the multi-launch streaming path, whose result agrees to rounding. */
    W4A16_FLAG_NO_COOPERATIVE = 1
} w4a16_flags;

/* Scale choice of mxfp4_quantize_pack. */
typedef enum w4a16_mxfp4_method {
    W4A16_MXFP4_RTN = 0,        /* exponent floor(log2 amax) - 2 (round-to-nearest)                  */
    W4A16_MXFP4_MSE = 1         /* exponent searched by weight MSE (see mxfp4_quantize_pack)          */
} w4a16_mxfp4_method;

/*
 * fp8_quantize_pack - per-output-channel FP8 E4M3 round-to-nearest.
 *
 * Page "Nex-N2.5-mini-mixed-NVFP4-FP8", What's quantized to what: the routed experts of
 * the six most sensitive layers in FP8 E4M3 with one scale per output channel, weights-only
 * round-to-nearest, no calibration.  For each row of each of n_mats matrices [rows, cols]:
 *     s = max |w| / 448            (fp32, IEEE division; 448 = the largest E4M3 value)
 *     q = E4M3( w / s )            (IEEE division, rounded to nearest even; s == 0: q = 0)
 *   w        device, [n_mats, rows, cols], fp32 or bf16 (w_dtype), finite
 *   cols     multiple of 4 (a multiple of 128 for use by moe_w4a16_forward)
 *   packed   device out, int32 [n_mats, rows, cols/4]: column c in byte c % 4 of word c/4
 *   scales   device out, fp32 [n_mats, rows]
 * Codes and scales are bit-identical to the definition above.  Errors as rtn_quantize_pack.
 */
int fp8_quantize_pack(const void* w, int w_dtype, int64_t n_mats, int64_t rows, int64_t cols, int32_t* packed,
                      float* scales, void* stream);

/*
 * mxfp4_quantize_pack - MXFP4 (E2M1 codes, one E8M0 power-of-two scale per 32 columns).
 *
 * Page "Nex-N2.5-mini-MXFP4-MxWave", Model summary (MXFP4 W4A16 routed experts) and
 * Quantization method.  For each block of 32 consecutive columns of a row, with
 * amax = max |w| over the block:
 *   W4A16_MXFP4_RTN: e = floor(log2 amax) - 2;
 *   W4A16_MXFP4_MSE: e minimises sum (w - Q_e(w))^2 over the candidates
 *       floor(log2(p / 6)) - 4 .. floor(log2(p / 6)) + 1 and the smallest e with
 *       amax <= 6 * 2^e, where p = a + (b - a) * 0.845 is the block's 99.5th percentile of
 *       |w| (a, b: its two largest |w|; fp64); the error is summed in fp64 in the fixed
 *       order (i + 16, i + 8, i + 4, i + 2, i + 1); equal errors take the smaller e;
 *   an all-zero block has e = -127; e is kept in [-127, 127];
 *   Q_e(w) = E2M1( w / 2^e ) * 2^e, rounded to nearest with ties to the even code and
 *       saturating at 6; the code's sign bit is w's sign bit.
 *   cols     multiple of 32 (a multiple of 128 for use by moe_w4a16_forward)
 *   packed   device out, int32 [n_mats, rows, cols/8]: column c in bits 4 (c % 8) of word c/8
 *   scales   device out, uint8 [n_mats, rows, cols/32]: e + 127
 * Codes and scales are bit-identical to the definition above.  Errors as rtn_quantize_pack.
 */
int mxfp4_quantize_pack(const void* w, int w_dtype, int64_t n_mats, int64_t rows, int64_t cols, int method,
                        int32_t* packed, uint8_t* scales, void* stream);

/*
 * Arguments of one routed-expert MoE FFN call.
 *
 * Shapes: T tokens, hidden H, expert intermediate I, E experts, top_k experts per token.
 * Limits: H % 128 == 0, I % 128 == 0, H <= 16384, I <= 8192, 1 <= top_k <= min(E, 16),
 * E <= 1024, T >= 0 (T == 0 is a no-op), T * top_k < 2^31, bits in {4, 8}, group == 128.
 *
 * Expert weights are the packed output of rtn_quantize_pack (same code layout).
 * The gate/up bank of expert e is one [2I, H] matrix: rows [0, I) are gate_proj, rows
 * [I, 2I) up_proj (the split of the fused gate_up_proj bank in the Int4-Int8Mix Recipe).
 *
 * Routing (router_logits != NULL, or router_w != NULL and the logits computed from x,
 * see the last fields): for each token the top_k largest fp32 logits are
 * chosen (equal logits: lower expert index first; slot j = j-th chosen) and weighted by
 * the softmax over all E logits renormalised over the chosen ones.  With
 * router_logits == NULL, topk_ids / topk_w are read as inputs instead (ids must be in
 * [0, E) and distinct within a token; an id outside [0, E) or a repeat of an earlier
 * slot's id contributes nothing).  Logits must not be NaN: a NaN logit is outside the
 * contract (the kernels rank it like -inf, the oracle below every number), and so is a
 * row whose logits are all -inf (its weights are not defined).
 *
 * Output: y[t] = residual[t] + sum_j w[t,j] * down_e( SiLU(gate_e x_t) * up_e x_t )
 *              + g[t] * shared( x_t )                 (e = topk_ids[t,j]; g = 1 without
 *                                                       shared_gate_w)
 * accumulated in fp32 and rounded once to bf16 (residual and shared terms only when
 * given).  The shared expert, when shared_bits != 0, is one always-on expert of
 * intermediate size shared_I with weight 1 (the Int4-Int8Mix Recipe keeps one shared
 * expert per layer next to the routed ones, INT8 group 128).
 */
typedef struct moe_w4a16_args {
    int64_t T, H, I, E, top_k;
    int32_t bits;                  /* routed expert code width: 4 or 8                      */
    int32_t group;                 /* must be 128                                           */
    const uint16_t* x;             /* bf16 [T, H]                                           */
    const float* router_logits;    /* fp32 [T, E], or NULL: topk_ids / topk_w are inputs    */
    const int32_t* w13;            /* [E, 2I, H*bits/32] packed gate (rows < I) and up rows */
    const uint16_t* s13;           /* bf16 [E, 2I, H/128]                                   */
    const int32_t* w2;             /* [E, H, I*bits/32] packed down projection              */
    const uint16_t* s2;            /* bf16 [E, H, I/128]                                    */
    int32_t shared_bits;           /* 0: no shared expert; else 4 or 8                      */
    int64_t shared_I;              /* shared expert intermediate size (multiple of 128)     */
    const int32_t* shared_w13;     /* [2*shared_I, H*shared_bits/32]                        */
    const uint16_t* shared_s13;    /* bf16 [2*shared_I, H/128]                              */
    const int32_t* shared_w2;      /* [H, shared_I*shared_bits/32]                          */
    const uint16_t* shared_s2;     /* bf16 [H, shared_I/128]                                */
    const uint16_t* residual;      /* bf16 [T, H] added to the output, or NULL              */
    uint16_t* y;                   /* bf16 [T, H] output (may alias residual, not x)        */
    int32_t* topk_ids;             /* int32 [T, top_k]: output, or input when logits NULL;  */
    float* topk_w;                 /* fp32  [T, top_k]: may be NULL when an output          */
    int32_t* expert_counts;        /* optional out, int32 [E]: pairs routed to each expert  */
    int32_t* expert_offsets;       /* optional out, int32 [E+1]: exclusive prefix of counts */
    int32_t* sorted_pairs;         /* optional out, int32 [T*top_k]: pair ids t*top_k+j by   */
                                   /* (expert, token) ascending                              */
    void* workspace;               /* device scratch, >= moe_w4a16_workspace_size(...);     */
                                   /* its first W4A16_WORKSPACE_HEAD_BYTES must be zero     */
                                   /* before the first call (moe_w4a16_workspace_init) and  */
                                   /* then stay owned by the library across calls; calls    */
                                   /* that may overlap on the GPU need workspaces of their  */
                                   /* own                                                    */
    size_t workspace_bytes;
    /* Router and shared-expert gate in bf16 (Int4-Int8Mix Recipe table: routers and
     * shared_expert_gate stay BF16).  With router_w the logits are computed from x,
     * logit[t, e] = sum_h x[t, h] * router_w[e, h] (fp32 accumulation), and router_logits
     * must be NULL; the routing then proceeds as above.  With shared_gate_w the shared
     * expert's output for token t is scaled by g[t] = 1 / (1 + exp(-sum_h x[t, h] *
     * shared_gate_w[h])) instead of 1 (needs shared_bits != 0). */
    const uint16_t* router_w;      /* bf16 [E, H], or NULL                                  */
    const uint16_t* shared_gate_w; /* bf16 [H], or NULL                                     */
    float* logits_out;             /* optional out, fp32 [T, E]: logits from router_w       */
    float* shared_gate_out;        /* optional out, fp32 [T]: g from shared_gate_w          */
    /* Routed experts' weight format (w4a16_format).  FP8_E4M3 (bits 8): w13/w2 hold E4M3
     * bytes as fp8_quantize_pack writes them and s13/s2 point to fp32 [E, 2I] / [E, H] row
     * scales (NVFP4-FP8 page, What's quantized to what).  MXFP4 (bits 4): E2M1 nibbles as
     * mxfp4_quantize_pack writes them and s13/s2 point to E8M0 bytes [E, 2I, H/32] /
     * [E, H, I/32] (MXFP4-MxWave page, Model summary).  The shared expert stays INT. */
    int32_t weight_format;
    int32_t flags;                 /* w4a16_flags, or 0                                      */
} moe_w4a16_args;

/* Device workspace bytes moe_w4a16_forward needs for T tokens, hidden H, intermediate I,
 * E experts, top_k, and a shared expert of intermediate size shared_I (0: none).  The
 * size does not depend on the code widths.  Returns 0 when the shapes are invalid (the
 * same checks as moe_w4a16_forward; w4a16_last_error() says which). */
size_t moe_w4a16_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, int64_t shared_I);

/* Bytes at the start of every workspace that carry state from one forward to the next. */
#define W4A16_WORKSPACE_HEAD_BYTES 147456
/* Byte offset, inside the head, of the sticky time-out word (uint32, 0 = no time-out). */
#define W4A16_WORKSPACE_ERROR_OFFSET 12928

/*
 * moe_w4a16_workspace_init - zero the head of a new workspace (its first
 * W4A16_WORKSPACE_HEAD_BYTES), once, before the workspace's first forward.  The head
 * belongs to the single-launch path for tiny batches (T * top_k <= 16, H <= 4096), whose
 * gate/up workgroups hand their results to the down-projection workgroups of the same
 * kernel: exit counters (zero between calls), an epoch number that each call advances, and
 * the handed-over values, each tagged with the epoch of the call that wrote it; and to the
 * small-batch routing from logits over several workgroups (25..64 tokens), whose last
 * workgroup to arrive finishes the routing: its arrival counter (zero between calls).  A
 * workspace needs this once, not per call (a zero-filled allocation needs none).
 * Enqueued on `stream` as a small fill kernel (no memset node, so it may be captured in a
 * graph).  Errors: W4A16_ERR_INVALID_ARG for NULL or a misaligned pointer,
 * W4A16_ERR_WORKSPACE when workspace_bytes < W4A16_WORKSPACE_HEAD_BYTES.
 */
int moe_w4a16_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_w4a16_workspace_check - surface a time-out of the single-launch path.
 *
 * The single-launch path (T * top_k <= 16) hands values from its gate/up workgroups to
 * its down workgroups inside one kernel, relying on both being resident together.  Each
 * wait is bounded: when one times out (the GPU was shared so that the producers could
 * not run), the kernel sets the workspace's sticky time-out word, and from then on every
 * single-launch forward on that workspace writes quiet NaN (bf16 0x7FC0) to the output
 * rows it owns instead of waiting, so a wrong result is never silent.  The rows of the
 * call that timed out that depend on the missing values are NaN as well.
 *
 * This call synchronises `stream` (so every forward enqueued on it has finished), reads
 * the word, and when it is set clears the whole head (epoch, counters, tagged values and
 * the word itself, as moe_w4a16_workspace_init does) and returns W4A16_ERR_TIMEOUT;
 * otherwise W4A16_OK.  Forwards after it run normally again.  Errors:
 * W4A16_ERR_INVALID_ARG (NULL or misaligned workspace), W4A16_ERR_WORKSPACE (smaller
 * than the head), W4A16_ERR_HIP.
 */
int moe_w4a16_workspace_check(void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_w4a16_forward - routing, fused dequant gate/up + SiLU(gate)*up, fused dequant down
 * projection and router-weighted un-permute, enqueued on `stream`.
 * The result is bitwise deterministic: the fp32 sum over a token's experts is formed in
 * slot order on every path (no atomics take part in it).
 * Two forwards must not use one workspace at the same time (on different streams).
 */
int moe_w4a16_forward(const moe_w4a16_args* args, void* stream);

/*
 * moe_w4a16_forward_noalloc - moe_w4a16_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): it allocates nothing, directly or through any library.
 *
 * args->workspace and args->workspace_bytes are ignored.  The scratch is instead one
 * static device array of W4A16_NOALLOC_SCRATCH_BYTES per GPU, in the library's code
 * object, held by each GPU the library runs on until the process ends.  Its address is
 * taken on the first call on each device, which also zeroes its head with a small fill
 * kernel on `stream` (as moe_w4a16_workspace_init does for a caller's workspace).
 * Shapes whose moe_w4a16_workspace_size exceeds that size return W4A16_ERR_UNSUPPORTED
 * before anything is enqueued (64 MiB holds the full 256-expert, hidden-2048 layer up to
 * 64 decode tokens, or about 1000 prefill tokens, with a shared expert).
 *
 * Every call on one GPU shares that GPU's array and finds the previous call's contents
 * in it: calls that may overlap on one GPU (different streams, no ordering between them)
 * race and must not be made.  This entry point never takes the single-launch path of
 * tiny batches (whose workgroups wait on each other), so no time-out state can arise in
 * the shared array; tiny batches run on the streaming decode kernels instead, and the
 * output agrees with moe_w4a16_forward's to the tolerance of the path, bit for bit
 * whenever both take the same kernels (T * top_k > 16).  Other arguments, results and
 * errors are those of moe_w4a16_forward.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_w4a16_forward_noalloc(const moe_w4a16_args* args, void* stream);

/*
 * w4a16_linear - a dense projection y = x . W^T (+ residual) with quantized W.
 *
 * Page "Nex-N2.5-mini Int4-Int8Mix", Recipe table: the attention q/k/v/o projections and
 * the Gated DeltaNet in_proj_qkv, in_proj_z and out_proj are INT8, symmetric, group 128.
 * Every code format of moe_w4a16_forward is accepted.  Up to 64 tokens (when K / 128 splits
 * into at most 16 equal ranges of 1, 2 or 4 groups) one weight-streaming kernel computes y;
 * otherwise the routed experts' down-projection kernels run it as one expert that every
 * token uses with weight 1.
 *   T tokens, K input columns (multiple of 128, <= 8192), N output rows (multiple of 128,
 *   <= 16384); bits / weight_format as in moe_w4a16_args (INT: bits 4 or 8, group 128).
 *   x        bf16 [T, K]
 *   w, s     W packed [N, K*bits/32] and its scales, as the matching quantizer writes them
 *            (INT: bf16 [N, K/128]; FP8: fp32 [N]; MXFP4: E8M0 bytes [N, K/32])
 *   residual bf16 [T, N] added before the one rounding, or NULL; y may alias it, not x
 *   y        bf16 [T, N]: fp32 accumulation, rounded once
 *   workspace device scratch of w4a16_linear_workspace_size(T, K, N) bytes (no state is
 *            kept in it between calls; the one-kernel small-batch path leaves it untouched)
 * Errors as moe_w4a16_forward.
 */
typedef struct w4a16_linear_args {
    int64_t T, K, N;
    int32_t bits, group, weight_format;
    const uint16_t* x;
    const int32_t* w;
    const void* s;
    const uint16_t* residual;
    uint16_t* y;
    void* workspace;
    size_t workspace_bytes;
} w4a16_linear_args;

size_t w4a16_linear_workspace_size(int64_t T, int64_t K, int64_t N);
int w4a16_linear(const w4a16_linear_args* args, void* stream);

/*
 * moe_w4a16_forward_timed - the same work as moe_w4a16_forward, each kernel launched with
 * a start and a stop HIP event bound to its own dispatch (hipExtLaunchKernelGGL), then a
 * wait for the last stop event (this call synchronises with the stream's work up to that
 * point).
 *   kernel_ms     out, [max_kernels]: execution time of each kernel in launch order, in ms
 *                 (start to stop event of that dispatch; the gap between dispatches is
 *                 not counted)
 *   kernel_names  out, [max_kernels]: static name of each kernel (owned by the library)
 *   n_kernels     out: number of entries written (<= max_kernels)
 * A profiling aid for per-kernel roofline measurements; the output y is identical.
 */
int moe_w4a16_forward_timed(const moe_w4a16_args* args, void* stream, int max_kernels, float* kernel_ms,
                            const char** kernel_names, int* n_kernels);

/*
 * w4a16_stream_read - a plain streaming read of `bytes` bytes at device address `buf`
 * (16-byte aligned, bytes a multiple of 16): every 32-bit word is read once and their XOR
 * is XOR-ed into the device word *sink.  Asynchronous on `stream`.  A measurement aid: its
 * launch time is the achievable time to read that many bytes in one kernel, the reference
 * for the decode kernels' reads of the same byte count.
 * Errors: W4A16_ERR_INVALID_ARG for a NULL pointer, a misaligned buffer or a byte count
 * that is negative or not a multiple of 16.
 */
int w4a16_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
