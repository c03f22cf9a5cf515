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
 *   - The caller owns every buffer.  The library allocates no device memory and keeps
 *     no state between calls except a per-thread error message.
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

#define W4A16_ABI_VERSION 3

typedef enum w4a16_status {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misaligned pointer, k > E, ...    */
    W4A16_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement          */
    W4A16_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than moe_w4a16_workspace_size() */
    W4A16_ERR_HIP = 4          /* a HIP launch reported an error                            */
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
 * Routing (router_logits != NULL): for each token the top_k largest fp32 logits are
 * chosen (equal logits: lower expert index first; slot j = j-th chosen) and weighted by
 * the softmax over all E logits renormalised over the chosen ones.  With
 * router_logits == NULL, topk_ids / topk_w are read as inputs instead (ids must be in
 * [0, E) and distinct within a token; an id outside [0, E) or a repeat of an earlier
 * slot's id contributes nothing).
 *
 * Output: y[t] = residual[t] + sum_j w[t,j] * down_e( SiLU(gate_e x_t) * up_e x_t )
 *              + shared( x_t )                        (e = topk_ids[t,j])
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
    void* workspace;               /* device scratch, >= moe_w4a16_workspace_size(args);    */
                                   /* its first W4A16_WORKSPACE_HEAD_BYTES must be zero     */
                                   /* before the first call (moe_w4a16_workspace_init) and  */
                                   /* then stay owned by the library across calls; calls    */
                                   /* that may overlap on the GPU need workspaces of their  */
                                   /* own                                                    */
    size_t workspace_bytes;
} moe_w4a16_args;

/* Device workspace bytes moe_w4a16_forward needs for these shapes (reads T, H, I, E,
 * top_k, shared_bits and shared_I only).  Returns 0 when the shapes are invalid. */
size_t moe_w4a16_workspace_size(const moe_w4a16_args* args);

/* Bytes at the start of every workspace that carry state from one forward to the next. */
#define W4A16_WORKSPACE_HEAD_BYTES 147456

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
 * moe_w4a16_forward - routing, fused dequant gate/up + SiLU(gate)*up, fused dequant down
 * projection and router-weighted un-permute, enqueued on `stream`.
 * The result is bitwise deterministic: the fp32 sum over a token's experts is formed in
 * slot order on every path (no atomics take part in it).
 * Two forwards must not use one workspace at the same time (on different streams).
 */
int moe_w4a16_forward(const moe_w4a16_args* args, void* stream);

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

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
