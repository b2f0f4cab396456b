/*
 * wsgemv: batch-1 weight-streaming GEMV for LLM decode on MI355X (gfx950).
 *
 * The operation (MiniCPM-V 4.6 on Orange Pi AIPro (Ascend 310B) post,
 * baseline paragraph and closing paragraph): during decode M = 1, so each
 * linear layer is a vector-matrix product, and every weight is read once per
 * generated token; the step is bound by memory bandwidth.  With W stored
 * [N, K] row-major (K contiguous) and activation x[K]:
 *
 *     y[n] = sum_k W[n, k] * x[k]          (fp32 accumulation, fp32 y)
 *
 * Conventions shared by every call below
 *  - Pointers named W, x, y, ws, ... are DEVICE pointers owned by the caller;
 *    the library never frees or retains them beyond the call (a decode-step
 *    plan retains the pointers it was created with, see there).
 *  - Calls are asynchronous on the caller's stream (a hipStream_t passed as
 *    wsg_stream_t; NULL means the null stream).  They never synchronise and
 *    never allocate device memory, except wsg_decode_step_create.
 *  - Every argument is validated before any HIP call; on any error nothing
 *    is launched and the outputs are untouched.
 *  - Return value: a wsg_status (0 = WSG_OK).  No C++ exception crosses the
 *    ABI.  WSG_ERR_HIP keeps the hipError_t in wsg_last_hip_error() (per
 *    thread).
 *  - N == 0 is a no-op.  K == 0 writes y = 0 (the empty sum).
 *  - A shape whose launch would need more than 2^32 - 1 work-items (HIP's
 *    32-bit grid: beyond tens to hundreds of millions of rows, fewer with
 *    many forced slices) returns WSG_ERR_UNSUPPORTED before anything is
 *    launched, as do the per-call limits stated below.
 *  - Outputs must not alias inputs.  Inputs must stay alive until the
 *    stream has reached the work.
 *
 * Split-K.  A call may cut the k-sum into S contiguous slices, computed by
 * different workgroups, whose fp32 (int32 for W8A8) partial sums are then
 * added on the device in fixed slice order 0..S-1, so results are
 * bit-identical from run to run.  This follows the same post, second change:
 * the ~248k-row lm_head is cut into slices at load time and the slice
 * results reduced (there on the host; here on the device, in the
 * caller-provided workspace).  `splits` = 0 lets the library's per-shape
 * launch table choose S (the EdgeFM summary, section 2B, dispatches
 * operators by tensor-shape signature); `splits` >= 1 forces S.  The
 * workspace must hold wsg_workspace_bytes(...) bytes, 256-byte aligned; it
 * may be NULL when that size is 0.  One workspace must not serve two calls
 * that are in flight at the same time.
 *
 * The last workgroup to finish a row tile adds that tile's partials (no
 * second kernel); it finds out through one arrival counter per row tile,
 * kept in the workspace after the partials (from the next 256-byte
 * boundary).  So a split workspace must be zero-filled before its first use
 * (hipMemset, torch.zeros); every call leaves the counters zero again, so
 * one zero fill serves every later call.
 */
#ifndef WSGEMV_H
#define WSGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *wsg_stream_t; /* a hipStream_t */
typedef int32_t wsg_status;

enum {
    WSG_OK = 0,
    WSG_ERR_NULL = 1,        /* a required pointer is NULL */
    WSG_ERR_SHAPE = 2,       /* negative or inconsistent sizes, K not a multiple of the vector width */
    WSG_ERR_ALIGN = 3,       /* a pointer is not aligned as stated */
    WSG_ERR_UNSUPPORTED = 4, /* a valid request the library does not implement (e.g. M > 8) */
    WSG_ERR_WORKSPACE = 5,   /* workspace missing or too small for the chosen split */
    WSG_ERR_HIP = 6,         /* a HIP runtime call failed; see wsg_last_hip_error() */
    WSG_ERR_NOMEM = 7,       /* host or device allocation failed (plan creation only) */
    WSG_ERR_STATE = 8        /* NULL, destroyed or unknown plan handle (a new plan may later reuse a
                                destroyed one's address, so do not keep destroyed handles) */
};

enum { WSG_F16 = 0, WSG_W8A8 = 1, WSG_W4A16 = 2, WSG_W4A8 = 3, WSG_W8A8_DYN = 4 }; /* wsg_linear.kind */

const char *wsg_status_string(wsg_status s);
int32_t wsg_last_hip_error(void);
const char *wsg_build_info(void);

/* The split S the launch table picks for this shape (kind, M, N, K). */
int32_t wsg_plan_splits(int32_t kind, int64_t M, int64_t N, int64_t K);

/* Workspace bytes a call of this shape needs with `splits` (0 = the table's
 * choice): S * M * N * 4 when S > 1, else 0. */
size_t wsg_workspace_bytes(int32_t kind, int64_t M, int64_t N, int64_t K, int32_t splits);

/*
 * fp16 weights, M = 1 (same post: FP16 weights read once per step).
 *   W  fp16 [N, K] row-major, 16-byte aligned, K % 8 == 0
 *   x  fp16 [K], 16-byte aligned
 *   y  fp32 [N], 4-byte aligned:  y[n] = sum_k W[n,k] x[k], fp32 accumulate
 */
wsg_status gemv_f16(const void *W, const void *x, float *y, int64_t N, int64_t K,
                    int32_t splits, void *ws, size_t ws_bytes, wsg_stream_t stream);

/*
 * gemv_f16 for callers that cannot allocate device memory or pass a
 * workspace: code under stream or graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments and result as gemv_f16
 * without (ws, ws_bytes).  The split-K partials (S * N * 4 bytes when S > 1)
 * live in a fixed device array of WSG_STATIC_SCRATCH_BYTES inside the library,
 * one per GPU, held until the process ends; its address is looked up on the
 * first call on each device; a second kernel adds them (the array keeps no
 * arrival counters, so nothing in it needs to start at zero).  A shape whose
 * partials do not fit returns WSG_ERR_WORKSPACE before anything is launched.  The call allocates nothing
 * (no hipMalloc, no hipFree).  Every call on one GPU uses that GPU's array:
 * two calls whose work overlaps in time on one GPU (different streams, or
 * different threads) race on it, so serialise them.
 */
enum { WSG_STATIC_SCRATCH_BYTES = 16 << 20 };
wsg_status gemv_f16_static(const void *W, const void *x, float *y, int64_t N, int64_t K,
                           int32_t splits, wsg_stream_t stream);

/*
 * int8 weights x int8 activations, M = 1 (vLLM Arm CPU optimisation post,
 * INT8 W8A8 section: 8-bit weights and 8-bit activations multiplied with an
 * integer multiply-accumulate; same MiniCPM-V post, closing paragraph: INT8
 * dequantisation fused into the product).
 *   Wq      int8 [N, K] row-major, 16-byte aligned, K % 16 == 0
 *   w_scale fp32 [N] per output channel
 *   xq      int8 [K], 16-byte aligned
 *   x_scale fp32 [1] per-tensor activation scale (device memory)
 *   acc[n]  = sum_k Wq[n,k] * xq[k], exact int32 (wrap-free for |acc| < 2^31)
 *   y[n]    = ((float)acc[n] * w_scale[n]) * x_scale, fp32, round to nearest even
 *   acc_out int32 [N] receives acc when non-NULL.
 */
wsg_status gemv_w8a8(const int8_t *Wq, const float *w_scale, const int8_t *xq,
                     const float *x_scale, float *y, int32_t *acc_out, int64_t N, int64_t K,
                     int32_t splits, void *ws, size_t ws_bytes, wsg_stream_t stream);

/*
 * int8 weights x fp16 activations quantised per token inside the kernel, M = 1
 * (vLLM Arm CPU optimisation post, INT8 W8A8 section: the activations are
 * quantised to 8 bits at run time).  The quantiser is gemv_w4a8's:
 *   Wq, w_scale  as for gemv_w8a8
 *   x        fp16 [K], 16-byte aligned, K % 16 == 0
 *   s_x      = fp32(max_k |x_k|) / 127; xq[k] = clamp(rint(x[k] / s_x), -127, 127)
 *            (fp32 division, ties to even); max|x| == 0 gives s_x = 0, xq = 0
 *   acc[n]   = sum_k Wq[n,k] * xq[k], exact int32
 *   y[n]     = ((float)acc[n] * w_scale[n]) * s_x, fp32
 *   acc_out  optional int32 [N]; xq_out optional int8 [K] (16-byte aligned);
 *            sx_out optional fp32 [1].  ws as for gemv_w8a8 (WSG_W8A8_DYN in
 *            wsg_workspace_bytes): with splits > 1 it holds the split
 *            partials, the s_x that the first work unit publishes, and the
 *            arrival counters (zero before the first use, see Split-K).
 */
wsg_status gemv_w8a8_dyn(const int8_t *Wq, const float *w_scale, const void *x, float *y,
                         int32_t *acc_out, int8_t *xq_out, float *sx_out, int64_t N, int64_t K,
                         int32_t splits, void *ws, size_t ws_bytes, wsg_stream_t stream);

/*
 * INT4 weights, load-time packing (vLLM Arm CPU optimisation post, dense
 * weight prepacking section: weights are put into the kernel's layout once
 * during warm-up and reused).  Canonical input:
 *   Wc  uint32 [N, K/8]; element k of row n is the 4-bit field at bits
 *       [4*(k%8), 4*(k%8)+3] of Wc[n, k/8], value q in 0..15, weight
 *       (q - 8) * s4[n, k/group]  (zero-point 8)
 *   s4  fp16 [N, K/group] row-major
 * Output: Wp (wsg_w4_packed_weight_bytes) and Sp (wsg_w4_packed_scale_bytes),
 * 16-byte aligned device buffers in the kernels' tile layout: 16-row x 128-k
 * tiles of 1 KiB, each 64-lane wave reading one tile with one 16-byte load
 * per lane, the same layout for the M = 1 and the M = 2..8 kernels.  Rows are
 * padded to a multiple of 16 with zero weights.  group must be 128,
 * K % 128 == 0.
 */
size_t wsg_w4_packed_weight_bytes(int64_t N, int64_t K);
size_t wsg_w4_packed_scale_bytes(int64_t N, int64_t K, int64_t group);
wsg_status wsg_pack_w4(const uint32_t *Wc, const void *s4, void *Wp, void *Sp,
                       int64_t N, int64_t K, int64_t group, wsg_stream_t stream);

/*
 * INT4 weights x fp16 activations with the dequantisation fused into the
 * product (MiniCPM-V post, closing paragraph: fused INT4 dequantisation;
 * vLLM Arm post, INT8 W4A8 section: 4-bit weights cut the bytes streamed).
 * M = 1 is the decode product; M = 2..8 is a speculative-verify block
 * (EdgeFM summary, section 2C: the base model checks a block of drafted
 * tokens against the same weights), computed with MFMA.
 *   Wp, Sp  packed by wsg_pack_w4 for this (N, K, group)
 *   x       fp16 [M, K] row-major, 16-byte aligned
 *   y       fp32 [M, N]:  y[m,n] = sum_g s4[n,g] * sum_{k in g} (q[n,k]-8) x[m,k]
 */
wsg_status gemv_w4a16(const void *Wp, const void *Sp, const void *x, float *y,
                      int64_t M, int64_t N, int64_t K, int64_t group,
                      int32_t splits, void *ws, size_t ws_bytes, wsg_stream_t stream);

/*
 * INT4 weights x INT8 activations with dynamic per-token activation
 * quantisation fused into the product, M = 1 (vLLM Arm CPU optimisation
 * post, INT8 W4A8 section: 4-bit weights with 8-bit activations, which cut
 * memory-bandwidth pressure further than W8A8).
 *   Wp, Sp   packed by wsg_pack_w4 (the same packed weights as gemv_w4a16)
 *   x        fp16 [K], 16-byte aligned
 *   s_x      = fp32(max_k |x_k|) / 127 (fp32, round to nearest even);
 *   xq[k]    = clamp(rint(x[k] / s_x), -127, 127) (fp32 division, ties to
 *              even); max|x| == 0 gives s_x = 0 and xq = 0
 *   y[n]     = s_x * sum_g s4[n,g] * sum_{k in g} (q[n,k] - 8) * xq[k], the
 *              inner sums exact in int32, fp32 y
 *   xq_out   optional int8 [K] (8-byte aligned) receives xq; sx_out optional
 *            fp32 [1] receives s_x.
 */
wsg_status gemv_w4a8(const void *Wp, const void *Sp, const void *x, float *y, int8_t *xq_out,
                     float *sx_out, int64_t N, int64_t K, int64_t group,
                     int32_t splits, void *ws, size_t ws_bytes, wsg_stream_t stream);

/*
 * Greedy token choice (MiniCPM-V 4.6 on Orange Pi AIPro post, second change:
 * the lm_head's sliced results are reduced, there on the host, to pick the
 * next token; here the reduce stays on the device and runs inside the
 * producing kernel).  The token is the index of the largest value: values
 * compare as IEEE numbers (-0 equals +0), a NaN is below every number, and
 * among equal values the lowest index wins.
 *
 * Every workgroup that produces values folds them into one 64-bit key and
 * stores it in its own slot of a key array in the workspace; a one-workgroup
 * finish kernel, next on the stream, reduces the keys and writes the token.
 * No atomics and no state between calls: the result does not depend on the
 * order in which workgroups run, and the workspace needs no initialisation.
 *
 * wsg_argmax_f32: token over a given fp32 vector y [N], N = 1..INT32_MAX.
 *   token        int32 [1] (out); token_logit optional fp32 [1] (out, y[token];
 *                a -0 comes back as +0)
 *   ws           at least WSG_ARGMAX_WS_BYTES, 256-byte aligned
 */
enum { WSG_ARGMAX_WS_BYTES = 8192, WSG_WITH_ARGMAX = 0x100 };
wsg_status wsg_argmax_f32(const float *y, int64_t N, int32_t *token, float *token_logit, void *ws,
                          size_t ws_bytes, wsg_stream_t stream);

/*
 * wsg_topk_f32: the k largest values of fp32 y [N] in the same order (larger
 * first, NaN below every number, -0 equal to +0, lower index first among
 * equals): idx int32 [k] (out, in that order), val optional fp32 [k] (out).
 * k = 1..WSG_TOPK_MAX and k <= N <= INT32_MAX.  Selection passes keep each
 * workgroup's k best keys as a sorted list until at most 256 lists remain.
 * Up to 16 lists are merged by one workgroup; more are first merged in
 * groups of 32 by several workgroups (one launch), whose results one
 * workgroup then merges (a second launch).  No atomics.
 *   ws   wsg_topk_ws_bytes(N, k) bytes, 256-byte aligned (two key buffers)
 */
enum { WSG_TOPK_MAX = 64 };
size_t wsg_topk_ws_bytes(int64_t N, int32_t k);
wsg_status wsg_topk_f32(const float *y, int64_t N, int32_t k, int32_t *idx, float *val, void *ws,
                        size_t ws_bytes, wsg_stream_t stream);

/*
 * gemv_f16_argmax: gemv_f16 (y = W . x, fp32 logits, written in full) with
 * the greedy token over y fused into the kernel that writes y (with
 * splits > 1, into the last workgroup of each row tile, which adds the
 * partials).  This is the lm_head of a decode step.
 *   N = 1..INT32_MAX; token int32 [1]; token_logit optional fp32 [1]
 *   ws           wsg_workspace_bytes(WSG_F16 | WSG_WITH_ARGMAX, 1, N, K,
 *                splits) bytes (the key array, then the split-K partials
 *                and counters), 256-byte aligned; zero before the first use
 *                when the call splits k (see Split-K)
 */
wsg_status gemv_f16_argmax(const void *W, const void *x, float *y, int32_t *token, float *token_logit,
                           int64_t N, int64_t K, int32_t splits, void *ws, size_t ws_bytes,
                           wsg_stream_t stream);

/*
 * One decode step of a causal depthwise 1-D convolution (MiniCPM-V 4.6 on
 * Orange Pi AIPro post, third change: the causal-conv1d of each decode step,
 * replaced there by a vectorised step kernel; the page gives no formula, and
 * this is the usual short causal convolution over each channel's last W
 * inputs).  For every channel c < C:
 *   window = (state[c][0], ..., state[c][W-2], x[c])     (oldest first)
 *   pre    = bias[c] + sum_j w[c][j] * window[j]         (fp32)
 *   out[c] = silu ? pre / (1 + exp(-pre)) : pre
 *   state[c] <- (window[1], ..., window[W-1])
 *   x      fp32 [C];  w fp16 [C, W];  bias optional fp32 [C];  state fp32
 *          [C, W-1] read and updated;  out fp32 [C]; W = 2..8.  out and
 *          state must not alias each other or the inputs.
 * A decode-step linear can run this step over its own output y inside the
 * kernel that writes y (wsg_linear.conv_*).
 */
wsg_status causal_conv1d_step(const float *x, const void *w, const float *bias, float *state, float *out,
                              int64_t C, int32_t W, int32_t silu, wsg_stream_t stream);

/*
 * Decode step: a fixed list of linears replayed once per token (EdgeFM
 * summary, section 2C: an execution graph is captured once and reused on
 * every decode iteration to cut kernel-launch overhead).
 *
 * wsg_decode_step_create validates every descriptor, builds the launch plan,
 * allocates the plan's own split-K partials and work table (the only device
 * allocation in this library), and, when the step has at least
 * WSG_STEP_GRAPH_MIN_LAUNCHES launches, captures them into a hipGraph on an
 * internal stream.  A graph launch costs more host and device time than a
 * few direct kernel launches on this platform (about 22 us of host time per
 * hipGraphLaunch against about 3 us per kernel launch), so shorter plans
 * (GROUPED is usually one launch) launch directly.  The descriptors'
 * pointers are frozen into the plan:
 * later calls read the buffers at those addresses (write new activations into
 * the same x buffers between steps).
 *   mode WSG_STEP_ORDERED: one kernel node per linear, in list order.
 *   mode WSG_STEP_GROUPED: the linears of each kind run as one launch over a
 *     work table of (linear, row tile, k-slice) units.  Valid because every
 *     linear of the list reads its own x and writes its own y; a list whose
 *     linears feed each other (through y16) must use ORDERED.
 *   | WSG_STEP_EAGER: never capture; decode_step_linears launches directly.
 *   | WSG_STEP_FORCE_GRAPH: always capture, whatever the launch count.
 *   mode WSG_STEP_PERSISTENT (no flags): the whole list, dependent linears
 *     included, runs as ONE cooperative launch per step whose workgroups are
 *     all resident at once.  A linear's input is either a buffer no linear of
 *     the list writes, or lies wholly inside the fp16 output (y16) of one
 *     EARLIER linear: the consumer starts its weight loads before that input
 *     is ready and takes each input value once the producer has published it
 *     for this step (the decode chain of the MiniCPM-V post's step, without a
 *     launch per linear; EdgeFM summary, section 2C, one executable step per
 *     decode iteration).  Supported: WSG_F16, M = 1, K <= 4096, splits 0 or 1,
 *     no argmax/conv epilogue, K > 0; an input taken from a y16 must start
 *     a multiple of 8 values into it; an input that overlaps any fp32 y, a
 *     later or the same linear's y16, or two y16s returns
 *     WSG_ERR_UNSUPPORTED.  Outputs are bit-identical from step to step.
 *     Every wait inside the launch is bounded; a wait that gives up leaves
 *     that step's results invalid and is counted (wsg_decode_step_status).
 *     Creation allocates the plan's tables and a tagged copy (4 bytes per
 *     output) of every y16 that feeds another linear.
 * decode_step_linears enqueues one step on `stream`.  A plan is not
 * thread-safe and one plan's steps must not overlap each other in time.
 */
typedef struct wsg_linear {
    int32_t kind;        /* WSG_F16, WSG_W8A8, WSG_W4A16, WSG_W4A8 or WSG_W8A8_DYN */
    int32_t M;           /* 1; or 1..8 for WSG_W4A16 */
    int64_t N, K;
    const void *W;       /* F16: fp16 [N,K]; W8A8, W8A8_DYN: int8 [N,K]; W4A16, W4A8: packed Wp */
    const void *scale;   /* W8A8, W8A8_DYN: fp32 [N]; W4A16, W4A8: packed Sp; F16: NULL */
    const void *x;       /* F16, W4A16, W4A8, W8A8_DYN: fp16 [M,K]; W8A8: int8 [K] */
    const float *x_scale;/* W8A8: fp32 [1]; otherwise NULL (W8A8_DYN computes it) */
    float *y;            /* fp32 [M,N] */
    int32_t *acc_out;    /* W8A8, W8A8_DYN: optional int32 [N]; otherwise NULL */
    int32_t group;       /* W4A16, W4A8: 128; otherwise 0 */
    int32_t splits;      /* 0 = table's choice; ORDERED mode only */
    int32_t *argmax_idx; /* optional int32 [M]: the greedy token of each output row
                            y[m] (the rule of wsg_argmax_f32; for a verify block, one
                            token per drafted position); N must be 1..INT32_MAX */
    float *argmax_val;   /* optional fp32 [M]: their logits; only with argmax_idx */
    /* Any kind with M = 1: optional causal-conv1d decode step over y, fused
       where y is final (see causal_conv1d_step; its C is N).  conv_out NULL =
       none; set with M > 1: WSG_ERR_UNSUPPORTED. */
    const void *conv_w;  /* fp16 [N, conv_width] */
    const float *conv_bias; /* optional fp32 [N] */
    float *conv_state;   /* fp32 [N, conv_width - 1], updated */
    float *conv_out;     /* fp32 [N] */
    int32_t conv_width;  /* 2..8 */
    int32_t conv_silu;   /* nonzero: SiLU on the conv output */
    /* Optional fp16 [M,N] copy of y, rounded to nearest even (overflow to
       inf), written where y is final.  It is how one linear feeds the next:
       a later linear of an ORDERED plan may take it, or a contiguous part of
       it, as its x.  A GROUPED plan rejects (WSG_ERR_UNSUPPORTED) a list in
       which any linear's x overlaps any linear's y16, since its units run in
       no fixed order.  2-byte aligned; must not alias any input. */
    void *y16;
} wsg_linear;

typedef struct wsg_step wsg_step;

enum { WSG_STEP_ORDERED = 0, WSG_STEP_GROUPED = 1, WSG_STEP_PERSISTENT = 2, WSG_STEP_EAGER = 0x100,
       WSG_STEP_FORCE_GRAPH = 0x200, WSG_STEP_GRAPH_MIN_LAUNCHES = 8 };

wsg_status wsg_decode_step_create(const wsg_linear *linears, int32_t n, int32_t mode,
                                  wsg_stream_t stream, wsg_step **out);
wsg_status decode_step_linears(wsg_step *step, wsg_stream_t stream);
wsg_status wsg_decode_step_destroy(wsg_step *step);
/* Launches per step (kernel nodes), work units of the plan, and whether the
 * step replays a captured graph (1) or launches directly (0).  Any output
 * pointer may be NULL. */
wsg_status wsg_decode_step_info(const wsg_step *step, int32_t *launches, int64_t *units, int32_t *graph);

/*
 * Waits of a WSG_STEP_PERSISTENT plan that gave up since the last call
 * (0 for other plans): synchronises `stream`, reads the plan's counter into
 * *give_ups, then clears it.  A nonzero count means some step enqueued
 * before this call produced invalid outputs.
 */
wsg_status wsg_decode_step_status(wsg_step *step, wsg_stream_t stream, uint32_t *give_ups);

/*
 * Per-unit timestamps of a WSG_STEP_PERSISTENT plan, to see where a
 * dependent step spends its time (EdgeFM summary, section 2C: the step as
 * one executable unit per decode iteration; the time between its linears is
 * what remains to account for).  `trace`: a device buffer of at least
 * 4 * units 64-bit words (units from wsg_decode_step_info), 8-byte aligned,
 * owned by the caller and kept alive while traced steps run; NULL stops
 * tracing.  Every step enqueued afterwards writes, for the plan's work unit u
 * (units in list order, linear by linear): trace[4u] the chip's 100 MHz
 * real-time clock when a workgroup starts the unit, trace[4u + 1] when its
 * input is staged, trace[4u + 2] when the whole workgroup has finished it,
 * and trace[4u + 3] = linear index | (workgroup << 32).  Tracing adds one
 * workgroup barrier per unit; outputs are unchanged.  Errors: WSG_ERR_STATE
 * for a NULL or destroyed plan, WSG_ERR_UNSUPPORTED for other modes,
 * WSG_ERR_ALIGN, WSG_ERR_SHAPE when capacity (in words) < 4 * units.
 */
wsg_status wsg_decode_step_trace(wsg_step *step, uint64_t *trace, int64_t capacity);

/*
 * Test hooks for plan creation on a machine without a GPU.  They only work
 * when the environment variable WSG_ENABLE_TEST_HOOKS is "1" (otherwise
 * WSG_ERR_UNSUPPORTED).  wsg_test_set_fault(mode): mode >= 0 makes
 * wsg_decode_step_create build plans in host memory (such a plan cannot be
 * launched: decode_step_linears returns WSG_ERR_STATE) and, for mode 1, 2 or
 * 3, makes its device allocation, upload or graph capture fail (creation
 * then returns WSG_ERR_NOMEM, WSG_ERR_HIP, WSG_ERR_HIP and frees what it
 * made); mode -1 restores normal creation.  wsg_test_live_blocks(): host
 * blocks of such plans not yet freed.
 */
wsg_status wsg_test_set_fault(int32_t mode);
int64_t wsg_test_live_blocks(void);

/*
 * Grid of a persistent launch: min(units, min(blocks_per_cu, cap_per_cu) * cus),
 * i.e. never more workgroups than the work units, nor than can be resident
 * at once (blocks_per_cu from the occupancy of the kernel, cap_per_cu <= 0
 * meaning no cap).  0 when any count is <= 0.  Pure function.
 */
int64_t wsg_chain_grid(int64_t units, int32_t blocks_per_cu, int32_t cus, int32_t cap_per_cu);

/*
 * HBM read ceiling: every lane streams 16-byte loads over buf[0, bytes) and
 * the workgroups write one fp32 partial each into out[grid] (so the loads
 * cannot be removed).  bytes % 16 == 0; grid = 0 picks a full-chip grid.
 * Gives the attainable read bandwidth next to the nominal peak.
 */
wsg_status wsg_read_probe(const void *buf, size_t bytes, float *out, int32_t grid,
                          wsg_stream_t stream);
int32_t wsg_read_probe_grid(size_t bytes);

/*
 * Launch-table overrides for tuning sweeps only.  Keys: "nt" (0/1
 * non-temporal weight loads), "dense_R"/"dense_CH" (rows and vectors per
 * lane per wave step of single fp16/int8 calls; set both), "dense_rows"
 * (rows per work unit), "group_R"/"group_CH"/"group_unit_kb" (the same for
 * grouped decode-step launches), "w4_R" (16-row tiles per wave step), "w4_B" (128-k blocks per
 * wave step: 4, 8),
 * "w4_tiles" / "group_w4_tiles" (tiles per work unit), "w4_mfma_m1" (1: W4A16
 * at M = 1 on the matrix-core kernel), "probe_U" (loads in flight per lane:
 * 4, 8, 16), "probe_chunked" (0/1), "split_fuse" (0: split-K partials summed
 * by a separate reduce kernel instead of the last workgroup of each row tile),
 * and for WSG_STEP_PERSISTENT plans "chain_unit_kb" (weight KiB per work
 * unit) and "chain_blocks_per_cu" (cap on resident workgroups per compute
 * unit), read when a plan is created, and "chain_spin_limit" (polls before a
 * wait gives up), "chain_sleep" (s_sleep(1) calls between polls) and
 * "chain_test_stale" (1: consumers wait for a tag no producer writes, to
 * exercise the give-up path), read at every launch.  value < 0 restores the
 * table's choice.  Process-wide, not thread-safe; plans capture the values
 * in force when they are created, except the three read at launch.  No
 * result depends on these settings beyond the summation order, except
 * chain_test_stale.  Unknown keys and kernel shapes that are not built
 * return WSG_ERR_UNSUPPORTED and leave the setting unchanged.
 */
wsg_status wsg_tune_set(const char *key, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* WSGEMV_H */
