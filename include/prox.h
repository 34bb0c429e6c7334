/*
 * prox.h -- C ABI of the MI355X (gfx950) Prox sparse SwiGLU FFN library.
 *
 * Prox ("Prox: Training-Free FFN Activation Sparsity via Approximate
 * Intermediate-Channel Salience in LLMs") runs a SwiGLU FFN
 *     y = W_down (silu(W_gate x) * (W_up x))
 * in two stages (technical summary, "Methodology: The Prox Framework"):
 *   Stage 1 (Lightweight Proxy Construction): sparsify x by magnitude, run it
 *     through quantized proxy copies of W_gate and W_up, score every
 *     intermediate channel by |silu(g~) * u~| and keep the top k channels as
 *     one mask shared by all three projections;
 *   Stage 2 (Exact Sparse Computation): compute gate, up, SiLU-multiply and
 *     down exactly, with the original weights, on the selected channels only.
 *
 * Conventions for every entry point:
 *  - Pointers named "device" point to device memory (any allocator); the
 *    library never allocates or frees device memory and keeps no state
 *    between calls.  Host pointers are read or written before return.
 *  - Work is enqueued on the caller's HIP stream and runs asynchronously; no
 *    call synchronizes.  Results are bitwise deterministic run to run.
 *  - Argument errors are reported before anything is enqueued, with nothing
 *    written.  A failed launch returns PROX_ERR_HIP.  No call aborts and no
 *    C++ exception crosses this interface.
 *  - Device pointers must be 16-byte aligned.  x and out must not alias.
 *  - Shapes: d_model % 8 == 0 (int4-g128 proxy: % 128), d_ff % 16 == 0,
 *    8 <= d_model <= 16384, 16 <= d_ff <= 65520, 1 <= batch <= 16
 *    (int4-g128 proxy: batch <= 4); other sizes return PROX_ERR_UNSUPPORTED.
 *    The method targets single-token decoding and names large batches as
 *    beyond its scope (technical summary, "Significance and Claims"): one
 *    token is the tuned case, small batches share one mask.
 *  - One workspace must not be used by two calls that may run concurrently.
 *    Its first 278528 bytes hold counters that must be zero before the
 *    workspace's first use (prox_workspace_init, or any zero fill); every
 *    call leaves them zero again, except one word counting bounded waits
 *    that gave up (prox_workspace_check).  After a call that returned
 *    PROX_ERR_HIP its kernels may have stopped part-way: zero them again
 *    before the next use.  The rest means nothing between calls.
 *
 * Notation: d = d_model, F = d_ff, B = batch, bf16 = bfloat16 bit patterns.
 */
#ifndef PROX_H
#define PROX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PROX_OK = 0,
    PROX_ERR_INVALID_ARG = -1, /* null/misaligned pointer, NaN or out-of-range fraction, bad batch */
    PROX_ERR_UNSUPPORTED = -2, /* shape, dtype or mode outside the supported set above */
    PROX_ERR_WORKSPACE = -3,   /* workspace_bytes smaller than prox_workspace_size() */
    PROX_ERR_HIP = -4,         /* a kernel launch failed (hipGetLastError) */
    PROX_ERR_SCRATCH_LIMIT = -5 /* prox_ffn_forward_noalloc: the layer's workspace exceeds
                                   PROX_STATIC_SCRATCH_BYTES */
} prox_status;

/* Element type of x, out and the full-precision weights (one type per call).
 * Accumulation is always fp32. */
typedef enum { PROX_F32 = 0, PROX_BF16 = 1 } prox_dtype;

/* Proxy weight format.  The pages specify INT4 proxies without a scheme;
 * both formats are symmetric absmax with fp32 scales and round-to-nearest-
 * even codes:  INT8_ROW = one scale per output channel, codes in [-127,127];
 * INT4_G128 = one scale per (channel, 128 consecutive inputs), codes in
 * [-7,7]. */
typedef enum { PROX_Q_INT8_ROW = 0, PROX_Q_INT4_G128 = 1 } prox_qmode;

/* Storage of the exact weights Stage 2 reads.  The pages say Prox composes
 * with FP8 model quantization (technical summary, Experimental Results and
 * Significance and Claims) without fixing a scheme.  PROX_W_FP8_E4M3 is OCP
 * E4M3 (bias 7, largest finite 448) with one fp32 scale per output row:
 * scale = fl32(amax / 448), code = nearest E4M3 value to fl32(w / scale),
 * ties to the even code, saturating; an all-zero row has scale 0.  Weight
 * value = scale * decode(code).  Activations and accumulation are unchanged. */
typedef enum { PROX_W_NATIVE = 0, PROX_W_FP8_E4M3 = 1 } prox_wformat;

/* Exact weights in the library's channel-major layout (produced by
 * prox_pack_weights, or prox_pack_weights_fp8):
 *   w_gu     [F][2][d]  row j*2 = gate row j, row j*2+1 = up row j, so the two
 *                       rows a selected channel needs are one contiguous run;
 *   w_down_t [F][d]     = W_down^T: row j holds the d outputs channel j feeds.
 * dtype is the type of x and out, and of the weights when wformat is
 * PROX_W_NATIVE.  With PROX_W_FP8_E4M3 both arrays hold E4M3 codes (one byte
 * each), gu_scales [F][2] holds the scales of gate row j and up row j, and
 * down_scales [d] the scale of W_down's row m (column m of w_down_t); the
 * FP8 path needs d % 16 == 0.  A zero-filled tail (wformat 0, NULL scales)
 * is the native layout. */
typedef struct {
    int64_t d_model, d_ff;
    prox_dtype dtype;
    const void *w_gu;          /* device */
    const void *w_down_t;      /* device */
    prox_wformat wformat;
    const float *gu_scales;    /* device, FP8 only */
    const float *down_scales;  /* device, FP8 only */
} prox_weights;

/* Quantized proxy of W_gate and W_up (produced by prox_quantize_proxy).
 * Layout, input-major so that a skipped input is a skipped contiguous run:
 *   INT8_ROW:  codes  int8  [d][2][F]        codes[i][0][j] = q_gate[j][i],
 *                                            codes[i][1][j] = q_up[j][i]
 *              scales fp32  [2][F]
 *   INT4_G128: codes  uint8 [d][2][F/2]      byte p of half h of input row i holds
 *                                            channel 2p in bits 0..3 and 2p+1 in
 *                                            bits 4..7, each as (q + 8) in [1,15]
 *              scales fp32  [d/128][2][F]    scales[g][h][j] for inputs g*128..+127
 * Dequantized proxy weight = scale * q. */
typedef struct {
    prox_qmode mode;
    int64_t d_model, d_ff;
    const void *codes;  /* device */
    const void *scales; /* device */
} prox_proxy;

/* Sparsity allocation (technical summary, Sparsity Allocation: Stage-2
 * sparsity anchored near 70%, Stage 1 keeping at least 30% of the inputs, a
 * cost model choosing both for a target effective sparsity at the least
 * normalized cost, counting the proxy's overhead).  The pages give no
 * formula; the reading taken:
 *   t1(keep)  = stage1_fixed_us + stage1_per_keep_us * keep   (Stage 1)
 *   t2(kappa) = stage2_fixed_us + stage2_per_kept_us * kappa  (Stage 2,
 *               kappa = 1 - ffn_sparsity, the kept channel fraction)
 * fitted from measured times on the device (bench.py --calibrate), and
 *   effective sparsity = 1 - (t1(keep) + t2(kappa)) / dense_us.
 * All host-only. */
typedef struct {
    double stage1_fixed_us, stage1_per_keep_us;
    double stage2_fixed_us, stage2_per_kept_us;
    double dense_us;
} prox_cost_model;

/* Effective sparsity of (input_keep, ffn_sparsity) under the model.
 * Requires dense_us > 0, keep and sparsity in [0,1]. */
prox_status prox_effective_sparsity(const prox_cost_model *m, double input_keep, double ffn_sparsity,
                                    double *effective);

/* (input_keep, ffn_sparsity) for a target effective sparsity, the target
 * read as a time budget (1 - target) * dense_us split between the stages:
 *   1. hold ffn_sparsity at s2_anchor and solve for input_keep;
 *   2. if that keep is above 1, keep every input and spend the rest on more
 *      exact channels (ffn_sparsity below the anchor, not below 0);
 *   3. if it is below min_keep, keep min_keep and raise ffn_sparsity.
 * A keep-independent Stage 1 (stage1_per_keep_us == 0) keeps every input.
 * Returns PROX_ERR_UNSUPPORTED when even ffn_sparsity = 1 at min_keep misses
 * the target; PROX_ERR_INVALID_ARG for a negative cost, dense_us <= 0,
 * stage2_per_kept_us <= 0, s2_anchor outside [0,1], min_keep outside (0,1]
 * or a target not below 1. */
prox_status prox_allocate_sparsity(const prox_cost_model *m, double target_effective, double s2_anchor,
                                   double min_keep, double *input_keep_out, double *ffn_sparsity_out);

/* Measurement aid, not part of the method: reads `bytes` (a multiple of 16)
 * of device memory at buf (16-byte aligned) once, in 16-byte non-temporal
 * loads spread over the whole device, and XORs every 32-bit word read into
 * *sink (device, caller-initialized; the result is the XOR of the buffer's
 * words, so the read is checkable).  Timed over a buffer far larger than the
 * 256 MB Infinity Cache, it gives the sustained HBM read rate the forward's
 * kernels are compared with, beside the nominal peak.  Bad pointers or sizes:
 * PROX_ERR_INVALID_ARG. */
prox_status prox_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char *prox_status_string(int status);

/* Library version string, e.g. "prox-gfx950 0.1". */
const char *prox_version(void);

/* Counts of kept inputs per token and kept channels, as the library computes
 * them (Sparsity Allocation: input sparsity keeps a fraction of input entries,
 * Stage-2 sparsity drops a fraction of intermediate channels):
 *   k_in = clamp(floor(input_keep * d + 1/2), 1, d)
 *   k    = clamp(floor((1 - ffn_sparsity) * F + 1/2), 0, F)
 * evaluated in binary64 on the binary32 arguments.  input_keep in (0,1],
 * ffn_sparsity in [0,1], both not NaN, else PROX_ERR_INVALID_ARG.  Host-only. */
prox_status prox_counts(int64_t d_model, int64_t d_ff, float input_keep, float ffn_sparsity,
                        int64_t *k_in, int64_t *k);

/* Offline: repack nn.Linear weights into the channel-major layout above.
 *   w_gate, w_up [F][d], w_down [d][F] (device, row-major, dtype)
 *   w_gu_out [F][2][d], w_down_t_out [F][d] (device, dtype; caller-allocated)
 * Inputs and outputs must not overlap. */
prox_status prox_pack_weights(const void *w_gate, const void *w_up, const void *w_down,
                              int64_t d_model, int64_t d_ff, prox_dtype dtype,
                              void *w_gu_out, void *w_down_t_out, hipStream_t stream);

/* Offline: FP8 (E4M3) copy of nn.Linear weights in the same layout, with the
 * scales described at prox_wformat.
 *   w_gate, w_up [F][d], w_down [d][F] (device, row-major, dtype, finite)
 *   w_gu_out uint8 [F][2][d], gu_scales_out fp32 [F][2],
 *   w_down_t_out uint8 [F][d], down_scales_out fp32 [d] (device; caller-allocated)
 * d % 16 == 0, else PROX_ERR_UNSUPPORTED.  Inputs and outputs must not
 * overlap.  Fill a prox_weights with wformat = PROX_W_FP8_E4M3, these four
 * outputs, and dtype = the activations' type. */
prox_status prox_pack_weights_fp8(const void *w_gate, const void *w_up, const void *w_down,
                                  int64_t d_model, int64_t d_ff, prox_dtype dtype,
                                  void *w_gu_out, float *gu_scales_out, void *w_down_t_out,
                                  float *down_scales_out, hipStream_t stream);

/* Bytes of the proxy buffers for a shape and mode (host-only). */
prox_status prox_proxy_sizes(int64_t d_model, int64_t d_ff, prox_qmode mode,
                             size_t *codes_bytes, size_t *scales_bytes);

/* Offline: quantize the proxy of W_gate and W_up from packed weights
 * (Stage 1, "Input Sparsity & Quantization": quantized proxy copies of the up
 * and gate projections).  Per segment (a channel's row for INT8_ROW, a
 * channel's 128-input group for INT4_G128): a = max |w| (binary32),
 * scale = a / qmax rounded to binary32, q = clamp(rint(w / scale)) with
 * round-to-nearest-even binary32 division; a == 0 gives scale 0 and q 0.
 * With FP8 weights, w is the binary32 value fl32(scale * decode(code)).
 * codes, scales: device buffers of prox_proxy_sizes() bytes. */
prox_status prox_quantize_proxy(const prox_weights *w, prox_qmode mode, void *codes, void *scales,
                                hipStream_t stream);

/* Workspace bytes a forward call with these sizes needs (host-only). */
prox_status prox_workspace_size(int64_t d_model, int64_t d_ff, int64_t batch, prox_qmode mode,
                                size_t *bytes);

/* Zero the counters of a workspace before its first use (enqueued on the
 * stream).  workspace: device, workspace_bytes >= 278528.  Needed once per
 * allocation, not per call: the cross-workgroup reductions elect their last
 * workgroup with ticket counters that each call returns to zero. */
prox_status prox_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Health of a workspace after the calls enqueued before this one on the
 * stream (host-only; synchronizes the stream).  Reads the counter block:
 * *fallbacks receives the number of bounded waits that gave up since the
 * workspace was last zeroed (each was completed without the awaited data, so
 * no result was wrong).  Returns PROX_ERR_WORKSPACE if any ticket or arrival
 * counter is nonzero, i.e. a call stopped part-way (after PROX_ERR_HIP) and
 * the workspace needs prox_workspace_init before its next use; PROX_ERR_HIP if
 * the copy or the synchronization fails. */
prox_status prox_workspace_check(const void *workspace, size_t workspace_bytes, uint32_t *fallbacks,
                                 hipStream_t stream);

/* The Prox FFN forward (both stages).
 *   x   [B][d] device, w->dtype: the FFN input (already normalized).
 *   out [B][d] device, w->dtype: y = sum over selected j of W_down[:, j] *
 *       silu(W_gate[j] . x) * (W_up[j] . x), fp32 accumulation, rounded to
 *       nearest-even on store.
 *   sel_idx_out: nullable device int32 [k]; receives the mask as ascending
 *       channel indices.
 * Stage 1 keeps, per token, the k_in largest |x_i| (ties: lower i), scores
 * channel j by score_j = sum_b |silu(g~_bj) * u~_bj| with the proxy
 * projections of the sparsified x, and selects the k largest scores (ties:
 * lower j) as one mask for the whole batch.  Stage 2 uses the dense x.
 * k == F skips Stage 1 (every channel is selected); k == 0 writes zeros. */
prox_status prox_ffn_forward(const void *x, int64_t batch, const prox_weights *w,
                             const prox_proxy *p, float input_keep, float ffn_sparsity, void *out,
                             int32_t *sel_idx_out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* As prox_ffn_forward, then out = residual + y (the add in fp32, one rounding).
 * residual [B][d] device, may alias out (in-place residual update) but not x. */
prox_status prox_ffn_forward_residual(const void *x, int64_t batch, const prox_weights *w,
                                      const prox_proxy *p, float input_keep, float ffn_sparsity,
                                      const void *residual, void *out, int32_t *sel_idx_out,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Gate activation h = act(g).  SILU: silu(z) = z / (1 + exp(-z)) (SwiGLU).
 * GELU_TANH: z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) (GeGLU FFNs, e.g.
 * the Gemma family the pages evaluate, technical summary, Key
 * Contributions).  Used by the salience and by Stage 2, s = act(g) * u. */
typedef enum { PROX_ACT_SILU = 0, PROX_ACT_GELU_TANH = 1 } prox_activation;

/* Channel-selection signal (technical summary, Problem Statement: the exact
 * intermediate state s = u (.) h is the ideal signal, prior methods use one
 * branch, h or u):
 *   S       |h~ u~| of the proxy (Prox; the default);
 *   H       |h~|, the proxy gate branch alone;
 *   U       |u~|, the proxy up branch alone;
 *   EXACT_S |h u| of the exact state: exact gate/up of every channel with the
 *           dense x (dense Stage-2 gate/up cost), no proxy -- the ideal mask,
 *           a diagnostic.
 * Each is summed over the batch before the top-k. */
typedef enum { PROX_SIGNAL_S = 0, PROX_SIGNAL_H = 1, PROX_SIGNAL_U = 2, PROX_SIGNAL_EXACT_S = 3 } prox_signal;

/* wait_limit_ticks: workgroups of one launch hand work to each other through
 * bounded waits.  A wait gives up after this many ticks of the device's
 * 100 MHz real-time counter (0: half a second).  In the single-token Stage 2
 * the workgroup then computes what it waited for itself, so the result is
 * the same, bitwise, only later; each such wait adds one to the count
 * prox_workspace_check reports.  The single-launch layer (below) waits on
 * grid barriers of workgroups that are all resident; a wait there that gives
 * up is a failure: the output is NaN and prox_workspace_check returns
 * PROX_ERR_HIP.  Negative: PROX_ERR_INVALID_ARG.
 * flags: PROX_FLAG_SINGLE_LAUNCH runs both stages of the layer in one launch
 * of one 1024-thread workgroup per CU, its phases joined by grid barriers,
 * where the shape allows it (one bf16 token, bf16 weights, int8 proxy,
 * d_model 4096 or 8192, d_ff <= 16384); elsewhere it is ignored.  Its
 * results agree with the default two-launch path within rounding, not
 * bitwise.  On MI355X it is slower than the default (61 against 53.5 us at
 * 4096 x 14336, 70% sparsity): the barriers cost more than the launch gap.
 * Unknown flags: PROX_ERR_UNSUPPORTED. */
#define PROX_FLAG_SINGLE_LAUNCH 1
typedef struct {
    prox_activation activation;
    prox_signal signal;
    int64_t wait_limit_ticks;
    int32_t flags;
} prox_options;

/* prox_ffn_forward with options (opt NULL = SILU and S, i.e. prox_ffn_forward)
 * and an optional residual (nullable; as prox_ffn_forward_residual).  With
 * PROX_SIGNAL_EXACT_S, p may be NULL (no proxy is read); the workspace is then
 * sized for PROX_Q_INT8_ROW.  Unknown options: PROX_ERR_UNSUPPORTED. */
prox_status prox_ffn_forward_ex(const void *x, int64_t batch, const prox_weights *w,
                                const prox_proxy *p, float input_keep, float ffn_sparsity,
                                const prox_options *opt, const void *residual, void *out,
                                int32_t *sel_idx_out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of prox_ffn_forward_residual (residual nullable) without a workspace
 * argument.  The workspace is a device array inside the library, one per
 * device, PROX_STATIC_SCRATCH_BYTES (64 MiB) large and held from the first
 * call on a device until the process ends; its counters are cleared by a
 * kernel on `stream` at that first call, and every call leaves them at zero.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 * Layers whose prox_workspace_size exceeds the limit (e.g. batch 16 at
 * 4096 x 14336, or batch above 4 at 8192 x 28672) return
 * PROX_ERR_SCRATCH_LIMIT before touching the device; every batch-1 layer of
 * the supported shapes fits.  All calls on one device share the array: calls
 * that may overlap in time on one device (different streams, host threads
 * without ordering) race and must not be issued.  The stream must belong to
 * the current device.  Results are bitwise those of prox_ffn_forward_residual
 * with its own workspace. */
#define PROX_STATIC_SCRATCH_BYTES (64u << 20)
prox_status prox_ffn_forward_noalloc(const void *x, int64_t batch, const prox_weights *w,
                                     const prox_proxy *p, float input_keep, float ffn_sparsity,
                                     const void *residual, void *out, int32_t *sel_idx_out,
                                     hipStream_t stream);

/* prox_ffn_forward with timing marks: events[0..5] (host array of six
 * hipEvent_t the caller created) are recorded on the stream before the input
 * selection, the proxy GEMV, the top-k, the gate/up GEMV and the down
 * projection, and after the down projection, so that hipEventElapsedTime of
 * consecutive pairs gives each step's duration on the device.  Without Stage 1
 * (k == 0 or k == F) events[1] and events[2] coincide.  A single token with
 * d <= 8192 and F <= 16384 runs all of Stage 1 as one kernel, between
 * events[0] and events[1]; events[1] and events[2] then coincide.  A single
 * token runs all of Stage 2 as one kernel, between events[3] and events[4];
 * events[4] and events[5] then coincide. */
prox_status prox_ffn_forward_timed(const void *x, int64_t batch, const prox_weights *w,
                                   const prox_proxy *p, float input_keep, float ffn_sparsity, void *out,
                                   int32_t *sel_idx_out, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream, hipEvent_t *events);

/* Stage 1 alone (technical summary, "Stage 1: Lightweight Proxy
 * Construction": sparsify x by magnitude, proxy gate/up projections with the
 * quantized weights, salience |silu(g~) u~|, top-k channels): the mask, and
 * optionally the fp32 channel scores.
 *   sel_idx_out: device int32 [k] ascending (k from prox_counts);
 *   scores_out:  nullable device fp32 [F] (score_j as above).
 * Requires k < F (k == F needs no Stage 1). */
prox_status prox_stage1_select(const void *x, int64_t batch, const prox_weights *w,
                               const prox_proxy *p, float input_keep, float ffn_sparsity,
                               int32_t *sel_idx_out, float *scores_out, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Top-k of a score vector, the mask-generation step on its own.
 *   scores [n] device fp32 (finite); sel_idx_out [k] device int32, receives
 *   the k indices with the largest |scores| (ties: lower index), ascending.
 *   1 <= n <= 65535, 0 <= k <= n.  workspace, workspace_bytes: unused (the
 *   selection runs in one workgroup's LDS and registers). */
prox_status prox_topk(const float *scores, int64_t n, int64_t k, int32_t *sel_idx_out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Stage 2 alone (technical summary, "Stage 2: Exact Sparse Computation": the
 * gate and up projections with the original weights and the dense x on the
 * selected channels, the SiLU-multiply, then the down projection over the
 * same channels): exact masked SwiGLU on a given mask.
 *   sel_idx [k] device int32, distinct channels in [0, F) in ascending order
 *   (entries outside [0, F) are clamped into it: wrong values, no stray
 *   access); out [B][d] device.  0 <= k <= F. */
prox_status prox_stage2_exact(const void *x, int64_t batch, const prox_weights *w,
                              const int32_t *sel_idx, int64_t k, void *out, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* prox_stage2_exact with options (the activation and the wait limit apply;
 * opt NULL = SILU and the default limit). */
prox_status prox_stage2_exact_ex(const void *x, int64_t batch, const prox_weights *w,
                                 const int32_t *sel_idx, int64_t k, const prox_options *opt, void *out,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* RMSNorm with unit gain: out = h / sqrt(mean(h^2) + eps), fp32 math, rounded
 * to the dtype.  h, out [B][d] device (may alias).  1 <= B <= 4096; d % 8 ==
 * 0 and 8 <= d <= 16384, else PROX_ERR_UNSUPPORTED; eps >= 0 and not NaN.
 * (The pages do not describe the layers around the FFN; this is the glue of
 * the layer stack below.) */
prox_status prox_rmsnorm(const void *h, int64_t batch, int64_t d_model, prox_dtype dtype, float eps,
                         void *out, hipStream_t stream);

/* A stack of n_layers Prox FFN layers with pre-norm residual adds, in place:
 *   for l in 0..n_layers-1:  h <- h + FFN_l(RMSNorm(h))
 * h [B][d] device (dtype of the layers); layers[l], proxies[l] host arrays of
 * descriptors with identical shapes and dtype.  The workspace must hold
 * prox_workspace_size(d, F, B, mode) + 256 + B*d*4 bytes (the normalized
 * input is staged there).  Each layer's result equals, bitwise, prox_rmsnorm
 * of h followed by prox_ffn_forward of that with residual h; with a sparse
 * mask Stage 1 computes the norm itself instead of a separate launch. */
prox_status prox_chain_forward(void *h, int64_t batch, const prox_weights *layers,
                               const prox_proxy *proxies, int64_t n_layers, float eps,
                               float input_keep, float ffn_sparsity, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PROX_H */
