/*
 * qmoe.h -- C ABI of the MI355X (gfx950) quantized top-k Mixture-of-Experts layer.
 *
 * The layer is the forward pass of a top-k routed MoE SwiGLU FFN whose experts
 * hold low-bit weights, as described on the source pages:
 *   - "Quantized Mixture of Experts (Q-MoE)", section 3 components table: a
 *     gating network selects the top-k experts per input (e.g. top-2); an expert
 *     quantizer owns each expert's precision (INT8, FP8, ...); a sparse execution
 *     engine runs only the activated experts. Section 4: INT4/INT8 quantization.
 *   - IT Donga article on DREAM-MoE / SRA-MoE, DREAM-MoE section: 4-bit and 3-bit
 *     weight-quantized MoE LLMs.
 *   - "FineRMoE" (aitrends), architecture paragraph: an expert is gate, up and
 *     down projections with an activation; shared experts sit beside sparse
 *     ones; the selected experts' outputs are mixed by the router's softmax
 *     probabilities.
 *   - "OmniMoE", technical summary 2.1 (an always-on shared dense MLP) and 2.2
 *     (expert-centric scheduling: flatten all routing decisions into a task
 *     list, group by expert id, order by token id inside each group, then a
 *     grouped GEMM that loads each expert's weights once for all its tokens).
 *
 * The three calls map onto those three components:
 *   qmoe_pack_experts  -- the expert quantizer (host quantization + device layout)
 *   qmoe_route_topk    -- the gating network's selection and task list
 *   qmoe_forward       -- the sparse execution engine (router, dispatch, experts,
 *                         combine), every step a HIP kernel on the caller's stream
 *   qmoe_destroy       -- releases what qmoe_pack_experts allocated
 *
 * Conventions (all entry points):
 *   - Return QMOE_OK (0) on success, a negative QMOE_E* code on failure; nothing
 *     throws across the ABI. qmoe_last_error() returns a thread-local message
 *     describing the last failure on the calling thread.
 *   - Asynchronous calls (route, forward) report argument and launch errors at
 *     once; execution errors surface at the caller's next stream synchronisation.
 *   - A context serves one stream at a time: its workspace is shared by calls.
 *   - "device" pointers are HIP device memory on the context's device; "host"
 *     pointers are ordinary CPU memory. The library never frees caller memory.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 */
#ifndef QMOE_H
#define QMOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_OK 0
#define QMOE_EINVAL (-1)       /* bad argument: null pointer, shape, T > max_tokens, ... */
#define QMOE_EHIP (-2)         /* a HIP runtime call or kernel launch failed */
#define QMOE_ENOMEM (-3)       /* device or host allocation failed */
#define QMOE_EUNSUPPORTED (-4) /* valid request outside what the library supports */

typedef struct qmoe_ctx qmoe_ctx; /* opaque; owns all device memory it allocates */

/* Expert weight formats (the expert quantizer's precision choices).
 * Rounding: fp32 arithmetic, round half to even; the stored scale is the one
 * used to form the codes; a row or group whose stored scale is zero gets
 * scale 1 and all-zero codes (and zero point 0).
 *   INT8_SYM_CH       s_n = amax_n/127 (fp32, per output row); q = clamp(rint(w/s), -127, 127)
 *   INT4_ASYM_G128    per (row, 128-wide group along the input dim): range widened to
 *                     include 0, s = fp16((max-min)/15), z = clamp(rint(-min/s), 0, 15)
 *                     stored as fp16, q = clamp(rint(w/s)+z, 0, 15); W = (q-z)*s
 *   INT4_SYM_G128     s = fp16(amax/7), q = clamp(rint(w/s), -8, 7); W = q*s
 *   INT3_SYM_G128_IN4 s = fp16(amax/3), q = clamp(rint(w/s), -4, 3), stored in 4-bit
 *                     containers exactly like INT4_SYM_G128
 *   FP8E4M3_CH        s_n = amax_n/448 (fp32, per row); q = OCP e4m3fn(w/s), nearest
 *                     even, saturating at 448; the sign bit follows w/s
 * fp16 scales saturate at 65504. */
typedef enum {
    QMOE_W_INT8_SYM_CH = 0,
    QMOE_W_INT4_ASYM_G128 = 1,
    QMOE_W_INT4_SYM_G128 = 2,
    QMOE_W_INT3_SYM_G128_IN4 = 3,
    QMOE_W_FP8E4M3_CH = 4
} qmoe_wformat;

/* Router weight quantization (config field router_quant). */
typedef enum { QMOE_RQ_NONE = 0, QMOE_RQ_INT8_CH = 1, QMOE_RQ_FP8E4M3_CH = 2 } qmoe_router_quant;

/* Layer configuration, fixed at pack time.
 *   d_model      input and output width d; multiple of 256
 *   d_ff         routed expert width F; multiple of 128
 *   n_experts    routed experts E, 1..1024
 *   top_k        experts per token k, 1..min(E, 64)
 *   n_shared     always-on shared experts S >= 0 (mixing weight 1, same format)
 *   d_ff_shared  shared expert width (multiple of 128; ignored when S = 0)
 *   wformat      a qmoe_wformat value (the format of every expert unless
 *                expert_wformat is given)
 *   group_size   must be 128 for the group formats (ignored otherwise)
 *   router_fp32  1: router weight is fp32 [E][d]; 0: bf16 [E][d]
 *   router_quant a qmoe_router_quant value: QMOE_RQ_NONE routes with the
 *                router weight as given; QMOE_RQ_INT8_CH / QMOE_RQ_FP8E4M3_CH
 *                quantize it per expert row at pack time with the rules of
 *                QMOE_W_INT8_SYM_CH / QMOE_W_FP8E4M3_CH above (the weight's
 *                values, fp32 or bf16, are the quantizer's input), and the
 *                logits become s_e * (x . q_e) + bias_e (fp32 accumulation).
 *                Quantized routing is the Q-MoE page's section 4 option and the
 *                routing-shift concern of the IT Donga DREAM-MoE section.
 *   renormalize  1: weights = softmax over the selected k (they sum to 1);
 *                0: weights = full-softmax probability of each selected expert
 *   expert_wformat  NULL, or host array [n_experts + n_shared] of qmoe_wformat
 *                values giving each expert its own format (routed experts
 *                first, then shared; read during qmoe_pack_experts only); NULL:
 *                every expert in `wformat`. Per-expert precision is the Q-MoE
 *                page's expert quantizer (section 3 components table: each
 *                expert keeps its own precision, e.g. INT8 for frequently
 *                chosen experts and INT4 for the rest)
 *   max_tokens   largest T a forward may pass; sizes the workspace
 *                (max_tokens <= 2^20, max_tokens * (top_k + n_shared) <= 2^21
 *                and max_tokens * d_model < 2^31)
 *   device       HIP device ordinal that holds the weights and runs the layer */
typedef struct {
    int32_t d_model, d_ff, n_experts, top_k, n_shared, d_ff_shared;
    int32_t wformat;
    int32_t group_size;
    int32_t router_fp32;
    int32_t renormalize;
    int32_t max_tokens;
    int32_t device;
    int32_t router_quant;
    const int32_t *expert_wformat;
} qmoe_config;

/* Caller-owned device buffers that receive routing results; any may be NULL.
 *   logits    [T][E] fp32   router logits x.W_r^T + bias (forward only)
 *   topk_idx  [T][k] int32  selected experts, descending logit, ties to the
 *                           lower index
 *   topk_w    [T][k] fp32   their mixing weights
 *   counts    [E]    int32  tasks (token, slot) per expert
 *   offsets   [E+1]  int32  exclusive scan of counts
 *   perm      [T*k]  int32  task list: perm[row] = t*k + j, rows grouped by
 *                           expert in expert order, tokens ascending inside */
typedef struct {
    float *logits;
    int32_t *topk_idx;
    float *topk_w;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
} qmoe_route_out;

/* The expert quantizer (Q-MoE page, section 3, "Expert Quantizer"; section 4
 * INT4/INT8 quantization). Synchronous.
 *   cfg        layer configuration (copied)
 *   w_gate     host array of E+S host pointers, each fp32 row-major [F][d]
 *              (routed experts 0..E-1, then shared experts, whose F is d_ff_shared)
 *   w_up       same shape as w_gate
 *   w_down     E+S host pointers, each fp32 row-major [d][F]
 *   w_router   host [E][d], fp32 or bf16 bit patterns per cfg->router_fp32
 *   router_bias host [E] fp32 added to every logit, or NULL
 *   out        receives the new context; *out is NULL on failure
 * Host arrays are only read during the call. Quantizes every matrix on the
 * host, lays the codes out for the device kernels, allocates the weight arena
 * and a workspace sized for cfg->max_tokens on cfg->device. */
int qmoe_pack_experts(const qmoe_config *cfg, const float *const *w_gate, const float *const *w_up,
                      const float *const *w_down, const void *w_router, const float *router_bias, qmoe_ctx **out);

/* The expert quantizer on the device: the same layer as qmoe_pack_experts, from
 * bf16 expert weights that are already in device memory (Q-MoE page, section
 * 3: the expert quantizer; quantization at load time without a host round
 * trip). Each expert matrix is quantized by HIP kernels with the rules above
 * (the bf16 values widen exactly to the fp32 the host quantizer would read), so
 * the packed arena is byte for byte the one qmoe_pack_experts builds from the
 * same values. Synchronous: the kernels run on `stream` (a hipStream_t, NULL
 * for the default stream) and are complete on return.
 *   w_gate, w_up, w_down  host arrays of E+S DEVICE pointers, each bf16 bit
 *              patterns row-major [F][d] / [F][d] / [d][F] on cfg->device,
 *              only read during the call
 *   w_router, router_bias, out  as for qmoe_pack_experts (host memory)
 * Errors as for qmoe_pack_experts; QMOE_EHIP if a kernel fails. */
int qmoe_pack_experts_device(const qmoe_config *cfg, const uint16_t *const *w_gate, const uint16_t *const *w_up,
                             const uint16_t *const *w_down, const void *w_router, const float *router_bias,
                             void *stream, qmoe_ctx **out);

/* The gating network's selection and the expert-centric task list, from given
 * logits (Q-MoE page, section 3 "Gating Network"; OmniMoE technical summary
 * 2.2, task collection and grouping). Asynchronous on `stream`.
 *   logits  device [T][E] fp32 (any bias already added); finite values only
 *   T       0 <= T <= max_tokens (T = 0 is a no-op)
 *   out     device buffers to fill (logits member ignored); NULL members skipped
 *   stream  hipStream_t (NULL = the null stream) */
int qmoe_route_topk(qmoe_ctx *ctx, const float *logits, int32_t T, qmoe_route_out *out, void *stream);

/* The sparse execution engine: y = sum_j w_tj * Expert_{e_tj}(x_t) + sum_s Shared_s(x_t),
 * Expert(x) = W_down (silu(W_gate x) * (W_up x)) on the quantized weights.
 * Asynchronous on `stream`; never synchronises with the host.
 *   x       device [T][d] bf16
 *   T       0 <= T <= max_tokens (T = 0 is a no-op)
 *   y       device [T][d] bf16 output (may not alias x)
 *   dbg     NULL, or device buffers that receive this call's routing
 *   stream  hipStream_t (NULL = the null stream)
 * The call issues only kernel launches (plus device-to-device copies for dbg)
 * and allocates nothing, so a caller may record it into a HIP graph on a
 * capturing stream and replay it (with kernel timing, qmoe_profile_enable,
 * switched off while capturing).
 * Numerics: fp32 accumulation throughout; H (the SwiGLU product) is held in
 * bf16 before the down projection; for batches on the prefill tiles each
 * weighted expert output is held as a 16-bit code with one power-of-two scale
 * per 16 consecutive columns until the sum (error at most 2^-15 of the
 * block's largest magnitude, magnitudes below 2^127); y is rounded once to
 * bf16. */
int qmoe_forward(qmoe_ctx *ctx, const uint16_t *x, int32_t T, uint16_t *y, qmoe_route_out *dbg, void *stream);

/* qmoe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, kernels and results as qmoe_forward, but the forward's workspace
 * (logits, routing tables, task list, H, O, row sums) lives in the library's
 * static per-device scratch array instead of the context's workspace, and the
 * call allocates nothing (no hipMalloc/hipFree, no events: the context's
 * kernel timing is not recorded by this call). The array holds 32 MiB per
 * device for the life of the process; a T whose workspace does not fit
 * returns QMOE_EUNSUPPORTED (at d_model = 2048, top-8, d_ff = 768 about 400
 * tokens fit; at d_model = 4096, top-2, d_ff = 14336 about 350). Every call on
 * one device shares that device's array: calls that overlap on a device (any
 * context, any stream) race and must be serialised by the caller. Nothing in
 * the array needs clearing between calls. */
int qmoe_forward_static(qmoe_ctx *ctx, const uint16_t *x, int32_t T, uint16_t *y, qmoe_route_out *dbg, void *stream);

/* Frees the context and its device memory. NULL is a no-op. The caller must
 * have synchronised every stream that used the context. */
void qmoe_destroy(qmoe_ctx *ctx);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char *qmoe_last_error(void);

/* Reads one packed matrix back in canonical form (synchronous; for tests).
 *   expert  0..E-1 routed, E..E+S-1 shared
 *   matrix  0 gate [F][d], 1 up [F][d], 2 down [d][F]
 *   codes   host [N][K] int8: signed q (symmetric formats), 0..15 (INT4_ASYM),
 *           raw e4m3 byte (FP8)
 *   scales  host fp32 [N][K/128] (group formats) or [N] (per-channel)
 *   zeros   host, same shape as scales (0 except INT4_ASYM), or NULL */
int qmoe_export_packed(qmoe_ctx *ctx, int32_t expert, int32_t matrix, int8_t *codes, float *scales, float *zeros);

/* ---- Atomic experts --------------------------------------------------------
 * The OmniMoE page's routed branch (technical summary 2.1-2.2): N = n_rows x
 * n_cols vector experts E_i(x) = silu(x . w_in_i) * w_out_i whose parameters
 * are two global matrices W (rows w_in_i) and V (rows w_out_i), chosen by a
 * Cartesian product router: row logits x . R_r^T and column logits x . R_c^T
 * (fp32 accumulation); expert i = a * n_cols + b scores l_r[a] + l_c[b] (fp32);
 * the top-k scores win (ties to the lower i) and the weights are the softmax
 * over the k selected scores; y_t = sum_j w_tj E_{i_tj}(x_t), rounded once to
 * bf16. The always-on dense MLP of that page is the shared-expert path of
 * qmoe_forward. All matrices are bf16 bit patterns, row-major [rows][d_model].
 *   d_model   multiple of 512, at most 8192
 *   n_rows, n_cols  1..1024 each (N = n_rows * n_cols experts)
 *   top_k     1..min(8, N)
 *   max_tokens  1..2^20 with max_tokens * top_k <= 2^21 */
typedef struct qmoe_atomic_ctx qmoe_atomic_ctx;
typedef struct {
    int32_t d_model, n_rows, n_cols, top_k, max_tokens, device;
} qmoe_atomic_config;

/* Caller-owned device buffers that receive the routing of a forward; any may
 * be NULL: logits_rows [T][n_rows], logits_cols [T][n_cols] fp32, topk_idx
 * [T][k] int32 (flat expert index, best first), topk_w [T][k] fp32; perm
 * [T*k] int32, written by the expert-centric schedule only: its task list,
 * perm[row] = t*k + j, rows grouped by expert group (group of flat index i:
 * i / ceil(N/256), groups in ascending order) and tokens ascending inside a
 * group. */
typedef struct {
    float *logits_rows, *logits_cols;
    int32_t *topk_idx;
    float *topk_w;
    int32_t *perm;
} qmoe_atomic_route_out;

/* Uploads W, V [N][d] and R_r [n_rows][d], R_c [n_cols][d] (host bf16 arrays,
 * only read during the call) to cfg->device and sizes a workspace for
 * cfg->max_tokens. Synchronous. */
int qmoe_atomic_create(const qmoe_atomic_config *cfg, const uint16_t *w_in, const uint16_t *w_out,
                       const uint16_t *router_rows, const uint16_t *router_cols, qmoe_atomic_ctx **out);

/* Schedules of qmoe_atomic_forward (OmniMoE technical summary 2.2):
 *   EXPERT_CENTRIC  routing decisions flattened into a task list, grouped by
 *                   contiguous ranges of expert ids and by token inside a group
 *                   (the dispatch of qmoe_forward); the tasks run in that
 *                   order, so the tasks of one group, computed side by side,
 *                   share its W and V rows through the cache
 *   TOKEN_CENTRIC   each token gathers its own k experts' rows (the baseline
 *                   the page replaces; kept for comparison) */
#define QMOE_SCHEDULE_EXPERT_CENTRIC 0
#define QMOE_SCHEDULE_TOKEN_CENTRIC 1

/* y [T][d] bf16 (device) from x [T][d] bf16 (device), asynchronous on `stream`;
 * T = 0 is a no-op, T > max_tokens is QMOE_EINVAL. */
int qmoe_atomic_forward(qmoe_atomic_ctx *ctx, const uint16_t *x, int32_t T, uint16_t *y, int32_t schedule,
                        qmoe_atomic_route_out *dbg, void *stream);

/* Releases what qmoe_atomic_create allocated; NULL is a no-op. */
void qmoe_atomic_destroy(qmoe_atomic_ctx *ctx);

/* Kernel timing with HIP events recorded on the launch stream around every
 * kernel of qmoe_forward / qmoe_route_topk (for measurement).
 *   qmoe_profile_enable   slot_mask != 0 starts recording the kernel slots
 *                         whose bits are set (bit i = slot i; -1 = all) and
 *                         clears the totals; 0 stops. Each recorded launch
 *                         adds two event records to the stream, which delay
 *                         the next kernel by a few microseconds: time only the
 *                         slots of interest when the step time matters.
 *   qmoe_profile_read     synchronises the recorded events and returns, per
 *                         kernel slot (QMOE_NUM_KERNELS), the summed elapsed
 *                         milliseconds and the number of launches
 *   qmoe_kernel_name      name of a kernel slot */
#define QMOE_NUM_KERNELS 10
int qmoe_profile_enable(qmoe_ctx *ctx, int32_t slot_mask);
int qmoe_profile_read(qmoe_ctx *ctx, double *total_ms, int64_t *launches);
const char *qmoe_kernel_name(int32_t slot);

/* Shader clock probe (for measurement): launches one wavefront on `stream`
 * that, until duration_ticks of the device's constant-rate real-time counter
 * have passed (hipDeviceAttributeWallClockRate kHz; a bounded wait, so it
 * always ends), writes up to max_samples pairs (shader-cycle counter,
 * real-time counter) about period_ticks apart to samples (device memory,
 * uint64 [max_samples][2]; entries past the last sample are left as they
 * were). Launched on a second stream beside a timed region, the ratio of
 * cycle and tick differences over a window, times the real-time rate, is the
 * shader clock during that window. *wall_khz (host) receives the real-time
 * counter's rate in kHz. Asynchronous; runs on the current device. */
int qmoe_clock_probe(void *stream, int64_t duration_ticks, int64_t period_ticks, int32_t max_samples,
                     uint64_t *samples, int64_t *wall_khz);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
