/*
 * kda.h -- C ABI of libkda, the fused KDA (Kimi Delta Attention) token step
 * for AMD Instinct MI355X (gfx950).
 *
 * One call runs, for every (sequence, head) pair and every token in order:
 *
 *   1. causal depthwise 4-tap conv + SiLU on the raw q | k | v channels, the
 *      conv window carried in and out
 *        ("Kimi K3 Metal Gap Analysis", §2 KDA Attention, row "Conv4 + SiLU";
 *         "Metal (Apple GPU) backend for Kimi K3", Design notes, "Fused KDA
 *         token": conv_silu for each of q, k, v);
 *   2. per-head L2 normalisation of q and k
 *        (Gap Analysis §2, row "L2 normalize q/k");
 *   3. the per-key-channel decay alpha = exp(gk), gk from A_log, dt_bias and
 *      the decay pre-activation f (Gap Analysis §2, row "Decay compute");
 *   4. the gated delta-rule update of the fp32 dk x dv state
 *        S <- (I - beta k k^T) Diag(alpha) S + beta k v^T
 *        (Gap Analysis §2, row "Recurrence"; beta as in "Metal (Apple GPU)
 *         backend for Kimi K3", Correctness, token-0 zero-state check);
 *   5. the readout o = S^T q from the updated state;
 *   6. y = sigmoid(g) * gamma * o / sqrt(mean(o^2) + rms_eps)
 *        (Gap Analysis §2, row "O projection": the gate and the per-head
 *         RMSNorm around St*q; the W_o and W_g matmuls are not part of it).
 *
 * Conventions (readings of the pages, stated once here):
 *   - conv: tap 3 multiplies the current raw row, tap 0 the oldest; no bias;
 *     the window holds the last 3 RAW rows, oldest first, channel order
 *     q | k | v, in fp32;
 *   - L2: x / sqrt(sum(x^2) + l2_eps); no scale on q;
 *   - gate: see kda_gate_mode; gamma has shape [dv], shared by all heads.
 *
 * Layouts (all device memory, C-contiguous, row = token index * H + head):
 *   q, k  [T, H, 128] act dtype     v, g  [T, H, 128] act dtype
 *   f     [T, H, 128] fp32          beta  [T, H]      fp32
 *   conv_w [H, 384, 4] fp32         A_log, dt_bias [H, 128] fp32
 *   gamma [128] fp32                y     [T, H, 128] act dtype
 *   state [N, H, 128, 128] fp32, row index = key channel, in/out
 *   conv_win [N, H, 3, 384] fp32, in/out
 *   o_raw [T, H, 128] fp32, optional (the pre-norm readout; test hook)
 * Every pointer must be 16-byte aligned, except beta (4-byte aligned, so that
 * one decode step's rows can be a slice of a longer run).  q, k, v, f, beta, g, conv_w, A_log,
 * dt_bias and gamma must not overlap y, o_raw, state or conv_win.
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer after
 * a call returns and allocates no device memory.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns at once.  A kernel fault surfaces at the
 * caller's next synchronisation, as for any HIP launch.  kda_sequence may
 * also use a second stream the caller passes (see there).
 *
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_DEVICE and
 * KDA_ERR_SCRATCH_LIMIT mean nothing was enqueued and no buffer was touched,
 * so the caller may run another implementation instead (the pages' fused
 * dispatch checks the return value and falls back to its CPU path: "Metal
 * (Apple GPU) backend for Kimi K3", CPU fallback).  KDA_ERR_LAUNCH means the
 * HIP runtime refused a launch; for a call that enqueues several kernels, the
 * ones before it stay enqueued.  The library itself never computes on the
 * CPU.
 *
 * Thread safety: the library keeps no streams, events or locks between
 * calls; its only process-wide state is a per-device cache of the device
 * kind and compute-unit count, and the static scratch of
 * kda_lowrank_gates_noalloc.  Calls on different streams with disjoint
 * buffers may run concurrently (the no-allocation call excepted).
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 2

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or enum */
    KDA_ERR_UNSUPPORTED = -2,   /* dims other than dk = dv = 128, 4 taps     */
    KDA_ERR_DEVICE = -3,        /* no current HIP device, or not gfx950      */
    KDA_ERR_LAUNCH = -4,        /* the HIP runtime refused the launch        */
    KDA_ERR_SCRATCH_LIMIT = -5  /* a no-allocation call needs more than the
                                   library's static scratch                  */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,                /* q, k, v, g, y in fp32                     */
    KDA_BF16 = 1                /* q, k, v, g, y in bf16 (math stays fp32)  */
} kda_dtype;

/* Decay gate forms ("Kimi K3 Metal Gap Analysis", §2, row "Decay compute").
 * The extracted text reads gk = -5 * (exp(A_log) * (f + dt_bias)), which is
 * not a decay when f + dt_bias < 0; a squashing function was evidently lost.
 * BOUNDED is the reading taken by default; the other two are exact forms. */
typedef enum kda_gate_mode {
    KDA_GATE_BOUNDED = 0,       /* gk = lb * sigmoid(exp(A_log) * (f + dt_bias)) */
    KDA_GATE_LITERAL = 1,       /* gk = lb * exp(A_log) * (f + dt_bias)         */
    KDA_GATE_RAW = 2            /* gk = f (the caller supplies the log-decay)   */
} kda_gate_mode;

/* Which prefill kernel kda_sequence runs.  All compute the same function
 * within the fp32 tolerance.  Where the gate allows the chunk form, AUTO
 * takes SHORT when the sequences hold fewer than 4 tokens on average
 * (total_tokens < 4 * num_seqs); else SCAN for at most 64 (sequence, head)
 * pairs averaging 128 tokens or more when the workspace is large enough;
 * else CHUNK_SHORT for sequences averaging at most 16 tokens, or at most 64
 * tokens from 512 pairs on; else CHUNK.  With the other gates AUTO takes
 * SHORT below 8 tokens on average, else SPLIT for few pairs and FUSED for
 * many.  SPLIT
 * spreads each pair's state columns over several workgroups (for few pairs,
 * e.g. one long sequence) and needs an fp32 buffer for the pre-norm readout:
 * o_raw, or else a workspace of the size kda_sequence_workspace_size reports.
 * CHUNK applies the recurrence 16 tokens at a time as small matrix products
 * on the matrix cores (bf16 operands split into high and low parts, about
 * 2^-16 relative error per product, fp32 accumulation and state). */
typedef enum kda_prefill_path {
    KDA_PREFILL_AUTO = 0,
    KDA_PREFILL_FUSED = 1,      /* one workgroup per (sequence, head)        */
    KDA_PREFILL_SPLIT = 2,      /* state columns split across workgroups    */
    KDA_PREFILL_CHUNK = 3,      /* 16-token chunks on the matrix cores; needs
                                   KDA_GATE_BOUNDED with |lb| <= 7.5, else
                                   KDA_ERR_UNSUPPORTED                       */
    KDA_PREFILL_SHORT = 4,      /* the decode step's layout with a token loop,
                                   for sequences of a few tokens; needs
                                   total_tokens * H * 512 < 2^32, else
                                   KDA_ERR_UNSUPPORTED                       */
    KDA_PREFILL_SCAN = 5        /* CHUNK in two passes: every chunk's
                                   input-only operands at once, then the
                                   chunks in order with each pair's state
                                   columns over 16 wavefronts; for few pairs of
                                   long sequences.  Same gate rule as CHUNK;
                                   needs the workspace kda_sequence_workspace_size
                                   reports (less the readout part when o_raw
                                   is given), else KDA_ERR_INVALID_ARG       */,
    KDA_PREFILL_CHUNK_SHORT = 6 /* CHUNK for sequences of a few chunks: each
                                   pair's chunks in turn without a pipeline,
                                   two workgroups per compute unit so that one
                                   pair's state load and store overlap another
                                   pair's arithmetic.  Same gate rule as CHUNK */
} kda_prefill_path;

typedef struct kda_config {
    int32_t num_heads;          /* H >= 1                                    */
    int32_t head_dim_k;         /* dk: must be 128                           */
    int32_t head_dim_v;         /* dv: must be 128                           */
    int32_t conv_taps;          /* must be 4                                 */
    int32_t act_dtype;          /* kda_dtype                                 */
    int32_t gate_mode;          /* kda_gate_mode                             */
    float gate_lower_bound;     /* lb, -5 in the pages                       */
    float l2_eps;               /* e.g. 1e-6                                 */
    float rms_eps;              /* e.g. 1e-6                                 */
    int32_t prefill_path;       /* kda_prefill_path (kda_sequence only)      */
} kda_config;

typedef struct kda_tensors {
    const void *q;              /* [T, H, 128] act dtype, raw (pre-conv)     */
    const void *k;              /* [T, H, 128] act dtype, raw                */
    const void *v;              /* [T, H, 128] act dtype, raw                */
    const float *f;             /* [T, H, 128] decay pre-activation          */
    const float *beta;          /* [T, H]                                    */
    const void *g;              /* [T, H, 128] act dtype, output-gate input  */
    const float *conv_w;        /* [H, 384, 4]                               */
    const float *A_log;         /* [H, 128]                                  */
    const float *dt_bias;       /* [H, 128]                                  */
    const float *gamma;         /* [128]                                     */
    float *state;               /* [N, H, 128, 128] in/out                   */
    float *conv_win;            /* [N, H, 3, 384] in/out                     */
    void *y;                    /* [T, H, 128] act dtype, out                */
    float *o_raw;               /* [T, H, 128] fp32 out, or NULL             */
} kda_tensors;

/*
 * Decode: one token for each of num_seqs sequences (T = num_seqs, token row
 * n belongs to sequence n): the whole token step of "Kimi K3 Metal Gap
 * Analysis", §2 KDA Attention (rows Conv4 + SiLU through O projection), as
 * "Metal (Apple GPU) backend for Kimi K3", Design notes, "Fused KDA token"
 * runs it for one token, with the state persisting in place between calls
 * (Design notes, zero-copy state persistence).  One kernel launch; each
 * (sequence, head) state is read once and written once.  num_seqs == 0 is a
 * no-op that returns KDA_OK after checking cfg (the tensor pointers are not
 * inspected).  Equivalent to kda_sequence with every sequence of length 1.
 */
kda_status kda_token_step(const kda_config *cfg, const kda_tensors *t,
                          int32_t num_seqs, void *stream);

/*
 * Prefill: the same step over num_seqs sequences packed along the token axis,
 * token by token in order within each sequence ("Kimi K3 Metal Gap
 * Analysis", §2 KDA Attention; "Metal (Apple GPU) backend for Kimi K3",
 * table "What runs where": the fused KDA row runs the step once per token,
 * and Performance: the 13-token prompt prefill goes through it).
 *   cu_seqlens  device int32 [num_seqs + 1] token offsets, or NULL for a
 *               dense batch of num_seqs sequences of total_tokens / num_seqs
 *               tokens each (total_tokens must divide evenly).
 *               Precondition (not checkable without a sync): cu[0] = 0,
 *               non-decreasing, cu[num_seqs] = total_tokens.  The kernel
 *               clamps every range to [0, total_tokens), so a violation gives
 *               wrong results but no out-of-bounds access.
 *   cu_seqlens_host  NULL, or a host copy of the same num_seqs + 1 offsets
 *               (only with a device cu_seqlens).  It is checked: cu[0] = 0,
 *               non-decreasing and cu[num_seqs] = total_tokens, else
 *               KDA_ERR_INVALID_ARG and nothing is enqueued.  It must hold
 *               the device array's values (not checkable).  It lets the
 *               library plan with the lengths: ragged batches of a few
 *               sequences then take the segmented two-pass schedule below.
 *               Not kept after the call.
 *   seq_order   device int32 [num_seqs] or NULL: the order in which sequences
 *               are scheduled (e.g. longest first).  Must be a permutation of
 *               0..num_seqs-1; entries outside that range are skipped.
 *   total_tokens  T, the number of token rows of q, k, v, f, beta, g, y.
 *   workspace, workspace_bytes  optional device scratch (see
 *               kda_sequence_workspace_size); NULL / 0 is always allowed.
 *   stream      the stream the call is ordered on.
 *   side_stream NULL, or a second stream of the same device (not `stream`,
 *               else KDA_ERR_INVALID_ARG).  The two-pass path of long
 *               sequences over at most 32 (sequence, head) pairs then runs
 *               the operand passes of later chunk segments and the finished
 *               segments' RMSNorm + gate on it, beside the state passes on
 *               `stream`.  The call joins the two with events it creates and
 *               releases: its work starts after everything enqueued on
 *               `stream` (and on side_stream) before the call, and
 *               everything enqueued on `stream` after the call starts after
 *               all of it; work enqueued on side_stream after the call may
 *               start before the call's work on `stream` is done.  With NULL
 *               everything runs on `stream` (same results).
 * Sequences of length 0 leave their state and window unchanged;
 * total_tokens == 0 is a no-op that returns KDA_OK after checking cfg (the
 * tensor pointers, which may then be NULL, are not inspected).  State and
 * window are carried in and out, so splitting a sequence across calls gives
 * the same result as one call (up to fp32 rounding order).
 */
kda_status kda_sequence(const kda_config *cfg, const kda_tensors *t,
                        int32_t num_seqs, const int32_t *cu_seqlens,
                        const int32_t *cu_seqlens_host, const int32_t *seq_order,
                        int64_t total_tokens, void *workspace, int64_t workspace_bytes,
                        void *stream, void *side_stream);

/*
 * Prefill with the decay pre-activation formed inside the step from the
 * low-rank factor: f[t, h, i] = sum_j w_fb[h * 128 + i, j] a[t, j] ("Kimi K3
 * Metal Gap Analysis", §2 KDA Attention, row "Decay compute": the decay is
 * formed from W_fb W_fa x), so f never goes through memory.  Everything else
 * as kda_sequence, with t->f NULL (else KDA_ERR_INVALID_ARG) and:
 *   a      [total_tokens, rank] fp32, device, 16-byte aligned: W_fa x of each
 *          token row (kda_lowrank_factor); read-only
 *   w_fb   [H * 128, rank] fp32, device, 16-byte aligned; read-only
 *   rank   a multiple of 32 up to 128 (above: KDA_ERR_UNSUPPORTED; use
 *          kda_lowrank_gates and kda_sequence)
 * It runs the one-pass chunk kernel (cfg->prefill_path AUTO or CHUNK, else
 * KDA_ERR_UNSUPPORTED), so it has the chunk form's gate rule (bounded gate,
 * |lb| <= 7.5, else KDA_ERR_UNSUPPORTED) and needs no workspace.  f is a
 * split-bf16 matrix-core product in the step (about 2^-16 relative error,
 * fp32 sums): the results agree with kda_lowrank_gates + kda_sequence within
 * the step's tolerance, not bit for bit.
 */
kda_status kda_sequence_lowrank(const kda_config *cfg, const kda_tensors *t, int32_t num_seqs,
                                const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                const int32_t *seq_order, int64_t total_tokens, const float *a,
                                const float *w_fb, int32_t rank, void *stream);

/*
 * Bytes of device workspace with which kda_sequence (above; same passages)
 * runs its faster path for
 * this shape (num_seqs sequences, total_tokens token rows, cfg->num_heads
 * heads, cfg->prefill_path); 0 if that path needs none.  A negative value is
 * a kda_status for bad arguments.  SPLIT uses it for its fp32 readout, which
 * o_raw replaces when given; SCAN for every chunk's operands (about 2.2 KiB
 * per token and head) followed by the readout (not needed with o_raw).
 * CHUNK (and AUTO where it takes CHUNK) asks for 256 bytes: a counter of
 * (sequence, head) pairs, which the call zeroes on `stream` before its kernel
 * runs.  With it the kernel runs one workgroup per compute unit, each taking
 * pairs in the scheduling order until none are left, so that compute units
 * running at different clocks share the work evenly; without it, one
 * workgroup per pair.  The results are the same bit for bit.  With
 * a smaller or NULL workspace kda_sequence falls back under
 * KDA_PREFILL_AUTO (to CHUNK or FUSED) and fails with KDA_ERR_INVALID_ARG
 * under KDA_PREFILL_SPLIT and KDA_PREFILL_SCAN.  Caller-owned, 16-byte
 * aligned, no initialisation needed, not kept after the call; its contents
 * are scratch (two calls in flight at once need a workspace each).
 */
int64_t kda_sequence_workspace_size(const kda_config *cfg, int32_t num_seqs,
                                    int64_t total_tokens);

/*
 * Projections on either side of the step: matrix products on the matrix
 * cores, one token row at a time (rows are independent).  Not part of the
 * step; they produce its f, beta and g inputs and consume its output y.
 * Layouts: row-major, device memory, 16-byte aligned (beta: 4-byte); no
 * output may overlap an input or another output.  An fp32 operand enters the
 * matrix cores split into two bf16 parts, the product formed from three bf16
 * products (about 2^-16 relative error each, fp32 sums); bf16 x bf16
 * products are exact, with fp32 sums.  Errors as for the step: nothing is
 * enqueued unless KDA_OK or KDA_ERR_LAUNCH comes back; tokens == 0 is a no-op
 * after cfg is checked; cfg->num_heads may be at most 65536 here.  workspace
 * (caller-owned, 16-byte aligned, scratch)
 * lets calls with few token rows split each sum across more workgroups; its
 * size for the fastest run is kda_projection_workspace_size.
 */
typedef enum kda_projection {
    KDA_PROJ_LOWRANK_GATES = 0,  /* kda_lowrank_gates     */
    KDA_PROJ_GATE = 1,           /* kda_gate_projection   */
    KDA_PROJ_OUTPUT = 2,         /* kda_output_projection */
    KDA_PROJ_LOWRANK_FACTOR = 3  /* kda_lowrank_factor    */
} kda_projection;

/*
 * Bytes of workspace for the fastest run of projection `which` (rank is read
 * for KDA_PROJ_LOWRANK_GATES only), or a negative kda_status.  The
 * projections are those of "Kimi K3 Metal Gap Analysis", §2 KDA Attention,
 * rows "Decay compute" and "O projection" (below).
 */
int64_t kda_projection_workspace_size(const kda_config *cfg, int32_t which, int32_t hidden,
                                      int32_t rank, int64_t tokens);

/*
 * The decay pre-activation and beta from the layer's hidden rows
 * ("Kimi K3 Metal Gap Analysis", §2 KDA Attention, row "Decay compute": the
 * decay is formed from W_fb W_fa x; "Metal (Apple GPU) backend for Kimi K3",
 * table "What runs where": fa, fb and bp are fp32 low-rank products; beta as
 * the sigmoid of the bp product is a reading).  For each token row t:
 *   a[t]       = W_fa x[t]                               (rank values)
 *   f[t, h, i] = sum_j W_fb[h * 128 + i, j] a[t, j]
 *   beta[t, h] = sigmoid(W_bp[h] . x[t])
 * x [tokens, hidden] act dtype; w_fa_bp [rank + H, hidden] fp32 (the rank
 * rows of W_fa, then the H rows of W_bp, so that one pass over x serves
 * both); w_fb [H * 128, rank] fp32; f [tokens, H, 128] fp32 out and beta
 * [tokens, H] fp32 out: the f and beta inputs of kda_token_step and
 * kda_sequence.  workspace: required, at least tokens * rank * 4 bytes
 * rounded up to 256 (it holds a).  From 512 token rows, with the bytes
 * kda_projection_workspace_size reports, it also holds w_fa_bp split into
 * bf16 parts once per call (the product then reads those instead of
 * splitting the fp32 weights itself; the results are the same).  hidden: a
 * positive multiple of 32; rank: a multiple of 32 in [32, 1024].
 */
kda_status kda_lowrank_gates(const kda_config *cfg, const void *x, const float *w_fa_bp,
                             const float *w_fb, int32_t hidden, int32_t rank, int64_t tokens,
                             float *f, float *beta, void *workspace, int64_t workspace_bytes,
                             void *stream);

/*
 * The first low-rank product alone, for kda_sequence_lowrank: for each token
 * row t, a[t] = W_fa x[t] (rank values, fp32) and beta[t, h] =
 * sigmoid(W_bp[h] . x[t]) (Gap Analysis §2, row "Decay compute"; PR table
 * "What runs where", KDA low-rank fa, fb, bp).  Arguments as for
 * kda_lowrank_gates, with a [tokens, rank] fp32 out in place of f; workspace
 * optional (with the bytes kda_projection_workspace_size reports for
 * KDA_PROJ_LOWRANK_FACTOR the weights are split into bf16 parts once and few
 * token rows split their sums; results equal).
 */
kda_status kda_lowrank_factor(const kda_config *cfg, const void *x, const float *w_fa_bp, int32_t hidden,
                              int32_t rank, int64_t tokens, float *a, float *beta, void *workspace,
                              int64_t workspace_bytes, void *stream);

/*
 * kda_lowrank_gates without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as
 * kda_lowrank_gates, except that the workspace is the library's own static
 * scratch: a device array of KDA_NOALLOC_SCRATCH_BYTES (16 MiB) that each
 * device the library runs on holds until the process ends.  The call
 * allocates nothing.  Limit: tokens * rank * 4 bytes, rounded up to 256, must
 * fit in the scratch, else KDA_ERR_SCRATCH_LIMIT and nothing is enqueued;
 * the bf16 weight parts and the split-K partial sums use what is left of it
 * when they fit (the results equal those of kda_lowrank_gates with a
 * workspace of the same size).  Every call on a device shares that device's
 * scratch: calls that overlap in time on one device (different streams,
 * threads or processes) race and must not be issued.  A failure to reach the
 * scratch on the current device returns KDA_ERR_DEVICE.
 */
#define KDA_NOALLOC_SCRATCH_BYTES 16777216
kda_status kda_lowrank_gates_noalloc(const kda_config *cfg, const void *x, const float *w_fa_bp,
                                     const float *w_fb, int32_t hidden, int32_t rank, int64_t tokens,
                                     float *f, float *beta, void *stream);

/*
 * g = W_g x, the input of the step's output gate (Gap Analysis §2, row "O
 * projection").  x [tokens, hidden] act dtype; w_g [H * 128, hidden] act
 * dtype; g [tokens, H, 128] act dtype out.  hidden: a positive multiple of
 * 32.  workspace optional.
 */
kda_status kda_gate_projection(const kda_config *cfg, const void *x, const void *w_g,
                               int32_t hidden, int64_t tokens, void *g,
                               void *workspace, int64_t workspace_bytes, void *stream);

/*
 * out = W_o y, the output projection of the step's output (Gap Analysis §2,
 * row "O projection").  y [tokens, H, 128] act dtype; w_o [hidden, H * 128]
 * act dtype; out [tokens, hidden] act dtype.  hidden: a positive multiple of
 * 4.  workspace optional.
 */
kda_status kda_output_projection(const kda_config *cfg, const void *y, const void *w_o,
                                 int32_t hidden, int64_t tokens, void *out,
                                 void *workspace, int64_t workspace_bytes, void *stream);

/* Static description of a status code (never NULL).  The codes are the
 * checked return of the fused dispatch ("Metal (Apple GPU) backend for Kimi
 * K3", CPU fallback: a failed GPU call falls back instead of misbehaving). */
const char *kda_status_string(int32_t status);

/* KDA_VERSION of the built library (the interface of this header). */
int32_t kda_version(void);

/*
 * KDA_OK if the current HIP device is a gfx950 part the library was built
 * for, else KDA_ERR_DEVICE.  Cheap after the first call on a device.  (The
 * GPU path is reachable only when a usable device exists: "Metal (Apple GPU)
 * backend for Kimi K3", CPU fallback.)
 */
kda_status kda_device_check(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
