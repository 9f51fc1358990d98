/*
 * kda_oracle.c -- plain CPU oracle for the fused KDA (Kimi Delta Attention)
 * token step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU-baseline
 * leg use it.  It shares no code, header, table or constant with the HIP
 * library; the two meet only through seeded inputs.
 *
 * What it computes (one (sequence, head) pair at a time, tokens in order):
 *
 *   1. Causal depthwise conv, 4 taps, then SiLU, on the q|k|v channels, with
 *      the conv window carried across calls
 *        -- "Kimi K3 Metal Gap Analysis", §2 KDA Attention, row "Conv4 + SiLU"
 *           (causal convolution of q/k/v with conv-state management);
 *        -- "Metal (Apple GPU) backend for Kimi K3", Design notes, "Fused KDA
 *           token" (conv_silu applied to each of q, k, v).
 *   2. Per-head L2 normalisation of q and k (v is not normalised)
 *        -- Gap Analysis §2, row "L2 normalize q/k".
 *   3. Per-key-channel decay gk built from A_log, dt_bias and the decay
 *      pre-activation f (the page's W_fb W_fa x), alpha = exp(gk)
 *        -- Gap Analysis §2, row "Decay compute".
 *   4. Gated delta-rule update of the dk x dv state,
 *        S <- (I - beta k k^T) Diag(alpha) S + beta k v^T
 *        -- Gap Analysis §2, row "Recurrence" (beta is lost from the extracted
 *           text; it is present in "Metal (Apple GPU) backend for Kimi K3",
 *           Correctness, token-0 zero-state check).
 *   5. Readout o = S^T q, taken AFTER the update
 *        -- Gap Analysis §2, row "O projection" (St*q); the order follows the
 *           token-0 check, where a zero state still gives a nonzero output.
 *   6. Per-head RMSNorm of o, times gamma, times sigmoid of the output-gate
 *      pre-activation g
 *        -- Gap Analysis §2, row "O projection" (sig(W_g x) * RMSNorm_head).
 *   7. State and window persist in place across calls
 *        -- "Metal (Apple GPU) backend for Kimi K3", Design notes, zero-copy
 *           state persistence.
 *
 * Readings taken where the pages are silent or garbled:
 *   - gate (BOUNDED, default): gk = lb * sigmoid(exp(A_log) * (f + dt_bias)),
 *     lb = -5.  The extracted text shows lb * exp(A_log) * (f + dt_bias) with
 *     no squashing function; that literal form is gate mode LITERAL, and
 *     gate mode RAW takes gk = f directly.
 *   - conv: cross-correlation, tap (taps-1) multiplies the current token,
 *     tap 0 the oldest; no bias; the window keeps the last taps-1 RAW rows,
 *     oldest first, channel order q|k|v.
 *   - L2: x / sqrt(sum x^2 + l2_eps).  RMSNorm: o / sqrt(mean o^2 + rms_eps),
 *     gamma has shape [dv] and is shared by every head, the gate multiplies
 *     after the norm.  No scale factor on q.
 *
 * Arithmetic is fp64 throughout (kda_oracle_run, the parity reference; a
 * single-precision copy of the same loops, kda_oracle_run_f32, at the end of
 * this file, is what the CPU baseline times).  Per-token inputs and parameters arrive as
 * fp32 (the data itself; widening is exact); state, window and outputs are
 * fp64.  The steps run in the order the pages give them -- decay, then
 * u = S^T k, then the rank-1 correction, then the readout -- with no fusion.
 *
 * Parity pins (see tests/test_oracle_pins.py): zero-state first token
 * o = beta (q.k) v; alpha = beta = 1 with q = k maps k to v; beta = 0 leaves
 * S alone; alpha = 0 resets S; dense matrix-product brute force at tiny dims;
 * one-hot taps; split and ragged invariance; closed forms of every gate mode.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

enum { ORACLE_GATE_BOUNDED = 0, ORACLE_GATE_LITERAL = 1, ORACLE_GATE_RAW = 2 };

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

int32_t kda_oracle_version(void) { return 1; }

/*
 * Run the KDA step over N sequences x H heads.
 *   cu       [N+1]        token offsets of each sequence (cu[0] = 0)
 *   q, k     [T, H, dk]   raw (pre-conv) query / key rows
 *   v        [T, H, dv]   raw value rows
 *   f        [T, H, dk]   decay pre-activation (gk itself in RAW mode)
 *   beta     [T, H]
 *   g        [T, H, dv]   output-gate pre-activation
 *   conv_w   [H, C, taps] C = 2*dk + dv
 *   A_log    [H, dk], dt_bias [H, dk], gamma [dv]
 *   state    [N, H, dk, dv]      in/out
 *   win      [N, H, taps-1, C]   in/out (oldest row first)
 *   y        [T, H, dv]   out
 *   o_raw    [T, H, dv]   out, may be NULL
 * Returns 0, or -1 on a bad argument.
 */
int32_t kda_oracle_run(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t taps,
                       const int64_t *cu,
                       const float *q, const float *k, const float *v,
                       const float *f, const float *beta, const float *g,
                       const float *conv_w, const float *A_log,
                       const float *dt_bias, const float *gamma,
                       int32_t gate_mode, double lower_bound,
                       double l2_eps, double rms_eps,
                       double *state, double *win, double *y, double *o_raw)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || taps < 1) return -1;
    if (gate_mode < 0 || gate_mode > 2) return -1;
    const int64_t C = 2 * (int64_t)dk + dv;
    const int64_t P = taps - 1;
    const int64_t units = (int64_t)N * H;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        double *S = state + unit * dk * dv;
        double *W = win + unit * P * C;
        double *x = (double *)malloc(sizeof(double) * (size_t)(4 * C + 4 * dk + 2 * dv));
        double *a = x + C;
        double *qh = a + C;
        double *kh = qh + dk;
        double *alpha = kh + dk;
        double *u = alpha + dk;
        double *o = u + dv;
        double *c = o + dv;

        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t row = t * H + h;

            /* 1. gather the raw channels q|k|v of this token */
            for (int64_t i = 0; i < dk; ++i) x[i] = q[row * dk + i];
            for (int64_t i = 0; i < dk; ++i) x[dk + i] = k[row * dk + i];
            for (int64_t j = 0; j < dv; ++j) x[2 * dk + j] = v[row * dv + j];

            /* causal depthwise conv over [window rows..., current row] */
            for (int64_t ch = 0; ch < C; ++ch) {
                const float *w = conv_w + ((int64_t)h * C + ch) * taps;
                double acc = 0.0;
                for (int64_t j = 0; j < P; ++j) acc += (double)w[j] * W[j * C + ch];
                acc += (double)w[P] * x[ch];
                c[ch] = acc;
            }
            /* SiLU */
            for (int64_t ch = 0; ch < C; ++ch) a[ch] = c[ch] * sigmoid(c[ch]);
            /* window <- drop the oldest row, append the raw current row */
            for (int64_t j = 0; j + 1 < P; ++j)
                for (int64_t ch = 0; ch < C; ++ch) W[j * C + ch] = W[(j + 1) * C + ch];
            if (P > 0)
                for (int64_t ch = 0; ch < C; ++ch) W[(P - 1) * C + ch] = x[ch];

            /* 2. L2 normalisation of q and k */
            double sq = 0.0, sk = 0.0;
            for (int64_t i = 0; i < dk; ++i) sq += a[i] * a[i];
            for (int64_t i = 0; i < dk; ++i) sk += a[dk + i] * a[dk + i];
            const double nq = sqrt(sq + l2_eps), nk = sqrt(sk + l2_eps);
            for (int64_t i = 0; i < dk; ++i) qh[i] = a[i] / nq;
            for (int64_t i = 0; i < dk; ++i) kh[i] = a[dk + i] / nk;
            const double *vv = a + 2 * dk;

            /* 3. per-channel decay */
            for (int64_t i = 0; i < dk; ++i) {
                const double fi = f[row * dk + i];
                double gk;
                if (gate_mode == ORACLE_GATE_RAW) {
                    gk = fi;
                } else {
                    const double z = exp((double)A_log[(int64_t)h * dk + i]) *
                                     (fi + (double)dt_bias[(int64_t)h * dk + i]);
                    gk = (gate_mode == ORACLE_GATE_BOUNDED) ? lower_bound * sigmoid(z)
                                                            : lower_bound * z;
                }
                alpha[i] = exp(gk);
            }

            /* 4. S <- Diag(alpha) S; u = S^T k; S <- S + beta k (v - u)^T */
            const double b = beta[row];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= alpha[i];
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += S[i * dv + j] * kh[i];
                u[j] = acc;
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += b * kh[i] * (vv[j] - u[j]);

            /* 5. readout from the updated state */
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += S[i * dv + j] * qh[i];
                o[j] = acc;
            }

            /* 6. RMSNorm over dv, gamma, sigmoid output gate */
            double ms = 0.0;
            for (int64_t j = 0; j < dv; ++j) ms += o[j] * o[j];
            ms /= (double)dv;
            const double r = 1.0 / sqrt(ms + rms_eps);
            for (int64_t j = 0; j < dv; ++j) {
                y[row * dv + j] = sigmoid((double)g[row * dv + j]) * (double)gamma[j] * o[j] * r;
                if (o_raw) o_raw[row * dv + j] = o[j];
            }
        }
        free(x);
    }
    return 0;
}

/*
 * The same step in single precision, for timing the CPU baseline.
 *
 * Identical loops and order to kda_oracle_run above (conv, SiLU, window
 * shift, L2, decay, Diag(alpha) S, u = S^T k, rank-1 correction, readout,
 * RMSNorm + gate), with every intermediate, the state and the window held in
 * float.  state, win, y and o_raw are float arrays; state and win are updated
 * in place, so a decode run can call this once per step on the step's token
 * rows (cu = 0, 1, ..., N) without copying the state.  It is not the parity
 * reference: kda_oracle_run (fp64) is; this one is pinned to it on the
 * 64-token single-head workload.
 */
static float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

int32_t kda_oracle_run_f32(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t taps,
                           const int64_t *cu,
                           const float *q, const float *k, const float *v,
                           const float *f, const float *beta, const float *g,
                           const float *conv_w, const float *A_log,
                           const float *dt_bias, const float *gamma,
                           int32_t gate_mode, float lower_bound,
                           float l2_eps, float rms_eps,
                           float *state, float *win, float *y, float *o_raw)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || taps < 1) return -1;
    if (gate_mode < 0 || gate_mode > 2) return -1;
    const int64_t C = 2 * (int64_t)dk + dv;
    const int64_t P = taps - 1;
    const int64_t units = (int64_t)N * H;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        float *S = state + unit * dk * dv;
        float *W = win + unit * P * C;
        float *x = (float *)malloc(sizeof(float) * (size_t)(4 * C + 4 * dk + 2 * dv));
        float *a = x + C;
        float *qh = a + C;
        float *kh = qh + dk;
        float *alpha = kh + dk;
        float *u = alpha + dk;
        float *o = u + dv;
        float *c = o + dv;

        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t row = t * H + h;

            /* 1. raw channels, causal conv, SiLU, window shift */
            for (int64_t i = 0; i < dk; ++i) x[i] = q[row * dk + i];
            for (int64_t i = 0; i < dk; ++i) x[dk + i] = k[row * dk + i];
            for (int64_t j = 0; j < dv; ++j) x[2 * dk + j] = v[row * dv + j];
            for (int64_t ch = 0; ch < C; ++ch) {
                const float *w = conv_w + ((int64_t)h * C + ch) * taps;
                float acc = 0.0f;
                for (int64_t j = 0; j < P; ++j) acc += w[j] * W[j * C + ch];
                acc += w[P] * x[ch];
                c[ch] = acc;
            }
            for (int64_t ch = 0; ch < C; ++ch) a[ch] = c[ch] * sigmoidf_(c[ch]);
            for (int64_t j = 0; j + 1 < P; ++j)
                for (int64_t ch = 0; ch < C; ++ch) W[j * C + ch] = W[(j + 1) * C + ch];
            if (P > 0)
                for (int64_t ch = 0; ch < C; ++ch) W[(P - 1) * C + ch] = x[ch];

            /* 2. L2 normalisation of q and k */
            float sq = 0.0f, sk = 0.0f;
            for (int64_t i = 0; i < dk; ++i) sq += a[i] * a[i];
            for (int64_t i = 0; i < dk; ++i) sk += a[dk + i] * a[dk + i];
            const float nq = sqrtf(sq + l2_eps), nk = sqrtf(sk + l2_eps);
            for (int64_t i = 0; i < dk; ++i) qh[i] = a[i] / nq;
            for (int64_t i = 0; i < dk; ++i) kh[i] = a[dk + i] / nk;
            const float *vv = a + 2 * dk;

            /* 3. per-channel decay */
            for (int64_t i = 0; i < dk; ++i) {
                const float fi = f[row * dk + i];
                float gk;
                if (gate_mode == ORACLE_GATE_RAW) {
                    gk = fi;
                } else {
                    const float z = expf(A_log[(int64_t)h * dk + i]) * (fi + dt_bias[(int64_t)h * dk + i]);
                    gk = (gate_mode == ORACLE_GATE_BOUNDED) ? lower_bound * sigmoidf_(z) : lower_bound * z;
                }
                alpha[i] = expf(gk);
            }

            /* 4. S <- Diag(alpha) S; u = S^T k; S <- S + beta k (v - u)^T */
            const float b = beta[row];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= alpha[i];
            for (int64_t j = 0; j < dv; ++j) {
                float acc = 0.0f;
                for (int64_t i = 0; i < dk; ++i) acc += S[i * dv + j] * kh[i];
                u[j] = acc;
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += b * kh[i] * (vv[j] - u[j]);

            /* 5. readout from the updated state */
            for (int64_t j = 0; j < dv; ++j) {
                float acc = 0.0f;
                for (int64_t i = 0; i < dk; ++i) acc += S[i * dv + j] * qh[i];
                o[j] = acc;
            }

            /* 6. RMSNorm over dv, gamma, sigmoid output gate */
            float ms = 0.0f;
            for (int64_t j = 0; j < dv; ++j) ms += o[j] * o[j];
            ms /= (float)dv;
            const float r = 1.0f / sqrtf(ms + rms_eps);
            for (int64_t j = 0; j < dv; ++j) {
                y[row * dv + j] = sigmoidf_(g[row * dv + j]) * gamma[j] * o[j] * r;
                if (o_raw) o_raw[row * dv + j] = o[j];
            }
        }
        free(x);
    }
    return 0;
}
