// kda_prefill.hip -- multi-token KDA over dense or ragged (cu_seqlens) batches,
// with state and conv window carried in and out.
//
// In the recurrent form every token touches every state element a few times
// (two dot products and the update) against almost no memory traffic, so the
// kernel is built around keeping the state resident and the VALU busy:
//   * one 128-thread workgroup (two wavefronts) per (sequence, head); the
//     128 x 128 fp32 state lives in registers for the whole token run,
//     128 floats per lane: lane (rg, cg) holds rows 16 rg .. 16 rg + 15 and
//     columns 8 cg .. 8 cg + 7, with rg in the low 3 lane bits so the
//     reductions over rows are 3 DPP steps inside a group of 8 lanes;
//   * tokens run in chunks of TC.  Per chunk, phase P computes everything
//     that depends only on inputs, in parallel over the chunk: the conv4 +
//     SiLU pre-step and L2 norms token by token (one wavefront per token),
//     and the decays key row by key row (one thread per row); phase Q
//     combines them into per-row coefficients in LDS; phase R runs the serial
//     recurrence reading those as LDS broadcasts; the RMSNorm + gate epilogue
//     of a chunk runs token-parallel in the next phase P, off the serial chain;
//   * the readout uses the pre-update state, o = S^T(alpha q) + beta (q.k)
//     (v - u), so one read of the registers feeds both dot products
//     ("Kimi K3 Metal Gap Analysis", §2, rows "Recurrence" and
//     "O projection", expanded).
//
// Decay folding (FOLD = true).  Inside a chunk the registers hold
// X_t = D_t^{-1} S_t, with D_t = Diag(alpha_1 ... alpha_t) the decay
// accumulated since the chunk start.  Then
//     u_t = X_{t-1}^T (D_t k),  p_t = X_{t-1}^T (D_t q),
//     X_t = X_{t-1} + (D_t^{-1} k) delta_t^T,
// so each state element costs 3 FMAs per token instead of 4 operations, and
// S = D X is restored once per chunk.  Rounding is of the same size as in the
// direct form (every product has the same magnitude once the D factors are
// applied).  It needs D_t to stay well inside fp32 range, which holds when
// the decay is bounded below: the bounded gate with lb * TC >= -60.  Other
// gate forms (unbounded log-decay) take the direct form.
#include "kda_device.hpp"

namespace kda {

namespace {

constexpr int PF_THREADS = 128;
constexpr int TC = 8;              // tokens per chunk
constexpr int HALF = TC / 2;       // chunk slots handled by each wavefront in phase P
constexpr int RGS = 17;            // LDS slots per row group: 16 key rows + 1 pad (bank spread)
constexpr float FOLD_MIN_LOG_DECAY = -60.0f;   // lowest chunk log-decay the folded form accepts

template <typename Act>
struct Ctx {
    const void *q, *k, *v;
    const float *W;   // carried-in window of this (sequence, head); read-only until the end
    int64_t lo;       // first token row of the sequence
    int H, h, lane;

    // raw row j of the history (j < 0: window row j + PAST), channels 2 lane, 2 lane + 1
    __device__ __forceinline__ void hist(int64_t j, float2 &xq, float2 &xk, float2 &xv) const {
        if (j >= 0) {
            const int64_t r = ((lo + j) * H + h) * DK + 2 * lane;
            xq = Act::load2(q, r);
            xk = Act::load2(k, r);
            xv = Act::load2(v, r);
        } else {
            const float *wr = W + (j + PAST) * CH + 2 * lane;
            xq = *reinterpret_cast<const float2 *>(wr);
            xk = *reinterpret_cast<const float2 *>(wr + DK);
            xv = *reinterpret_cast<const float2 *>(wr + 2 * DK);
        }
    }
};

__device__ __forceinline__ float conv4(float4 w, float a, float b, float c, float x) {
    return w.x * a + w.y * b + w.z * c + w.w * x;
}

// LDS slot of key row i in the padded row-group layout
__device__ __forceinline__ int row_slot(int i) { return (i >> 4) * RGS + (i & 15); }

template <typename Act, bool FOLD>
__global__ __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(Params p) {
    const int slot_n = blockIdx.x / p.H;
    const int h = blockIdx.x - slot_n * p.H;
    int n = slot_n;
    if (p.seq_order) {
        n = p.seq_order[slot_n];
        if (n < 0 || n >= p.num_seqs) return;
    }
    const Range rng = seq_range(p, n);
    if (rng.len <= 0) return;
    const int64_t L = rng.len;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rg = lane & 7;                   // row group: rows 16 rg .. 16 rg + 15
    const int cg = wave * 8 + (lane >> 3);     // column group: columns 8 cg .. 8 cg + 7
    const int64_t unit = (int64_t)n * p.H + h;

    // per-row coefficients for the dot products: FOLD (D k, D q), else (alpha k, alpha q)
    __shared__ float2 s_dot[TC][8 * RGS];
    // per-row coefficients for the update: FOLD (k / D, -), else (alpha, k)
    __shared__ float2 s_upd[TC][8 * RGS];
    __shared__ float s_col[TC][DV];            // activated v, overwritten by the readout o
    __shared__ float2 s_tok[TC];               // (beta, q_hat . k_hat)
    __shared__ float s_kh[TC][DK];             // k_hat of each chunk token
    __shared__ float s_qh[TC][DK];             // q_hat of each chunk token
    __shared__ float s_dec[TC][DK];            // FOLD: D_t (decay since chunk start); else alpha_t

    float *S = p.state + unit * (DK * DV);
    float *Wout = p.win + unit * (PAST * CH);
    const Ctx<Act> cx{p.q, p.k, p.v, Wout, rng.lo, p.H, h, lane};

    float4 s[16][2];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float *src = S + (16 * rg + m) * DV + 8 * cg;
        s[m][0] = *reinterpret_cast<const float4 *>(src);
        s[m][1] = *reinterpret_cast<const float4 *>(src + 4);
    }

    const int s0 = wave * HALF;                // this wavefront's chunk slots in phase P

    // Phase P issues every global load of a helper before the first use, so a
    // chunk pays one memory latency per helper rather than one per token.

    // token-parallel epilogue of slots [s0, s0 + HALF) of the chunk starting at c0
    auto epilogue = [&](int64_t c0, int nvalid) {
        const float2 gm = *reinterpret_cast<const float2 *>(p.gamma + 2 * lane);
        float2 gg[HALF];
#pragma unroll
        for (int sl = 0; sl < HALF; ++sl) {
            const int slot = s0 + sl;
            gg[sl] = slot < nvalid
                ? Act::load2(p.g, ((rng.lo + c0 + slot) * p.H + h) * DV + 2 * lane)
                : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int sl = 0; sl < HALF; ++sl) {
            const int slot = s0 + sl;
            if (slot >= nvalid) break;
            const float2 o = *reinterpret_cast<const float2 *>(&s_col[slot][2 * lane]);
            const float ss = sum64(o.x * o.x + o.y * o.y);
            const float r = rsqrtf(ss * (1.0f / DV) + p.rms_eps);
            const int64_t orow = ((rng.lo + c0 + slot) * p.H + h) * DV + 2 * lane;
            float2 y;
            y.x = sigmoid(gg[sl].x) * gm.x * o.x * r;
            y.y = sigmoid(gg[sl].y) * gm.y * o.y * r;
            Act::store2(p.y, orow, y);
            if (p.o_raw) *reinterpret_cast<float2 *>(p.o_raw + orow) = o;
        }
    };

    // token pre-step of slots [s0, s0 + HALF) of the chunk starting at c0:
    // conv4 + SiLU over the raw rows j0 - 3 .. j0 + HALF - 1, L2 norms, beta, q.k
    auto prestep_tokens = [&](int64_t c0) {
        const int64_t j0 = c0 + s0;
        if (j0 >= L) return;
        const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);
        const int c = 2 * lane;
        const float4 wq0 = *reinterpret_cast<const float4 *>(cw + c * TAPS);
        const float4 wq1 = *reinterpret_cast<const float4 *>(cw + (c + 1) * TAPS);
        const float4 wk0 = *reinterpret_cast<const float4 *>(cw + (DK + c) * TAPS);
        const float4 wk1 = *reinterpret_cast<const float4 *>(cw + (DK + c + 1) * TAPS);
        const float4 wv0 = *reinterpret_cast<const float4 *>(cw + (2 * DK + c) * TAPS);
        const float4 wv1 = *reinterpret_cast<const float4 *>(cw + (2 * DK + c + 1) * TAPS);

        float2 xq[PAST + HALF], xk[PAST + HALF], xv[PAST + HALF];
        float bta[HALF];
#pragma unroll
        for (int r = 0; r < PAST + HALF; ++r) {
            const int64_t j = j0 - PAST + r;
            if (j < L) {
                cx.hist(j, xq[r], xk[r], xv[r]);
            } else {
                xq[r] = xk[r] = xv[r] = make_float2(0.f, 0.f);
            }
        }
#pragma unroll
        for (int sl = 0; sl < HALF; ++sl)
            bta[sl] = (lane == 0 && j0 + sl < L) ? p.beta[(rng.lo + j0 + sl) * p.H + h] : 0.f;

#pragma unroll
        for (int sl = 0; sl < HALF; ++sl) {
            if (j0 + sl >= L) break;
            const float aq0 = silu(conv4(wq0, xq[sl].x, xq[sl + 1].x, xq[sl + 2].x, xq[sl + 3].x));
            const float aq1 = silu(conv4(wq1, xq[sl].y, xq[sl + 1].y, xq[sl + 2].y, xq[sl + 3].y));
            const float ak0 = silu(conv4(wk0, xk[sl].x, xk[sl + 1].x, xk[sl + 2].x, xk[sl + 3].x));
            const float ak1 = silu(conv4(wk1, xk[sl].y, xk[sl + 1].y, xk[sl + 2].y, xk[sl + 3].y));
            const float av0 = silu(conv4(wv0, xv[sl].x, xv[sl + 1].x, xv[sl + 2].x, xv[sl + 3].x));
            const float av1 = silu(conv4(wv1, xv[sl].y, xv[sl + 1].y, xv[sl + 2].y, xv[sl + 3].y));

            const float qq = sum64(aq0 * aq0 + aq1 * aq1);
            const float kk = sum64(ak0 * ak0 + ak1 * ak1);
            const float qk = sum64(aq0 * ak0 + aq1 * ak1);
            const float rq = rsqrtf(qq + p.l2_eps), rk = rsqrtf(kk + p.l2_eps);

            const int slot = s0 + sl;
            *reinterpret_cast<float2 *>(&s_qh[slot][c]) = make_float2(aq0 * rq, aq1 * rq);
            *reinterpret_cast<float2 *>(&s_kh[slot][c]) = make_float2(ak0 * rk, ak1 * rk);
            *reinterpret_cast<float2 *>(&s_col[slot][c]) = make_float2(av0, av1);
            if (lane == 0) s_tok[slot] = make_float2(bta[sl], qk * rq * rk);
        }
    };

    // row pre-step of the chunk starting at c0 (thread tid = key row): the
    // decays of its nv tokens, accumulated from the chunk start when folding
    const float eA = __expf(p.A_log[h * DK + tid]);
    const float dtb = p.dt_bias[h * DK + tid];
    auto prestep_rows = [&](int64_t c0, int nv) {
        float fv[TC];
#pragma unroll
        for (int t = 0; t < TC; ++t)
            fv[t] = t < nv ? p.f[((rng.lo + c0 + t) * p.H + h) * DK + tid] : 0.f;
        float D = 1.0f;
#pragma unroll
        for (int t = 0; t < TC; ++t) {
            if (t >= nv) break;
            const float al = decay(fv[t], eA, dtb, p.gate_mode, p.lb);
            if constexpr (FOLD) {
                D *= al;
                s_dec[t][tid] = D;
            } else {
                s_dec[t][tid] = al;
            }
        }
    };

    // phase Q (thread tid = key row): per-row coefficients of the chunk's tokens
    auto combine_rows = [&](int nv) {
        const int slot = row_slot(tid);
#pragma unroll 1
        for (int t = 0; t < nv; ++t) {
            const float kh = s_kh[t][tid], qh = s_qh[t][tid], dd = s_dec[t][tid];
            s_dot[t][slot] = make_float2(dd * kh, dd * qh);
            if constexpr (FOLD)
                s_upd[t][slot] = make_float2(kh * fast_rcp(dd), 0.0f);
            else
                s_upd[t][slot] = make_float2(dd, kh);
        }
    };

#pragma unroll 1
    for (int64_t c0 = 0; c0 < L; c0 += TC) {
        const int nv = (int)((L - c0) < TC ? (L - c0) : TC);
        if (c0 > 0) epilogue(c0 - TC, TC);
        prestep_tokens(c0);
        prestep_rows(c0, nv);
        __syncthreads();
        combine_rows(nv);
        __syncthreads();

#pragma unroll 1
        for (int t = 0; t < nv; ++t) {
            const float2 bt = s_tok[t];
            float u[8], pq[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) { u[c] = 0.f; pq[c] = 0.f; }
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float2 rd = s_dot[t][rg * RGS + m];
                u[0] += s[m][0].x * rd.x; u[1] += s[m][0].y * rd.x;
                u[2] += s[m][0].z * rd.x; u[3] += s[m][0].w * rd.x;
                u[4] += s[m][1].x * rd.x; u[5] += s[m][1].y * rd.x;
                u[6] += s[m][1].z * rd.x; u[7] += s[m][1].w * rd.x;
                pq[0] += s[m][0].x * rd.y; pq[1] += s[m][0].y * rd.y;
                pq[2] += s[m][0].z * rd.y; pq[3] += s[m][0].w * rd.y;
                pq[4] += s[m][1].x * rd.y; pq[5] += s[m][1].y * rd.y;
                pq[6] += s[m][1].z * rd.y; pq[7] += s[m][1].w * rd.y;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) { u[c] = sum8(u[c]); pq[c] = sum8(pq[c]); }

            const float4 v0 = *reinterpret_cast<const float4 *>(&s_col[t][8 * cg]);
            const float4 v1 = *reinterpret_cast<const float4 *>(&s_col[t][8 * cg + 4]);
            const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            float d[8], o[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                d[c] = bt.x * (vv[c] - u[c]);
                o[c] = pq[c] + bt.y * d[c];
            }
            if constexpr (FOLD) {
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const float ck = s_upd[t][rg * RGS + m].x;   // k_hat / D_t
                    s[m][0].x += ck * d[0]; s[m][0].y += ck * d[1];
                    s[m][0].z += ck * d[2]; s[m][0].w += ck * d[3];
                    s[m][1].x += ck * d[4]; s[m][1].y += ck * d[5];
                    s[m][1].z += ck * d[6]; s[m][1].w += ck * d[7];
                }
            } else {
                // decay in place, then the rank-1 FMA into the same register (this
                // order lets the state keep its registers across iterations)
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const float2 rd = s_upd[t][rg * RGS + m];   // (alpha, k_hat)
                    s[m][0].x = __builtin_fmaf(rd.y, d[0], s[m][0].x * rd.x);
                    s[m][0].y = __builtin_fmaf(rd.y, d[1], s[m][0].y * rd.x);
                    s[m][0].z = __builtin_fmaf(rd.y, d[2], s[m][0].z * rd.x);
                    s[m][0].w = __builtin_fmaf(rd.y, d[3], s[m][0].w * rd.x);
                    s[m][1].x = __builtin_fmaf(rd.y, d[4], s[m][1].x * rd.x);
                    s[m][1].y = __builtin_fmaf(rd.y, d[5], s[m][1].y * rd.x);
                    s[m][1].z = __builtin_fmaf(rd.y, d[6], s[m][1].z * rd.x);
                    s[m][1].w = __builtin_fmaf(rd.y, d[7], s[m][1].w * rd.x);
                }
            }
            if (rg == 0) {
                *reinterpret_cast<float4 *>(&s_col[t][8 * cg]) = make_float4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<float4 *>(&s_col[t][8 * cg + 4]) = make_float4(o[4], o[5], o[6], o[7]);
            }
        }
        if constexpr (FOLD) {
            // back to the true state: S = D X with the decay of the whole chunk
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float dd = s_dec[nv - 1][16 * rg + m];
                s[m][0].x *= dd; s[m][0].y *= dd; s[m][0].z *= dd; s[m][0].w *= dd;
                s[m][1].x *= dd; s[m][1].y *= dd; s[m][1].z *= dd; s[m][1].w *= dd;
            }
        }
        __syncthreads();
    }

    // epilogue of the last chunk
    const int64_t last = ((L - 1) / TC) * TC;
    epilogue(last, (int)(L - last));

#pragma unroll
    for (int m = 0; m < 16; ++m) {
        float *dst = S + (16 * rg + m) * DV + 8 * cg;
        *reinterpret_cast<float4 *>(dst) = s[m][0];
        *reinterpret_cast<float4 *>(dst + 4) = s[m][1];
    }

    // window out: the last PAST raw rows (old window rows when L < PAST).
    // Only wavefront 0 touches the window; it reads all three sources before
    // writing, and wavefront 1 finished its last read of the window (phase P)
    // before the final barrier of the loop.
    if (wave == 0) {
        float2 xq[3], xk[3], xv[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) cx.hist(L - 3 + r, xq[r], xk[r], xv[r]);
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            float *wr = Wout + r * CH + 2 * lane;
            *reinterpret_cast<float2 *>(wr) = xq[r];
            *reinterpret_cast<float2 *>(wr + DK) = xk[r];
            *reinterpret_cast<float2 *>(wr + 2 * DK) = xv[r];
        }
    }
}

template <bool FOLD>
hipError_t launch_prefill_as(const Params &p, bool bf16, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.num_seqs * p.H)), block(PF_THREADS);
    if (bf16)
        hipLaunchKernelGGL((prefill_kernel<BF16, FOLD>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<F32, FOLD>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Params &p, bool bf16, hipStream_t stream) {
    const bool fold = p.gate_mode == GATE_BOUNDED && p.lb <= 0.0f && p.lb * TC >= FOLD_MIN_LOG_DECAY;
    return fold ? launch_prefill_as<true>(p, bf16, stream) : launch_prefill_as<false>(p, bf16, stream);
}

}  // namespace kda
