// kda_prefill_split.hip -- prefill for workloads with few (sequence, head)
// pairs, e.g. one long sequence over 32 heads.
//
// The fused kernel gives each pair one workgroup, so 32 pairs keep 64 of the
// GPU's 1024 SIMDs busy and every token waits on a long per-pair chain.  The
// recurrence never mixes state columns -- column j of S evolves from
// (k, alpha, beta, v_j) alone ("Kimi K3 Metal Gap Analysis", §2, row
// "Recurrence": every term of the update is a row scaling or a rank-1 term
// with column factor v_j - u_j) -- so here each pair's 128 columns are spread
// over G = 128 / (16 C) workgroups of 256 threads:
//   * lane (rg, cl) of a workgroup holds key rows 8 rg .. 8 rg + 7 of state
//     columns cl * C .. cl * C + C - 1 of the slice; rg is the low 4 lane bits,
//     so the reductions over rows are 4 DPP steps inside a row of 16 lanes;
//   * every workgroup runs the pre-step for its chunk (all 128 key rows, only
//     its own value channels) -- duplicated G times, but on otherwise idle
//     CUs -- and the same folded / direct recurrence as the fused kernel,
//     the folding period being 8 tokens (two per 16-token chunk);
//   * the pre-norm readout o goes to a buffer; the RMSNorm + gate epilogue
//     (which needs all 128 columns) and the window update (which must wait
//     until every slice has read the old window) run as two small kernels
//     afterwards.
#include "kda_device.hpp"

namespace kda {

namespace {

constexpr int SP_THREADS = 256;
constexpr int STC = 16;            // tokens per chunk
constexpr int SQ = STC / 4;        // chunk slots per wavefront in the token pre-step
constexpr int SRG = 9;             // LDS float4 slots per row group: 8 key rows + 1 pad
constexpr int SFP = 8;             // folding period: D restarts every SFP tokens
static_assert(STC == 2 * SFP, "the decay pre-step gives each half of the workgroup one period");
constexpr float SPLIT_FOLD_MIN_LOG_DECAY = -60.0f;   // lowest log-decay over one period

__device__ __forceinline__ int srow_slot(int i) { return (i >> 3) * SRG + (i & 7); }

__device__ __forceinline__ float conv4s(float4 w, float a, float b, float c, float x) {
    return w.x * a + w.y * b + w.z * c + w.w * x;
}

__device__ __forceinline__ const void *chan_src(const Params &p, int ch) {
    return ch < DK ? p.q : (ch < 2 * DK ? p.k : p.v);
}

template <typename Act, bool FOLD, int C>
__global__ __launch_bounds__(SP_THREADS) void prefill_split_kernel(Params p, float *obuf) {
    constexpr int CW = 16 * C;         // state columns of this workgroup
    constexpr int G = DV / CW;         // workgroups per (sequence, head)
    const int units = p.num_seqs * p.H;
    const int g = blockIdx.x / units;  // slices of one pair share an XCD when units % 8 == 0
    const int slot_u = blockIdx.x - g * units;
    const int slot_n = slot_u / p.H;
    const int h = slot_u - slot_n * p.H;
    int n = slot_n;
    if (p.seq_order) {
        n = p.seq_order[slot_n];
        if (n < 0 || n >= p.num_seqs) return;
    }
    const Range rng = seq_range(p, n);
    if (rng.len <= 0 || g >= G) return;
    const int64_t L = rng.len;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rg = tid & 15;                   // rows 8 rg .. 8 rg + 7
    const int cl = tid >> 4;                   // columns g CW + cl C .. + C - 1
    const int col0 = g * CW + cl * C;
    const int64_t unit = (int64_t)n * p.H + h;

    __shared__ float4 s_row[STC][16 * SRG];    // FOLD (Dk, Dq, k/D, -); else (alpha k, alpha q, alpha, k)
    __shared__ float s_kh[STC][DK];
    __shared__ float s_qh[STC][DK];
    __shared__ float s_dec[STC][DK];           // FOLD: D_t since the chunk start; else alpha_t
    __shared__ float s_v[STC][CW];             // activated v of this slice
    __shared__ float2 s_tok[STC];              // (beta, q_hat . k_hat)

    float *S = p.state + unit * (DK * DV);
    const float *W = p.win + unit * (PAST * CH);   // read-only here; the window kernel writes it

    float s[8][C];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int c = 0; c < C; ++c) s[m][c] = S[(8 * rg + m) * DV + col0 + c];

    // raw row j (j < 0: window row) of channels ch, ch + 1 of one tensor
    auto hist2 = [&](int64_t j, int ch) -> float2 {
        if (j >= 0) {
            const int64_t r = ((rng.lo + j) * p.H + h) * DK + (ch & (DK - 1));
            return Act::load2(chan_src(p, ch), r);
        }
        return *reinterpret_cast<const float2 *>(W + (j + PAST) * CH + ch);
    };

    const float eA = __expf(p.A_log[h * DK + (tid & (DK - 1))]);
    const float dtb = p.dt_bias[h * DK + (tid & (DK - 1))];
    const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);
    const bool has_v = 2 * lane < CW;
    const int chq = 2 * lane, chk = DK + 2 * lane, chv = 2 * DK + g * CW + (has_v ? 2 * lane : 0);

    // All global inputs of a chunk's phase P.  The next chunk's are loaded
    // while the current chunk runs its serial phase R, so phase P never
    // waits on memory.
    struct ChunkIn {
        float2 xq[PAST + SQ], xk[PAST + SQ], xv[PAST + SQ];   // raw rows j0 - 3 .. j0 + SQ - 1
        float bta[SQ];
        float fv[SFP];                                          // decay inputs of one key row
    };
    const int drow = tid & (DK - 1);           // key row of this thread's decay pre-step
    const int dt0 = (tid >> 7) * SFP;          // its folding period in the chunk
    auto load_chunk = [&](int64_t c0, ChunkIn &in) {
        const int64_t j0 = c0 + wave * SQ;
#pragma unroll
        for (int r = 0; r < PAST + SQ; ++r) {
            const int64_t j = j0 - PAST + r;
            const bool ok = j < L;
            in.xq[r] = ok ? hist2(j, chq) : make_float2(0.f, 0.f);
            in.xk[r] = ok ? hist2(j, chk) : make_float2(0.f, 0.f);
            in.xv[r] = (ok && has_v) ? hist2(j, chv) : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int sl = 0; sl < SQ; ++sl)
            in.bta[sl] = (lane == 0 && j0 + sl < L) ? p.beta[(rng.lo + j0 + sl) * p.H + h] : 0.f;
#pragma unroll
        for (int t = 0; t < SFP; ++t)
            in.fv[t] = (c0 + dt0 + t < L) ? p.f[((rng.lo + c0 + dt0 + t) * p.H + h) * DK + drow] : 0.f;
    };
    const float4 wq0 = *reinterpret_cast<const float4 *>(cw + chq * TAPS);
    const float4 wq1 = *reinterpret_cast<const float4 *>(cw + (chq + 1) * TAPS);
    const float4 wk0 = *reinterpret_cast<const float4 *>(cw + chk * TAPS);
    const float4 wk1 = *reinterpret_cast<const float4 *>(cw + (chk + 1) * TAPS);
    const float4 wv0 = *reinterpret_cast<const float4 *>(cw + chv * TAPS);
    const float4 wv1 = *reinterpret_cast<const float4 *>(cw + (chv + 1) * TAPS);

    ChunkIn cur;
    load_chunk(0, cur);

#pragma unroll 1
    for (int64_t c0 = 0; c0 < L; c0 += STC) {
        const int nv = (int)((L - c0) < STC ? (L - c0) : STC);

        // ---- phase P: token pre-step (wavefront w: slots SQ w .. SQ w + SQ - 1)
        const int64_t j0 = c0 + wave * SQ;
        if (j0 < L) {
#pragma unroll
            for (int sl = 0; sl < SQ; ++sl) {
                if (j0 + sl >= L) break;
                const float2 *xq = cur.xq + sl, *xk = cur.xk + sl, *xv = cur.xv + sl;
                const float aq0 = silu(conv4s(wq0, xq[0].x, xq[1].x, xq[2].x, xq[3].x));
                const float aq1 = silu(conv4s(wq1, xq[0].y, xq[1].y, xq[2].y, xq[3].y));
                const float ak0 = silu(conv4s(wk0, xk[0].x, xk[1].x, xk[2].x, xk[3].x));
                const float ak1 = silu(conv4s(wk1, xk[0].y, xk[1].y, xk[2].y, xk[3].y));
                const float qq = sum64(aq0 * aq0 + aq1 * aq1);
                const float kk = sum64(ak0 * ak0 + ak1 * ak1);
                const float qk = sum64(aq0 * ak0 + aq1 * ak1);
                const float rq = rsqrtf(qq + p.l2_eps), rk = rsqrtf(kk + p.l2_eps);
                const int slot = wave * SQ + sl;
                *reinterpret_cast<float2 *>(&s_qh[slot][chq]) = make_float2(aq0 * rq, aq1 * rq);
                *reinterpret_cast<float2 *>(&s_kh[slot][chq]) = make_float2(ak0 * rk, ak1 * rk);
                if (has_v) {
                    const float av0 = silu(conv4s(wv0, xv[0].x, xv[1].x, xv[2].x, xv[3].x));
                    const float av1 = silu(conv4s(wv1, xv[0].y, xv[1].y, xv[2].y, xv[3].y));
                    *reinterpret_cast<float2 *>(&s_v[slot][2 * lane]) = make_float2(av0, av1);
                }
                if (lane == 0) s_tok[slot] = make_float2(cur.bta[sl], qk * rq * rk);
            }
        }
        // ---- phase P: decays of key row drow over the folding period of this
        // half of the workgroup -- each period's decay accumulates from its own
        // start, so the two halves work independently
        {
            float D = 1.0f;
#pragma unroll
            for (int t = 0; t < SFP; ++t) {
                if (dt0 + t >= nv) break;
                const float al = decay(cur.fv[t], eA, dtb, p.gate_mode, p.lb);
                if constexpr (FOLD) {
                    D *= al;
                    s_dec[dt0 + t][drow] = D;
                } else {
                    s_dec[dt0 + t][drow] = al;
                }
            }
        }
        __syncthreads();

        // ---- phase Q: per-row coefficients (row tid & 127, every other token)
        {
            const int i = tid & (DK - 1);
            const int slot = srow_slot(i);
#pragma unroll 1
            for (int t = tid >> 7; t < nv; t += 2) {
                const float kh = s_kh[t][i], qh = s_qh[t][i], dd = s_dec[t][i];
                if constexpr (FOLD)
                    s_row[t][slot] = make_float4(dd * kh, dd * qh, kh * fast_rcp(dd), 0.0f);
                else
                    s_row[t][slot] = make_float4(dd * kh, dd * qh, dd, kh);
            }
        }
        __syncthreads();

        if (c0 + STC < L) load_chunk(c0 + STC, cur);   // phase P's inputs are consumed

        // ---- phase R: the serial recurrence over the chunk.  Everything token
        // t + 1 reads from LDS (beta, q.k, v, row coefficients) is loaded while
        // token t computes, scalars first, so no LDS latency sits on the chain.
        float4 rd[8];
        float2 bt = s_tok[0];
        float vv[C];
#pragma unroll
        for (int c = 0; c < C; ++c) vv[c] = s_v[0][cl * C + c];
#pragma unroll
        for (int m = 0; m < 8; ++m) rd[m] = s_row[0][rg * SRG + m];
#pragma unroll 1
        for (int t = 0; t < nv; ++t) {
            const int tn = t + 1 < nv ? t + 1 : t;
            const float2 btn = s_tok[tn];
            float vn[C];
#pragma unroll
            for (int c = 0; c < C; ++c) vn[c] = s_v[tn][cl * C + c];
            float4 rn[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) rn[m] = s_row[tn][rg * SRG + m];
            // two partial sums per dot product halve the FMA chain
            float u0[C], u1[C], p0[C], p1[C];
#pragma unroll
            for (int c = 0; c < C; ++c) { u0[c] = u1[c] = p0[c] = p1[c] = 0.f; }
#pragma unroll
            for (int m = 0; m < 8; m += 2)
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    u0[c] += s[m][c] * rd[m].x;
                    p0[c] += s[m][c] * rd[m].y;
                    u1[c] += s[m + 1][c] * rd[m + 1].x;
                    p1[c] += s[m + 1][c] * rd[m + 1].y;
                }
            float d[C], o[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const float u = sum16(u0[c] + u1[c]);
                const float pq = sum16(p0[c] + p1[c]);
                d[c] = bt.x * (vv[c] - u);
                o[c] = pq + bt.y * d[c];
            }
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    if constexpr (FOLD)
                        s[m][c] += rd[m].z * d[c];
                    else
                        s[m][c] = __builtin_fmaf(rd[m].w, d[c], s[m][c] * rd[m].z);
                }
            if (rg == 0) {
                float *dst = obuf + ((rng.lo + c0 + t) * p.H + h) * DV + col0;
#pragma unroll
                for (int c = 0; c < C; ++c) dst[c] = o[c];
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) rd[m] = rn[m];
            bt = btn;
#pragma unroll
            for (int c = 0; c < C; ++c) vv[c] = vn[c];
            if constexpr (FOLD) {
                if (t % SFP == SFP - 1 || t == nv - 1) {
                    // end of a folding period: back to the true state, S = D X
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const float dd = s_dec[t][8 * rg + m];
#pragma unroll
                        for (int c = 0; c < C; ++c) s[m][c] *= dd;
                    }
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int c = 0; c < C; ++c) S[(8 * rg + m) * DV + col0 + c] = s[m][c];
}

// RMSNorm over the 128 readouts of one (token, head) row, gamma, sigmoid gate,
// one wavefront per row, for rows [row_lo, row_lo + rows) after
// seq_rows * blockIdx.y
template <typename Act>
__global__ __launch_bounds__(256) void split_epilogue_kernel(Params p, const float *obuf, int64_t row_lo,
                                                             int64_t rows, int64_t seq_rows) {
    const int64_t base = (int64_t)blockIdx.y * seq_rows + row_lo;
    const int lane = threadIdx.x & 63;
    const float2 gm = *reinterpret_cast<const float2 *>(p.gamma + 2 * lane);
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
        const int64_t off = (base + row) * DV + 2 * lane;
        const float2 o = *reinterpret_cast<const float2 *>(obuf + off);
        const float ss = sum64(o.x * o.x + o.y * o.y);
        const float r = rsqrtf(ss * (1.0f / DV) + p.rms_eps);
        const float2 gg = Act::load2(p.g, off);
        float2 y;
        y.x = sigmoid(gg.x) * gm.x * o.x * r;
        y.y = sigmoid(gg.y) * gm.y * o.y * r;
        Act::store2(p.y, off, y);
    }
}

// window out for every (sequence, head): the last PAST raw rows (old window
// rows when the sequence is shorter than PAST); each thread reads all the
// sources of its channels before writing them
template <typename Act>
__global__ __launch_bounds__(128) void split_window_kernel(Params p) {
    const int unit = blockIdx.x;
    const int n = unit / p.H, h = unit - n * p.H;
    const Range rng = seq_range(p, n);
    if (rng.len <= 0) return;
    float *W = p.win + (int64_t)unit * (PAST * CH);
    for (int ch = threadIdx.x; ch < CH; ch += 128) {
        const void *src = ch < DK ? p.q : (ch < 2 * DK ? p.k : p.v);
        float x[PAST];
#pragma unroll
        for (int r = 0; r < PAST; ++r) {
            const int64_t j = rng.len - PAST + r;
            x[r] = j >= 0 ? Act::load1(src, ((rng.lo + j) * p.H + h) * DK + (ch & (DK - 1)))
                          : W[(j + PAST) * CH + ch];
        }
#pragma unroll
        for (int r = 0; r < PAST; ++r) W[r * CH + ch] = x[r];
    }
}

template <typename Act>
hipError_t launch_epilogue_as(const Params &p, const float *obuf, int64_t row_lo, int64_t rows, int64_t seq_rows,
                              int32_t nseq, hipStream_t stream) {
    if (rows <= 0 || nseq <= 0) return hipSuccess;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL((split_epilogue_kernel<Act>),
                       dim3((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20)), (unsigned)nseq), dim3(256), 0,
                       stream, p, obuf, row_lo, rows, seq_rows);
    return hipGetLastError();
}

template <typename Act, bool FOLD, int C>
hipError_t launch_split_as(const Params &p, float *obuf, hipStream_t stream) {
    constexpr int G = DV / (16 * C);
    const int64_t units = (int64_t)p.num_seqs * p.H;
    hipLaunchKernelGGL((prefill_split_kernel<Act, FOLD, C>), dim3((unsigned)(units * G)),
                       dim3(SP_THREADS), 0, stream, p, obuf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_epilogue_as<Act>(p, obuf, 0, p.total_tokens * p.H, 0, 1, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((split_window_kernel<Act>), dim3((unsigned)units), dim3(128), 0, stream, p);
    return hipGetLastError();
}

template <typename Act, bool FOLD>
hipError_t launch_split_cols(const Params &p, float *obuf, int C, hipStream_t stream) {
    switch (C) {
        case 1: return launch_split_as<Act, FOLD, 1>(p, obuf, stream);
        case 2: return launch_split_as<Act, FOLD, 2>(p, obuf, stream);
        default: return launch_split_as<Act, FOLD, 4>(p, obuf, stream);
    }
}

template <typename Act>
hipError_t launch_window_as(const Params &p, hipStream_t stream) {
    const int64_t units = (int64_t)p.num_seqs * p.H;
    hipLaunchKernelGGL((split_window_kernel<Act>), dim3((unsigned)units), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_split_finish(const Params &p, bool bf16, const float *obuf, hipStream_t stream) {
    hipError_t e = launch_split_epilogue(p, bf16, obuf, 0, p.total_tokens * p.H, 0, 1, stream);
    if (e != hipSuccess) return e;
    return bf16 ? launch_window_as<BF16>(p, stream) : launch_window_as<F32>(p, stream);
}

hipError_t launch_split_epilogue(const Params &p, bool bf16, const float *obuf, int64_t row_lo, int64_t rows,
                                 int64_t seq_rows, int32_t nseq, hipStream_t stream) {
    return bf16 ? launch_epilogue_as<BF16>(p, obuf, row_lo, rows, seq_rows, nseq, stream)
                : launch_epilogue_as<F32>(p, obuf, row_lo, rows, seq_rows, nseq, stream);
}

hipError_t launch_split_window(const Params &p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_window_as<BF16>(p, stream) : launch_window_as<F32>(p, stream);
}

int prefill_split_cols(int64_t units) {
    if (units <= 48) return 1;      // 8 workgroups per pair
    if (units <= 96) return 2;      // 4
    if (units <= 192) return 4;     // 2
    return 0;
}

hipError_t launch_prefill_split(const Params &p, bool bf16, float *obuf, int C, hipStream_t stream) {
    const bool fold = p.gate_mode == GATE_BOUNDED && p.lb <= 0.0f && p.lb * SFP >= SPLIT_FOLD_MIN_LOG_DECAY;
    if (bf16)
        return fold ? launch_split_cols<BF16, true>(p, obuf, C, stream)
                    : launch_split_cols<BF16, false>(p, obuf, C, stream);
    return fold ? launch_split_cols<F32, true>(p, obuf, C, stream)
                : launch_split_cols<F32, false>(p, obuf, C, stream);
}

}  // namespace kda
