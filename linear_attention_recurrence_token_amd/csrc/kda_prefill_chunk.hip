// kda_prefill_chunk.hip -- chunkwise KDA prefill on fp32 MFMA.
//
// The recurrence of "Kimi K3 Metal Gap Analysis" (§2, row "Recurrence"),
// S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T, is applied to a
// chunk of C = 16 tokens at once.  With G_t the per-channel log-decay
// accumulated since the chunk start (G_t = sum of log a over tokens 0..t) and
// S_0 the state entering the chunk, unrolling the recurrence gives (exact
// algebra; the token-by-token delta d_t = b_t (v_t - u_t), u_t the value the
// state predicts for k_t):
//     u_t = (e^{G_t} . k_t)^T S_0 + sum_{s<t} L_ts d_s,
//         L_ts = sum_i k_ti k_si e^{G_ti - G_si}           (strictly lower)
//     o_t = (e^{G_t} . q_t)^T S_0 + sum_{s<=t} M_ts d_s,
//         M_ts = sum_i q_ti k_si e^{G_ti - G_si}           (lower, diagonal q.k)
//     S_C = Diag(e^{G_C}) S_0 + sum_s (e^{G_C - G_s} . k_s) d_s^T
// so with P = (e^G . K) S_0 and R = (e^G . Q) S_0 (C x 128 each):
//     (I + Diag(b) L) Delta = Diag(b) (V - P),  O = R + M Delta,
//     S_C = Diag(e^{G_C}) S_0 + E^T Delta,  E_s = e^{G_C - G_s} . k_s.
// Every product is a small dense GEMM, done with v_mfma_f32_16x16x4_f32:
// the work per token is the same ~7 dk dv flops as the recurrent form, but on
// the matrix cores, which run fp32 at twice the rate of the (unpacked) VALU.
//
// Exponent ranges: L and M use factors e^{G_t - r} and e^{r - G_s} with r the
// log-decay at the chunk middle, so every factor lies within e^{+-|lb| C / 2};
// with the bounded gate and |lb| <= 7.5 that is at most e^{60}, far inside
// fp32.  (Products above the diagonal can reach e^{|lb| C}; they are masked
// by selection, never multiplied.)  Other gate forms take the recurrent path.
//
// Layout.  One 256-thread workgroup (4 wavefronts) per (sequence, head).
// Wavefront w owns state columns 32 w .. 32 w + 31 as 8 x 2 MFMA accumulator
// tiles: lane l holds S[16 rt + 4 (l / 16) + r][32 w + 16 j + l % 16] in
// element r of tile (rt, j).  The state never leaves the accumulators between
// chunks: it feeds P and R as the B operand directly, by ordering the sum over
// key channels so that MFMA step (rt, r) takes channel 16 rt + 4 (l / 16) + r
// in lane l (the A operand is read from LDS in the matching order).
#include "kda_device.hpp"

namespace kda {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CK_THREADS = 256;
constexpr int CC = 16;             // tokens per chunk
constexpr int CQ = CC / 4;         // tokens per wavefront in the token pre-step
constexpr int KP = DK + 4;         // padded LDS row
constexpr float CHUNK_MAX_HALF_LOG_DECAY = 60.0f;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float cconv4(float4 w, float a, float b, float c, float x) {
    return w.x * a + w.y * b + w.z * c + w.w * x;
}

template <typename Act>
__global__ __launch_bounds__(CK_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_chunk_kernel(Params p) {
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
    const int n16 = lane & 15, g4 = lane >> 4;
    const int64_t unit = (int64_t)n * p.H + h;
    const int col0 = 32 * wave;

    // LDS, [token][channel] unless noted.  Rows read as 16 tokens x float4 by
    // one wavefront are padded to 132 floats so the 16 rows hit distinct banks.
    __shared__ float s_ka[CC][KP];     // k_hat, then e^G . k_hat            (A operand of P)
    __shared__ float s_qa[CC][KP];     // q_hat, then e^G . q_hat            (A operand of R)
    __shared__ float s_v[CC][DV];      // activated v
    __shared__ float s_G[CC][DK];      // log-decay accumulated from the chunk start
    __shared__ float s_kt[CC][KP];     // e^{G - r} . k_hat, then the readout o of the chunk
    __shared__ float s_qt[CC][KP];     // e^{G - r} . q_hat
    __shared__ float s_kb[CC][KP];     // e^{r - G} . k_hat
    __shared__ float s_E[DK][CC + 4];  // [channel][token]: e^{G_C - G} . k_hat (padded rows)
    __shared__ float s_gC[DK];         // e^{G_C}: decay of the whole chunk
    __shared__ float s_beta[CC];
    __shared__ float s_Lp[4][CC][CC];  // per-wavefront partial L (channel quarters)
    __shared__ float s_Mp[4][CC][CC];
    __shared__ float s_T[CC][CC + 4];  // (I + Diag(b) L)^{-1}
    __shared__ float s_M[CC][CC + 4];

    const float *W = p.win + unit * (PAST * CH);   // read-only; the window kernel writes it

    // ---- state into the accumulator tiles.  Buffer accesses: lane offset
    // (row 4 g4 + r, column col0 + 16 j + n16), row tile rt as the scalar offset.
    const Rsrc rs_state = make_rsrc(p.state + unit * (DK * DV), DK * DV * 4);
    f32x4 st[8][2];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st[rt][j][r] = bld_f32(rs_state, ((4 * g4 + r) * DV + col0 + 16 * j + n16) * 4,
                                       rt * 16 * DV * 4);

    // Per-chunk buffer resources over token rows [lo + base, lo + end): inputs
    // of the pre-step (from PAST rows before the chunk) and of the epilogue.
    const int64_t rowsz = (int64_t)p.H * DK;       // elements per token row
    auto tok_rsrc = [&](const void *t, uint32_t elem, int64_t base, int64_t end) -> Rsrc {
        return make_rsrc(static_cast<const char *>(t) + (rng.lo + base) * rowsz * elem,
                         (uint32_t)((end - base) * rowsz * elem));
    };
    const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);
    const int chq = 2 * lane, chk = DK + 2 * lane, chv = 2 * DK + 2 * lane;
    const float4 wq0 = *reinterpret_cast<const float4 *>(cw + chq * TAPS);
    const float4 wq1 = *reinterpret_cast<const float4 *>(cw + (chq + 1) * TAPS);
    const float4 wk0 = *reinterpret_cast<const float4 *>(cw + chk * TAPS);
    const float4 wk1 = *reinterpret_cast<const float4 *>(cw + (chk + 1) * TAPS);
    const float4 wv0 = *reinterpret_cast<const float4 *>(cw + chv * TAPS);
    const float4 wv1 = *reinterpret_cast<const float4 *>(cw + (chv + 1) * TAPS);
    const int dch = tid & (DK - 1);    // key channel of this thread's decay / combine work
    const float eA = __expf(p.A_log[h * DK + dch]);
    const float dtb = p.dt_bias[h * DK + dch];
    const float2 gm = *reinterpret_cast<const float2 *>(p.gamma + 2 * lane);

    // RMSNorm + gate of the chunk starting at c0 (readout in s_kt), tokens CQ w ..
    auto epilogue = [&](int64_t c0, int nvalid) {
        const Rsrc rs_g = tok_rsrc(p.g, BufAct<Act>::ELEM, c0, c0 + nvalid);
        const Rsrc rs_y = tok_rsrc(p.y, BufAct<Act>::ELEM, c0, c0 + nvalid);
        const Rsrc rs_o = tok_rsrc(p.o_raw, 4, c0, c0 + nvalid);
#pragma unroll
        for (int sl = 0; sl < CQ; ++sl) {
            const int t = wave * CQ + sl;
            if (t >= nvalid) break;
            const float2 o = *reinterpret_cast<const float2 *>(&s_kt[t][2 * lane]);
            const float ss = sum64(o.x * o.x + o.y * o.y);
            const float r = rsqrtf(ss * (1.0f / DV) + p.rms_eps);
            const uint32_t e = (uint32_t)(t * rowsz + h * DV + 2 * lane);
            const float2 gg = BufAct<Act>::load2(rs_g, e);
            float2 y;
            y.x = sigmoid(gg.x) * gm.x * o.x * r;
            y.y = sigmoid(gg.y) * gm.y * o.y * r;
            BufAct<Act>::store2(rs_y, e, y);
            if (p.o_raw) bst_f32x2(rs_o, o, e * 4);
        }
    };

#pragma unroll 1
    for (int64_t c0 = 0; c0 < L; c0 += CC) {
        const int nv = (int)((L - c0) < CC ? (L - c0) : CC);

        // ================= phase P: everything that depends on inputs only
        if (c0 > 0) epilogue(c0 - CC, CC);
        {
            // token pre-step: wavefront w, tokens CQ w .. CQ w + CQ - 1 (zeros past the end)
            const int64_t j0 = c0 + wave * CQ;
            const int64_t base = c0 >= PAST ? c0 - PAST : 0;
            const int64_t end = (c0 + CC < L) ? c0 + CC : L;
            const Rsrc rq = tok_rsrc(p.q, BufAct<Act>::ELEM, base, end);
            const Rsrc rk = tok_rsrc(p.k, BufAct<Act>::ELEM, base, end);
            const Rsrc rv = tok_rsrc(p.v, BufAct<Act>::ELEM, base, end);
            float2 xq[PAST + CQ], xk[PAST + CQ], xv[PAST + CQ];
            float bta[CQ];
#pragma unroll
            for (int r = 0; r < PAST + CQ; ++r) {
                const int64_t jj = j0 - PAST + r;
                if (jj < 0) {            // from the carried-in window
                    const float *wr = W + (jj + PAST) * CH;
                    xq[r] = *reinterpret_cast<const float2 *>(wr + chq);
                    xk[r] = *reinterpret_cast<const float2 *>(wr + chk);
                    xv[r] = *reinterpret_cast<const float2 *>(wr + chv);
                } else {                 // rows at or past the end read as 0
                    const uint32_t e = (uint32_t)((jj - base) * rowsz + h * DK + 2 * lane);
                    xq[r] = BufAct<Act>::load2(rq, e);
                    xk[r] = BufAct<Act>::load2(rk, e);
                    xv[r] = BufAct<Act>::load2(rv, e);
                }
            }
#pragma unroll
            for (int sl = 0; sl < CQ; ++sl)
                bta[sl] = (lane == 0 && j0 + sl < L) ? p.beta[(rng.lo + j0 + sl) * p.H + h] : 0.f;
#pragma unroll
            for (int sl = 0; sl < CQ; ++sl) {
                const int t = wave * CQ + sl;
                const bool valid = j0 + sl < L;       // wavefront-uniform
                float2 qh = make_float2(0.f, 0.f), kh = qh, vh = qh;
                if (valid) {
                    const float aq0 = silu(cconv4(wq0, xq[sl].x, xq[sl + 1].x, xq[sl + 2].x, xq[sl + 3].x));
                    const float aq1 = silu(cconv4(wq1, xq[sl].y, xq[sl + 1].y, xq[sl + 2].y, xq[sl + 3].y));
                    const float ak0 = silu(cconv4(wk0, xk[sl].x, xk[sl + 1].x, xk[sl + 2].x, xk[sl + 3].x));
                    const float ak1 = silu(cconv4(wk1, xk[sl].y, xk[sl + 1].y, xk[sl + 2].y, xk[sl + 3].y));
                    vh.x = silu(cconv4(wv0, xv[sl].x, xv[sl + 1].x, xv[sl + 2].x, xv[sl + 3].x));
                    vh.y = silu(cconv4(wv1, xv[sl].y, xv[sl + 1].y, xv[sl + 2].y, xv[sl + 3].y));
                    const float rq = rsqrtf(sum64(aq0 * aq0 + aq1 * aq1) + p.l2_eps);
                    const float rk = rsqrtf(sum64(ak0 * ak0 + ak1 * ak1) + p.l2_eps);
                    qh = make_float2(aq0 * rq, aq1 * rq);
                    kh = make_float2(ak0 * rk, ak1 * rk);
                }
                *reinterpret_cast<float2 *>(&s_qa[t][chq]) = qh;
                *reinterpret_cast<float2 *>(&s_ka[t][chq]) = kh;
                *reinterpret_cast<float2 *>(&s_v[t][chq]) = vh;
                if (lane == 0) s_beta[t] = bta[sl];
            }
            // log-decay accumulated over the chunk, one key channel per thread;
            // held constant past the last valid token
            if (tid < DK) {
                const Rsrc rf = tok_rsrc(p.f, 4, c0, c0 + nv);
                float fv[CC];
#pragma unroll
                for (int t = 0; t < CC; ++t)      // rows past the end read as 0
                    fv[t] = bld_f32(rf, (uint32_t)((h * DK + dch) * 4), (uint32_t)(t * rowsz * 4));
                float G = 0.f;
#pragma unroll
                for (int t = 0; t < CC; ++t) {
                    if (t < nv) G += p.lb * sigmoid(eA * (fv[t] + dtb));
                    s_G[t][dch] = G;
                }
            }
        }
        __syncthreads();

        // ================= phase Q: decay-weighted operands (channel dch, 8 tokens)
        {
            const int t0 = (tid >> 7) * (CC / 2);
            const float gr = s_G[CC / 2 - 1][dch];     // reference: middle of the chunk
            const float gc = s_G[CC - 1][dch];
#pragma unroll
            for (int u = 0; u < CC / 2; ++u) {
                const int t = t0 + u;
                const float G = s_G[t][dch];
                const float kh = s_ka[t][dch], qh = s_qa[t][dch];
                const float eg = __expf(G), ef = __expf(G - gr), eb = __expf(gr - G);
                s_ka[t][dch] = eg * kh;
                s_qa[t][dch] = eg * qh;
                s_kt[t][dch] = ef * kh;
                s_qt[t][dch] = ef * qh;
                s_kb[t][dch] = eb * kh;
                s_E[dch][t] = __expf(gc - G) * kh;
            }
            if (tid < DK) s_gC[dch] = __expf(gc);
        }
        __syncthreads();

        // ================= phase M1: P, R (this wavefront's columns); L, M partials
        f32x4 Pt[2], Rt[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) { Pt[j] = f32x4{0.f, 0.f, 0.f, 0.f}; Rt[j] = Pt[j]; }
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const float4 ak = *reinterpret_cast<const float4 *>(&s_ka[n16][16 * rt + 4 * g4]);
            const float4 aq = *reinterpret_cast<const float4 *>(&s_qa[n16][16 * rt + 4 * g4]);
            const float akv[4] = {ak.x, ak.y, ak.z, ak.w};
            const float aqv[4] = {aq.x, aq.y, aq.z, aq.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    Pt[j] = mfma4(akv[r], st[rt][j][r], Pt[j]);
                    Rt[j] = mfma4(aqv[r], st[rt][j][r], Rt[j]);
                }
        }
        {
            // channels 32 w + 8 (l / 16) + s, s = 0..7, in MFMA step s
            const float *kt = &s_kt[n16][col0 + 8 * g4];
            const float *qt = &s_qt[n16][col0 + 8 * g4];
            const float *kb = &s_kb[n16][col0 + 8 * g4];
            f32x4 Lt = {0.f, 0.f, 0.f, 0.f}, Mt = Lt;
#pragma unroll
            for (int s4 = 0; s4 < 2; ++s4) {
                const float4 a = *reinterpret_cast<const float4 *>(kt + 4 * s4);
                const float4 c = *reinterpret_cast<const float4 *>(qt + 4 * s4);
                const float4 b = *reinterpret_cast<const float4 *>(kb + 4 * s4);
                Lt = mfma4(a.x, b.x, Lt); Mt = mfma4(c.x, b.x, Mt);
                Lt = mfma4(a.y, b.y, Lt); Mt = mfma4(c.y, b.y, Mt);
                Lt = mfma4(a.z, b.z, Lt); Mt = mfma4(c.z, b.z, Mt);
                Lt = mfma4(a.w, b.w, Lt); Mt = mfma4(c.w, b.w, Mt);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s_Lp[wave][4 * g4 + r][n16] = Lt[r];
                s_Mp[wave][4 * g4 + r][n16] = Mt[r];
            }
        }
        __syncthreads();

        // ================= phase T: (I + Diag(b) L)^{-1} by forward substitution
        // (wavefront 0, lane j < 16 builds column j); the other lanes idle here
        if (wave == 0 && lane < CC) {
            const int jc = lane;
            float Tcol[CC];
#pragma unroll
            for (int t = 0; t < CC; ++t) {
                float acc = (t == jc) ? 1.0f : 0.0f;
                const float bt = s_beta[t];
#pragma unroll
                for (int s = 0; s < t; ++s) {
                    const float lts = s_Lp[0][t][s] + s_Lp[1][t][s] + s_Lp[2][t][s] + s_Lp[3][t][s];
                    acc -= bt * lts * Tcol[s];
                }
                Tcol[t] = acc;
                s_T[t][jc] = acc;
            }
            // M: lower triangle with diagonal, row t
#pragma unroll
            for (int t = 0; t < CC; ++t) {
                const float m = s_Mp[0][t][jc] + s_Mp[1][t][jc] + s_Mp[2][t][jc] + s_Mp[3][t][jc];
                s_M[t][jc] = (jc <= t) ? m : 0.0f;
            }
        }
        // W = Diag(b) (V - P), this wavefront's columns, accumulator layout (rows 4 g4 + r)
        f32x4 Wt[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                Wt[j][r] = s_beta[t] * (s_v[t][col0 + 16 * j + n16] - Pt[j][r]);
            }
        __syncthreads();

        // ================= phase M2: Delta = T W; O = R + M Delta; state update
        f32x4 Dt[2], Ot[2];
        {
            const float4 tr = *reinterpret_cast<const float4 *>(&s_T[n16][4 * g4]);
            const float4 mr = *reinterpret_cast<const float4 *>(&s_M[n16][4 * g4]);
            const float trv[4] = {tr.x, tr.y, tr.z, tr.w};
            const float mrv[4] = {mr.x, mr.y, mr.z, mr.w};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                Dt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) Dt[j] = mfma4(trv[r], Wt[j][r], Dt[j]);
                Ot[j] = Rt[j];
#pragma unroll
                for (int r = 0; r < 4; ++r) Ot[j] = mfma4(mrv[r], Dt[j][r], Ot[j]);
            }
        }
        // readout of the chunk into s_kt (its L operand is no longer needed)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_kt[4 * g4 + r][col0 + 16 * j + n16] = Ot[j][r];
        // S <- Diag(e^{G_C}) S + E^T Delta
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const float4 dc = *reinterpret_cast<const float4 *>(&s_gC[16 * rt + 4 * g4]);
            const float4 er = *reinterpret_cast<const float4 *>(&s_E[16 * rt + n16][4 * g4]);
            const float dcv[4] = {dc.x, dc.y, dc.z, dc.w};
            const float erv[4] = {er.x, er.y, er.z, er.w};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) st[rt][j][r] *= dcv[r];
#pragma unroll
                for (int r = 0; r < 4; ++r) st[rt][j] = mfma4(erv[r], Dt[j][r], st[rt][j]);
            }
        }
        __syncthreads();
    }

    // epilogue of the last chunk, then the state
    const int64_t last = ((L - 1) / CC) * CC;
    epilogue(last, (int)(L - last));
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                bst_f32(rs_state, st[rt][j][r], ((4 * g4 + r) * DV + col0 + 16 * j + n16) * 4,
                        rt * 16 * DV * 4);
}

// window out (same as after the column-split path): every thread reads all
// sources of its channels before writing them
template <typename Act>
__global__ __launch_bounds__(128) void chunk_window_kernel(Params p) {
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
hipError_t launch_chunk_as(const Params &p, hipStream_t stream) {
    const int64_t units = (int64_t)p.num_seqs * p.H;
    hipLaunchKernelGGL((prefill_chunk_kernel<Act>), dim3((unsigned)units), dim3(CK_THREADS), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_window_kernel<Act>), dim3((unsigned)units), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool prefill_chunk_supported(const Params &p) {
    // the per-chunk buffer resources span (CC + PAST) token rows of H * 128 elements
    return p.gate_mode == GATE_BOUNDED && p.lb <= 0.0f && -p.lb * (CC / 2) <= CHUNK_MAX_HALF_LOG_DECAY &&
           p.H <= 4096;
}

hipError_t launch_prefill_chunk(const Params &p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_chunk_as<BF16>(p, stream) : launch_chunk_as<F32>(p, stream);
}

}  // namespace kda
