// kda_decode.hip -- one decode token for each of N sequences, all heads, in
// one launch.
//
// The step is HBM-bound: per (sequence, head) it must stream the 64 KiB fp32
// state in and 64 KiB out, against ~115 K flops.  So the design is about the
// memory stream:
//   * one workgroup of NT threads per (sequence, head); the 128 x 128 state is
//     held in registers (16384 / NT floats per thread), loaded with coalesced
//     16-byte loads issued right after the pre-step's few input loads, so the
//     whole 64 KiB is in flight while the pre-step runs;
//   * the pre-step (conv4 + SiLU, window shift, L2 norms, decay) runs from
//     the raw inputs while those loads are outstanding;
//   * one pass over the registers gives both dot products the step needs,
//     u = S^T (alpha * k) and p = S^T (alpha * q), because the readout of the
//     updated state equals p + beta (q.k) (v - u)  (expand S_new^T q with
//     S_new = Diag(alpha) S + beta k (v - u)^T, "Kimi K3 Metal Gap Analysis",
//     §2, rows "Recurrence" and "O projection"); the thread of key channel i
//     stores (alpha_i q_i, alpha_i k_i, alpha_i, k_i) once, so a row costs one
//     LDS read, and the L2 norms scale the two sums instead of every row;
//   * the update is written back in place with 16-byte stores; the RMSNorm +
//     sigmoid gate epilogue needs only a 32-lane reduction.
//
// Thread layout: tid = 32 * rg + cg.  Thread (rg, cg) owns rows rg + NRG m
// (m = 0 .. 128 / NRG - 1, NRG = NT / 32 row groups) and columns 4 cg ..
// 4 cg + 3.  A wavefront covers two adjacent rows per load instruction: 1 KiB
// contiguous.
#include "kda_device.hpp"

#include <atomic>

namespace kda {

namespace {

template <int NT>
struct DecodeShape {
    static constexpr int NW = NT / 64;        // wavefronts
    static constexpr int NRG = NT / 32;       // row groups
    static constexpr int RPT = DK / NRG;      // rows per thread
    static_assert(NT == 128 || NT == 256 || NT == 512, "decode workgroup size");
};


// 16 bytes of state through the pair's buffer resource; nontemporal (the
// cache policy's NT bit) or not
constexpr int CPOL_NT = 2;
template <bool NTMP>
__device__ __forceinline__ float4 ld_state(Rsrc r, uint32_t voff, uint32_t soff) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NTMP ? CPOL_NT : 0);
    return make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
}

// (bst_f32x4_at: the whole offset per lane, so that the compiler separates
// the store from later writes to its data registers; with an SGPR scalar
// offset it did not, and a few state rows per launch were lost at random)
template <bool NTMP>
__device__ __forceinline__ void st_state(Rsrc r, float4 v, uint32_t voff, uint32_t off) {
    bst_f32x4_at<NTMP ? CPOL_NT : 0>(r, v, voff + off);
}

// Row owned by row group rg at step m: interleaved (rg + NRG m: one load
// instruction of a wavefront covers two adjacent rows) or blocked (RPT rg + m:
// a wavefront's loads cover one contiguous 2 * RPT-row region).
template <int NT, bool BLOCKED>
__device__ __forceinline__ int dec_row(int rg, int m) {
    using Sh = DecodeShape<NT>;
    return BLOCKED ? Sh::RPT * rg + m : rg + Sh::NRG * m;
}

template <typename Act, int NT, bool NT_LOAD, bool NT_STORE, bool BLOCKED = false, int WPE = 1>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE)))
void decode_kernel(Params p) {
    using Sh = DecodeShape<NT>;
    const int unit = blockIdx.x;           // n * H + h == token row of sequence n
    const int h = unit % p.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid & 31, rg = tid >> 5;

    // key row i: (a_i q_i, a_i k_i, a_i, k_i) with q, k after conv + SiLU and
    // before the L2 norms, which are applied to the sums over rows instead
    __shared__ float4 s_row[DK];
    __shared__ float s_v[DV];              // activated v of this token
    __shared__ float s_red[Sh::NW][4];     // per-wave partial sums (qq, kk, qk)
    __shared__ float4 s_up[Sh::NW][32][2]; // per-wave partial u, p per column group

    float *S = p.state + (int64_t)unit * (DK * DV);
    float *W = p.win + (int64_t)unit * (PAST * CH);
    const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);
    const int64_t row = (int64_t)unit * DK;   // DK == DV

    // ---- 1. the pre-step's inputs first: loads return in issue order, so
    // issuing these few before the state lets the pre-step run while the
    // 64 KiB of state is still arriving.  Task i < 128 is the (q_i, k_i)
    // channel pair and the decay of key channel i, task 128 + j the v channel j.
    constexpr int TPT = (2 * DK + NT - 1) / NT;   // pre-step tasks per thread
    float x0[TPT], x1[TPT], w0[TPT][PAST], w1[TPT][PAST], fa[TPT], fb[TPT], fc[TPT];
    float4 c0[TPT], c1[TPT];
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
        const int task = tid + r * NT;
        if (task < DK) {
            const int i = task;
            x0[r] = Act::load1(p.q, row + i);
            x1[r] = Act::load1(p.k, row + i);
            c0[r] = *reinterpret_cast<const float4 *>(cw + i * TAPS);
            c1[r] = *reinterpret_cast<const float4 *>(cw + (DK + i) * TAPS);
#pragma unroll
            for (int j = 0; j < PAST; ++j) { w0[r][j] = W[j * CH + i]; w1[r][j] = W[j * CH + DK + i]; }
            fa[r] = p.f[row + i];
            fb[r] = p.A_log[h * DK + i];
            fc[r] = p.dt_bias[h * DK + i];
        } else if (task < 2 * DK) {
            const int j = task - DK;
            x0[r] = Act::load1(p.v, row + j);
            c0[r] = *reinterpret_cast<const float4 *>(cw + (2 * DK + j) * TAPS);
#pragma unroll
            for (int jj = 0; jj < PAST; ++jj) w0[r][jj] = W[jj * CH + 2 * DK + j];
        }
    }
    const float b = p.beta[unit];

    // ---- 2. put the whole state in flight: one buffer resource for the
    // pair's 64 KiB, a per-lane offset, and each row step's offset a constant
    const Rsrc rs = make_rsrc(S, DK * DV * 4);
    const uint32_t s_lane = (uint32_t)(dec_row<NT, BLOCKED>(rg, 0) * DV + 4 * cg) * 4;
    constexpr uint32_t ROW_STEP = (BLOCKED ? 1 : Sh::NRG) * DV * 4;
    float4 s[Sh::RPT];
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) s[m] = ld_state<NT_LOAD>(rs, s_lane, m * ROW_STEP);

    // ---- 3. pre-step: conv4 + SiLU, window shift, L2 partial sums, decay
    float qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
        const int task = tid + r * NT;
        if (task < DK) {
            const int i = task;
            const float aq = silu(c0[r].x * w0[r][0] + c0[r].y * w0[r][1] + c0[r].z * w0[r][2] + c0[r].w * x0[r]);
            const float ak = silu(c1[r].x * w1[r][0] + c1[r].y * w1[r][1] + c1[r].z * w1[r][2] + c1[r].w * x1[r]);
            W[i] = w0[r][1]; W[CH + i] = w0[r][2]; W[2 * CH + i] = x0[r];
            W[DK + i] = w1[r][1]; W[CH + DK + i] = w1[r][2]; W[2 * CH + DK + i] = x1[r];
            const float al = decay(fa[r], __expf(fb[r]), fc[r], p.gate_mode, p.lb);
            s_row[i] = make_float4(al * aq, al * ak, al, ak);
            qq += aq * aq; kk += ak * ak; qk += aq * ak;
        } else if (task < 2 * DK) {
            const int j = task - DK;
            s_v[j] = silu(c0[r].x * w0[r][0] + c0[r].y * w0[r][1] + c0[r].z * w0[r][2] + c0[r].w * x0[r]);
            W[2 * DK + j] = w0[r][1]; W[CH + 2 * DK + j] = w0[r][2]; W[2 * CH + 2 * DK + j] = x0[r];
        }
    }
    qq = sum64(qq); kk = sum64(kk); qk = sum64(qk);
    if (lane == 0) { s_red[wave][0] = qq; s_red[wave][1] = kk; s_red[wave][2] = qk; }
    __syncthreads();

    qq = 0.f; kk = 0.f; qk = 0.f;
#pragma unroll
    for (int w = 0; w < Sh::NW; ++w) { qq += s_red[w][0]; kk += s_red[w][1]; qk += s_red[w][2]; }
    const float rq = rsqrtf(qq + p.l2_eps);
    const float rk = rsqrtf(kk + p.l2_eps);
    qk *= rq * rk;

    // ---- 3. one pass: u = S^T (alpha k_hat), p = S^T (alpha q_hat), summed
    // over rows with the unnormalised q, k and scaled by 1/|k|, 1/|q| after
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f), pq = u;
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) {
        const float4 rw = s_row[dec_row<NT, BLOCKED>(rg, m)];
        u.x += s[m].x * rw.y; u.y += s[m].y * rw.y; u.z += s[m].z * rw.y; u.w += s[m].w * rw.y;
        pq.x += s[m].x * rw.x; pq.y += s[m].y * rw.x; pq.z += s[m].z * rw.x; pq.w += s[m].w * rw.x;
    }
    // the two row groups of this wavefront, then the wavefronts
    u.x += __shfl_xor(u.x, 32); u.y += __shfl_xor(u.y, 32);
    u.z += __shfl_xor(u.z, 32); u.w += __shfl_xor(u.w, 32);
    pq.x += __shfl_xor(pq.x, 32); pq.y += __shfl_xor(pq.y, 32);
    pq.z += __shfl_xor(pq.z, 32); pq.w += __shfl_xor(pq.w, 32);
    if (lane < 32) { s_up[wave][cg][0] = u; s_up[wave][cg][1] = pq; }
    __syncthreads();
    u = s_up[0][cg][0]; pq = s_up[0][cg][1];
#pragma unroll
    for (int w = 1; w < Sh::NW; ++w) {
        const float4 a = s_up[w][cg][0], c = s_up[w][cg][1];
        u.x += a.x; u.y += a.y; u.z += a.z; u.w += a.w;
        pq.x += c.x; pq.y += c.y; pq.z += c.z; pq.w += c.w;
    }
    u.x *= rk; u.y *= rk; u.z *= rk; u.w *= rk;
    pq.x *= rq; pq.y *= rq; pq.z *= rq; pq.w *= rq;

    // ---- 4. delta, readout, in-place update S <- Diag(alpha) S + k_hat delta^T
    // (k_hat_i delta = k_i (delta / |k|))
    const float4 vv = *reinterpret_cast<const float4 *>(&s_v[4 * cg]);
    float4 d, o, dk;
    d.x = b * (vv.x - u.x); d.y = b * (vv.y - u.y); d.z = b * (vv.z - u.z); d.w = b * (vv.w - u.w);
    o.x = pq.x + qk * d.x; o.y = pq.y + qk * d.y; o.z = pq.z + qk * d.z; o.w = pq.w + qk * d.w;
    dk.x = d.x * rk; dk.y = d.y * rk; dk.z = d.z * rk; dk.w = d.w * rk;
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) {
        const float2 ak = *reinterpret_cast<const float2 *>(&s_row[dec_row<NT, BLOCKED>(rg, m)].z);
        float4 t;
        t.x = ak.x * s[m].x + ak.y * dk.x; t.y = ak.x * s[m].y + ak.y * dk.y;
        t.z = ak.x * s[m].z + ak.y * dk.z; t.w = ak.x * s[m].w + ak.y * dk.w;
        st_state<NT_STORE>(rs, t, s_lane, m * ROW_STEP);
    }

    // ---- 5. RMSNorm over the 128 outputs (32 lanes x 4), gamma, sigmoid gate
    const float ss = sum32(o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w);
    if (tid < 32) {
        const float r = rsqrtf(ss * (1.0f / DV) + p.rms_eps);
        const float4 gm = *reinterpret_cast<const float4 *>(p.gamma + 4 * cg);
        const int64_t orow = row + 4 * cg;
        const float2 g01 = Act::load2(p.g, orow), g23 = Act::load2(p.g, orow + 2);
        float4 y;
        y.x = sigmoid(g01.x) * gm.x * o.x * r;
        y.y = sigmoid(g01.y) * gm.y * o.y * r;
        y.z = sigmoid(g23.x) * gm.z * o.z * r;
        y.w = sigmoid(g23.y) * gm.w * o.w * r;
        Act::store4(p.y, orow, y);
        if (p.o_raw) *reinterpret_cast<float4 *>(p.o_raw + orow) = o;
    }
}

// ---------------------------------------------------------------- persistent decode
// The same step as decode_kernel, with G workgroups that each take the pairs
// blockIdx.x, blockIdx.x + G, ... (G a multiple of H, so a workgroup keeps one
// head and loads its conv taps, A_log and dt_bias once).  Each pair's
// per-token inputs (q, k, v, f, beta, g and the conv window) are loaded while
// the previous pair is processed, right behind that pair's state loads, so
// they have a whole pair's time to arrive.  This matters when the state
// itself comes back fast: a state that fits in the Infinity Cache stays there
// between steps under the plain cache policy, while every step's inputs are
// new rows; with one pair per workgroup their latency sits on every pair's
// critical path.
struct DecodeIn {
    float x0, x1, w0[PAST], w1[PAST], fa, b;
    float2 g01, g23;
};

template <typename Act, bool NT_LOAD, bool NT_STORE>
__global__ __launch_bounds__(256) void decode_stream_kernel(Params p, int32_t G) {
    constexpr int NT = 256;
    using Sh = DecodeShape<NT>;
    const int P = p.num_seqs * p.H;
    int unit = blockIdx.x;
    if (unit >= P) return;
    const int h = unit % p.H;                    // the same for every pair of this workgroup
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid & 31, rg = tid >> 5;

    // per-pair values, by pair parity: a pair's writes never meet the reads of
    // the pair before it, and the two barriers of the pair in between keep
    // the pair two back finished
    __shared__ float4 s_row[2][DK];
    __shared__ float s_v[2][DV];
    __shared__ float s_red[2][Sh::NW][4];
    __shared__ float4 s_up[2][Sh::NW][32][2];

    // per-head constants, in LDS for the workgroup's life: the conv taps of
    // every channel, exp(A_log), dt_bias and gamma
    __shared__ float4 s_cw[CH];
    __shared__ float s_eA[DK], s_dtb[DK], s_gm[DV];
    {
        const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);
        for (int c = tid; c < CH; c += NT) s_cw[c] = *reinterpret_cast<const float4 *>(cw + c * TAPS);
        if (tid < DK) {
            s_eA[tid] = __expf(p.A_log[h * DK + tid]);
            s_dtb[tid] = p.dt_bias[h * DK + tid];
            s_gm[tid] = p.gamma[tid];
        }
    }
    __syncthreads();                             // the per-head constants in LDS
    // thread tid < 128: q, k channel tid and the decay of key channel tid;
    // thread 128 + j: v channel j (wavefront-uniform split)
    const bool qk = tid < DK;
    const int ch = qk ? tid : tid - DK;

    // Every thread issues the same twelve loads in the same order, so that
    // the compiler's wait counts are exact on every wavefront: the v threads'
    // second channel, second window column and decay input repeat addresses
    // in range (their values are unused), and every thread reads a g pair
    // (those of lanes 0-31 are used).
    const void *x1src = qk ? p.k : p.v;
    const int w0col = qk ? ch : 2 * DK + ch, w1col = qk ? DK + ch : 2 * DK + ch;
    auto load_in = [&](int u, DecodeIn &in) {
        const int64_t row = (int64_t)u * DK;
        const float *W = p.win + (int64_t)u * (PAST * CH);
        in.x0 = Act::load1(qk ? p.q : p.v, row + ch);
        in.x1 = Act::load1(x1src, row + ch);
#pragma unroll
        for (int j = 0; j < PAST; ++j) { in.w0[j] = W[j * CH + w0col]; in.w1[j] = W[j * CH + w1col]; }
        in.fa = p.f[row + (ch & (DK - 1))];
        in.b = p.beta[u];
        in.g01 = Act::load2(p.g, row + 4 * cg);
        in.g23 = Act::load2(p.g, row + 4 * cg + 2);
    };

    const uint32_t s_lane = (uint32_t)(rg * DV + 4 * cg) * 4;
    constexpr uint32_t ROW_STEP = Sh::NRG * DV * 4;

    auto issue_state = [&](int u, float4 (&s)[Sh::RPT]) {
        const Rsrc rs = make_rsrc(p.state + (int64_t)u * (DK * DV), DK * DV * 4);
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) s[m] = ld_state<NT_LOAD>(rs, s_lane, m * ROW_STEP);
    };
    // the step of pair u from its inputs and its state registers (loads in flight)
    auto pair_body = [&](int u, const DecodeIn &in, float4 (&s)[Sh::RPT], const int b) {
        const Rsrc rs = make_rsrc(p.state + (int64_t)u * (DK * DV), DK * DV * 4);
        // pre-step of this pair from its prefetched inputs
        float *W = p.win + (int64_t)u * (PAST * CH);
        float qq = 0.f, kk = 0.f, qkd = 0.f;
        // window shift: six stores by every thread (a v thread writes its
        // three values twice), so the store count is the same on every path
#pragma unroll
        for (int j = 0; j < PAST; ++j) {
            W[j * CH + w0col] = j + 1 < PAST ? in.w0[j + 1] : in.x0;
            W[j * CH + w1col] = qk ? (j + 1 < PAST ? in.w1[j + 1] : in.x1) : (j + 1 < PAST ? in.w0[j + 1] : in.x0);
        }
        if (qk) {
            const float4 c0 = s_cw[ch], c1 = s_cw[DK + ch];
            const float aq = silu(c0.x * in.w0[0] + c0.y * in.w0[1] + c0.z * in.w0[2] + c0.w * in.x0);
            const float ak = silu(c1.x * in.w1[0] + c1.y * in.w1[1] + c1.z * in.w1[2] + c1.w * in.x1);
            const float al = decay(in.fa, s_eA[ch], s_dtb[ch], p.gate_mode, p.lb);
            s_row[b][ch] = make_float4(al * aq, al * ak, al, ak);
            qq = aq * aq; kk = ak * ak; qkd = aq * ak;
        } else {
            const float4 c0 = s_cw[2 * DK + ch];
            s_v[b][ch] = silu(c0.x * in.w0[0] + c0.y * in.w0[1] + c0.z * in.w0[2] + c0.w * in.x0);
        }
        qq = sum64(qq); kk = sum64(kk); qkd = sum64(qkd);
        if (lane == 0) { s_red[b][wave][0] = qq; s_red[b][wave][1] = kk; s_red[b][wave][2] = qkd; }
        __syncthreads();
        qq = 0.f; kk = 0.f; qkd = 0.f;
#pragma unroll
        for (int w = 0; w < Sh::NW; ++w) { qq += s_red[b][w][0]; kk += s_red[b][w][1]; qkd += s_red[b][w][2]; }
        const float rq = rsqrtf(qq + p.l2_eps);
        const float rk = rsqrtf(kk + p.l2_eps);
        qkd *= rq * rk;

        // u = S^T (alpha k_hat), p = S^T (alpha q_hat) in one pass
        float4 uu = make_float4(0.f, 0.f, 0.f, 0.f), pq = uu;
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) {
            const float4 rw = s_row[b][rg + Sh::NRG * m];
            uu.x += s[m].x * rw.y; uu.y += s[m].y * rw.y; uu.z += s[m].z * rw.y; uu.w += s[m].w * rw.y;
            pq.x += s[m].x * rw.x; pq.y += s[m].y * rw.x; pq.z += s[m].z * rw.x; pq.w += s[m].w * rw.x;
        }
        uu.x += __shfl_xor(uu.x, 32); uu.y += __shfl_xor(uu.y, 32);
        uu.z += __shfl_xor(uu.z, 32); uu.w += __shfl_xor(uu.w, 32);
        pq.x += __shfl_xor(pq.x, 32); pq.y += __shfl_xor(pq.y, 32);
        pq.z += __shfl_xor(pq.z, 32); pq.w += __shfl_xor(pq.w, 32);
        if (lane < 32) { s_up[b][wave][cg][0] = uu; s_up[b][wave][cg][1] = pq; }
        __syncthreads();
        uu = s_up[b][0][cg][0]; pq = s_up[b][0][cg][1];
#pragma unroll
        for (int w = 1; w < Sh::NW; ++w) {
            const float4 a = s_up[b][w][cg][0], c = s_up[b][w][cg][1];
            uu.x += a.x; uu.y += a.y; uu.z += a.z; uu.w += a.w;
            pq.x += c.x; pq.y += c.y; pq.z += c.z; pq.w += c.w;
        }
        uu.x *= rk; uu.y *= rk; uu.z *= rk; uu.w *= rk;
        pq.x *= rq; pq.y *= rq; pq.z *= rq; pq.w *= rq;

        // delta, readout, in-place update
        const float4 vv = *reinterpret_cast<const float4 *>(&s_v[b][4 * cg]);
        float4 d, o, dk;
        d.x = in.b * (vv.x - uu.x); d.y = in.b * (vv.y - uu.y); d.z = in.b * (vv.z - uu.z); d.w = in.b * (vv.w - uu.w);
        o.x = pq.x + qkd * d.x; o.y = pq.y + qkd * d.y; o.z = pq.z + qkd * d.z; o.w = pq.w + qkd * d.w;
        dk.x = d.x * rk; dk.y = d.y * rk; dk.z = d.z * rk; dk.w = d.w * rk;
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) {
            const float2 ak = *reinterpret_cast<const float2 *>(&s_row[b][rg + Sh::NRG * m].z);
            float4 t;
            t.x = ak.x * s[m].x + ak.y * dk.x; t.y = ak.x * s[m].y + ak.y * dk.y;
            t.z = ak.x * s[m].z + ak.y * dk.z; t.w = ak.x * s[m].w + ak.y * dk.w;
            st_state<NT_STORE>(rs, t, s_lane, m * ROW_STEP);
        }

        // RMSNorm + gamma + sigmoid gate
        const float ssq = sum32(o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w);
        if (tid < 32) {
            const float r = rsqrtf(ssq * (1.0f / DV) + p.rms_eps);
            const int64_t orow = (int64_t)u * DK + 4 * cg;
            const float4 gm = *reinterpret_cast<const float4 *>(&s_gm[4 * cg]);
            float4 y;
            y.x = sigmoid(in.g01.x) * gm.x * o.x * r;
            y.y = sigmoid(in.g01.y) * gm.y * o.y * r;
            y.z = sigmoid(in.g23.x) * gm.z * o.z * r;
            y.w = sigmoid(in.g23.y) * gm.w * o.w * r;
            Act::store4(p.y, orow, y);
            if (p.o_raw) *reinterpret_cast<float4 *>(p.o_raw + orow) = o;
        }
    };

    // The next pair's inputs are loaded right behind this pair's state loads,
    // at an in-range index on every path (the last pair repeats its own index
    // and ignores the values), so that every path issues the same loads and
    // the compiler's wait counts stay exact.
    DecodeIn inA, inB;
    float4 st[Sh::RPT];
    load_in(unit, inA);
#pragma unroll 1
    while (true) {
        const int n1 = unit + G;
        issue_state(unit, st);
        load_in(n1 < P ? n1 : unit, inB);
        pair_body(unit, inA, st, 0);
        if (n1 >= P) break;
        unit = n1;
        const int n2 = unit + G;
        issue_state(unit, st);
        load_in(n2 < P ? n2 : unit, inA);
        pair_body(unit, inB, st, 1);
        if (n2 >= P) break;
        unit = n2;
    }
}

// ---------------------------------------------------------------- short sequences
// kda_sequence for sequences of a few tokens: the decode step's layout with a
// token loop.  The state stays in registers for all of the sequence's tokens
// (read once, written once), the conv window shifts in registers, and each
// token's inputs are loaded while the previous token is processed.
//   thread i < 128:   q_i, k_i (conv, SiLU) and the decay a_i of key channel i;
//                     it stores (a q_i, a k_i) and (a_i, k_i), unnormalised
//   thread 128 + j:   v_j
// The L2 norms are applied after the dot products: u = |k|^-1 S^T (a . k),
// p = |q|^-1 S^T (a . q), and the update adds (k_i / |k|) delta_j.  Two
// barriers per token; the per-token LDS values are double-buffered by token
// parity.  Memory goes through buffer resources (32-bit offsets; the host
// keeps the sequence's rows under 4 GiB per tensor).
template <typename Act>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void short_seq_kernel(Params p) {
    constexpr int NT = 256;
    using Sh = DecodeShape<NT>;
    typedef BufAct<Act> BA;
    const int slot_n = blockIdx.x / p.H;
    const int h = blockIdx.x - slot_n * p.H;
    int n = slot_n;
    if (p.seq_order) {
        n = p.seq_order[slot_n];
        if (n < 0 || n >= p.num_seqs) return;
    }
    const Range rng = seq_range(p, n);
    if (rng.len <= 0) return;
    const int64_t unit = (int64_t)n * p.H + h;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid & 31, rg = tid >> 5;

    __shared__ float2 s_aqk[2][DK];        // (a q, a k) per key channel, by token parity
    __shared__ float2 s_ak[2][DK];         // (a, k) per key channel
    __shared__ float s_v[2][DV];           // activated v
    __shared__ float s_red[Sh::NW][4];
    __shared__ float4 s_up[Sh::NW][32][2];

    float *W = p.win + unit * (PAST * CH);
    const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);

    const bool qk_task = tid < DK;
    const int ch = qk_task ? tid : tid - DK;
    const int wch = qk_task ? ch : 2 * DK + ch;       // conv / window channel of x0
    const float4 c0 = *reinterpret_cast<const float4 *>(cw + wch * TAPS);
    const float4 c1 = *reinterpret_cast<const float4 *>(cw + (qk_task ? DK + ch : wch) * TAPS);
    float w0[PAST], w1[PAST];              // raw rows before the current token, oldest first
#pragma unroll
    for (int j = 0; j < PAST; ++j) {
        w0[j] = W[j * CH + wch];
        w1[j] = qk_task ? W[j * CH + DK + ch] : 0.f;
    }
    const float eA = qk_task ? __expf(p.A_log[h * DK + ch]) : 0.f;
    const float dtb = qk_task ? p.dt_bias[h * DK + ch] : 0.f;

    // the sequence's token rows: element offset of (token t, this head, channel c)
    // is t * rowsz + h * DK + c
    const int64_t rowsz = (int64_t)p.H * DK;
    auto rows = [&](const void *base, uint32_t elem) -> Rsrc {
        return make_rsrc(static_cast<const char *>(base) + rng.lo * rowsz * elem,
                         (uint32_t)(rng.len * rowsz * elem));
    };
    const Rsrc r_q = rows(p.q, BA::ELEM);
    const Rsrc r_k = rows(p.k, BA::ELEM);
    const Rsrc r_v = rows(p.v, BA::ELEM);
    const Rsrc r_f = rows(p.f, 4);
    const Rsrc r_g = rows(p.g, BA::ELEM);
    const Rsrc r_y = rows(p.y, BA::ELEM);
    const Rsrc r_o = rows(p.o_raw, 4);
    const Rsrc r_b = make_rsrc(p.beta + rng.lo * p.H, (uint32_t)(rng.len * p.H * 4));
    const uint32_t e_ch = (uint32_t)(h * DK + ch), e_out = (uint32_t)(h * DV + 4 * cg);

    float x0, x1, fa, bt;
    float2 g01 = make_float2(0.f, 0.f), g23 = g01;
    auto load_token = [&](int64_t t) {
        const uint32_t tr = (uint32_t)(t * rowsz);
        if (qk_task) {                     // wavefronts 0 and 1
            x0 = bld_one<Act>(r_q, tr + e_ch);
            x1 = bld_one<Act>(r_k, tr + e_ch);
            fa = bld_f32(r_f, (tr + e_ch) * 4);
        } else {
            x0 = bld_one<Act>(r_v, tr + e_ch);
            x1 = 0.f;
            fa = 0.f;
        }
        bt = bld_f32(r_b, (uint32_t)((t * p.H + h) * 4));
        if (tid < 32) {
            g01 = BA::load2(r_g, tr + e_out);
            g23 = BA::load2(r_g, tr + e_out + 2);
        }
    };
    load_token(0);

    // state rows rg + 8 m, columns 4 cg .. 4 cg + 3: lane offset plus m as the scalar offset
    const Rsrc r_s = make_rsrc(p.state + unit * (DK * DV), DK * DV * 4);
    const uint32_t s_lane = (uint32_t)((rg * DV + 4 * cg) * 4);
    float4 s[Sh::RPT];
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) s[m] = bld_f32x4(r_s, s_lane, (uint32_t)(m * Sh::NRG * DV * 4));

#pragma unroll 1
    for (int64_t t = 0; t < rng.len; ++t) {
        const int par = (int)(t & 1);
        const float cx0 = x0, cx1 = x1, cfa = fa, b = bt;
        const float2 cg01 = g01, cg23 = g23;
        if (t + 1 < rng.len) load_token(t + 1);

        // ---- pre-step of token t
        float qq = 0.f, kk = 0.f, qk = 0.f;
        const float a0 = silu(c0.x * w0[0] + c0.y * w0[1] + c0.z * w0[2] + c0.w * cx0);
        if (qk_task) {
            const float ak = silu(c1.x * w1[0] + c1.y * w1[1] + c1.z * w1[2] + c1.w * cx1);
            const float al = decay(cfa, eA, dtb, p.gate_mode, p.lb);
            s_aqk[par][ch] = make_float2(al * a0, al * ak);
            s_ak[par][ch] = make_float2(al, ak);
            qq = a0 * a0; kk = ak * ak; qk = a0 * ak;
        } else {
            s_v[par][ch] = a0;
        }
        w0[0] = w0[1]; w0[1] = w0[2]; w0[2] = cx0;
        w1[0] = w1[1]; w1[1] = w1[2]; w1[2] = cx1;
        qq = sum64(qq); kk = sum64(kk); qk = sum64(qk);
        if (lane == 0) { s_red[wave][0] = qq; s_red[wave][1] = kk; s_red[wave][2] = qk; }
        __syncthreads();
        qq = 0.f; kk = 0.f; qk = 0.f;
#pragma unroll
        for (int w = 0; w < Sh::NW; ++w) { qq += s_red[w][0]; kk += s_red[w][1]; qk += s_red[w][2]; }
        const float rq = rsqrtf(qq + p.l2_eps);
        const float rk = rsqrtf(kk + p.l2_eps);
        qk *= rq * rk;

        // ---- unnormalised S^T (a . k), S^T (a . q) over this thread's rows
        float4 u = make_float4(0.f, 0.f, 0.f, 0.f), pq = u;
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) {
            const float2 c = s_aqk[par][rg + Sh::NRG * m];
            u.x += s[m].x * c.y; u.y += s[m].y * c.y; u.z += s[m].z * c.y; u.w += s[m].w * c.y;
            pq.x += s[m].x * c.x; pq.y += s[m].y * c.x; pq.z += s[m].z * c.x; pq.w += s[m].w * c.x;
        }
        u.x += __shfl_xor(u.x, 32); u.y += __shfl_xor(u.y, 32);
        u.z += __shfl_xor(u.z, 32); u.w += __shfl_xor(u.w, 32);
        pq.x += __shfl_xor(pq.x, 32); pq.y += __shfl_xor(pq.y, 32);
        pq.z += __shfl_xor(pq.z, 32); pq.w += __shfl_xor(pq.w, 32);
        if (lane < 32) { s_up[wave][cg][0] = u; s_up[wave][cg][1] = pq; }
        __syncthreads();
        u = s_up[0][cg][0]; pq = s_up[0][cg][1];
#pragma unroll
        for (int w = 1; w < Sh::NW; ++w) {
            const float4 a = s_up[w][cg][0], c = s_up[w][cg][1];
            u.x += a.x; u.y += a.y; u.z += a.z; u.w += a.w;
            pq.x += c.x; pq.y += c.y; pq.z += c.z; pq.w += c.w;
        }

        // ---- delta, readout, update in registers
        const float4 vv = *reinterpret_cast<const float4 *>(&s_v[par][4 * cg]);
        float4 d, o, dk;
        d.x = b * (vv.x - rk * u.x); d.y = b * (vv.y - rk * u.y);
        d.z = b * (vv.z - rk * u.z); d.w = b * (vv.w - rk * u.w);
        o.x = rq * pq.x + qk * d.x; o.y = rq * pq.y + qk * d.y;
        o.z = rq * pq.z + qk * d.z; o.w = rq * pq.w + qk * d.w;
        dk.x = rk * d.x; dk.y = rk * d.y; dk.z = rk * d.z; dk.w = rk * d.w;
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) {
            const float2 c = s_ak[par][rg + Sh::NRG * m];      // (a_i, k_i)
            s[m].x = c.x * s[m].x + c.y * dk.x; s[m].y = c.x * s[m].y + c.y * dk.y;
            s[m].z = c.x * s[m].z + c.y * dk.z; s[m].w = c.x * s[m].w + c.y * dk.w;
        }

        // ---- RMSNorm over the 128 outputs, gamma, sigmoid gate
        const float ss = sum32(o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w);
        if (tid < 32) {
            const float r = rsqrtf(ss * (1.0f / DV) + p.rms_eps);
            const float4 gm = *reinterpret_cast<const float4 *>(p.gamma + 4 * cg);
            const uint32_t e = (uint32_t)(t * rowsz) + e_out;
            float2 y01, y23;
            y01.x = sigmoid(cg01.x) * gm.x * o.x * r;
            y01.y = sigmoid(cg01.y) * gm.y * o.y * r;
            y23.x = sigmoid(cg23.x) * gm.z * o.z * r;
            y23.y = sigmoid(cg23.y) * gm.w * o.w * r;
            BA::store2(r_y, e, y01);
            BA::store2(r_y, e + 2, y23);
            if (p.o_raw) {
                bst_f32x2(r_o, make_float2(o.x, o.y), e * 4);
                bst_f32x2(r_o, make_float2(o.z, o.w), (e + 2) * 4);
            }
        }
    }

    // ---- state and window out
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) bst_f32x4_at(r_s, s[m], s_lane + (uint32_t)(m * Sh::NRG * DV * 4));
#pragma unroll
    for (int j = 0; j < PAST; ++j) {
        W[j * CH + wch] = w0[j];
        if (qk_task) W[j * CH + DK + ch] = w1[j];
    }
}

template <int NT, bool NT_LOAD, bool NT_STORE, bool BLOCKED = false, int WPE = 1>
hipError_t launch_decode_as(const Params &p, bool bf16, hipStream_t stream) {
    const dim3 grid((unsigned)(p.num_seqs * p.H)), block(NT);
    if (bf16)
        hipLaunchKernelGGL((decode_kernel<BF16, NT, NT_LOAD, NT_STORE, BLOCKED, WPE>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<F32, NT, NT_LOAD, NT_STORE, BLOCKED, WPE>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// Compute units of each device, read on first use.
constexpr int STREAM_DEVICES = 64;
std::atomic<int> g_stream_cus[STREAM_DEVICES];

// Grid of the persistent kernel: one workgroup per compute unit, its size a
// multiple of H; batches of at most two pairs per compute unit keep one pair
// per workgroup.  Measured at 64 x 32 (2048 pairs, plain cache policy): 256
// workgroups of 8 pairs 46.8 us per step, 512 of 4 48.0, 768 of 2 or 3 47.9;
// grids that leave some workgroups one pair more than others lose the tail
// (640: 52.0, 384: 52.0).  Prefetching the next pair's state as well (two
// state register sets) measured slower: 49.1 us at 256 workgroups.
template <typename Act, bool NT_LOAD, bool NT_STORE>
hipError_t launch_stream_as(const Params &p, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = dev >= 0 && dev < STREAM_DEVICES ? g_stream_cus[dev].load(std::memory_order_relaxed) : 0;
    if (cus <= 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (cus <= 0) cus = 1;
        if (dev >= 0 && dev < STREAM_DEVICES) g_stream_cus[dev].store(cus, std::memory_order_relaxed);
    }
    const int64_t pairs = (int64_t)p.num_seqs * p.H;
    int64_t G = pairs;
    if (pairs > 2 * (int64_t)cus) G = cus >= p.H ? (int64_t)cus / p.H * p.H : p.H;
    hipLaunchKernelGGL((decode_stream_kernel<Act, NT_LOAD, NT_STORE>), dim3((unsigned)G), dim3(256), 0,
                       stream, p, (int32_t)G);
    return hipGetLastError();
}

}  // namespace

// Cache policy of the state: a state that fits comfortably in the 256 MB
// Infinity Cache (with the window and the step's other rows) stays there
// from one step to the next under the plain policy; larger ones stream
// better nontemporally, and above the cache size the blocked row order of
// the one-pair-per-workgroup kernel streams best (6.3 vs 6.0 TB/s at 1 GiB).
hipError_t launch_decode(const Params &p, bool bf16, hipStream_t stream) {
    const int64_t state_bytes = (int64_t)p.num_seqs * p.H * (DK * DV * 4);
    if (state_bytes > (int64_t(256) << 20))
        return launch_decode_as<256, true, true, true>(p, bf16, stream);
    return bf16 ? launch_stream_as<BF16, false, false>(p, stream) : launch_stream_as<F32, false, false>(p, stream);
}

bool short_supported(int64_t total_tokens, int32_t num_heads) {
    // per-tensor token rows of one sequence addressed with 32-bit byte offsets
    return total_tokens * num_heads * DK * 4 < (int64_t(1) << 32);
}

hipError_t launch_short(const Params &p, bool bf16, hipStream_t stream) {
    const dim3 grid((unsigned)(p.num_seqs * p.H)), block(256);
    if (bf16)
        hipLaunchKernelGGL((short_seq_kernel<BF16>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((short_seq_kernel<F32>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
