// kda_prefill_scan.hip -- chunkwise KDA prefill in two passes, for batches of
// few (sequence, head) pairs.
//
// The chunk form (kda_prefill_chunk.hip; "Kimi K3 Metal Gap Analysis", §2,
// row "Recurrence") splits each 16-token chunk's work in two:
//   * quantities that depend only on the chunk's own inputs -- the activated
//     and normalised q, k, v, the decays, (e^G . K), (e^G . Q), E,
//     T = (I + Diag(b) L)^{-1} and M -- and
//   * the products with the state entering the chunk, which chain the chunks.
// The one-pass kernel gives a (sequence, head) pair one workgroup that does
// both, chunk after chunk; with few pairs most of the GPU then idles.  Here
// pass 1 computes the first kind for every chunk of every pair at once (one
// workgroup per chunk and head, all independent) into a record per chunk in
// the caller's workspace, and pass 2 walks the chunks of a pair with only the
// state products left, its 128 state columns spread over 16 wavefronts in
// four workgroups (each 16-column block split in two 64-row halves).  The pre-norm readout goes to an fp32 buffer; the RMSNorm +
// gate and the window are written by the column-split path's finishing
// kernels.
//
// Arithmetic is that of the one-pass kernel: state products on bf16 MFMA with
// split operands (hi + lo, about 2^-16 relative error per product, fp32
// sums and state); L and M in fp32 with the chunk-middle reference r = G at
// token 7 keeping every exponential inside e^{+-|lb| C / 2}.
#include "kda_device.hpp"

namespace kda {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void *lds_ptr;

constexpr int CC = 16;                 // tokens per chunk

// ---- the per-chunk record (bytes); bf16 parts as [hi block][lo block]
//   KA, QA  split e^G . k_hat, e^G . q_hat in the order of the state product:
//           16-byte slot (m, g, t) holds channels 32 m + 4 g + {0..3} and
//           32 m + 16 + 4 g + {0..3} of token t, at slot index (m * 4 + g) * 16 + t
//   E       split e^{G_C - G_t} . k_hat_t, [channel][token]
//   T, M    split (I + Diag(b) L)^{-1} and M (lower, with the diagonal), [row][column]
//   GC      e^{G_C} per channel, fp32
//   V       activated v, [token][channel] fp32 (zero past the sequence end)
//   B       beta per token (zero past the end)
constexpr int R_KA = 0, R_QA = 8192, R_E = 16384, R_T = 24576, R_M = 25600, R_GC = 26624,
              R_V = 27136, R_B = 35328, REC = 35840;   // REC: 35 KiB
static_assert(REC % 1024 == 0, "a record is a whole number of 1 KiB load blocks");

__device__ __forceinline__ uint16_t bf16_hi(float x) { return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu); }
__device__ __forceinline__ void split_store(uint8_t *rec, int off_hi, int part_bytes, int idx, float x) {
    const uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;
    const float lo = x - __uint_as_float(h << 16);
    reinterpret_cast<uint16_t *>(rec + off_hi)[idx] = (uint16_t)h;
    reinterpret_cast<uint16_t *>(rec + off_hi + part_bytes)[idx] = bf16_hi(lo);
}

// two fp32 values as packed bf16 high parts and packed bf16 remainders (the
// first value in the low half)
struct Split2 {
    uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split2(float x0, float x1) {
    const uint32_t hb = pack_bf16x2(x0, x1);
    return {hb, pack_bf16x2(x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u))};
}

__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// record slot of chunk c of sequence n: slots floor(cu[n] / 16) + n + c never
// collide (a sequence of len tokens has at most floor(len / 16) + 1 chunks)
__device__ __forceinline__ int64_t slot_base(const Params &p, int n) {
    const int64_t lo = p.cu_seqlens ? (int64_t)p.cu_seqlens[n] : (int64_t)n * p.dense_len;
    const int64_t c = lo < 0 ? 0 : (lo > p.total_tokens ? p.total_tokens : lo);
    return c / CC + n;
}

// four consecutive activations at byte offset o of a buffer (reads 0 out of range)
template <typename Act> __device__ __forceinline__ float4 ld_act4(Rsrc r, uint32_t o);
template <> __device__ __forceinline__ float4 ld_act4<F32>(Rsrc r, uint32_t o) { return bld_f32x4(r, o); }
template <> __device__ __forceinline__ float4 ld_act4<BF16>(Rsrc r, uint32_t o) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

// ---------------------------------------------------------------- pass 1
constexpr int PREP_THREADS = 256;
constexpr int XP = CH + 4;              // raw / activated row length in LDS
// raw rows: a thread loads 4 channels of one row of q, k or v at a time, the
// workgroup RAW_GRP rows of a tensor per pass
constexpr int RAW_ROWS = CC + PAST;
constexpr int RAW_GRP = PREP_THREADS / (DK / 4);
constexpr int RAW_PASSES = (RAW_ROWS + RAW_GRP - 1) / RAW_GRP;
constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every range here: reads 0

// LDS of the operand pass: the raw / activated rows, later each wavefront's
// partial L, M in the same bytes; the conv taps, later the decay sums in the
// same bytes
constexpr int R1_BYTES = (CC + PAST) * XP * 4;
constexpr int G_BYTES = CC * DK * 4, CW_BYTES = CH * TAPS * 4;
constexpr int R2_BYTES = G_BYTES > CW_BYTES ? G_BYTES : CW_BYTES;

template <typename Act>
__global__ __launch_bounds__(PREP_THREADS) __attribute__((amdgpu_waves_per_eu(3)))
void scan_prep_kernel(Params p, uint8_t *records, int32_t seg_lo) {
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    int n;
    int64_t slot, c;
    if (seg_lo < 0) {
        // the whole batch: one workgroup per record slot; the sequence owning
        // this slot is the last n with slot_base(n) <= slot
        slot = blockIdx.x;
        int lo = 0, hi = p.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (slot_base(p, mid) <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        c = slot - slot_base(p, n);
    } else {
        // one segment of chunks: chunk seg_lo + x of sequence z
        n = blockIdx.z;
        c = seg_lo + (int64_t)blockIdx.x;
        slot = slot_base(p, n) + c;
    }
    const Range rng = seq_range(p, n);
    const int64_t c0 = c * CC;
    if (c < 0 || c0 >= rng.len) return;
    const int nv = (int)(rng.len - c0 < CC ? rng.len - c0 : CC);
    uint8_t *rec = records + (slot * p.H + h) * REC;

    __shared__ __attribute__((aligned(16))) uint8_t smem[R1_BYTES + R2_BYTES];
    // raw rows c0 - 3 .. c0 + 15, then activated rows 3 .. 18
    float(*s_x)[XP] = reinterpret_cast<float(*)[XP]>(smem);
    // each wavefront's partial L, M (after the last read of s_x)
    float(*s_part)[2][CC * CC] = reinterpret_cast<float(*)[2][CC * CC]>(smem);
    static_assert(PREP_THREADS / 64 * 2 * CC * CC * 4 <= R1_BYTES, "partials in the raw rows' bytes");
    f32x4 lp, mp;
    float(*s_cw)[TAPS] = reinterpret_cast<float(*)[TAPS]>(smem + R1_BYTES);
    // log-decay summed from the chunk start (after the conv's last read of s_cw)
    float(*s_G)[DK] = reinterpret_cast<float(*)[DK]>(smem + R1_BYTES);
    __shared__ float s_nrm[CC][2];          // L2 scales of q, k
    __shared__ float s_A[CC][CC], s_b[CC];

    const int64_t rowsz = (int64_t)p.H * DK;
    // every global load of the chunk first (they are independent), then LDS.
    // Raw rows c0 - 3 .. c0 + 15: a row before the sequence comes from the
    // carried window, a row past its end reads 0; both loads are issued for
    // every row, one of them out of its buffer's range (reading 0), so the
    // pair adds up to the row without a branch.
    const int64_t rb0 = c0 - PAST < 0 ? 0 : c0 - PAST;   // first token row loaded
    const int64_t rend = rng.len < c0 + CC ? rng.len : c0 + CC;
    const Rsrc r_win = make_rsrc(p.win + ((int64_t)n * p.H + h) * (PAST * CH), PAST * CH * 4);
    const int rg = tid / (DK / 4), c4 = 4 * (tid % (DK / 4));
    float4 xr[3][RAW_PASSES];
#pragma unroll
    for (int ten = 0; ten < 3; ++ten) {
        const void *src = ten == 0 ? p.q : (ten == 1 ? p.k : p.v);
        const Rsrc r_tok = make_rsrc(static_cast<const char *>(src) + (rng.lo + rb0) * rowsz * BufAct<Act>::ELEM,
                                     (uint32_t)((rend - rb0) * rowsz * BufAct<Act>::ELEM));
#pragma unroll
        for (int u = 0; u < RAW_PASSES; ++u) {
            const int r = rg + RAW_GRP * u;
            const int64_t j = c0 - PAST + r;
            const bool live = r < RAW_ROWS;
            const uint32_t to = (live && j >= 0) ? (uint32_t)(((j - rb0) * rowsz + (int64_t)h * DK + c4) * BufAct<Act>::ELEM) : OOB;
            const uint32_t wo = (live && j < 0) ? (uint32_t)(((j + PAST) * CH + ten * DK + c4) * 4) : OOB;
            const float4 a = ld_act4<Act>(r_tok, to), b = bld_f32x4(r_win, wo);
            xr[ten][u] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        }
    }
    float fv[CC];
    float eA = 0.f, dtb = 0.f, bt = 0.f;
    if (tid < DK) {
        // (rows past the sequence end read 0)
        const Rsrc r_f = make_rsrc(p.f + (rng.lo + c0) * rowsz, (uint32_t)(nv * rowsz * 4));
#pragma unroll
        for (int t = 0; t < CC; ++t) fv[t] = bld_f32(r_f, (uint32_t)((h * DK + tid) * 4), (uint32_t)(t * rowsz * 4));
        eA = p.A_log[h * DK + tid];
        dtb = p.dt_bias[h * DK + tid];
    } else if (tid < DK + CC) {
        const int t = tid - DK;
        bt = t < nv ? p.beta[(rng.lo + c0 + t) * p.H + h] : 0.f;
    }
    float4 cw0 = *reinterpret_cast<const float4 *>(p.conv_w + ((int64_t)h * CH + tid) * TAPS);
    float4 cw1 = tid < CH - PREP_THREADS
                     ? *reinterpret_cast<const float4 *>(p.conv_w + ((int64_t)h * CH + PREP_THREADS + tid) * TAPS)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4 *>(s_cw[tid]) = cw0;
    if (tid < CH - PREP_THREADS) *reinterpret_cast<float4 *>(s_cw[PREP_THREADS + tid]) = cw1;
#pragma unroll
    for (int ten = 0; ten < 3; ++ten)
#pragma unroll
        for (int u = 0; u < RAW_PASSES; ++u) {
            const int r = rg + RAW_GRP * u;
            if (r < RAW_ROWS) *reinterpret_cast<float4 *>(&s_x[r][ten * DK + c4]) = xr[ten][u];
        }
    __syncthreads();
    // conv + SiLU (tokens past the end give zeros); each thread keeps its
    // results in registers until every tap has been read
    float act[(CC * CH) / PREP_THREADS];
#pragma unroll
    for (int u = 0; u < (CC * CH) / PREP_THREADS; ++u) {
        const int idx = tid + u * PREP_THREADS;
        const int t = idx / CH, ch = idx - t * CH;
        const float4 w = *reinterpret_cast<const float4 *>(s_cw[ch]);
        const float a = w.x * s_x[t][ch] + w.y * s_x[t + 1][ch] + w.z * s_x[t + 2][ch] + w.w * s_x[t + 3][ch];
        act[u] = t < nv ? silu(a) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (CC * CH) / PREP_THREADS; ++u) {
        const int idx = tid + u * PREP_THREADS;
        const int t = idx / CH, ch = idx - t * CH;
        s_x[PAST + t][ch] = act[u];
    }
    // decays: channel i's log-decay summed over the chunk's tokens
    if (tid < DK) {
        const int i = tid;
        eA = __expf(eA);
        float G = 0.f;                         // held constant past the last token
#pragma unroll
        for (int t = 0; t < CC; ++t) {
            if (t < nv) G += p.lb * sigmoid(eA * (fv[t] + dtb));
            s_G[t][i] = G;
        }
    } else if (tid < DK + CC) {
        const int t = tid - DK;
        s_b[t] = bt;
        reinterpret_cast<float *>(rec + R_B)[t] = bt;
    }
    __syncthreads();
    // L2 scales: 8 lanes per (token, q or k)
    {
        const int grp = tid >> 3, sub = tid & 7;
        const int t = grp >> 1, which = grp & 1;
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < DK / 8; ++u) {
            const float a = s_x[PAST + t][which * DK + sub * (DK / 8) + u];
            ss += a * a;
        }
        ss = sum8(ss);
        if (sub == 0) s_nrm[t][which] = rsqrtf(ss + p.l2_eps);
    }
    __syncthreads();
    // operands of the state products, one 16-byte record slot per thread:
    // token t, channels 32 m + 4 g + {0..3} and 32 m + 16 + 4 g + {0..3}; and
    // the L, M factors of those channels.  The slot's q_hat, k_hat are read
    // now: the factors go into the bytes of s_x after the next barrier.
    const int st_t = tid & 15, st_g = (tid >> 4) & 3, st_m = tid >> 6;
    float sq[8], sk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = 32 * st_m + 16 * (e >> 2) + 4 * st_g + (e & 3);
        sq[e] = s_x[PAST + st_t][i] * s_nrm[st_t][0];
        sk[e] = s_x[PAST + st_t][DK + i] * s_nrm[st_t][1];
    }
    // E: one channel's 16 tokens per thread; and e^{G_C}
    if (tid < DK) {
        const int i = tid;
        const float GC = s_G[CC - 1][i];
        u32x4 eh[2], el[2];
#pragma unroll
        for (int t2 = 0; t2 < CC / 2; ++t2) {
            const float e0 = __expf(GC - s_G[2 * t2][i]) * (s_x[PAST + 2 * t2][DK + i] * s_nrm[2 * t2][1]);
            const float e1 = __expf(GC - s_G[2 * t2 + 1][i]) * (s_x[PAST + 2 * t2 + 1][DK + i] * s_nrm[2 * t2 + 1][1]);
            const Split2 a = split2(e0, e1);
            eh[t2 >> 2][t2 & 3] = a.hi;
            el[t2 >> 2][t2 & 3] = a.lo;
        }
        *reinterpret_cast<u32x4 *>(rec + R_E + i * 32) = eh[0];
        *reinterpret_cast<u32x4 *>(rec + R_E + i * 32 + 16) = eh[1];
        *reinterpret_cast<u32x4 *>(rec + R_E + 4096 + i * 32) = el[0];
        *reinterpret_cast<u32x4 *>(rec + R_E + 4096 + i * 32 + 16) = el[1];
        reinterpret_cast<float *>(rec + R_GC)[i] = __expf(GC);
    }
    // v: four channels per store
#pragma unroll
    for (int u = 0; u < (CC * DV / 4) / PREP_THREADS; ++u) {
        const int idx = tid + u * PREP_THREADS;
        const int t = idx / (DV / 4), i4 = (idx - t * (DV / 4)) * 4;
        *reinterpret_cast<float4 *>(rec + R_V + (t * DV + i4) * 4) =
            *reinterpret_cast<const float4 *>(&s_x[PAST + t][2 * DK + i4]);
    }
    __syncthreads();                           // s_x is dead from here on
    {
        float ka[8], qa[8], fl[8], fm[8], fr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 32 * st_m + 16 * (e >> 2) + 4 * st_g + (e & 3);
            const float G = s_G[st_t][i], r = s_G[CC / 2 - 1][i];
            const float eg = __expf(G);
            ka[e] = eg * sk[e];
            qa[e] = eg * sq[e];
            const float ef = __expf(G - r), eb = __expf(r - G);
            fl[e] = ef * sk[e];
            fm[e] = ef * sq[e];
            fr[e] = eb * sk[e];
        }
        // the partial L, M over this wavefront's 32 channels as one 16x16x32
        // step per split part: lane l holds token l % 16 and eight channels as
        // k = 8 (l / 16) + e, both for the rows (fl, fm) and for the columns
        // (fr), so the lane's own factors are the operands
        u32x4 lh, ll, mh, ml, rh, rl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const Split2 a = split2(fl[2 * e], fl[2 * e + 1]), b = split2(fm[2 * e], fm[2 * e + 1]);
            const Split2 c = split2(fr[2 * e], fr[2 * e + 1]);
            lh[e] = a.hi; ll[e] = a.lo;
            mh[e] = b.hi; ml[e] = b.lo;
            rh[e] = c.hi; rl[e] = c.lo;
        }
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        lp = mfma32(lh, rh, mfma32(lh, rl, mfma32(ll, rh, z4)));
        mp = mfma32(mh, rh, mfma32(mh, rl, mfma32(ml, rh, z4)));
        const int so = (((st_m * 4 + st_g) * CC) + st_t) * 16;
        u32x4 kh4, kl4, qh4, ql4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const Split2 a = split2(ka[2 * e], ka[2 * e + 1]), b = split2(qa[2 * e], qa[2 * e + 1]);
            kh4[e] = a.hi;
            kl4[e] = a.lo;
            qh4[e] = b.hi;
            ql4[e] = b.lo;
        }
        *reinterpret_cast<u32x4 *>(rec + R_KA + so) = kh4;
        *reinterpret_cast<u32x4 *>(rec + R_KA + 4096 + so) = kl4;
        *reinterpret_cast<u32x4 *>(rec + R_QA + so) = qh4;
        *reinterpret_cast<u32x4 *>(rec + R_QA + 4096 + so) = ql4;
    }
    __syncthreads();
    // the four wavefronts' partials (lane l: rows 4 (l / 16) + r of column
    // l % 16) through LDS, in the bytes the raw rows used
    {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s_part[st_m][0][(4 * st_g + r) * CC + st_t] = lp[r];
            s_part[st_m][1][(4 * st_g + r) * CC + st_t] = mp[r];
        }
    }
    __syncthreads();
    // L (strictly lower, times beta: the matrix A of the solve) and M (lower
    // with the diagonal): one (t, s) pair per thread, the partials added in
    // wavefront order
    {
        const int t = tid >> 4, s = tid & 15;
        float l = s_part[0][0][tid], mm = s_part[0][1][tid];
#pragma unroll
        for (int w = 1; w < PREP_THREADS / 64; ++w) {
            l += s_part[w][0][tid];
            mm += s_part[w][1][tid];
        }
        s_A[t][s] = s < t ? s_b[t] * l : 0.f;
        split_store(rec, R_M, 512, t * CC + s, s <= t ? mm : 0.f);
    }
    __syncthreads();
    // T = (I + A)^{-1} by forward substitution, one column per thread
    if (tid < CC) {
        const int col = tid;
        float x[CC];
#pragma unroll
        for (int t = 0; t < CC; ++t) {
            float y = (t == col) ? 1.0f : 0.0f;
#pragma unroll
            for (int s = 0; s < t; ++s) y = fmaf(-s_A[t][s], x[s], y);
            x[t] = t < col ? 0.f : y;
            split_store(rec, R_T, 512, t * CC + col, x[t]);
        }
    }
}

// ---------------------------------------------------------------- pass 2
// Wavefront w of a workgroup: state columns 16 (2 grp + w / 2) .. + 15, key
// rows 64 (w % 2) .. + 63; the two row halves of a column block add their
// partial P, R through LDS.
constexpr int SCAN_WAVES = 4;
constexpr int SCAN_COLS = 2;            // 16-column blocks per workgroup
constexpr int SCAN_GROUPS = DV / (16 * SCAN_COLS);
constexpr int XCDS = 8;
constexpr int RING = 4;                 // record buffers per workgroup (3 loading while 1 is used)

__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b),
                                                     c, 0, 0, 0);
}
__device__ __forceinline__ void split4(f32x4 d, u32x2 &h, u32x2 &l) {
    const Split2 a = split2(d[0], d[1]), b = split2(d[2], d[3]);
    h = u32x2{a.hi, b.hi};
    l = u32x2{a.lo, b.lo};
}
// c + a b with both operands split
__device__ __forceinline__ f32x4 mma32(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
    c = mfma32(al, bh, c);
    c = mfma32(ah, bl, c);
    return mfma32(ah, bh, c);
}
__device__ __forceinline__ f32x4 mma16(u32x2 ah, u32x2 al, u32x2 bh, u32x2 bl, f32x4 c) {
    c = mfma16(al, bh, c);
    c = mfma16(ah, bl, c);
    return mfma16(ah, bh, c);
}

// wait until at most N of this wavefront's loads are outstanding and its LDS
// reads are complete, then the workgroup barrier (no fence: that would wait
// for the loads still in flight).  The wait is the builtin, which the
// compiler's own wait counting sees: it then knows the record loads older
// than the last N have landed and adds no wait for them before the record's
// LDS reads (behind a wait in inline asm it waited for every load in flight
// once per loop trip).  The barrier is asm with a memory clobber, so that no
// LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
    static_assert(N < 64, "vmcnt has 6 bits");
    // s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt 11:8 (0)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    asm volatile("s_barrier" ::: "memory");
}
// LDS writes complete, then the workgroup barrier (loads may stay in flight)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// a record into LDS: 35 blocks of 1 KiB, block b by wavefront b % 4
constexpr int REC_BLOCKS = REC / 1024;
constexpr int LOADS_PER_WAVE = (REC_BLOCKS + SCAN_WAVES - 1) / SCAN_WAVES;   // 9 (the last is partial)
__device__ __forceinline__ void rec_issue(Rsrc r, uint8_t *dst, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < LOADS_PER_WAVE; ++j) {
        const int b = wave + SCAN_WAVES * j;
        // every wavefront issues the same number of loads (the wait counts
        // assume it): past the record's last block the load repeats block 0
        // into a spare block of the buffer
        const int bb = b < REC_BLOCKS ? b : 0;
        const int db = b < REC_BLOCKS ? b : REC_BLOCKS;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(dst + db * 1024), 16, bb * 1024 + lane * 16, 0, 0, 0);
    }
}

// chunks [c_lo, c_hi) of each pair: the state is read at the start and
// written at the end, so consecutive ranges chain through it
__global__ __launch_bounds__(64 * SCAN_WAVES) void scan_kernel(Params p, const uint8_t *records, float *obuf,
                                                               int32_t c_lo, int32_t c_hi) {
    // one LDS buffer per record in flight (+1 spare block each), separate
    // arrays so that the compiler's waits track each one alone
    __shared__ __attribute__((aligned(1024))) uint8_t sR0[REC + 1024], sR1[REC + 1024], sR2[REC + 1024],
        sR3[REC + 1024];
    // workgroups are dealt to the XCDs in turn: the SCAN_GROUPS workgroups
    // of one (sequence, head) pair are XCDS apart in the grid, so that they
    // share one XCD and its L2 fetches each record once for all of them
    const int xcd = blockIdx.x % XCDS;
    const int grp = blockIdx.x / XCDS % SCAN_GROUPS;
    const int pair = blockIdx.x / (XCDS * SCAN_GROUPS) * XCDS + xcd;
    if (pair >= p.num_seqs * p.H) return;
    const int slot_n = pair / p.H;
    const int h = pair - slot_n * p.H;
    int n = slot_n;
    if (p.seq_order) {
        n = p.seq_order[slot_n];
        if (n < 0 || n >= p.num_seqs) return;
    }
    const Range rng = seq_range(p, n);
    if (rng.len <= 0) return;
    const int64_t NCS = (rng.len + CC - 1) / CC;
    const int64_t NC = NCS < c_hi ? NCS : c_hi;    // one past this launch's last chunk
    if (c_lo >= NC) return;
    // the wavefront index is uniform: read it into a scalar register, so that
    // the record loads' LDS destinations are scalar too
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int rh = wave & 1;                               // key rows 64 rh .. 64 rh + 63
    const int col0 = 16 * (grp * SCAN_COLS + (wave >> 1));
    const int64_t unit = (int64_t)n * p.H + h;
    const int64_t sb = slot_base(p, n);
    const uint8_t *recs = records + (sb * p.H + h) * REC;   // chunk c at + c * H * REC
    // partial P, R of each wavefront: [wave][P, R][element r][lane]
    __shared__ __attribute__((aligned(16))) float sX[SCAN_WAVES][2][4][64];

    // the state: tile j, element r = S[16 (4 rh + j) + 4 g4 + r][col0 + n16]
    const Rsrc rs_state = make_rsrc(p.state + unit * (DK * DV), DK * DV * 4);
    f32x4 st[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            st[j][r] = bld_f32(rs_state, ((4 * g4 + r) * DV + col0 + n16) * 4, (4 * rh + j) * 16 * DV * 4);

    auto rec_rsrc = [&](int64_t c) { return make_rsrc(recs + c * p.H * REC, REC); };
    const int64_t rowsz = (int64_t)p.H * DV;

    // O rows of a chunk through a buffer resource per chunk: the lane offsets
    // are constant, and rows past the sequence end fall outside the buffer's
    // range, where stores are dropped
    uint32_t o_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o_off[r] = (uint32_t)(((4 * g4 + r) * rowsz + n16) * 4);
    auto chunk = [&](int64_t c, const uint8_t *R) {
        // partial P, R over this wavefront's key rows: steps m = 2 rh, 2 rh + 1
        // (rows 32 m .. 32 m + 31, tiles 2 (m - 2 rh), + 1); the three parts of
        // each split product accumulate in one chain
        // (LDS reads complete in order: the products' operands are read first,
        // then the chunk's other record fields that the chain after the
        // exchange needs, so that their latency runs under the products; the
        // scheduling barriers keep that order)
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 Pp = z4, Rp = z4;
        u32x4 ka_h[2], ka_l[2], qa_h[2], qa_l[2];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const int so = (((2 * rh + mm) * 4 + g4) * CC + n16) * 16;
            ka_h[mm] = *reinterpret_cast<const u32x4 *>(R + R_KA + so);
            ka_l[mm] = *reinterpret_cast<const u32x4 *>(R + R_KA + 4096 + so);
            qa_h[mm] = *reinterpret_cast<const u32x4 *>(R + R_QA + so);
            qa_l[mm] = *reinterpret_cast<const u32x4 *>(R + R_QA + 4096 + so);
        }
        __builtin_amdgcn_sched_barrier(0);
        // beta, v, T and M of the chunk, behind the products' operands
        const float4 bt = *reinterpret_cast<const float4 *>(R + R_B + 16 * g4);   // beta of tokens 4 g4 + r
        float vt[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) vt[r] = reinterpret_cast<const float *>(R + R_V)[(4 * g4 + r) * DK + col0 + n16];
        const int to = (n16 * CC + 4 * g4) * 2;
        const u32x2 th = *reinterpret_cast<const u32x2 *>(R + R_T + to);
        const u32x2 tl = *reinterpret_cast<const u32x2 *>(R + R_T + 512 + to);
        const u32x2 mh = *reinterpret_cast<const u32x2 *>(R + R_M + to);
        const u32x2 ml = *reinterpret_cast<const u32x2 *>(R + R_M + 512 + to);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const u32x4 kah = ka_h[mm], kal = ka_l[mm], qah = qa_h[mm], qal = qa_l[mm];
            const Split2 x0 = split2(st[2 * mm][0], st[2 * mm][1]);
            const Split2 x1 = split2(st[2 * mm][2], st[2 * mm][3]);
            const Split2 x2 = split2(st[2 * mm + 1][0], st[2 * mm + 1][1]);
            const Split2 x3 = split2(st[2 * mm + 1][2], st[2 * mm + 1][3]);
            const u32x4 sh = {x0.hi, x1.hi, x2.hi, x3.hi}, sl = {x0.lo, x1.lo, x2.lo, x3.lo};
            Pp = mfma32(kal, sh, Pp);
            Rp = mfma32(qal, sh, Rp);
            Pp = mfma32(kah, sl, Pp);
            Rp = mfma32(qah, sl, Rp);
            Pp = mfma32(kah, sh, Pp);
            Rp = mfma32(qah, sh, Rp);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sX[wave][0][r][lane] = Pp[r];
            sX[wave][1][r][lane] = Rp[r];
        }
        lds_barrier();
        // the update's operands from the record, read before the chain of W,
        // Delta and O, which they then wait under
        float4 dc[4];
        u32x2 eh[4], el[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rt = 4 * rh + j;
            dc[j] = *reinterpret_cast<const float4 *>(R + R_GC + (16 * rt + 4 * g4) * 4);
            const int eo = ((16 * rt + n16) * CC + 4 * g4) * 2;
            eh[j] = *reinterpret_cast<const u32x2 *>(R + R_E + eo);
            el[j] = *reinterpret_cast<const u32x2 *>(R + R_E + 4096 + eo);
        }
        // whole P, R: the lower row half's part plus the upper's, in that order
        // in both wavefronts, so that both form the same Delta
        f32x4 Pt, Rt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float po = sX[wave ^ 1][0][r][lane], ro = sX[wave ^ 1][1][r][lane];
            Pt[r] = rh == 0 ? Pp[r] + po : po + Pp[r];
            Rt[r] = rh == 0 ? Rp[r] + ro : ro + Rp[r];
        }
        // W = Diag(b) (V - P) (rows 4 g4 + r); Delta = T W; O = R + M Delta
        const f32x4 Wt = {bt.x * (vt[0] - Pt[0]), bt.y * (vt[1] - Pt[1]), bt.z * (vt[2] - Pt[2]), bt.w * (vt[3] - Pt[3])};
        u32x2 wh, wl, dh, dl;
        split4(Wt, wh, wl);
        const f32x4 Dt = mma16(th, tl, wh, wl, f32x4{0.f, 0.f, 0.f, 0.f});
        split4(Dt, dh, dl);
        if (rh == 0) {
            const f32x4 Ot = mma16(mh, ml, dh, dl, Rt);
            const int64_t nv = rng.len - c * CC < CC ? rng.len - c * CC : CC;
            const Rsrc ro = make_rsrc(obuf + (rng.lo + c * CC) * rowsz + (int64_t)h * DV + col0,
                                      (uint32_t)(((nv - 1) * rowsz + DV) * 4));
#pragma unroll
            for (int r = 0; r < 4; ++r) bst_f32(ro, Ot[r], o_off[r]);
        }
        // S <- Diag(e^{G_C}) S + E^T Delta on this wavefront's rows
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            st[j][0] *= dc[j].x;
            st[j][1] *= dc[j].y;
            st[j][2] *= dc[j].z;
            st[j][3] *= dc[j].w;
            st[j] = mma16(eh[j], el[j], dh, dl, st[j]);
        }
    };
    // chunk c: its record landed everywhere (and every wavefront is done with
    // chunk c - 1's buffer), the chunk, then the record RING - 1 chunks ahead
    // into that buffer.  (Issued before the chunk, those loads made the
    // compiler wait for every load in flight before the chunk's record reads
    // once per loop trip: it cannot tell the buffers' loads apart there.)
    auto step = [&](int64_t c, const uint8_t *cur, uint8_t *prev) {
        if (c >= NC) return;
        const int64_t after = NC - 1 - c < RING - 2 ? NC - 1 - c : RING - 2;
        if (after >= 2)
            wait_then_barrier<2 * LOADS_PER_WAVE>();
        else if (after == 1)
            wait_then_barrier<LOADS_PER_WAVE>();
        else
            wait_then_barrier<0>();
        chunk(c, cur);
        if (c + RING - 1 < NC) rec_issue(rec_rsrc(c + RING - 1), prev, wave, lane);
    };
    rec_issue(rec_rsrc(c_lo), sR0, wave, lane);
    if (NC > c_lo + 1) rec_issue(rec_rsrc(c_lo + 1), sR1, wave, lane);
    if (NC > c_lo + 2) rec_issue(rec_rsrc(c_lo + 2), sR2, wave, lane);
#pragma unroll 1
    for (int64_t c = c_lo; c < NC; c += RING) {
        step(c, sR0, sR3);
        step(c + 1, sR1, sR0);
        step(c + 2, sR2, sR1);
        step(c + 3, sR3, sR2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            bst_f32(rs_state, st[j][r], ((4 * g4 + r) * DV + col0 + n16) * 4, (4 * rh + j) * 16 * DV * 4);
}

// ---- the schedule
//
// A pair's state pass keeps one workgroup per CU busy (its LDS), so with at
// most 32 pairs it fills at most half of the 256 CUs, and the operand pass,
// which has the whole GPU to itself, would otherwise run first and alone.
// With enough chunks, and a second stream from the caller, the chunks are
// cut into segments: segment s + 1's operand pass runs on the second stream,
// on the idle CUs, while segment s's state pass runs, and each state-pass
// launch continues from the state the previous one wrote.  The two streams
// are ordered by events that the call creates and releases.
constexpr int SEG_MAX = 4;              // segments at most
constexpr int SEG_CHUNKS = 128;         // chunks per segment aimed at (at least 2 segments from here)
constexpr int64_t SEG_MAX_PAIRS = 32;   // state-pass workgroups on at most half the CUs

// chunks of the longest sequence when the host knows it (dense batches, a
// single sequence, or the caller's host copy of the offsets), else 0
int64_t scan_max_chunks(const Params &p, const int32_t *cu_host) {
    if (!p.cu_seqlens) return ((int64_t)p.dense_len + CC - 1) / CC;
    if (cu_host) {
        int64_t mx = 0;
        for (int n = 0; n < p.num_seqs; ++n) {
            const int64_t len = (int64_t)cu_host[n + 1] - cu_host[n];
            mx = len > mx ? len : mx;
        }
        return (mx + CC - 1) / CC;
    }
    if (p.num_seqs == 1) return (p.total_tokens + CC - 1) / CC;
    return 0;
}

// ragged batches of more sequences than this finish with one epilogue launch
// (a segment's rows are one launch per sequence)
constexpr int SEG_MAX_RAGGED_SEQS = 8;

int scan_segments(const Params &p, const int32_t *cu_host) {
    const int64_t pairs = (int64_t)p.num_seqs * p.H;
    if (p.cu_seqlens && p.num_seqs > 1 && (!cu_host || p.num_seqs > SEG_MAX_RAGGED_SEQS)) return 1;
    const int64_t nc = scan_max_chunks(p, cu_host);
    if (pairs > SEG_MAX_PAIRS || nc < SEG_CHUNKS) return 1;
    const int64_t s = nc / SEG_CHUNKS;
    return (int)(s < 2 ? 2 : (s < SEG_MAX ? s : SEG_MAX));
}

// events ordering the two streams of one call: created by the call, released
// once enqueued (a recorded event lives until the device has passed it)
struct CallEvents {
    hipEvent_t ev[2 * SEG_MAX] = {};
    int n = 0;
    hipError_t create(int count) {
        for (n = 0; n < count; ++n) {
            const hipError_t e = hipEventCreateWithFlags(&ev[n], hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    ~CallEvents() {
        for (int i = 0; i < n; ++i) (void)hipEventDestroy(ev[i]);
    }
};

template <typename Act>
hipError_t launch_prep(const Params &p, uint8_t *records, int64_t c_lo, int64_t c_hi, bool whole,
                       hipStream_t stream) {
    if (whole) {
        const int64_t slots = p.total_tokens / CC + p.num_seqs;
        hipLaunchKernelGGL((scan_prep_kernel<Act>), dim3((unsigned)slots, (unsigned)p.H), dim3(PREP_THREADS), 0,
                           stream, p, records, -1);
    } else {
        hipLaunchKernelGGL((scan_prep_kernel<Act>), dim3((unsigned)(c_hi - c_lo), (unsigned)p.H, (unsigned)p.num_seqs),
                           dim3(PREP_THREADS), 0, stream, p, records, (int32_t)c_lo);
    }
    return hipGetLastError();
}

hipError_t launch_state_pass(const Params &p, const uint8_t *records, float *obuf, int64_t c_lo, int64_t c_hi,
                             hipStream_t stream) {
    const int64_t pairs = (int64_t)p.num_seqs * p.H;
    const int64_t blocks = (pairs + XCDS - 1) / XCDS * XCDS * SCAN_GROUPS;
    hipLaunchKernelGGL(scan_kernel, dim3((unsigned)blocks), dim3(64 * SCAN_WAVES), 0, stream, p, records, obuf,
                       (int32_t)c_lo, (int32_t)(c_hi < INT32_MAX ? c_hi : INT32_MAX));
    return hipGetLastError();
}

template <typename Act>
hipError_t launch_scan_as(const Params &p, bool bf16, uint8_t *records, float *obuf, hipStream_t stream,
                          hipStream_t side, const int32_t *cu_host) {
    const int nseg = side ? scan_segments(p, cu_host) : 1;
    hipError_t e;
    if (nseg == 1) {
        e = launch_prep<Act>(p, records, 0, 0, true, stream);
        if (e == hipSuccess) e = launch_state_pass(p, records, obuf, 0, INT64_MAX, stream);
        if (e == hipSuccess) e = launch_split_finish(p, bf16, obuf, stream);
        return e;
    }
    CallEvents events;
    e = events.create(2 * nseg);
    if (e != hipSuccess) return e;
    const int64_t nc = scan_max_chunks(p, cu_host);
    auto bound = [&](int s) { return nc * s / nseg; };
    // RMSNorm + gate of segment s: tokens [16 bound(s), 16 bound(s + 1)) of
    // every sequence (the last segment to the end).  Dense batches and a
    // single sequence take one launch; ragged batches one per sequence.
    auto epilogue = [&](int s, hipStream_t st) {
        const int64_t t0 = CC * bound(s), t1 = s + 1 < nseg ? CC * bound(s + 1) : INT64_MAX;
        if (!p.cu_seqlens || p.num_seqs == 1) {
            const int64_t len = p.cu_seqlens ? p.total_tokens : p.dense_len;
            const int32_t nseq = p.cu_seqlens ? 1 : p.num_seqs;
            const int64_t hi = t1 < len ? t1 : len;
            return launch_split_epilogue(p, bf16, obuf, t0 * p.H, (hi - t0) * p.H, len * p.H, nseq, st);
        }
        hipError_t r = hipSuccess;
        for (int n = 0; r == hipSuccess && n < p.num_seqs; ++n) {
            const int64_t len = (int64_t)cu_host[n + 1] - cu_host[n];
            const int64_t lo = t0 < len ? t0 : len, hi = t1 < len ? t1 : len;
            if (hi > lo)
                r = launch_split_epilogue(p, bf16, obuf, ((int64_t)cu_host[n] + lo) * p.H, (hi - lo) * p.H, 0, 1, st);
        }
        return r;
    };
    hipEvent_t *ev = events.ev;   // [0] start, [s] operands of s, [nseg + s] state pass of s, [2 nseg - 1] epilogues
    // segment 0's operands on the caller's stream; the others on the side
    // stream, after it (and so after the caller's earlier work)
    e = launch_prep<Act>(p, records, 0, bound(1), false, stream);
    if (e == hipSuccess) e = hipEventRecord(ev[0], stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, ev[0], 0);
    for (int s = 1; e == hipSuccess && s < nseg; ++s) {
        e = launch_prep<Act>(p, records, bound(s), bound(s + 1), false, side);
        if (e == hipSuccess) e = hipEventRecord(ev[s], side);
    }
    // the state passes in order on the caller's stream, each after its operands
    for (int s = 0; e == hipSuccess && s < nseg; ++s) {
        if (s > 0) e = hipStreamWaitEvent(stream, ev[s], 0);
        if (e == hipSuccess)
            e = launch_state_pass(p, records, obuf, bound(s), s + 1 < nseg ? bound(s + 1) : INT64_MAX, stream);
        if (e == hipSuccess && s + 1 < nseg) e = hipEventRecord(ev[nseg + s], stream);
    }
    // RMSNorm + gate of each finished segment on the side stream while the
    // later state passes run; the last segment's and the window (which the
    // first operand pass has read) on the caller's stream, after them
    for (int s = 0; e == hipSuccess && s + 1 < nseg; ++s) {
        e = hipStreamWaitEvent(side, ev[nseg + s], 0);
        if (e == hipSuccess) e = epilogue(s, side);
    }
    if (e == hipSuccess) e = hipEventRecord(ev[2 * nseg - 1], side);
    if (e == hipSuccess) e = epilogue(nseg - 1, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, ev[2 * nseg - 1], 0);
    if (e == hipSuccess) e = launch_split_window(p, bf16, stream);
    return e;
}

}  // namespace

int64_t prefill_scan_record_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads) {
    return (total_tokens / CC + num_seqs) * num_heads * (int64_t)REC;
}

hipError_t launch_prefill_scan(const Params &p, bool bf16, uint8_t *records, float *obuf, hipStream_t stream,
                               hipStream_t side_stream, const int32_t *cu_host) {
    return bf16 ? launch_scan_as<BF16>(p, true, records, obuf, stream, side_stream, cu_host)
                : launch_scan_as<F32>(p, false, records, obuf, stream, side_stream, cu_host);
}

}  // namespace kda
