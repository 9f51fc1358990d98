// kda_prefill_chunk.hip -- chunkwise KDA prefill on the matrix cores.
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
//
// Arithmetic.  On gfx950 fp32 MFMA holds the SIMD's vector ALU for its whole
// duration, while bf16 MFMA runs beside it at 16x the rate.  Every product
// (P, R, the update, Delta, O, and the partial L and M) therefore runs on bf16
// MFMA with each operand split as x = hi + lo, hi = bf16(x), lo = bf16(x - hi),
// and a b ~ a_hi b_hi + a_hi b_lo + a_lo b_hi: relative error about 2^-16 per
// product, accumulated in fp32, the state itself kept in fp32.
// T = (I + Diag(b) L)^{-1} is solved by forward substitution in fp32.
//
// Exponent ranges: L and M use factors e^{G_t - r} and e^{r - G_s} with r the
// log-decay at the chunk middle, so every factor lies within e^{+-|lb| C / 2};
// with the bounded gate and |lb| <= 7.5 that is at most e^{60}, inside fp32.
// (Products above the diagonal can reach e^{|lb| C}; they are masked by
// selection, never multiplied.)  Other gate forms take the recurrent path.
//
// Layout and schedule.  One 1024-thread workgroup (16 wavefronts, four per
// SIMD) per (sequence, head) at a time, in two roles, each with its own loop over the
// chunks and the same two workgroup barriers per chunk:
//   state wavefronts w = 0..7 own state columns 16 w .. 16 w + 15 as 8 MFMA
//     accumulator tiles (lane l holds S[16 rt + 4 (l / 16) + r][16 w + l % 16]
//     in element r of tile rt) and do the matrix work: P, R, the update, the
//     partial L, M over key channels 16 w .. 16 w + 15, the solve for T and the
//     sum of M (wavefronts 0 and 1), and the RMSNorm epilogue of tokens 2 w,
//     2 w + 1;
//   token wavefronts 8 + u (u = 0..7) do the token-wise work of tokens 2 u,
//     2 u + 1 (conv, SiLU, L2 norm, the split operands) and the decay sums of
//     (channel, quarter) pairs 64 u .. 64 u + 63.
// A wavefront issues vector instructions at no more than about half its
// SIMD's rate, and the step's chains stall it far more often, so each SIMD
// holds four wavefronts: two of each role, whose matrix and vector work
// overlap; and the split keeps each role's registers (the state, the inputs
// loaded ahead) apart, within the 128 that four wavefronts allow.
// Chunk i:
//   half 1: state: P and R of chunk i, RMSNorm and gate of chunk i - 1, the
//           partial L, M of chunk i + 1; token: the split operands of chunk i + 1
//   half 2: state: Delta, O and the state update of chunk i, T and M of chunk
//           i + 1 (wavefronts 0 and 1); token: conv, SiLU, L2 norm and decay of
//           chunk i + 2 from registers loaded a chunk earlier, loads for chunk i + 3
// so that the two longest stretches, the pre-step and the update, share a half
// (the operands, T and M are therefore double-buffered, v and beta triple).
// The state never leaves the accumulators between chunks: it feeds P and R
// as the B operand of 16x16x32 steps directly, by ordering the sum over key
// channels so that step m takes, in lane l, the rows the lane holds of tiles
// 2 m and 2 m + 1; the A operands are stored in LDS in that order.
// Pairs in turn.  Given a pair counter, the grid is one workgroup per compute
// unit and each workgroup takes pairs from the counter until none are left:
// faster compute units (chiplets run at different clocks) take more pairs,
// and a pair's start overlaps the previous one's end, since the token role
// begins the next pair's chunk 0 (its taps, loads and pre-step) while the
// state role finishes the last RMSNorm and stores the state (chunk 0 writes
// none of the LDS that this tail reads).
#include <atomic>

#include "kda_device.hpp"

namespace kda {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CK_THREADS = 1024;   // 16 wavefronts: 8 state, 8 token
constexpr int LR_THREADS = 512;    // the low-rank form's kernel: 8 wavefronts
constexpr int CC = 16;             // tokens per chunk
constexpr int TW = CC / 8;         // tokens per wavefront in the token-wise work
constexpr int RAWR = PAST + TW;    // raw rows behind those tokens
constexpr int KP = DK + 4;         // padded fp32 LDS rows (rows read as float4 hit distinct banks)
constexpr int TP = CC + 4;
constexpr int OPR = 17;            // 16-byte slots per token row of the P / R operands (one pad slot)
constexpr int ER = (CC + 4) / 2;   // u32 per channel row of E (16 tokens as bf16, padded)
constexpr int EIR = CC + 4;        // u32 per channel row of E with hi and lo interleaved (padded)
constexpr int TR = (CC + 4) / 2;   // u32 per row of T and M (bf16, padded)
constexpr int NPART = 8;           // partial L, M over channel eighths
constexpr float CHUNK_MAX_HALF_LOG_DECAY = 60.0f;

struct Split2 {
    uint32_t hi, lo;   // bf16 pairs, first value in the low half
};
__device__ __forceinline__ Split2 split2(float x0, float x1) {
    const f32x2 x = {x0, x1};
    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    const f32x2 r = {x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u)};
    return {hb, __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2))};
}
// The split of values that are not needed afterwards: lo = x - hi as the bf16
// dot product of the packed hi parts with the pair (-1, 0) or (0, -1),
// accumulated onto x itself.  That is one instruction per value in place of a
// shift or mask and a subtraction, and exact: x - hi is representable in fp32
// (checked bit for bit against the subtraction over 2^22 values of every
// exponent, denormals included).  The two pairs come in scalar registers the
// compiler cannot see through: as an immediate it encodes the pair (-1, 0) as
// the inline constant -1.0, which the instruction reads as the fp32 pattern,
// that is as the pair (0, -1).
struct NegOne {
    uint32_t lo, hi;   // (-1, 0) and (0, -1) as bf16 pairs
};
__device__ __forceinline__ NegOne neg_one_pairs() {
    uint32_t a = 0x0000bf80u, b = 0xbf800000u;
    asm volatile("" : "+s"(a), "+s"(b));
    return {a, b};
}
__device__ __forceinline__ Split2 split2_dead(float x0, float x1, NegOne n) {
    const f32x2 x = {x0, x1};
    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    const bf16x2 h = __builtin_bit_cast(bf16x2, hb);
    const f32x2 r = {__builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, n.lo), x0, false),
                     __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, n.hi), x1, false)};
    return {hb, __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2))};
}
// c + a b with both operands split (16x16x32 and 16x16x16 bf16 steps)
__device__ __forceinline__ f32x4 mma32(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
    typedef bf16x8 B8;
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(B8, al), __builtin_bit_cast(B8, bh), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(B8, ah), __builtin_bit_cast(B8, bl), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(B8, ah), __builtin_bit_cast(B8, bh), c, 0, 0, 0);
}
// A split product over K = 16 (lane group g: k = 4 g .. 4 g + 3) in two
// steps: the cross terms a_lo b_hi + a_hi b_lo as one 16x16x32 step (each lane
// pairs its a_lo, a_hi with b_hi, b_lo of the same four k), and a_hi b_hi as a
// 16x16x16 step.  Both forms take the same time on gfx950, so this is two
// steps' time where three 16x16x16 steps would be three.
// A 16x16x16 step must not take a 16x16x32 step's result as its accumulator
// straight after it: the compiler puts no wait states between the two, and the
// second step then reads the accumulator from before the first (measured).
// Callers therefore either add the two results with vector instructions or
// keep other matrix steps between the two.
__device__ __forceinline__ f32x4 mma_cross(u32x2 ah, u32x2 al, u32x2 bh, u32x2 bl, f32x4 c) {
    typedef bf16x8 B8;
    const u32x4 a = {al.x, al.y, ah.x, ah.y}, b = {bh.x, bh.y, bl.x, bl.y};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(B8, a), __builtin_bit_cast(B8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_hihi(u32x2 ah, u32x2 bh, f32x4 c) {
    typedef bf16x4 B4;
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(B4, ah), __builtin_bit_cast(B4, bh), c, 0, 0, 0);
}
// The same cross-term step with a given as {a_lo, a_hi} in one 16-byte group,
// as the interleaved E rows hold it (the group goes to the matrix core as
// read, with no register moves to assemble it)
__device__ __forceinline__ f32x4 mma_cross_packed(u32x4 a, u32x2 bh, u32x2 bl, f32x4 c) {
    typedef bf16x8 B8;
    const u32x4 b = {bh.x, bh.y, bl.x, bl.y};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(B8, a), __builtin_bit_cast(B8, b), c, 0, 0, 0);
}
// c + a b with both operands split, over K = 16 as three 16x16x16 steps (the
// low-rank form's kernel)
__device__ __forceinline__ f32x4 mma16(u32x2 ah, u32x2 al, u32x2 bh, u32x2 bl, f32x4 c) {
    typedef bf16x4 B4;
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(B4, al), __builtin_bit_cast(B4, bh), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(B4, ah), __builtin_bit_cast(B4, bl), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(B4, ah), __builtin_bit_cast(B4, bh), c, 0, 0, 0);
}
// the four rows 4 g + r of an accumulator tile as the split B operand of a 16x16x16 step
__device__ __forceinline__ void split4(f32x4 d, u32x2 &h, u32x2 &l) {
    const Split2 a = split2(d[0], d[1]), b = split2(d[2], d[3]);
    h = u32x2{a.hi, b.hi};
    l = u32x2{a.lo, b.lo};
}
// (the same for a tile not needed afterwards)
__device__ __forceinline__ void split4_dead(f32x4 d, u32x2 &h, u32x2 &l, NegOne n) {
    const Split2 a = split2_dead(d[0], d[1], n), b = split2_dead(d[2], d[3], n);
    h = u32x2{a.hi, b.hi};
    l = u32x2{a.lo, b.lo};
}

__device__ __forceinline__ float cconv4(float4 w, float a, float b, float c, float x) {
    return w.x * a + w.y * b + w.z * c + w.w * x;
}
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float2 ld2(const float *p) { return *reinterpret_cast<const float2 *>(p); }
__device__ __forceinline__ void st4(float *p, float4 x) { *reinterpret_cast<float4 *>(p) = x; }

// G_t - r, the log-decay of a token of quarter tq relative to the chunk
// middle, from the sums that start as close to the token as possible: the
// token's own sum from its quarter's start (g), minus quarter 0 (c0) and the
// part of quarter 1 up to token 7 (g7) for quarter 0, minus g7 for quarter 1,
// plus quarter 2 (c2) for quarter 3.  The terms are chosen by coefficients 0
// or 1 per lane rather than by branches (x - 1 y and x + 0 y round exactly as
// x - y and x).
struct MidCoef {
    float a0, a1, a3;
};
// (formed anew at each use from an opaque copy of the lane's token, rather
// than kept in registers across a chunk loop)
__device__ __forceinline__ MidCoef mid_coef(int t) {
    asm volatile("" : "+v"(t));
    const int tq = t >> 2;
    return {tq == 0 ? 1.f : 0.f, tq <= 1 ? 1.f : 0.f, tq == 3 ? 1.f : 0.f};
}
__device__ __forceinline__ float rel_mid(MidCoef m, float g, float c0, float g7, float c2) {
    return fmaf(m.a3, c2, fmaf(-m.a1, g7, fmaf(-m.a0, c0, g)));
}

// the lane index, formed where it is used (from the lane count) and opaque to
// the compiler, so that addresses derived from it are not hoisted out of a
// chunk loop and kept (or spilled) for the workgroup's life
__device__ __forceinline__ int opaque_lane() {
    int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    return l;
}

// 1/sqrt(x) by the hardware instruction, without the scaling the library adds
// for denormal arguments: the same result for every x from the smallest normal
// float up (x is a sum of squares plus eps here, so only an eps below that
// bound, with an all but zero vector, can reach the difference)
__device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// The sums over the 64 lanes of two values at once, in every lane: the two
// share the cross-row lane swaps.  After the sums within rows of 16 lanes, the
// first swap and add leave a's pair sums (rows 0 + 1, 2 + 3) in rows 0 and 2
// and b's in rows 1 and 3; the second, a's total in rows 0 and 2 and b's in
// rows 1 and 3; the third hands every row both (each total is formed once, in
// one order, so all lanes hold the same bits).
__device__ __forceinline__ void sum64x2(float &a, float &b) {
    a = sum16(a);
    b = sum16(b);
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const float c = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    s = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(c), false, false);
    const float e = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    s = __builtin_amdgcn_permlane16_swap(__float_as_uint(e), __float_as_uint(e), false, false);
    a = __uint_as_float(s[0]);
    b = __uint_as_float(s[1]);
}

// LDS writes of this wavefront visible to its other lanes (no other wavefront)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <typename Act>
__global__ __launch_bounds__(CK_THREADS) void prefill_chunk_kernel(Params p) {
    typedef BufAct<Act> BA;
    typedef typename BA::Raw2 Raw2;
    // the (sequence, head) pair in hand: ticket tk of the scheduling order is
    // head tk % H of the sequence in slot tk / H.  Workgroup b starts with
    // ticket b; with a pair counter (p.tickets) it asks the counter for its
    // next ticket while it works on a pair (tickets past the grid's own, in
    // the order workgroups ask), so that compute units that run faster take
    // more of the pairs
    const int64_t tickets_total = (int64_t)p.num_seqs * p.H;
    int64_t tk = blockIdx.x;
    int h, n;
    Range rng;
    int64_t L, NC, unit;
    auto take = [&](int64_t t, int nn, Range r) {
        tk = t;
        h = (int)(t % p.H);
        n = nn;
        rng = r;
        L = r.len;
        NC = (L + CC - 1) / CC;
        unit = (int64_t)n * p.H + h;
    };
    {
        const int slot = (int)(tk / p.H);
        const int nn = p.seq_order ? p.seq_order[slot] : slot;
        const bool ok = nn >= 0 && nn < p.num_seqs;   // entries out of range are skipped
        take(tk, ok ? nn : 0, ok ? seq_range(p, nn) : Range{0, 0});
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // in a scalar register
    const int n16 = lane & 15, g4 = lane >> 4;
    const bool state_wave = wave < 8;               // the role (wavefront-uniform)
    const NegOne neg1 = neg_one_pairs();
    const int rw = wave & 7;                        // wavefront index within the role
    const int rtid = tid & (CK_THREADS / 2 - 1);    // thread index within the role
    const int t0 = TW * rw;                         // tokens of this wavefront's token-wise work
    const int64_t rowsz = (int64_t)p.H * DK;       // elements per token row of q, k, v, f, g, y

    __shared__ float s_kh[CC][KP];         // k_hat of the chunk being prepared
    __shared__ float s_qh[CC][KP];         // q_hat of the chunk being prepared
    // (the log-decay sums in base 2: log2(alpha) = log2(e) gk, so that each
    // factor e^{G...} below is one exp2)
    __shared__ float s_Gq[CC][KP];         // log2-decay summed from the start of the token's quarter
    __shared__ float s_Gt[4][DK];          // log2-decay summed over each quarter
    __shared__ float s_v[3][CC][DV + 4];   // activated v            (by chunk index mod 3)
    __shared__ float s_beta[3][CC];        //                        (by chunk index mod 3)
    // split bf16 operands e^G . k_hat, e^G . q_hat of P and R: slot (t, m, g)
    // holds channels 32 m + 4 g + {0..3} and 32 m + 16 + 4 g + {0..3} of token t
    // (by chunk parity)
    // (one array: k hi, k lo, q hi, q lo by the second index, so that a lane's
    // 16 reads of them per chunk share one address register)
    __shared__ __attribute__((aligned(16))) uint32_t s_pr[2][4][CC * OPR * 4];
    // [channel][token] split e^{G_C - G} . k_hat of the update (by chunk parity):
    // for tokens 4 g .. 4 g + 3, u32 4 g and 4 g + 1 hold the lo parts and
    // 4 g + 2 and 4 g + 3 the hi parts, so that one 16-byte read is the A
    // operand of a cross-term step as it stands
    __shared__ __attribute__((aligned(16))) uint32_t s_E[2][DK][EIR];
    __shared__ float s_gC[2][DK];          // e^{G_C}, decay of the whole chunk (by chunk parity)
    __shared__ float s_Lp[NPART][CC][CC];  // L, M summed over one channel eighth each
    __shared__ float s_Mp[NPART][CC][CC];
    __shared__ float s_A[CC][TP];          // Diag(b) L, strictly lower
    // (I + Diag(b) L)^{-1} and M (lower triangle with the diagonal), [row][column]
    // split bf16 (by chunk parity)
    // (one array: T hi, T lo, M hi, M lo by the second index)
    __shared__ __attribute__((aligned(16))) uint32_t s_tm[2][4][CC][TR];
    __shared__ float s_o[CC][DV + 4];      // readout of the chunk, before RMSNorm
    __shared__ long long s_nx[4];          // the next pair: ticket, sequence, first token, length

    // the next pair as published in s_nx (false: no pairs left)
    auto next_pair = [&]() -> bool {
        long long v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const long long x = s_nx[i];
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)x >> 32));
            v[i] = (long long)(((unsigned long long)hi << 32) | lo);
        }
        if (v[0] >= tickets_total) return false;
        take(v[0], (int)v[1], Range{v[2], v[3]});
        return true;
    };

    auto tok_rsrc = [&](const void *t, uint32_t elem, int64_t base, int64_t end) -> Rsrc {
        return make_rsrc(static_cast<const char *>(t) + (rng.lo + base) * rowsz * elem,
                         (uint32_t)((end - base) * rowsz * elem));
    };
    auto chunk_end = [&](int64_t c0) -> int64_t { return (c0 + CC < L) ? c0 + CC : L; };
    // lane: conv channels chq, chq + 1 of q, k, v; value (and output) channels chq, chq + 1
    const int chq = 2 * lane, chk = DK + 2 * lane, chv = 2 * DK + 2 * lane;

    // =========================================================== state role
    // T = (I + A)^{-1}, A = Diag(b) L strictly lower, by forward substitution
    // in blocks of 4 rows on one wavefront: lane (c = l / 4, r = l % 4) builds
    // row 4 b + r of column c in block b, and every lane of a quad keeps the
    // finished part of column c; the rows of a block couple through quad
    // broadcasts.  Masked entries of A are exact zeros.
    auto solve_T = [&](int vb, int tb) {
        {
            const int t = lane >> 2, s0 = 4 * (lane & 3);
            float4 a = ld4(&s_Lp[0][t][s0]);
#pragma unroll
            for (int q = 1; q < NPART; ++q) a += ld4(&s_Lp[q][t][s0]);
            const float bt = s_beta[vb][t];
            a.x = (s0 + 0 < t) ? bt * a.x : 0.f;
            a.y = (s0 + 1 < t) ? bt * a.y : 0.f;
            a.z = (s0 + 2 < t) ? bt * a.z : 0.f;
            a.w = (s0 + 3 < t) ? bt * a.w : 0.f;
            st4(&s_A[t][s0], a);
        }
        wave_lds_sync();
        const int c = lane >> 2, r = lane & 3;
        float Tc[CC];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int t = 4 * b + r;
            // y = e_c(t) - sum over the finished rows s < 4 b of A[t][s] T[s][c]
            float acc[4] = {(t == c) ? 1.0f : 0.0f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < b; ++s4) {
                const float4 a = ld4(&s_A[t][4 * s4]);
                acc[0] = fmaf(-a.x, Tc[4 * s4 + 0], acc[0]);
                acc[1] = fmaf(-a.y, Tc[4 * s4 + 1], acc[1]);
                acc[2] = fmaf(-a.z, Tc[4 * s4 + 2], acc[2]);
                acc[3] = fmaf(-a.w, Tc[4 * s4 + 3], acc[3]);
            }
            float y = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            // inside the block: row r subtracts A[t][4 b + r'] times finished row r' < r
            const float4 ab = ld4(&s_A[t][4 * b]);
            const float x0 = dpp<0x00>(y);
            y = fmaf(-ab.x, x0, y);
            const float x1 = dpp<0x55>(y);
            y = fmaf(-ab.y, x1, y);
            const float x2 = dpp<0xAA>(y);
            y = fmaf(-ab.z, x2, y);
            const float x3 = dpp<0xFF>(y);
            Tc[4 * b + 0] = x0;
            Tc[4 * b + 1] = x1;
            Tc[4 * b + 2] = x2;
            Tc[4 * b + 3] = x3;
            const Split2 x = split2(y, 0.f);
            reinterpret_cast<uint16_t *>(s_tm[tb][0][t])[c] = (uint16_t)x.hi;
            reinterpret_cast<uint16_t *>(s_tm[tb][1][t])[c] = (uint16_t)x.lo;
        }
    };
    auto reduce_M = [&](int tb) {
        const int l = opaque_lane();
        const int t = l >> 2, s0 = 4 * (l & 3);
        float4 m = ld4(&s_Mp[0][t][s0]);
#pragma unroll
        for (int q = 1; q < NPART; ++q) m += ld4(&s_Mp[q][t][s0]);
        m.x = (s0 + 0 <= t) ? m.x : 0.f;
        m.y = (s0 + 1 <= t) ? m.y : 0.f;
        m.z = (s0 + 2 <= t) ? m.z : 0.f;
        m.w = (s0 + 3 <= t) ? m.w : 0.f;
        const Split2 a = split2(m.x, m.y), b = split2(m.z, m.w);
        *reinterpret_cast<u32x2 *>(&s_tm[tb][2][t][s0 / 2]) = u32x2{a.hi, b.hi};
        *reinterpret_cast<u32x2 *>(&s_tm[tb][3][t][s0 / 2]) = u32x2{a.lo, b.lo};
    };

    // L_ts = sum_i (e^{G_ti - r_i} k_ti)(e^{r_i - G_si} k_si), M likewise with q_t,
    // over channel eighth rw of the prepared chunk (partial sums), r = G at the
    // chunk middle (token 7), as split bf16 products; lane l: token l % 16,
    // channels 16 rw + 4 (l / 16) + s
    auto partial_LM = [&]() {
        const int lc = 16 * rw + 4 * g4;
        const float4 k4 = ld4(&s_kh[n16][lc]);
        const float4 q4 = ld4(&s_qh[n16][lc]);
        const float4 gq = ld4(&s_Gq[n16][lc]);
        const float4 g7 = ld4(&s_Gq[CC / 2 - 1][lc]);   // quarter 1 up to token 7
        const float4 c0 = ld4(&s_Gt[0][lc]);
        const float4 c2 = ld4(&s_Gt[2][lc]);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
        const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
        const float gv[4] = {gq.x, gq.y, gq.z, gq.w};
        const float g7v[4] = {g7.x, g7.y, g7.z, g7.w};
        const float c0v[4] = {c0.x, c0.y, c0.z, c0.w};
        const float c2v[4] = {c2.x, c2.y, c2.z, c2.w};
        const MidCoef mc = mid_coef(n16);
        float fl[4], fm[4], fb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float d = rel_mid(mc, gv[s], c0v[s], g7v[s], c2v[s]);
            const float ef = __builtin_amdgcn_exp2f(d), eb = __builtin_amdgcn_exp2f(-d);
            fl[s] = ef * kv[s];
            fm[s] = ef * qv[s];
            fb[s] = eb * kv[s];
        }
        // one K = 16 step covers the lane's four channels s: the factors split
        // into bf16 parts, three 16x16x16 steps per product (the same form
        // throughout, so no step reads another form's result)
        const Split2 l0 = split2_dead(fl[0], fl[1], neg1), l1 = split2_dead(fl[2], fl[3], neg1);
        const Split2 m0 = split2_dead(fm[0], fm[1], neg1), m1 = split2_dead(fm[2], fm[3], neg1);
        const Split2 b0 = split2_dead(fb[0], fb[1], neg1), b1 = split2_dead(fb[2], fb[3], neg1);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const u32x2 bh = {b0.hi, b1.hi}, bl = {b0.lo, b1.lo};
        const f32x4 Lt = mma16(u32x2{l0.hi, l1.hi}, u32x2{l0.lo, l1.lo}, bh, bl, zero);
        const f32x4 Mt = mma16(u32x2{m0.hi, m1.hi}, u32x2{m0.lo, m1.lo}, bh, bl, zero);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s_Lp[rw][4 * g4 + r][n16] = Lt[r];
            s_Mp[rw][4 * g4 + r][n16] = Mt[r];
        }
    };

    if (state_wave) {
        const int col0 = 16 * rw;
        const float2 gm = ld2(p.gamma + 2 * lane);
        Raw2 rg[TW];                               // gate rows of the chunk whose epilogue comes next
        auto issue_gate = [&](int64_t c0) {
            const Rsrc ag = tok_rsrc(p.g, BA::ELEM, c0, chunk_end(c0));
#pragma unroll
            for (int sl = 0; sl < TW; ++sl)
                rg[sl] = BA::load_raw2(ag, (uint32_t)((t0 + sl) * rowsz + h * DV + 2 * lane));
        };
        // RMSNorm + gate of tokens t0, t0 + 1 of the chunk at c0 (readout in s_o,
        // gates in rg); the output buffers end at the sequence end, so stores of
        // tokens past it are dropped (no branch: the tokens' chains interleave)
        auto epilogue = [&](int64_t c0) {
            const int nve = (int)(L - c0 < CC ? L - c0 : CC);
            const Rsrc ay = tok_rsrc(p.y, BA::ELEM, c0, c0 + nve);
            const Rsrc ao = tok_rsrc(p.o_raw, 4, c0, c0 + nve);
            static_assert(TW == 2, "two tokens a wavefront: their sums share the lane swaps");
            const float2 o0 = ld2(&s_o[t0][chq]), o1 = ld2(&s_o[t0 + 1][chq]);
            float ss[TW] = {o0.x * o0.x + o0.y * o0.y, o1.x * o1.x + o1.y * o1.y};
            sum64x2(ss[0], ss[1]);
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                const int t = t0 + sl;
                const float2 o = sl == 0 ? o0 : o1;
                const float r = rsq(ss[sl] * (1.0f / DV) + p.rms_eps);
                const uint32_t e = (uint32_t)(t * rowsz + h * DV + chq);
                const float2 gg = BA::unpack2(rg[sl]);
                float2 y;
                y.x = sigmoid(gg.x) * gm.x * o.x * r;
                y.y = sigmoid(gg.y) * gm.y * o.y * r;
                BA::store2(ay, e, y);
                if (p.o_raw) bst_f32x2(ao, o, e * 4);
            }
        };

        // the state in the accumulator tiles (lane offset: row 4 g4 + r, column
        // col0 + n16; row tile rt as the scalar offset)
        f32x4 st[8];
        // lane 0 of wavefront 2 asks the counter for the next ticket at the
        // start of a pair, looks up its sequence after the first barrier and
        // publishes it with the sequence's token range before the third (the
        // others read s_nx after the pair, before their next barrier)
        const bool asker = p.tickets && rw == 2 && lane == 0;
        int32_t nx_a = 0, nx_n = -1;
        auto ask = [&]() { nx_a = __hip_atomic_fetch_add(p.tickets, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        auto look_up = [&]() {
            const int64_t t = (int64_t)gridDim.x + nx_a;
            const int slot = (int)(t / p.H);
            nx_n = t >= tickets_total ? -1 : (p.seq_order ? p.seq_order[slot] : slot);
        };
        auto publish = [&]() {
            const int64_t t = (int64_t)gridDim.x + nx_a;
            const bool ok = t < tickets_total && nx_n >= 0 && nx_n < p.num_seqs;
            const Range r = ok ? seq_range(p, nx_n) : Range{0, 0};
            s_nx[0] = t;
            s_nx[1] = ok ? nx_n : 0;
            s_nx[2] = r.lo;
            s_nx[3] = r.len;
        };

        f32x4 Pt, Rt;
        // P, R of the current chunk: step m covers state rows 32 m .. 32 m + 31
        // (tiles 2 m, 2 m + 1)
        auto products_PR = [&](int pb) {
            Pt = f32x4{0.f, 0.f, 0.f, 0.f};
            Rt = Pt;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int w = (n16 * OPR + m * 4 + g4) * 4;
                const u32x4 kah = *reinterpret_cast<const u32x4 *>(&s_pr[pb][0][w]);
                const u32x4 kal = *reinterpret_cast<const u32x4 *>(&s_pr[pb][1][w]);
                const u32x4 qah = *reinterpret_cast<const u32x4 *>(&s_pr[pb][2][w]);
                const u32x4 qal = *reinterpret_cast<const u32x4 *>(&s_pr[pb][3][w]);
                const Split2 x0 = split2(st[2 * m][0], st[2 * m][1]);
                const Split2 x1 = split2(st[2 * m][2], st[2 * m][3]);
                const Split2 x2 = split2(st[2 * m + 1][0], st[2 * m + 1][1]);
                const Split2 x3 = split2(st[2 * m + 1][2], st[2 * m + 1][3]);
                const u32x4 sh = {x0.hi, x1.hi, x2.hi, x3.hi}, sl = {x0.lo, x1.lo, x2.lo, x3.lo};
                Pt = mma32(kah, kal, sh, sl, Pt);
                Rt = mma32(qah, qal, sh, sl, Rt);
            }
        };
        // Delta, O and the state update of the current chunk
        auto update = [&](int vb, int cur) {
            // W = Diag(b) (V - P) (rows 4 g4 + r); Delta = T W; O = R + M Delta
            f32x4 Wt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                Wt[r] = s_beta[vb][t] * (s_v[vb][t][col0 + n16] - Pt[r]);
            }
            const u32x2 th = *reinterpret_cast<const u32x2 *>(&s_tm[cur][0][n16][2 * g4]);
            const u32x2 tl = *reinterpret_cast<const u32x2 *>(&s_tm[cur][1][n16][2 * g4]);
            const u32x2 mh = *reinterpret_cast<const u32x2 *>(&s_tm[cur][2][n16][2 * g4]);
            const u32x2 ml = *reinterpret_cast<const u32x2 *>(&s_tm[cur][3][n16][2 * g4]);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            u32x2 wh, wl, dh, dl;
            split4_dead(Wt, wh, wl, neg1);
            const f32x4 Dt = mma_cross(th, tl, wh, wl, zero) + mma_hihi(th, wh, zero);
            split4_dead(Dt, dh, dl, neg1);
            const f32x4 Ot = mma_cross(mh, ml, dh, dl, Rt) + mma_hihi(mh, dh, zero);
#pragma unroll
            for (int r = 0; r < 4; ++r) s_o[4 * g4 + r][col0 + n16] = Ot[r];
            // S <- Diag(e^{G_C}) S + E^T Delta: the cross-term steps of all
            // eight tiles, then their hi * hi steps (the empty asm keeps that
            // order, so seven steps separate each pair)
            u32x2 eh[8];
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const float4 dc = ld4(&s_gC[cur][16 * rt + 4 * g4]);
                const u32x4 e = *reinterpret_cast<const u32x4 *>(&s_E[cur][16 * rt + n16][4 * g4]);
                eh[rt] = u32x2{e.z, e.w};
                st[rt][0] *= dc.x;
                st[rt][1] *= dc.y;
                st[rt][2] *= dc.z;
                st[rt][3] *= dc.w;
                st[rt] = mma_cross_packed(e, dh, dl, st[rt]);
            }
            asm volatile("" : "+v"(st[0]), "+v"(st[1]), "+v"(st[2]), "+v"(st[3]),
                              "+v"(st[4]), "+v"(st[5]), "+v"(st[6]), "+v"(st[7]));
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) st[rt] = mma_hihi(eh[rt], dh, st[rt]);
        };

#pragma unroll 1
        for (;;) {
        if (L > 0) {
        const Rsrc rs_state = make_rsrc(p.state + unit * (DK * DV), DK * DV * 4);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st[rt][r] = bld_f32(rs_state, ((4 * g4 + r) * DV + col0 + n16) * 4, rt * 16 * DV * 4);
        if (asker) ask();
        __syncthreads();                           // chunk 0 prepared
        partial_LM();                              // L, M of chunk 0
        if (asker) look_up();
        __syncthreads();                           // chunk 0's operands, L and M
        if (rw == 0) solve_T(0, 0);
        else if (rw == 1) reduce_M(0);
        else if (asker) publish();
        __syncthreads();                           // T, M of chunk 0; chunk 1 prepared

        int vb = 0;                                // chunk i's index mod 3
#pragma unroll 1
        for (int64_t i = 0; i < NC; ++i) {
            const int cur = (int)(i & 1);
            const int vb1 = vb == 2 ? 0 : vb + 1;
            // ================= half 1: P, R of chunk i; epilogue of chunk i - 1;
            // partial L, M of chunk i + 1
            products_PR(cur);
            if (i >= 1) epilogue((i - 1) * CC);
            issue_gate(i * CC);
            if (i + 1 < NC) partial_LM();
            __syncthreads();
            // ================= half 2: update of chunk i; T and M of chunk i + 1
            update(vb, cur);
            if (i + 1 < NC) {
                if (rw == 0) solve_T(vb1, cur ^ 1);
                else if (rw == 1) reduce_M(cur ^ 1);
            }
            __syncthreads();
            vb = vb1;
        }
        epilogue((NC - 1) * CC);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                bst_f32(rs_state, st[rt][r], ((4 * g4 + r) * DV + col0 + n16) * 4, rt * 16 * DV * 4);
        } else if (p.tickets) {
            // an empty pair: its successor is asked for at once
            __syncthreads();                       // s_nx read by all
            if (asker) {
                ask();
                look_up();
                publish();
            }
            __syncthreads();                       // s_nx written
        }
        if (!p.tickets || !next_pair()) return;
        }
    }

    // =========================================================== token role
    // decay: key channel dch over the tokens of quarter dq
    const int dch = rtid & (DK - 1);
    const int dq = rtid >> 7;
    uint32_t foff;
    // sigmoid(exp(A_log) (f + dt_bias)) = 1 / (1 + 2^(nA f + nAd)), with nA =
    // -log2(e) exp(A_log) and nAd = nA dt_bias formed once a pair
    float nA, nAd;

    // registers loaded a chunk ahead: raw inputs of the next chunk to pre-step
    Raw2 rq[RAWR], rk[RAWR], rv[RAWR];
    auto unpack_q = [&](int r) { return BA::unpack2(rq[r]); };
    auto unpack_k = [&](int r) { return BA::unpack2(rk[r]); };
    auto unpack_v = [&](int r) { return BA::unpack2(rv[r]); };
    // conv taps of this lane's channels, kept in registers (their LDS reads
    // would queue behind the state wavefronts' operand reads every chunk)
    float4 wq0, wq1, wk0, wk1, wv0, wv1;
    constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
    const float l2_eps2 = p.l2_eps * (LOG2E * LOG2E);   // eps for the activations times log2(e)
    const float lb2 = p.lb * LOG2E;                     // the decay's bound in base 2
    float rf[4], rb;

    // loads of a chunk at c0 >= CC (its past rows are tokens, not the window);
    // rows past the sequence end read as 0
    auto issue_inputs = [&](int64_t c0) {
        const int64_t base = c0 - PAST, end = chunk_end(c0);
        const Rsrc aq = tok_rsrc(p.q, BA::ELEM, base, end);
        const Rsrc ak = tok_rsrc(p.k, BA::ELEM, base, end);
        const Rsrc av = tok_rsrc(p.v, BA::ELEM, base, end);
#pragma unroll
        for (int r = 0; r < RAWR; ++r) {
            const uint32_t e = (uint32_t)((t0 + r) * rowsz + h * DK + 2 * lane);
            rq[r] = BA::load_raw2(aq, e);
            rk[r] = BA::load_raw2(ak, e);
            rv[r] = BA::load_raw2(av, e);
        }
        {
            const Rsrc af = tok_rsrc(p.f, 4, c0, end);
#pragma unroll
            for (int u = 0; u < 4; ++u) rf[u] = bld_f32(af, foff, (uint32_t)(u * rowsz * 4));
        }
        const Rsrc ab = make_rsrc(p.beta + (rng.lo + c0) * p.H, (uint32_t)((end - c0) * p.H * 4));
        rb = bld_f32(ab, (uint32_t)(((t0 + (lane & (TW - 1))) * p.H + h) * 4));
    };

    // conv + SiLU + L2 norm of this wavefront's tokens of the chunk at c0 (zeros
    // past the end), decay sums of (dch, quarter dq); v, beta to buffer vb
    // (gq, gk, gv: row r of the raw window behind the tokens, as float2)
    auto prestep = [&](auto gq, auto gk, auto gv, int64_t c0, int vb) {
        const int nv = (int)(L - c0 < CC ? L - c0 : CC);
        // conv + SiLU of one of q, k, v for this wavefront's two tokens, times
        // log2(e): the taps in registers carry that factor, so that
        // e^{-conv} is one exp2 of the scaled sum (the factor drops out of
        // the L2 norms of q and k with eps scaled by log2(e)^2, and v is
        // scaled back)
        auto silu2 = [](float y) { return y * fast_rcp(1.0f + __builtin_amdgcn_exp2f(-y)); };
        auto act = [&](auto g, const float4 &w0, const float4 &w1, float (&a)[TW][2]) {
            float2 x[RAWR];
#pragma unroll
            for (int r = 0; r < RAWR; ++r) x[r] = g(r);
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                a[sl][0] = silu2(cconv4(w0, x[sl].x, x[sl + 1].x, x[sl + 2].x, x[sl + 3].x));
                a[sl][1] = silu2(cconv4(w1, x[sl].y, x[sl + 1].y, x[sl + 2].y, x[sl + 3].y));
            }
        };
        float aq[TW][2], ak[TW][2], av[TW][2];
        act(gq, wq0, wq1, aq);
        act(gk, wk0, wk1, ak);
        act(gv, wv0, wv1, av);
        // the L2 norms and the stores; a token past the end is computed and
        // then replaced by zeros, and the decay sum held constant past the last
        // token (only in a chunk the sequence ends inside: the condition is
        // wavefront-uniform, so a full chunk takes the branch without selects)
        auto finish = [&](auto masked) {
            // squared norms of q and k of the two tokens (pairs share lane swaps)
            float sq[TW], sk[TW];
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                sq[sl] = aq[sl][0] * aq[sl][0] + aq[sl][1] * aq[sl][1];
                sk[sl] = ak[sl][0] * ak[sl][0] + ak[sl][1] * ak[sl][1];
            }
            sum64x2(sq[0], sk[0]);
            sum64x2(sq[1], sk[1]);
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                // (no branch on the token: the two tokens' chains interleave)
                const int t = t0 + sl;
                const float nq = rsq(sq[sl] + l2_eps2);
                const float nk = rsq(sk[sl] + l2_eps2);
                float2 qh = make_float2(aq[sl][0] * nq, aq[sl][1] * nq);
                float2 kh = make_float2(ak[sl][0] * nk, ak[sl][1] * nk);
                float2 vh = make_float2(av[sl][0] * LN2, av[sl][1] * LN2);
                if (masked && t >= nv) qh = kh = vh = make_float2(0.f, 0.f);
                *reinterpret_cast<float2 *>(&s_qh[t][chq]) = qh;
                *reinterpret_cast<float2 *>(&s_kh[t][chq]) = kh;
                *reinterpret_cast<float2 *>(&s_v[vb][t][chq]) = vh;
            }
            if (lane < TW) s_beta[vb][t0 + lane] = (!masked || t0 + lane < nv) ? rb : 0.f;
            float G = 0.f;
            const int rem = nv - 4 * dq;           // tokens of quarter dq within the sequence
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float gk = lb2 * fast_rcp(1.0f + __builtin_amdgcn_exp2f(fmaf(nA, rf[u], nAd)));
                G += (!masked || u < rem) ? gk : 0.f;
                s_Gq[4 * dq + u][dch] = G;
            }
            s_Gt[dq][dch] = G;
        };
        if (nv == CC)
            finish(false);
        else
            finish(true);
    };

    // split operands of the prepared chunk (into buffer buf)
    auto operands = [&](int buf) {
        {
            // lane: channels chq, chq + 1 of this wavefront's tokens (quarter rw / 2)
            const int qt = t0 >> 2;
            const float2 gt0 = ld2(&s_Gt[0][chq]), gt1 = ld2(&s_Gt[1][chq]);
            const float2 gt2 = ld2(&s_Gt[2][chq]), gt3 = ld2(&s_Gt[3][chq]);
            // sums of the quarters before and after this one (qt is
            // wavefront-uniform: one scalar branch, no per-lane selects)
            float2 before, after;
            switch (qt) {
            case 0:
                before = make_float2(0.f, 0.f);
                after = make_float2((gt1.x + gt2.x) + gt3.x, (gt1.y + gt2.y) + gt3.y);
                break;
            case 1:
                before = gt0;
                after = make_float2(gt2.x + gt3.x, gt2.y + gt3.y);
                break;
            case 2:
                before = make_float2(gt0.x + gt1.x, gt0.y + gt1.y);
                after = gt3;
                break;
            default:
                before = make_float2((gt0.x + gt1.x) + gt2.x, (gt0.y + gt1.y) + gt2.y);
                after = make_float2(0.f, 0.f);
                break;
            }
            const float2 gq_end = ld2(&s_Gt[qt][chq]);
            const int m = chq >> 5, gg = (chq & 15) >> 2, e = ((chq & 31) >> 4) * 4 + (chq & 3);
            float E0[TW], E1[TW];
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                const int t = t0 + sl;
                const float2 gq = ld2(&s_Gq[t][chq]);
                const float2 kh = ld2(&s_kh[t][chq]);
                const float2 qh = ld2(&s_qh[t][chq]);
                const float eg0 = __builtin_amdgcn_exp2f(before.x + gq.x), eg1 = __builtin_amdgcn_exp2f(before.y + gq.y);
                const Split2 ka = split2_dead(eg0 * kh.x, eg1 * kh.y, neg1);
                const Split2 qa = split2_dead(eg0 * qh.x, eg1 * qh.y, neg1);
                const int w = (t * OPR + m * 4 + gg) * 4 + e / 2;
                s_pr[buf][0][w] = ka.hi; s_pr[buf][1][w] = ka.lo;
                s_pr[buf][2][w] = qa.hi; s_pr[buf][3][w] = qa.lo;
                // G_C - G_t = (rest of this quarter) + (later quarters)
                E0[sl] = __builtin_amdgcn_exp2f(gq_end.x - gq.x + after.x) * kh.x;
                E1[sl] = __builtin_amdgcn_exp2f(gq_end.y - gq.y + after.y) * kh.y;
            }
            const Split2 a0 = split2_dead(E0[0], E0[1], neg1), a1 = split2_dead(E1[0], E1[1], neg1);
            const int eo = 4 * (rw >> 1) + (rw & 1);   // tokens t0, t0 + 1 in their group of four
            s_E[buf][chq][eo] = a0.lo;
            s_E[buf][chq][eo + 2] = a0.hi;
            s_E[buf][chq + 1][eo] = a1.lo;
            s_E[buf][chq + 1][eo + 2] = a1.hi;
            if (rw == 0) {
                const float gc0 = gt0.x + gt1.x + gt2.x + gt3.x, gc1 = gt0.y + gt1.y + gt2.y + gt3.y;
                *reinterpret_cast<float2 *>(&s_gC[buf][chq]) =
                    make_float2(__builtin_amdgcn_exp2f(gc0), __builtin_amdgcn_exp2f(gc1));
            }
        }
    };

#pragma unroll 1
    for (;;) {
    if (L > 0) {
    // this head's taps times log2(e) (see the pre-step) and decay constants
    {
        const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);
        wq0 = ld4(cw + chq * TAPS) * LOG2E; wq1 = ld4(cw + (chq + 1) * TAPS) * LOG2E;
        wk0 = ld4(cw + chk * TAPS) * LOG2E; wk1 = ld4(cw + (chk + 1) * TAPS) * LOG2E;
        wv0 = ld4(cw + chv * TAPS) * LOG2E; wv1 = ld4(cw + (chv + 1) * TAPS) * LOG2E;
        foff = (uint32_t)((4 * dq * rowsz + h * DK + dch) * 4);
        nA = -1.4426950408889634f * __expf(p.A_log[h * DK + dch]);
        nAd = nA * p.dt_bias[h * DK + dch];
    }
    // ---- chunk 0 (its past rows come from the carried window)
    {
        const int64_t end = chunk_end(0);
        const Rsrc aq = tok_rsrc(p.q, BA::ELEM, 0, end);
        const Rsrc ak = tok_rsrc(p.k, BA::ELEM, 0, end);
        const Rsrc av = tok_rsrc(p.v, BA::ELEM, 0, end);
        const float *W = p.win + unit * (PAST * CH);
        float2 xq[RAWR], xk[RAWR], xv[RAWR];
#pragma unroll
        for (int r = 0; r < RAWR; ++r) {
            const int jj = t0 - PAST + r;
            if (jj < 0) {
                const float *wr = W + (jj + PAST) * CH;
                xq[r] = ld2(wr + chq);
                xk[r] = ld2(wr + chk);
                xv[r] = ld2(wr + chv);
            } else {
                const uint32_t e = (uint32_t)(jj * rowsz + h * DK + 2 * lane);
                xq[r] = BA::load2(aq, e);
                xk[r] = BA::load2(ak, e);
                xv[r] = BA::load2(av, e);
            }
        }
        {
            const Rsrc af = tok_rsrc(p.f, 4, 0, end);
#pragma unroll
            for (int u = 0; u < 4; ++u) rf[u] = bld_f32(af, foff, (uint32_t)(u * rowsz * 4));
        }
        const Rsrc ab = make_rsrc(p.beta + rng.lo * p.H, (uint32_t)(end * p.H * 4));
        rb = bld_f32(ab, (uint32_t)(((t0 + (lane & (TW - 1))) * p.H + h) * 4));
        prestep([&](int r) { return xq[r]; }, [&](int r) { return xk[r]; }, [&](int r) { return xv[r]; }, 0, 0);
        if (NC > 1) issue_inputs(CC);
    }
    __syncthreads();                               // chunk 0 prepared
    operands(0);
    __syncthreads();                               // chunk 0's operands, L and M
    // ---- chunk 1 (its rows were loaded with chunk 0's)
    if (NC > 1) {
        prestep(unpack_q, unpack_k, unpack_v, CC, 1);
        if (NC > 2) issue_inputs(2 * CC);
    }
    __syncthreads();                               // T, M of chunk 0; chunk 1 prepared

    // (the work of chunks past the last is skipped; the branches are uniform)
    int vb = 0;                                    // chunk i's index mod 3
#pragma unroll 1
    for (int64_t i = 0; i < NC; ++i) {
        const int cur = (int)(i & 1);
        const int vb1 = vb == 2 ? 0 : vb + 1, vb2 = vb1 == 2 ? 0 : vb1 + 1;
        // ================= half 1: operands of chunk i + 1
        if (i + 1 < NC) operands(cur ^ 1);
        __syncthreads();
        // ================= half 2: pre-step of chunk i + 2, loads for chunk i + 3
        if (i + 2 < NC) {
            prestep(unpack_q, unpack_k, unpack_v, (i + 2) * CC, vb2);
        }
        if (i + 3 < NC) issue_inputs((i + 3) * CC);
        __syncthreads();
        vb = vb1;
    }
    } else if (p.tickets) {
        __syncthreads();                           // s_nx read by all
        __syncthreads();                           // s_nx written
    }
    if (!p.tickets || !next_pair()) return;
    }
}

// The low-rank decay form (kda_sequence_lowrank) runs on this kernel: one
// role, 8 wavefronts (512 threads), each owning 16 state columns and two tokens
// of the token-wise work, as the 16-wavefront kernel's roles do together.  Its
// W_fb operand (32 registers per lane) does not fit beside either role of the
// 16-wavefront kernel within the 128 registers that four wavefronts per SIMD
// allow.  f = W_fb a for the chunk's 16 tokens is one more split-bf16 product
// per chunk (tokens x the wavefront's 16 key channels, K = rank): W_fb's rows
// for those channels stay in registers as the B operand for the workgroup's
// life, and each chunk's rank-r rows of a pass through LDS as the A operand.
// The accumulator gives lane l the channel 16 w + l % 16 over tokens
// 4 (l / 16) .. + 3, which is the unit the decay sums take, so f never goes
// through memory.
template <typename Act>
__global__ __launch_bounds__(LR_THREADS) void prefill_chunk_lr_kernel(Params p) {
    typedef BufAct<Act> BA;
    typedef typename BA::Raw2 Raw2;
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
    const int64_t NC = (L + CC - 1) / CC;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, g4 = lane >> 4;
    const int64_t unit = (int64_t)n * p.H + h;
    const int64_t rowsz = (int64_t)p.H * DK;       // elements per token row of q, k, v, f, g, y
    const int t0 = TW * wave;                       // this wavefront's tokens in the token-wise work
    const NegOne neg1 = neg_one_pairs();

    __shared__ float s_kh[CC][KP];         // k_hat of the chunk being prepared
    __shared__ float s_qh[CC][KP];         // q_hat of the chunk being prepared
    __shared__ float s_Gq[CC][KP];         // log-decay summed from the start of the token's quarter
    __shared__ float s_Gt[4][DK];          // log-decay summed over each quarter
    __shared__ float s_v[2][CC][DV + 4];   // activated v            (by chunk parity)
    __shared__ float s_beta[2][CC];        //                        (by chunk parity)
    // split bf16 operands e^G . k_hat, e^G . q_hat of P and R: slot (t, m, g)
    // holds channels 32 m + 4 g + {0..3} and 32 m + 16 + 4 g + {0..3} of token t
    __shared__ __attribute__((aligned(16))) uint32_t s_kah[CC * OPR * 4], s_kal[CC * OPR * 4];
    __shared__ __attribute__((aligned(16))) uint32_t s_qah[CC * OPR * 4], s_qal[CC * OPR * 4];
    // [channel][token] split e^{G_C - G} . k_hat of the update (by chunk parity)
    __shared__ __attribute__((aligned(16))) uint32_t s_Eh[2][DK][ER], s_El[2][DK][ER];
    __shared__ float s_gC[2][DK];          // e^{G_C}, decay of the whole chunk (by chunk parity)
    __shared__ float s_Lp[NPART][CC][CC];  // L, M summed over one channel eighth each
    __shared__ float s_Mp[NPART][CC][CC];
    __shared__ float s_A[CC][TP];          // Diag(b) L, strictly lower
    // (I + Diag(b) L)^{-1} and M (lower triangle with the diagonal), [row][column] split bf16
    __shared__ __attribute__((aligned(16))) uint32_t s_Th[CC][TR], s_Tl[CC][TR], s_Mh[CC][TR], s_Ml[CC][TR];
    __shared__ float s_o[CC][DV + 4];      // readout of the chunk, before RMSNorm
    __shared__ float s_cw[CH][TAPS];       // conv taps of this head
    // the chunk's rank-r rows of a split into bf16 parts, [token][k] with k
    // padded, by chunk parity
    constexpr int AKW = (LOWRANK_MAX_RANK + 8) / 2;
    __shared__ __attribute__((aligned(16))) uint32_t s_lah[2][CC][AKW], s_lal[2][CC][AKW];

    {
        const float *cw = p.conv_w + (int64_t)h * (CH * TAPS);
        for (int c = tid; c < CH; c += LR_THREADS) st4(s_cw[c], ld4(cw + c * TAPS));
    }

    auto tok_rsrc = [&](const void *t, uint32_t elem, int64_t base, int64_t end) -> Rsrc {
        return make_rsrc(static_cast<const char *>(t) + (rng.lo + base) * rowsz * elem,
                         (uint32_t)((end - base) * rowsz * elem));
    };
    auto chunk_end = [&](int64_t c0) -> int64_t { return (c0 + CC < L) ? c0 + CC : L; };

    // lane: conv channels chq, chq + 1 of q, k, v and value channels chq, chq + 1;
    // decay: key channel dch over the tokens of quarter dq
    const int chq = 2 * lane, chk = DK + 2 * lane, chv = 2 * DK + 2 * lane;
    // (the lane of the f product's accumulator)
    const int dch = 16 * wave + n16;
    const int dq = g4;
    const float eA = __expf(p.A_log[h * DK + dch]);
    const float dtb = p.dt_bias[h * DK + dch];
    const float2 gm = ld2(p.gamma + 2 * lane);

    // registers loaded a chunk ahead: raw inputs of the next chunk to pre-step,
    // and the gate pre-activations of the chunk whose epilogue comes next
    Raw2 rq[RAWR], rk[RAWR], rv[RAWR], rg[TW];
    float rf[4], rb;

    // W_fb's rows of this wavefront's key channels as split B operands:
    // step m holds k = 32 m + 8 g4 + {0..7} of channel 16 w + n16, zero from
    // the rank on; and the rank-r row piece of one token of a chunk in flight
    // (thread: token tid / 32, k = 4 (tid % 32) .. + 3)
    u32x4 wfh[4], wfl[4];
    float4 ra = make_float4(0.f, 0.f, 0.f, 0.f);
    const int la_t = tid >> 5, la_k = 4 * (tid & 31);
    {
        const float *wr = p.lr_wfb + ((int64_t)h * DK + 16 * wave + n16) * p.lr_rank;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int k0 = 32 * m + 8 * g4;
            const bool live = k0 < p.lr_rank;
            const float4 x0 = live ? ld4(wr + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 x1 = live ? ld4(wr + k0 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
            const Split2 a = split2(x0.x, x0.y), b = split2(x0.z, x0.w), c = split2(x1.x, x1.y), d = split2(x1.z, x1.w);
            wfh[m] = u32x4{a.hi, b.hi, c.hi, d.hi};
            wfl[m] = u32x4{a.lo, b.lo, c.lo, d.lo};
        }
    }
    auto issue_lowrank = [&](int64_t c0) {
        const int64_t end = chunk_end(c0);
        const Rsrc aa = make_rsrc(p.lr_a + (rng.lo + c0) * (int64_t)p.lr_rank,
                                  (uint32_t)((end - c0) * p.lr_rank * 4));
        // columns from the rank on repeat column 0 (unused, kept in range)
        ra = bld_f32x4(aa, (uint32_t)((la_t * p.lr_rank + (la_k < p.lr_rank ? la_k : 0)) * 4));
    };
    auto write_lowrank = [&](int buf) {
        const bool live = la_k < p.lr_rank;
        const Split2 a = split2(live ? ra.x : 0.f, live ? ra.y : 0.f);
        const Split2 b = split2(live ? ra.z : 0.f, live ? ra.w : 0.f);
        *reinterpret_cast<u32x2 *>(&s_lah[buf][la_t][la_k / 2]) = u32x2{a.hi, b.hi};
        *reinterpret_cast<u32x2 *>(&s_lal[buf][la_t][la_k / 2]) = u32x2{a.lo, b.lo};
    };
    // f of the chunk in buffer buf for (dch, quarter dq), into rf
    auto lowrank_f = [&](int buf) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const u32x4 ah = *reinterpret_cast<const u32x4 *>(&s_lah[buf][n16][16 * m + 4 * g4]);
            const u32x4 al = *reinterpret_cast<const u32x4 *>(&s_lal[buf][n16][16 * m + 4 * g4]);
            acc = mma32(ah, al, wfh[m], wfl[m], acc);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) rf[u] = acc[u];
    };

    // loads of a chunk at c0 >= CC (its past rows are tokens, not the window);
    // rows past the sequence end read as 0
    auto issue_inputs = [&](int64_t c0) {
        issue_lowrank(c0);                         // first: the next half waits for it alone
        const int64_t base = c0 - PAST, end = chunk_end(c0);
        const Rsrc aq = tok_rsrc(p.q, BA::ELEM, base, end);
        const Rsrc ak = tok_rsrc(p.k, BA::ELEM, base, end);
        const Rsrc av = tok_rsrc(p.v, BA::ELEM, base, end);
#pragma unroll
        for (int r = 0; r < RAWR; ++r) {
            const uint32_t e = (uint32_t)((t0 + r) * rowsz + h * DK + 2 * lane);
            rq[r] = BA::load_raw2(aq, e);
            rk[r] = BA::load_raw2(ak, e);
            rv[r] = BA::load_raw2(av, e);
        }
        const Rsrc ab = make_rsrc(p.beta + (rng.lo + c0) * p.H, (uint32_t)((end - c0) * p.H * 4));
        rb = bld_f32(ab, (uint32_t)(((t0 + (lane & (TW - 1))) * p.H + h) * 4));
    };
    auto issue_gate = [&](int64_t c0) {
        const Rsrc ag = tok_rsrc(p.g, BA::ELEM, c0, chunk_end(c0));
#pragma unroll
        for (int sl = 0; sl < TW; ++sl)
            rg[sl] = BA::load_raw2(ag, (uint32_t)((t0 + sl) * rowsz + h * DV + 2 * lane));
    };

    // conv + SiLU + L2 norm of this wavefront's tokens of the chunk at c0 (zeros
    // past the end), decay sums of (dch, quarter dq); v, beta to buffer buf
    auto prestep = [&](const float2 (&xq)[RAWR], const float2 (&xk)[RAWR], const float2 (&xv)[RAWR],
                       int64_t c0, int buf) {
        const int nv = (int)(L - c0 < CC ? L - c0 : CC);
        const float4 wq0 = ld4(s_cw[chq]), wq1 = ld4(s_cw[chq + 1]);
        const float4 wk0 = ld4(s_cw[chk]), wk1 = ld4(s_cw[chk + 1]);
        const float4 wv0 = ld4(s_cw[chv]), wv1 = ld4(s_cw[chv + 1]);
#pragma unroll
        for (int sl = 0; sl < TW; ++sl) {
            const int t = t0 + sl;
            float2 qh = make_float2(0.f, 0.f), kh = qh, vh = qh;
            if (t < nv) {                          // wavefront-uniform
                const float aq0 = silu(cconv4(wq0, xq[sl].x, xq[sl + 1].x, xq[sl + 2].x, xq[sl + 3].x));
                const float aq1 = silu(cconv4(wq1, xq[sl].y, xq[sl + 1].y, xq[sl + 2].y, xq[sl + 3].y));
                const float ak0 = silu(cconv4(wk0, xk[sl].x, xk[sl + 1].x, xk[sl + 2].x, xk[sl + 3].x));
                const float ak1 = silu(cconv4(wk1, xk[sl].y, xk[sl + 1].y, xk[sl + 2].y, xk[sl + 3].y));
                vh.x = silu(cconv4(wv0, xv[sl].x, xv[sl + 1].x, xv[sl + 2].x, xv[sl + 3].x));
                vh.y = silu(cconv4(wv1, xv[sl].y, xv[sl + 1].y, xv[sl + 2].y, xv[sl + 3].y));
                const float nq = rsq(sum64(aq0 * aq0 + aq1 * aq1) + p.l2_eps);
                const float nk = rsq(sum64(ak0 * ak0 + ak1 * ak1) + p.l2_eps);
                qh = make_float2(aq0 * nq, aq1 * nq);
                kh = make_float2(ak0 * nk, ak1 * nk);
            }
            *reinterpret_cast<float2 *>(&s_qh[t][chq]) = qh;
            *reinterpret_cast<float2 *>(&s_kh[t][chq]) = kh;
            *reinterpret_cast<float2 *>(&s_v[buf][t][chq]) = vh;
        }
        if (lane < TW) s_beta[buf][t0 + lane] = (t0 + lane < nv) ? rb : 0.f;
        float G = 0.f;                             // held constant past the last token
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = 4 * dq + u;
            if (t < nv) G += p.lb * sigmoid(eA * (rf[u] + dtb));
            s_Gq[t][dch] = G;
        }
        s_Gt[dq][dch] = G;
    };

    // split operands of the prepared chunk (into buffer buf) and the partial
    // L, M over channel eighth `wave`
    auto operands = [&](int buf) {
        {
            // lane: channels chq, chq + 1 of this wavefront's tokens (quarter wave / 2)
            const int qt = t0 >> 2;
            const float2 gt0 = ld2(&s_Gt[0][chq]), gt1 = ld2(&s_Gt[1][chq]);
            const float2 gt2 = ld2(&s_Gt[2][chq]), gt3 = ld2(&s_Gt[3][chq]);
            // sums of the quarters before and after this one (qt is
            // wavefront-uniform: one scalar branch, no per-lane selects)
            float2 before, after;
            switch (qt) {
            case 0:
                before = make_float2(0.f, 0.f);
                after = make_float2((gt1.x + gt2.x) + gt3.x, (gt1.y + gt2.y) + gt3.y);
                break;
            case 1:
                before = gt0;
                after = make_float2(gt2.x + gt3.x, gt2.y + gt3.y);
                break;
            case 2:
                before = make_float2(gt0.x + gt1.x, gt0.y + gt1.y);
                after = gt3;
                break;
            default:
                before = make_float2((gt0.x + gt1.x) + gt2.x, (gt0.y + gt1.y) + gt2.y);
                after = make_float2(0.f, 0.f);
                break;
            }
            const float2 gq_end = ld2(&s_Gt[qt][chq]);
            const int m = chq >> 5, gg = (chq & 15) >> 2, e = ((chq & 31) >> 4) * 4 + (chq & 3);
            float E0[TW], E1[TW];
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                const int t = t0 + sl;
                const float2 gq = ld2(&s_Gq[t][chq]);
                const float2 kh = ld2(&s_kh[t][chq]);
                const float2 qh = ld2(&s_qh[t][chq]);
                const float eg0 = __expf(before.x + gq.x), eg1 = __expf(before.y + gq.y);
                const Split2 ka = split2(eg0 * kh.x, eg1 * kh.y);
                const Split2 qa = split2(eg0 * qh.x, eg1 * qh.y);
                const int w = (t * OPR + m * 4 + gg) * 4 + e / 2;
                s_kah[w] = ka.hi; s_kal[w] = ka.lo;
                s_qah[w] = qa.hi; s_qal[w] = qa.lo;
                // G_C - G_t = (rest of this quarter) + (later quarters)
                E0[sl] = __expf(gq_end.x - gq.x + after.x) * kh.x;
                E1[sl] = __expf(gq_end.y - gq.y + after.y) * kh.y;
            }
            const Split2 a0 = split2(E0[0], E0[1]), a1 = split2(E1[0], E1[1]);
            reinterpret_cast<uint32_t *>(s_Eh[buf][chq])[wave] = a0.hi;
            reinterpret_cast<uint32_t *>(s_El[buf][chq])[wave] = a0.lo;
            reinterpret_cast<uint32_t *>(s_Eh[buf][chq + 1])[wave] = a1.hi;
            reinterpret_cast<uint32_t *>(s_El[buf][chq + 1])[wave] = a1.lo;
            if (wave == 0) {
                const float gc0 = gt0.x + gt1.x + gt2.x + gt3.x, gc1 = gt0.y + gt1.y + gt2.y + gt3.y;
                *reinterpret_cast<float2 *>(&s_gC[buf][chq]) = make_float2(__expf(gc0), __expf(gc1));
            }
        }
        // L_ts = sum_i (e^{G_ti - r_i} k_ti)(e^{r_i - G_si} k_si), M likewise with q_t,
        // r = G at the chunk middle (token 7), as split bf16 products over the
        // wavefront's 16 channels; lane l: token l % 16, channels 16 wave + 4 (l / 16) + s
        const int cb = 16 * wave + 4 * g4;
        const int tq = n16 >> 2;
        const float4 k4 = ld4(&s_kh[n16][cb]);
        const float4 q4 = ld4(&s_qh[n16][cb]);
        const float4 gq = ld4(&s_Gq[n16][cb]);
        const float4 g7 = ld4(&s_Gq[CC / 2 - 1][cb]);   // quarter 1 up to token 7
        const float4 c0 = ld4(&s_Gt[0][cb]);
        const float4 c2 = ld4(&s_Gt[2][cb]);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
        const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
        const float gv[4] = {gq.x, gq.y, gq.z, gq.w};
        const float g7v[4] = {g7.x, g7.y, g7.z, g7.w};
        const float c0v[4] = {c0.x, c0.y, c0.z, c0.w};
        const float c2v[4] = {c2.x, c2.y, c2.z, c2.w};
        float fl[4], fm[4], fb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // G_t - r from sums that start as close to both tokens as possible
            const float d = tq == 0 ? gv[s] - c0v[s] - g7v[s]
                          : tq == 1 ? gv[s] - g7v[s]
                          : tq == 2 ? gv[s] : gv[s] + c2v[s];
            const float ef = __expf(d), eb = __expf(-d);
            fl[s] = ef * kv[s];
            fm[s] = ef * qv[s];
            fb[s] = eb * kv[s];
        }
        // (one K = 16 step per part: three 16x16x16 steps per product)
        const Split2 l0 = split2_dead(fl[0], fl[1], neg1), l1 = split2_dead(fl[2], fl[3], neg1);
        const Split2 m0 = split2_dead(fm[0], fm[1], neg1), m1 = split2_dead(fm[2], fm[3], neg1);
        const Split2 b0 = split2_dead(fb[0], fb[1], neg1), b1 = split2_dead(fb[2], fb[3], neg1);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const u32x2 bh = {b0.hi, b1.hi}, bl = {b0.lo, b1.lo};
        const f32x4 Lt = mma16(u32x2{l0.hi, l1.hi}, u32x2{l0.lo, l1.lo}, bh, bl, zero);
        const f32x4 Mt = mma16(u32x2{m0.hi, m1.hi}, u32x2{m0.lo, m1.lo}, bh, bl, zero);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s_Lp[wave][4 * g4 + r][n16] = Lt[r];
            s_Mp[wave][4 * g4 + r][n16] = Mt[r];
        }
    };

    // T = (I + A)^{-1}, A = Diag(b) L strictly lower, by forward substitution
    // in blocks of 4 rows on one wavefront: lane (c = l / 4, r = l % 4) builds
    // row 4 b + r of column c in block b, and every lane of a quad keeps the
    // finished part of column c; the rows of a block couple through quad
    // broadcasts.  Masked entries of A are exact zeros.
    auto solve_T = [&](int buf) {
        {
            const int t = lane >> 2, s0 = 4 * (lane & 3);
            float4 a = ld4(&s_Lp[0][t][s0]);
#pragma unroll
            for (int q = 1; q < NPART; ++q) a += ld4(&s_Lp[q][t][s0]);
            const float bt = s_beta[buf][t];
            a.x = (s0 + 0 < t) ? bt * a.x : 0.f;
            a.y = (s0 + 1 < t) ? bt * a.y : 0.f;
            a.z = (s0 + 2 < t) ? bt * a.z : 0.f;
            a.w = (s0 + 3 < t) ? bt * a.w : 0.f;
            st4(&s_A[t][s0], a);
        }
        wave_lds_sync();
        const int c = lane >> 2, r = lane & 3;
        float Tc[CC];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int t = 4 * b + r;
            // y = e_c(t) - sum over the finished rows s < 4 b of A[t][s] T[s][c]
            float acc[4] = {(t == c) ? 1.0f : 0.0f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < b; ++s4) {
                const float4 a = ld4(&s_A[t][4 * s4]);
                acc[0] = fmaf(-a.x, Tc[4 * s4 + 0], acc[0]);
                acc[1] = fmaf(-a.y, Tc[4 * s4 + 1], acc[1]);
                acc[2] = fmaf(-a.z, Tc[4 * s4 + 2], acc[2]);
                acc[3] = fmaf(-a.w, Tc[4 * s4 + 3], acc[3]);
            }
            float y = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            // inside the block: row r subtracts A[t][4 b + r'] times finished row r' < r
            const float4 ab = ld4(&s_A[t][4 * b]);
            const float x0 = dpp<0x00>(y);
            y = fmaf(-ab.x, x0, y);
            const float x1 = dpp<0x55>(y);
            y = fmaf(-ab.y, x1, y);
            const float x2 = dpp<0xAA>(y);
            y = fmaf(-ab.z, x2, y);
            const float x3 = dpp<0xFF>(y);
            Tc[4 * b + 0] = x0;
            Tc[4 * b + 1] = x1;
            Tc[4 * b + 2] = x2;
            Tc[4 * b + 3] = x3;
            const Split2 x = split2(y, 0.f);
            reinterpret_cast<uint16_t *>(s_Th[t])[c] = (uint16_t)x.hi;
            reinterpret_cast<uint16_t *>(s_Tl[t])[c] = (uint16_t)x.lo;
        }
    };
    auto reduce_M = [&]() {
        const int t = lane >> 2, s0 = 4 * (lane & 3);
        float4 m = ld4(&s_Mp[0][t][s0]);
#pragma unroll
        for (int q = 1; q < NPART; ++q) m += ld4(&s_Mp[q][t][s0]);
        m.x = (s0 + 0 <= t) ? m.x : 0.f;
        m.y = (s0 + 1 <= t) ? m.y : 0.f;
        m.z = (s0 + 2 <= t) ? m.z : 0.f;
        m.w = (s0 + 3 <= t) ? m.w : 0.f;
        const Split2 a = split2(m.x, m.y), b = split2(m.z, m.w);
        *reinterpret_cast<u32x2 *>(&s_Mh[t][s0 / 2]) = u32x2{a.hi, b.hi};
        *reinterpret_cast<u32x2 *>(&s_Ml[t][s0 / 2]) = u32x2{a.lo, b.lo};
    };

    // RMSNorm + gate of this wavefront's tokens of the chunk at c0 (readout in s_o, gates in rg)
    auto epilogue = [&](int64_t c0) {
        const int nve = (int)(L - c0 < CC ? L - c0 : CC);
        const Rsrc ay = tok_rsrc(p.y, BA::ELEM, c0, c0 + nve);
        const Rsrc ao = tok_rsrc(p.o_raw, 4, c0, c0 + nve);
#pragma unroll
        for (int sl = 0; sl < TW; ++sl) {
            const int t = t0 + sl;
            if (t >= nve) break;                   // wavefront-uniform
            const float2 o = ld2(&s_o[t][chq]);
            const float r = rsq(sum64(o.x * o.x + o.y * o.y) * (1.0f / DV) + p.rms_eps);
            const uint32_t e = (uint32_t)(t * rowsz + h * DV + chq);
            const float2 gg = BA::unpack2(rg[sl]);
            float2 y;
            y.x = sigmoid(gg.x) * gm.x * o.x * r;
            y.y = sigmoid(gg.y) * gm.y * o.y * r;
            BA::store2(ay, e, y);
            if (p.o_raw) bst_f32x2(ao, o, e * 4);
        }
    };

    // ---- state into the accumulator tiles (lane offset: row 4 g4 + r,
    // column col0 + n16; row tile rt as the scalar offset)
    const int col0 = 16 * wave;
    const Rsrc rs_state = make_rsrc(p.state + unit * (DK * DV), DK * DV * 4);
    f32x4 st[8];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            st[rt][r] = bld_f32(rs_state, ((4 * g4 + r) * DV + col0 + n16) * 4, rt * 16 * DV * 4);

    __syncthreads();                               // conv taps in LDS
    // ---- chunk 0 (its past rows come from the carried window)
    {
        const int64_t end = chunk_end(0);
        const Rsrc aq = tok_rsrc(p.q, BA::ELEM, 0, end);
        const Rsrc ak = tok_rsrc(p.k, BA::ELEM, 0, end);
        const Rsrc av = tok_rsrc(p.v, BA::ELEM, 0, end);
        const float *W = p.win + unit * (PAST * CH);
        float2 xq[RAWR], xk[RAWR], xv[RAWR];
#pragma unroll
        for (int r = 0; r < RAWR; ++r) {
            const int jj = t0 - PAST + r;
            if (jj < 0) {
                const float *wr = W + (jj + PAST) * CH;
                xq[r] = ld2(wr + chq);
                xk[r] = ld2(wr + chk);
                xv[r] = ld2(wr + chv);
            } else {
                const uint32_t e = (uint32_t)(jj * rowsz + h * DK + 2 * lane);
                xq[r] = BA::load2(aq, e);
                xk[r] = BA::load2(ak, e);
                xv[r] = BA::load2(av, e);
            }
        }
        issue_lowrank(0);
        const Rsrc ab = make_rsrc(p.beta + rng.lo * p.H, (uint32_t)(end * p.H * 4));
        rb = bld_f32(ab, (uint32_t)(((t0 + (lane & (TW - 1))) * p.H + h) * 4));
        // f of chunk 0 from its rows of a (every wavefront's part in LDS first)
        write_lowrank(0);
        __syncthreads();
        lowrank_f(0);
        prestep(xq, xk, xv, 0, 0);
        if (NC > 1) issue_inputs(CC);
    }
    __syncthreads();
    operands(0);
    write_lowrank(1);                              // chunk 1's rows of a, read in the first half 1
    __syncthreads();

    f32x4 Pt, Rt;
    // P, R of the current chunk: step m covers state rows 32 m .. 32 m + 31
    // (tiles 2 m, 2 m + 1)
    auto products_PR = [&]() {
        Pt = f32x4{0.f, 0.f, 0.f, 0.f};
        Rt = Pt;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int w = (n16 * OPR + m * 4 + g4) * 4;
            const u32x4 kah = *reinterpret_cast<const u32x4 *>(&s_kah[w]);
            const u32x4 kal = *reinterpret_cast<const u32x4 *>(&s_kal[w]);
            const u32x4 qah = *reinterpret_cast<const u32x4 *>(&s_qah[w]);
            const u32x4 qal = *reinterpret_cast<const u32x4 *>(&s_qal[w]);
            const Split2 x0 = split2(st[2 * m][0], st[2 * m][1]);
            const Split2 x1 = split2(st[2 * m][2], st[2 * m][3]);
            const Split2 x2 = split2(st[2 * m + 1][0], st[2 * m + 1][1]);
            const Split2 x3 = split2(st[2 * m + 1][2], st[2 * m + 1][3]);
            const u32x4 sh = {x0.hi, x1.hi, x2.hi, x3.hi}, sl = {x0.lo, x1.lo, x2.lo, x3.lo};
            Pt = mma32(kah, kal, sh, sl, Pt);
            Rt = mma32(qah, qal, sh, sl, Rt);
        }
    };
    // token-wise work of half 1: pre-step of chunk i + 1, epilogue of chunk
    // i - 1, loads for chunk i + 2 (the epilogue waits for its gate loads
    // before the next chunk's loads are issued: the memory counter drains in
    // order)
    // (past the last chunk the pre-step and the operands run on masked tokens
    // into buffers nothing reads: running them unconditionally keeps each half
    // one straight-line block for the scheduler)
    auto tokens_half1 = [&](int64_t i, int cur) {
        lowrank_f(cur ^ 1);                        // f of chunk i + 1
        {
            float2 xq[RAWR], xk[RAWR], xv[RAWR];
#pragma unroll
            for (int r = 0; r < RAWR; ++r) {
                xq[r] = BA::unpack2(rq[r]);
                xk[r] = BA::unpack2(rk[r]);
                xv[r] = BA::unpack2(rv[r]);
            }
            prestep(xq, xk, xv, (i + 1) * CC, cur ^ 1);
        }
        if (i >= 1) epilogue((i - 1) * CC);
        if (i + 2 < NC) issue_inputs((i + 2) * CC);
        issue_gate(i * CC);
    };
    // Delta, O and the state update of the current chunk
    auto update = [&](int cur) {
        // W = Diag(b) (V - P) (rows 4 g4 + r); Delta = T W; O = R + M Delta
        f32x4 Wt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g4 + r;
            Wt[r] = s_beta[cur][t] * (s_v[cur][t][col0 + n16] - Pt[r]);
        }
        const u32x2 th = *reinterpret_cast<const u32x2 *>(&s_Th[n16][2 * g4]);
        const u32x2 tl = *reinterpret_cast<const u32x2 *>(&s_Tl[n16][2 * g4]);
        const u32x2 mh = *reinterpret_cast<const u32x2 *>(&s_Mh[n16][2 * g4]);
        const u32x2 ml = *reinterpret_cast<const u32x2 *>(&s_Ml[n16][2 * g4]);
        u32x2 wh, wl, dh, dl;
        split4(Wt, wh, wl);
        const f32x4 Dt = mma16(th, tl, wh, wl, f32x4{0.f, 0.f, 0.f, 0.f});
        split4(Dt, dh, dl);
        const f32x4 Ot = mma16(mh, ml, dh, dl, Rt);
#pragma unroll
        for (int r = 0; r < 4; ++r) s_o[4 * g4 + r][col0 + n16] = Ot[r];
        // S <- Diag(e^{G_C}) S + E^T Delta
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const float4 dc = ld4(&s_gC[cur][16 * rt + 4 * g4]);
            const u32x2 eh = *reinterpret_cast<const u32x2 *>(&s_Eh[cur][16 * rt + n16][2 * g4]);
            const u32x2 el = *reinterpret_cast<const u32x2 *>(&s_El[cur][16 * rt + n16][2 * g4]);
            st[rt][0] *= dc.x;
            st[rt][1] *= dc.y;
            st[rt][2] *= dc.z;
            st[rt][3] *= dc.w;
            st[rt] = mma16(eh, el, dh, dl, st[rt]);
        }
    };

    // The two wavefronts that share a SIMD (w and w + 4) take the matrix work
    // and the vector work of each half in opposite orders, so that one's
    // MFMAs run while the other issues vector instructions.
    const bool mfma_first = wave < 4;
#pragma unroll 1
    for (int64_t i = 0; i < NC; ++i) {
        const int cur = (int)(i & 1);
        // ================= half 1
        if (wave == 0) solve_T(cur);
        else if (wave == 1) reduce_M();
        if (mfma_first) {
            products_PR();
            tokens_half1(i, cur);
        } else {
            tokens_half1(i, cur);
            products_PR();
        }
        __syncthreads();
        // ================= half 2
        if (mfma_first) {
            update(cur);
            operands(cur ^ 1);
        } else {
            operands(cur ^ 1);
            update(cur);
        }
        // chunk i + 2's rows of a, loaded in half 1, for its f in the
        // next half 1 (past the last chunk: values nothing uses)
        write_lowrank(cur);
        __syncthreads();
    }

    epilogue((NC - 1) * CC);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            bst_f32(rs_state, st[rt][r], ((4 * g4 + r) * DV + col0 + n16) * 4, rt * 16 * DV * 4);
}

// Sequences of a few chunks.  The kernels above hold one workgroup per
// compute unit (1024 threads and 147 KB of LDS, or 512 threads at 256
// registers), so a pair's state load and store never overlap another pair's
// work; in a batch of short sequences that round trip (128 KiB per pair) is
// most of the bytes.  This kernel takes a pair's chunks one after the other,
// without a pipeline: 8 wavefronts (512 threads), one buffer of everything,
// 79 KB of LDS and at most 128 registers, so that two workgroups share a
// compute unit and one's loads and stores run beside the other's arithmetic.
// Wavefront w does the token-wise work of tokens 2 w, 2 w + 1 (as the token
// role above) and holds rows 64 (w % 2) .. + 63 of state columns 32 (w / 2)
// .. + 31: the two wavefronts of a column block add their partial P and R
// through LDS, and every state load and store covers 128 contiguous bytes of
// a row.  It writes the conv window out itself.  Per chunk, four workgroup
// barriers apart:
//   1. the chunk's loads (the first chunk: the carried window into LDS, the
//      state last); conv, SiLU, L2 norm and the decay sums of tokens 2 w,
//      2 w + 1 and of a channel quarter
//   2. the split operands; partial L (wavefronts 0-3, one key-channel quarter
//      each) or M (wavefronts 4-7)
//   3. T (wavefront 0) and M (wavefront 1); P and R over the wavefront's rows
//   4. the other half's P and R added; Delta, O, the state update, the sums
//      of O^2 over the wavefront's readout columns
//   then the RMSNorm and gate of the chunk and its stores.
constexpr int CS_THREADS = 512;
constexpr int CS_PART = 4;         // partial L, M over channel quarters

// four consecutive activations (element index i, a multiple of 4) through a buffer
template <typename Act> __device__ __forceinline__ float4 bld4(Rsrc r, uint32_t i);
template <> __device__ __forceinline__ float4 bld4<F32>(Rsrc r, uint32_t i) { return bld_f32x4(r, i * 4); }
template <> __device__ __forceinline__ float4 bld4<BF16>(Rsrc r, uint32_t i) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, i * 2, 0, 0);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}
template <typename Act> __device__ __forceinline__ void bst4(Rsrc r, uint32_t i, float4 x);
template <> __device__ __forceinline__ void bst4<F32>(Rsrc r, uint32_t i, float4 x) { bst_f32x4_at(r, x, i * 4); }
template <> __device__ __forceinline__ void bst4<BF16>(Rsrc r, uint32_t i, float4 x) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w)}, r, i * 2, 0, 0);
}

template <typename Act>
__global__ __launch_bounds__(CS_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4)))
void prefill_chunk_short_kernel(Params p) {
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
    const int64_t L = rng.len;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // in a scalar register
    auto lane_id = opaque_lane;
    const NegOne neg1 = neg_one_pairs();
    const int t0 = TW * wave;                       // tokens of this wavefront's token-wise work
    // its state block: rows 64 hb .. 64 hb + 63 of columns 32 cb .. 32 cb + 31
    const int cb = wave >> 1, hb = wave & 1;
    const int64_t unit = (int64_t)n * p.H + h;
    const int64_t rowsz = (int64_t)p.H * DK;       // elements per token row of q, k, v, f, g, y

    // k_hat, q_hat and the log-decay summed from the start of the token's
    // quarter; after the operands are formed from them, the partial P and R
    // that the two wavefronts of a column block exchange
    __shared__ __attribute__((aligned(16))) float s_pre[3][CC][KP];
    float (*s_kh)[KP] = s_pre[0];
    float (*s_qh)[KP] = s_pre[1];
    float (*s_Gq)[KP] = s_pre[2];
    float *s_xP = &s_pre[0][0][0];            // [wavefront][column tile][16][16]
    float *s_xR = s_xP + 8 * 2 * 256;         // [wavefront][16][16]
    static_assert(8 * 3 * 256 <= 3 * CC * KP, "exchange area");
    __shared__ float s_Gt[4][DK];          // log-decay summed over each quarter
    __shared__ float s_v[CC][DV + 4];      // activated v
    __shared__ float s_beta[CC];
    // split bf16 operands e^G . k_hat, e^G . q_hat of P and R: slot (t, m, g)
    // holds channels 32 m + 4 g + {0..3} and 32 m + 16 + 4 g + {0..3} of token
    // t; before the first chunk's operands, the carried conv window
    __shared__ __attribute__((aligned(16))) uint32_t s_ops[4][CC * OPR * 4];
    uint32_t *s_kah = s_ops[0], *s_kal = s_ops[1], *s_qah = s_ops[2], *s_qal = s_ops[3];
    float (*s_win)[CH] = reinterpret_cast<float (*)[CH]>(&s_ops[0][0]);
    static_assert(PAST * CH <= 4 * CC * OPR * 4, "window copy");
    // after the products, each wavefront's readout tile [token][n16], for the
    // stores of whole column runs
    float (*s_ox)[CC][16] = reinterpret_cast<float (*)[CC][16]>(&s_ops[0][0]);
    static_assert(8 * CC * 16 <= 4 * CC * OPR * 4, "readout exchange");
    // [channel][token] split e^{G_C - G} . k_hat of the update, hi and lo
    // interleaved by groups of four tokens (u32 4 g, 4 g + 1: lo; 4 g + 2,
    // 4 g + 3: hi), one 16-byte read per cross-term operand
    __shared__ __attribute__((aligned(16))) uint32_t s_E[DK][EIR];
    __shared__ float s_gC[DK];             // e^{G_C}, decay of the whole chunk
    // L, M summed over one channel quarter each; Diag(b) L (strictly lower)
    // over the partial L, which wavefront 0 reads before it writes; the sums
    // of O^2 over each wavefront's readout columns over the partial M (no
    // longer read by then)
    __shared__ __attribute__((aligned(16))) float s_LM[2][CS_PART][CC][CC];
    float (*s_Lp)[CC][CC] = s_LM[0];
    float (*s_Mp)[CC][CC] = s_LM[1];
    float (*s_A)[TP] = reinterpret_cast<float (*)[TP]>(&s_LM[0][0][0][0]);
    float (*s_ss)[CC] = reinterpret_cast<float (*)[CC]>(&s_LM[1][0][0][0]);
    static_assert(CC * TP <= CS_PART * CC * CC && 8 * CC <= CS_PART * CC * CC, "aliases");
    // (I + Diag(b) L)^{-1} and M (lower triangle with the diagonal), [row][column] split bf16
    __shared__ __attribute__((aligned(16))) uint32_t s_Th[CC][TR], s_Tl[CC][TR], s_Mh[CC][TR], s_Ml[CC][TR];
    __shared__ __attribute__((aligned(16))) float s_cw[CH][TAPS];   // conv taps of this head

    // the state in the accumulator tiles: in tile 4 ct + rl, lane (g4, n16)
    // holds row 64 hb + 16 rl + 4 g4 + r, column 32 cb + 2 n16 + ct in element
    // r.  The two column tiles interleave, so a lane's two columns are
    // adjacent and each load or store of a row covers 128 contiguous bytes
    // (a wavefront owning 16 columns would touch 64-byte halves of lines).
    // Loaded with the first chunk.
    const Rsrc rs_state = make_rsrc(p.state + unit * (DK * DV), DK * DV * 4);
    f32x4 st[8];
    auto st_off = [&](int l, int rl, int r) -> uint32_t {
        return (uint32_t)(((64 * hb + 16 * rl + 4 * (l >> 4) + r) * DV + 32 * cb + 2 * (l & 15)) * 4);
    };

    // one chunk; the first is its own copy, which also loads the state (after
    // the chunk's inputs: loads complete in order, so the pre-step waits for
    // the inputs alone and the state arrives during it)
    auto chunk = [&](int64_t c0, auto first) {
        // the lane's indices anew each chunk (from the lane count, opaque to
        // the compiler): otherwise every address derived from them is kept
        // live across the loop, beyond the registers two workgroups per
        // compute unit allow
        const int ti = wave * 64 + lane_id();
        const int lane = ti & 63;
        const int n16 = lane & 15, g4 = lane >> 4;
        auto tok_rsrc = [&](const void *t, uint32_t elem, int64_t base, int64_t end) -> Rsrc {
            return make_rsrc(static_cast<const char *>(t) + (rng.lo + base) * rowsz * elem,
                             (uint32_t)((end - base) * rowsz * elem));
        };
        // lane: conv channels chq, chq + 1 of q, k, v (and value channels chq, chq + 1);
        // decay: key channel dch over the tokens of quarter dq
        const int chq = 2 * lane, chk = DK + 2 * lane, chv = 2 * DK + 2 * lane;
        const int dch = ti & (DK - 1), dq = ti >> 7;
        const uint32_t foff = (uint32_t)((4 * dq * rowsz + h * DK + dch) * 4);
        const float eA = __expf(p.A_log[h * DK + dch]);
        const float dtb = p.dt_bias[h * DK + dch];
        // the epilogue's lane: token 8 hb + lane / 8, columns jq .. jq + 3
        const int te = 8 * hb + (lane >> 3), jq = 32 * cb + 4 * (lane & 7);

        // T = (I + A)^{-1} by forward substitution, as in the kernel above
        auto solve_T = [&]() {
            {
                const int t = lane >> 2, s0 = 4 * (lane & 3);
                float4 a = ld4(&s_Lp[0][t][s0]);
#pragma unroll
                for (int q = 1; q < CS_PART; ++q) a += ld4(&s_Lp[q][t][s0]);
                const float bt = s_beta[t];
                a.x = (s0 + 0 < t) ? bt * a.x : 0.f;
                a.y = (s0 + 1 < t) ? bt * a.y : 0.f;
                a.z = (s0 + 2 < t) ? bt * a.z : 0.f;
                a.w = (s0 + 3 < t) ? bt * a.w : 0.f;
                st4(&s_A[t][s0], a);
            }
            wave_lds_sync();
            const int c = lane >> 2, r = lane & 3;
            float Tc[CC];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int t = 4 * b + r;
                float acc[4] = {(t == c) ? 1.0f : 0.0f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < b; ++s4) {
                    const float4 a = ld4(&s_A[t][4 * s4]);
                    acc[0] = fmaf(-a.x, Tc[4 * s4 + 0], acc[0]);
                    acc[1] = fmaf(-a.y, Tc[4 * s4 + 1], acc[1]);
                    acc[2] = fmaf(-a.z, Tc[4 * s4 + 2], acc[2]);
                    acc[3] = fmaf(-a.w, Tc[4 * s4 + 3], acc[3]);
                }
                float y = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                const float4 ab = ld4(&s_A[t][4 * b]);
                const float x0 = dpp<0x00>(y);
                y = fmaf(-ab.x, x0, y);
                const float x1 = dpp<0x55>(y);
                y = fmaf(-ab.y, x1, y);
                const float x2 = dpp<0xAA>(y);
                y = fmaf(-ab.z, x2, y);
                const float x3 = dpp<0xFF>(y);
                Tc[4 * b + 0] = x0;
                Tc[4 * b + 1] = x1;
                Tc[4 * b + 2] = x2;
                Tc[4 * b + 3] = x3;
                const Split2 x = split2(y, 0.f);
                reinterpret_cast<uint16_t *>(s_Th[t])[c] = (uint16_t)x.hi;
                reinterpret_cast<uint16_t *>(s_Tl[t])[c] = (uint16_t)x.lo;
            }
        };
        auto reduce_M = [&]() {
            const int t = lane >> 2, s0 = 4 * (lane & 3);
            float4 m = ld4(&s_Mp[0][t][s0]);
#pragma unroll
            for (int q = 1; q < CS_PART; ++q) m += ld4(&s_Mp[q][t][s0]);
            m.x = (s0 + 0 <= t) ? m.x : 0.f;
            m.y = (s0 + 1 <= t) ? m.y : 0.f;
            m.z = (s0 + 2 <= t) ? m.z : 0.f;
            m.w = (s0 + 3 <= t) ? m.w : 0.f;
            const Split2 a = split2(m.x, m.y), b = split2(m.z, m.w);
            *reinterpret_cast<u32x2 *>(&s_Mh[t][s0 / 2]) = u32x2{a.hi, b.hi};
            *reinterpret_cast<u32x2 *>(&s_Ml[t][s0 / 2]) = u32x2{a.lo, b.lo};
        };
        // wavefronts 0-3: L over key channels 32 j .. 32 j + 31 (j = w); 4-7: M
        // over the same quarter (j = w - 4); lane l: token l % 16 and channels
        // 32 j + 8 (l / 16) + {0..7}; factors e^{+-(G - r)}, r the log-decay at
        // the chunk middle, as in the kernel above; split bf16 products, one
        // K = 16 step per half hh of the lane's channels (three 16x16x16 steps
        // each, accumulated in one form)
        auto partial_LM = [&]() {
            const int j = wave & 3;
            const bool is_M = wave >= 4;              // wavefront-uniform
            const MidCoef mc = mid_coef(n16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int lc = 32 * j + 8 * g4 + 4 * hh;
                const float4 k4 = ld4(&s_kh[n16][lc]);
                const float4 a4 = is_M ? ld4(&s_qh[n16][lc]) : k4;
                const float4 gq = ld4(&s_Gq[n16][lc]);
                const float4 g7 = ld4(&s_Gq[CC / 2 - 1][lc]);
                const float4 c0 = ld4(&s_Gt[0][lc]);
                const float4 c2 = ld4(&s_Gt[2][lc]);
                const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
                const float gv[4] = {gq.x, gq.y, gq.z, gq.w};
                const float g7v[4] = {g7.x, g7.y, g7.z, g7.w};
                const float c0v[4] = {c0.x, c0.y, c0.z, c0.w};
                const float c2v[4] = {c2.x, c2.y, c2.z, c2.w};
                float fa[4], fb[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float d = rel_mid(mc, gv[s], c0v[s], g7v[s], c2v[s]);
                    fa[s] = __expf(d) * av[s];
                    fb[s] = __expf(-d) * kv[s];
                }
                const Split2 a0 = split2_dead(fa[0], fa[1], neg1), a1 = split2_dead(fa[2], fa[3], neg1);
                const Split2 b0 = split2_dead(fb[0], fb[1], neg1), b1 = split2_dead(fb[2], fb[3], neg1);
                acc = mma16(u32x2{a0.hi, a1.hi}, u32x2{a0.lo, a1.lo}, u32x2{b0.hi, b1.hi}, u32x2{b0.lo, b1.lo}, acc);
            }
            float (*dst)[CC] = is_M ? s_Mp[j] : s_Lp[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[4 * g4 + r][n16] = acc[r];
        };
        // split operands of the chunk (lane: channels chq, chq + 1 of tokens t0, t0 + 1)
        auto operands = [&]() {
            const int qt = t0 >> 2;
            const float2 gt0 = ld2(&s_Gt[0][chq]), gt1 = ld2(&s_Gt[1][chq]);
            const float2 gt2 = ld2(&s_Gt[2][chq]), gt3 = ld2(&s_Gt[3][chq]);
            // sums of the quarters before and after this one (qt is
            // wavefront-uniform: one scalar branch, no per-lane selects)
            float2 before, after;
            switch (qt) {
            case 0:
                before = make_float2(0.f, 0.f);
                after = make_float2((gt1.x + gt2.x) + gt3.x, (gt1.y + gt2.y) + gt3.y);
                break;
            case 1:
                before = gt0;
                after = make_float2(gt2.x + gt3.x, gt2.y + gt3.y);
                break;
            case 2:
                before = make_float2(gt0.x + gt1.x, gt0.y + gt1.y);
                after = gt3;
                break;
            default:
                before = make_float2((gt0.x + gt1.x) + gt2.x, (gt0.y + gt1.y) + gt2.y);
                after = make_float2(0.f, 0.f);
                break;
            }
            const float2 gq_end = ld2(&s_Gt[qt][chq]);
            const int m = chq >> 5, gg = (chq & 15) >> 2, e = ((chq & 31) >> 4) * 4 + (chq & 3);
            float E0[TW], E1[TW];
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                const int t = t0 + sl;
                const float2 gq = ld2(&s_Gq[t][chq]);
                const float2 kh = ld2(&s_kh[t][chq]);
                const float2 qh = ld2(&s_qh[t][chq]);
                const float eg0 = __expf(before.x + gq.x), eg1 = __expf(before.y + gq.y);
                const Split2 ka = split2(eg0 * kh.x, eg1 * kh.y);
                const Split2 qa = split2(eg0 * qh.x, eg1 * qh.y);
                const int w = (t * OPR + m * 4 + gg) * 4 + e / 2;
                s_kah[w] = ka.hi; s_kal[w] = ka.lo;
                s_qah[w] = qa.hi; s_qal[w] = qa.lo;
                E0[sl] = __expf(gq_end.x - gq.x + after.x) * kh.x;
                E1[sl] = __expf(gq_end.y - gq.y + after.y) * kh.y;
            }
            const Split2 a0 = split2(E0[0], E0[1]), a1 = split2(E1[0], E1[1]);
            const int eo = 4 * (wave >> 1) + (wave & 1);   // this wavefront's two tokens in their group of four
            s_E[chq][eo] = a0.lo;
            s_E[chq][eo + 2] = a0.hi;
            s_E[chq + 1][eo] = a1.lo;
            s_E[chq + 1][eo + 2] = a1.hi;
            if (wave == 0) {
                const float gc0 = gt0.x + gt1.x + gt2.x + gt3.x, gc1 = gt0.y + gt1.y + gt2.y + gt3.y;
                *reinterpret_cast<float2 *>(&s_gC[chq]) = make_float2(__expf(gc0), __expf(gc1));
            }
        };

        const int64_t end = (c0 + CC < L) ? c0 + CC : L;
        const int nv = (int)(end - c0);
        // ================= 1: loads; conv, SiLU, L2 norm, decay sums
        // (rows before the sequence start come from the carried window, rows
        // past its end read as 0)
        // raw rows behind this wavefront's tokens: rows of the sequence (past
        // its end they read as 0) and, in the first chunk, rows of the carried
        // window, which are copied to LDS first (a token row's load is then
        // sent out of range and reads as 0, without a branch on the row)
        typename BA::Raw2 xq[RAWR], xk[RAWR], xv[RAWR];
        float rf[4], rb;
        float4 gg;                                 // gates of the epilogue's token and columns
        float wn[PAST];
        float4 cw4;                                // the head's conv taps, for LDS
        if constexpr (decltype(first)::value) {
            if (ti < CH) {
                const Rsrc rs_cw = make_rsrc(p.conv_w + (int64_t)h * (CH * TAPS), CH * TAPS * 4);
                const Rsrc rs_w = make_rsrc(p.win + unit * (PAST * CH), PAST * CH * 4);
                cw4 = bld_f32x4(rs_cw, (uint32_t)(ti * TAPS * 4));
#pragma unroll
                for (int r = 0; r < PAST; ++r) wn[r] = bld_f32(rs_w, (uint32_t)((r * CH + ti) * 4));
            }
        }
        {
            const int64_t base = c0 == 0 ? 0 : c0 - PAST;
            const Rsrc aq = tok_rsrc(p.q, BA::ELEM, base, end);
            const Rsrc ak = tok_rsrc(p.k, BA::ELEM, base, end);
            const Rsrc av = tok_rsrc(p.v, BA::ELEM, base, end);
#pragma unroll
            for (int r = 0; r < RAWR; ++r) {
                const int64_t jj = c0 + t0 - PAST + r;
                const uint32_t e = jj < 0 ? 0x40000000u : (uint32_t)((jj - base) * rowsz + h * DK + 2 * lane);
                xq[r] = BA::load_raw2(aq, e);
                xk[r] = BA::load_raw2(ak, e);
                xv[r] = BA::load_raw2(av, e);
            }
            const Rsrc af = tok_rsrc(p.f, 4, c0, end);
#pragma unroll
            for (int u = 0; u < 4; ++u) rf[u] = bld_f32(af, foff, (uint32_t)(u * rowsz * 4));
            const Rsrc ab = make_rsrc(p.beta + (rng.lo + c0) * p.H, (uint32_t)((end - c0) * p.H * 4));
            rb = bld_f32(ab, (uint32_t)(((t0 + (lane & (TW - 1))) * p.H + h) * 4));
            const Rsrc ag = tok_rsrc(p.g, BA::ELEM, c0, end);
            gg = bld4<Act>(ag, (uint32_t)(te * rowsz + h * DV + jq));
        }
        if constexpr (decltype(first)::value) {
#pragma unroll
            for (int rl = 0; rl < 4; ++rl)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float2 x = bld_f32x2(rs_state, st_off(lane, rl, r));
                    st[rl][r] = x.x;
                    st[4 + rl][r] = x.y;
                }
            if (ti < CH) {
#pragma unroll
                for (int r = 0; r < PAST; ++r) s_win[r][ti] = wn[r];
                st4(s_cw[ti], cw4);
            }
            __syncthreads();
        }
        {
            // (the conv window out: the sequence's last PAST raw rows, written
            // in the last chunk by the wavefront whose tokens they are, rows
            // before the chunk by wavefront 0; every read of the carried window
            // lies before the first chunk's barrier)
            const Rsrc rs_win = make_rsrc(p.win + unit * (PAST * CH), PAST * CH * 4);
            auto act = [&](const typename BA::Raw2 (&raw)[RAWR], int ch, float (&a)[TW][2]) {
                const float4 w0 = ld4(s_cw[ch]), w1 = ld4(s_cw[ch + 1]);
                float2 x[RAWR];
#pragma unroll
                for (int r = 0; r < RAWR; ++r) {
                    x[r] = BA::unpack2(raw[r]);
                    if constexpr (decltype(first)::value) {
                        if (t0 - PAST + r < 0) x[r] = ld2(&s_win[t0 + r][ch]);   // wavefront-uniform
                    }
                    const int64_t j = c0 + t0 - PAST + r;
                    if ((r >= PAST || wave == 0) && j >= L - PAST && j < L)    // wavefront-uniform
                        bst_f32x2(rs_win, x[r], (uint32_t)(((j - (L - PAST)) * CH + ch) * 4));
                }
#pragma unroll
                for (int sl = 0; sl < TW; ++sl) {
                    a[sl][0] = silu(cconv4(w0, x[sl].x, x[sl + 1].x, x[sl + 2].x, x[sl + 3].x));
                    a[sl][1] = silu(cconv4(w1, x[sl].y, x[sl + 1].y, x[sl + 2].y, x[sl + 3].y));
                }
            };
            float aq[TW][2], ak[TW][2], av[TW][2];
            act(xq, chq, aq);
            act(xk, chk, ak);
            act(xv, chv, av);
#pragma unroll
            for (int sl = 0; sl < TW; ++sl) {
                const int t = t0 + sl;
                const bool live = t < nv;
                const float nq = rsq(sum64(aq[sl][0] * aq[sl][0] + aq[sl][1] * aq[sl][1]) + p.l2_eps);
                const float nk = rsq(sum64(ak[sl][0] * ak[sl][0] + ak[sl][1] * ak[sl][1]) + p.l2_eps);
                const float2 qh = live ? make_float2(aq[sl][0] * nq, aq[sl][1] * nq) : make_float2(0.f, 0.f);
                const float2 kh = live ? make_float2(ak[sl][0] * nk, ak[sl][1] * nk) : make_float2(0.f, 0.f);
                const float2 vh = live ? make_float2(av[sl][0], av[sl][1]) : make_float2(0.f, 0.f);
                *reinterpret_cast<float2 *>(&s_qh[t][chq]) = qh;
                *reinterpret_cast<float2 *>(&s_kh[t][chq]) = kh;
                *reinterpret_cast<float2 *>(&s_v[t][chq]) = vh;
            }
            if (lane < TW) s_beta[t0 + lane] = (t0 + lane < nv) ? rb : 0.f;
            float G = 0.f;                         // held constant past the last token
            const int rem = nv - 4 * dq;           // tokens of quarter dq within the sequence
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float gk = p.lb * sigmoid(eA * (rf[u] + dtb));
                G += (u < rem) ? gk : 0.f;
                s_Gq[4 * dq + u][dch] = G;
            }
            s_Gt[dq][dch] = G;
        }
        __syncthreads();
        // ================= 2: split operands; partial L or M
        operands();
        partial_LM();
        __syncthreads();
        // ================= 3: T, M; P and R over this wavefront's 64 rows
        // (step m covers its row tiles 2 m, 2 m + 1: key channels from 64 hb +
        // 32 m, operand slot 2 hb + m), handed to the other wavefront of the
        // column block: both P tiles, and the R tile whose readout it forms
        if (wave == 0) solve_T();
        else if (wave == 1) reduce_M();
        f32x4 Pt[2], Rt[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Pt[ct] = Rt[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int w = (n16 * OPR + (2 * hb + m) * 4 + g4) * 4;
            const u32x4 kah = *reinterpret_cast<const u32x4 *>(&s_kah[w]);
            const u32x4 kal = *reinterpret_cast<const u32x4 *>(&s_kal[w]);
            const u32x4 qah = *reinterpret_cast<const u32x4 *>(&s_qah[w]);
            const u32x4 qal = *reinterpret_cast<const u32x4 *>(&s_qal[w]);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const f32x4 &a = st[4 * ct + 2 * m], &b = st[4 * ct + 2 * m + 1];
                const Split2 x0 = split2(a[0], a[1]), x1 = split2(a[2], a[3]);
                const Split2 x2 = split2(b[0], b[1]), x3 = split2(b[2], b[3]);
                const u32x4 sh = {x0.hi, x1.hi, x2.hi, x3.hi}, sl = {x0.lo, x1.lo, x2.lo, x3.lo};
                Pt[ct] = mma32(kah, kal, sh, sl, Pt[ct]);
                Rt[ct] = mma32(qah, qal, sh, sl, Rt[ct]);
            }
        }
        {
            // lane (g4, n16): rows 4 g4 + r of the 16 x 16 tiles
            float *xp = s_xP + wave * 512 + g4 * 64 + n16;
            float *xr = s_xR + wave * 256 + g4 * 64 + n16;
            const f32x4 &ro = hb ? Rt[0] : Rt[1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                xp[16 * r] = Pt[0][r];
                xp[256 + 16 * r] = Pt[1][r];
                xr[16 * r] = ro[r];
            }
        }
        __syncthreads();
        f32x4 Rs;                                   // R of this lane's readout column, whole
        {
            const int pw = wave ^ 1;
            const float *xp = s_xP + pw * 512 + g4 * 64 + n16;
            const float *xr = s_xR + pw * 256 + g4 * 64 + n16;
            const f32x4 &ri = hb ? Rt[1] : Rt[0];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Pt[0][r] += xp[16 * r];
                Pt[1][r] += xp[256 + 16 * r];
                Rs[r] = ri[r] + xr[16 * r];
            }
        }
        // ================= 4: Delta, O, the state update; sums of O^2
        f32x4 Ot;
        {
            // W = Diag(b) (V - P) for both column tiles (columns 32 cb + 2 n16 + ct)
            f32x4 Wt[2];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                const float2 v2 = ld2(&s_v[t][32 * cb + 2 * n16]);
                const float bt = s_beta[t];
                Wt[0][r] = bt * (v2.x - Pt[0][r]);
                Wt[1][r] = bt * (v2.y - Pt[1][r]);
            }
            const u32x2 th = *reinterpret_cast<const u32x2 *>(&s_Th[n16][2 * g4]);
            const u32x2 tl = *reinterpret_cast<const u32x2 *>(&s_Tl[n16][2 * g4]);
            const u32x2 mh = *reinterpret_cast<const u32x2 *>(&s_Mh[n16][2 * g4]);
            const u32x2 ml = *reinterpret_cast<const u32x2 *>(&s_Ml[n16][2 * g4]);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            u32x2 dh[2], dl[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                u32x2 wh, wl;
                split4(Wt[ct], wh, wl);
                const f32x4 Dt = mma_cross(th, tl, wh, wl, zero) + mma_hihi(th, wh, zero);
                split4(Dt, dh[ct], dl[ct]);
            }
            // O = R + M Delta for the readout column tile (ct = hb)
            const u32x2 &doh = hb ? dh[1] : dh[0], &dol = hb ? dl[1] : dl[0];
            Ot = mma_cross(mh, ml, doh, dol, Rs) + mma_hihi(mh, doh, zero);
            // rows 4 g4 + r: the sum over this wavefront's 16 readout columns,
            // written by lane n16 = r
            float ss[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ss[r] = sum16(Ot[r] * Ot[r]);
            if (n16 < 4) s_ss[wave][4 * g4 + n16] = n16 == 0 ? ss[0] : n16 == 1 ? ss[1] : n16 == 2 ? ss[2] : ss[3];
#pragma unroll
            for (int r = 0; r < 4; ++r) s_ox[wave][4 * g4 + r][n16] = Ot[r];
            // S <- Diag(e^{G_C}) S + E^T Delta on this wavefront's rows (key
            // channels 64 hb + 16 rl + ..): the cross-term steps of all eight
            // tiles, then their hi * hi steps (the empty asm keeps that order,
            // so seven steps separate each pair)
            u32x2 eh[4];
#pragma unroll
            for (int rl = 0; rl < 4; ++rl) {
                const int row = 64 * hb + 16 * rl;
                const float4 dc = ld4(&s_gC[row + 4 * g4]);
                const u32x4 e = *reinterpret_cast<const u32x4 *>(&s_E[row + n16][4 * g4]);
                eh[rl] = u32x2{e.z, e.w};
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    f32x4 &x = st[4 * ct + rl];
                    x[0] *= dc.x;
                    x[1] *= dc.y;
                    x[2] *= dc.z;
                    x[3] *= dc.w;
                    x = mma_cross_packed(e, dh[ct], dl[ct], x);
                }
            }
            asm volatile("" : "+v"(st[0]), "+v"(st[1]), "+v"(st[2]), "+v"(st[3]),
                              "+v"(st[4]), "+v"(st[5]), "+v"(st[6]), "+v"(st[7]));
#pragma unroll
            for (int rl = 0; rl < 4; ++rl)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) st[4 * ct + rl] = mma_hihi(eh[rl], dh[ct], st[4 * ct + rl]);
        }
        __syncthreads();
        // ================= RMSNorm + gate of token te, columns jq .. jq + 3
        // (columns 32 cb + 2 n16 + ct of the two tiles interleave; the output
        // buffers end at the sequence end: later tokens are dropped)
        {
            float s = s_ss[0][te];
#pragma unroll
            for (int w = 1; w < 8; ++w) s += s_ss[w][te];
            const float rr = rsq(s * (1.0f / DV) + p.rms_eps);
            const float2 o0 = ld2(&s_ox[2 * cb][te][2 * (lane & 7)]);
            const float2 o1 = ld2(&s_ox[2 * cb + 1][te][2 * (lane & 7)]);
            const float4 o = make_float4(o0.x, o1.x, o0.y, o1.y);
            const float4 gm = ld4(p.gamma + jq);
            const float4 y = make_float4(sigmoid(gg.x) * gm.x * o.x * rr, sigmoid(gg.y) * gm.y * o.y * rr,
                                         sigmoid(gg.z) * gm.z * o.z * rr, sigmoid(gg.w) * gm.w * o.w * rr);
            const uint32_t e = (uint32_t)(te * rowsz + h * DV + jq);
            bst4<Act>(tok_rsrc(p.y, BA::ELEM, c0, end), e, y);
            if (p.o_raw) bst4<F32>(tok_rsrc(p.o_raw, 4, c0, end), e, o);
        }
    };
    chunk(0, std::true_type{});
#pragma unroll 1
    for (int64_t c0 = CC; c0 < L; c0 += CC) chunk(c0, std::false_type{});
    const int lane = lane_id();
#pragma unroll
    for (int rl = 0; rl < 4; ++rl)
#pragma unroll
        for (int r = 0; r < 4; ++r) bst_f32x2(rs_state, make_float2(st[rl][r], st[4 + rl][r]), st_off(lane, rl, r));
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

// zeroes the pair counter before a launch that takes tickets from it (a
// kernel, not a memset, so that the call can be captured in a graph)
__global__ void ticket_reset_kernel(int32_t *c) {
    if (threadIdx.x == 0) *c = 0;
}

// Compute units of each device, read on first use.
constexpr int CHUNK_DEVICES = 64;
std::atomic<int> g_chunk_cus[CHUNK_DEVICES];

hipError_t device_cus(int &cus) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    cus = dev >= 0 && dev < CHUNK_DEVICES ? g_chunk_cus[dev].load(std::memory_order_relaxed) : 0;
    if (cus <= 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (cus <= 0) cus = 1;
        if (dev >= 0 && dev < CHUNK_DEVICES) g_chunk_cus[dev].store(cus, std::memory_order_relaxed);
    }
    return hipSuccess;
}

// With a pair counter the 16-wavefront kernel runs one workgroup per compute
// unit (its LDS allows no more) and each takes pairs until none are left;
// without one, one workgroup per pair.
template <typename Act>
hipError_t launch_chunk_as(const Params &p, bool lowrank, hipStream_t stream) {
    const int64_t units = (int64_t)p.num_seqs * p.H;
    if (lowrank) {
        hipLaunchKernelGGL((prefill_chunk_lr_kernel<Act>), dim3((unsigned)units), dim3(LR_THREADS), 0, stream, p);
    } else if (p.tickets) {
        int cus = 0;
        hipError_t e = device_cus(cus);
        if (e != hipSuccess) return e;
        const int64_t G = units < cus ? units : cus;
        hipLaunchKernelGGL(ticket_reset_kernel, dim3(1), dim3(64), 0, stream, p.tickets);
        hipLaunchKernelGGL((prefill_chunk_kernel<Act>), dim3((unsigned)G), dim3(CK_THREADS), 0, stream, p);
    } else {
        hipLaunchKernelGGL((prefill_chunk_kernel<Act>), dim3((unsigned)units), dim3(CK_THREADS), 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_window_kernel<Act>), dim3((unsigned)units), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool prefill_chunk_supported(int32_t gate_mode, float lb, int32_t num_heads) {
    // the per-chunk buffer resources span (CC + PAST) token rows of H * 128 elements
    return gate_mode == GATE_BOUNDED && lb <= 0.0f && -lb * (CC / 2) <= CHUNK_MAX_HALF_LOG_DECAY &&
           num_heads <= 4096;
}

hipError_t launch_prefill_chunk(const Params &p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_chunk_as<BF16>(p, false, stream) : launch_chunk_as<F32>(p, false, stream);
}

hipError_t launch_prefill_chunk_short(const Params &p, bool bf16, hipStream_t stream) {
    const int64_t units = (int64_t)p.num_seqs * p.H;
    if (bf16)
        hipLaunchKernelGGL((prefill_chunk_short_kernel<BF16>), dim3((unsigned)units), dim3(CS_THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_chunk_short_kernel<F32>), dim3((unsigned)units), dim3(CS_THREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_prefill_chunk_lowrank(const Params &p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_chunk_as<BF16>(p, true, stream) : launch_chunk_as<F32>(p, true, stream);
}

}  // namespace kda
