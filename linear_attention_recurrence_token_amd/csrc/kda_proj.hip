// kda_proj.hip -- the matrix products on either side of the KDA step, on the
// matrix cores ("Kimi K3 Metal Gap Analysis", §2 KDA Attention, rows "Decay
// compute" and "O projection"; "Metal (Apple GPU) backend for Kimi K3", table
// "What runs where (per layer)": the KDA projections and the fp32 low-rank
// products fa, fb, bp run as GPU matrix products):
//
//   C[m, n] = sum_k A[m, k] B[n, k]     A: token rows [M, K], B: weight rows [N, K]
//
// with an epilogue that stores columns [0, n_split) in the output type and
// passes columns [n_split, N) through a sigmoid (the beta logits).
//
// Precision.  Operands enter the 16x16x32 bf16 MFMA as bf16: bf16 data as it
// is, fp32 data split into hi = bf16(x) and lo = bf16(x - hi).  A product
// with an fp32 side is formed as hi*hi + hi*lo + lo*hi (the lo*lo term lies
// below fp32 rounding): about 2^-16 relative error per product, fp32
// accumulation -- the fp32 products of the pages at a third of the bf16
// matrix-core rate, still well above what fp32 MFMA gives.  bf16 x bf16 is
// exact in the products.
//
// Tiling.  256 threads = 4 wavefronts in a 2 x 2 grid; a workgroup tile of BM
// tokens x BN outputs, K consumed 32 columns per stage through a double-
// buffered LDS tile (rows padded to 80 bytes: the 16 rows a 16-lane group
// reads fall on distinct banks).  The next stage's global loads are issued
// before the current stage's MFMAs.  The weight tile is the MFMA's A operand
// and the token tile its B operand, so each lane's accumulator holds 4
// consecutive outputs of one token; the output tile then goes through LDS so
// that consecutive lanes write consecutive 16-byte pieces of one output row.
// Few tiles (decode-sized M) split K across workgroups into an fp32 scratch
// that a second kernel sums before the epilogue.
#include "kda_device.hpp"

#include <type_traits>

namespace kda {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Tiles of the direct-to-LDS bf16 kernel: 128 tokens x 256 outputs (64 x 128
// per wavefront), 3 stages in LDS (72 KiB), two workgroups per compute unit --
// measured the fastest of 256 x 256 with 4 stages and one workgroup, 256 x 128
// and 128 x 128.  Its limit is the rate at which tiles arrive from L2 (about
// 17 bytes per clock per compute unit on 32768 x 8192 x 8192), not the MFMA.
constexpr int DMA_BM = 128;      // token rows per tile
constexpr int DMA_BN = 256;      // outputs per tile
constexpr int DMA_NS = 3;        // K stages in LDS
constexpr int DMA_WPE = 2;       // waves per SIMD: two workgroups of four wavefronts per compute unit

constexpr int GT = 256;          // threads per workgroup
constexpr int BK = 32;           // K columns per stage
constexpr int BKP = BK + 8;      // LDS row length in bf16 elements (80 bytes)

template <typename T> struct Opnd;
template <> struct Opnd<F32> { static constexpr int PARTS = 2, ELEM = 4; };
template <> struct Opnd<BF16> { static constexpr int PARTS = 1, ELEM = 2; };
// fp32 operand already split into bf16 parts: the high parts of all N rows,
// then the low parts (ProjGemm::b_presplit); ELEM is the bytes per part
struct F32P {};
template <> struct Opnd<F32P> { static constexpr int PARTS = 2, ELEM = 2; };

struct GemmArgs {
    const void *A;               // [M, K] token rows
    const void *B;               // [N, K] weight rows
    int64_t M;
    int32_t N, K;
    int32_t k_len;               // K columns per split (multiple of BK)
    int32_t splits;
    int32_t tiles_m, tiles_n;
    void *C0;                    // columns [0, n_split), output type
    int64_t ldc0;
    float *C1;                   // columns [n_split, N) through a sigmoid, or null
    int64_t ldc1;
    int32_t n_split;
    int32_t np;                  // N rounded up to 4 (row length of the scratch)
    float *partial;              // [splits, M, np] fp32, or null (epilogue in place)
};

// one operand tile of R rows x BK columns: global (buffer) loads into
// registers, then into LDS as bf16 parts
template <typename T, int R>
struct Tile {
    static constexpr int ELEM = Opnd<T>::ELEM;
    static constexpr int CPR = BK * ELEM / 16;         // 16-byte chunks per row
    static constexpr int CHUNKS = R * CPR;
    static constexpr int PER = (CHUNKS + GT - 1) / GT;
    u32x4 v[PER];
    u32x4 v2[std::is_same<T, F32P>::value ? PER : 1];   // the low parts (F32P)

    // F32P: both parts, from the high and the low plane
    __device__ __forceinline__ void issue2(Rsrc r, Rsrc r2, int tid, uint32_t row_bytes, uint32_t kbyte) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = tid + GT * j;
            if (CHUNKS % GT == 0 || c < CHUNKS) {
                const uint32_t row = c / CPR, col = c % CPR;
                v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, row * row_bytes + kbyte + col * 16, 0, 0);
                v2[j] = __builtin_amdgcn_raw_buffer_load_b128(r2, row * row_bytes + kbyte + col * 16, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void issue(Rsrc r, int tid, uint32_t row_bytes, uint32_t kbyte) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = tid + GT * j;
            if (CHUNKS % GT == 0 || c < CHUNKS) {
                const uint32_t row = c / CPR, col = c % CPR;
                v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, row * row_bytes + kbyte + col * 16, 0, 0);
            }
        }
    }
    // s: [PARTS][R][BKP] bf16 bits
    __device__ __forceinline__ void store(uint16_t *s, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = tid + GT * j;
            if (CHUNKS % GT == 0 || c < CHUNKS) {
                const int row = c / CPR, col = c % CPR;
                if constexpr (std::is_same<T, F32P>::value) {
                    *reinterpret_cast<u32x4 *>(s + row * BKP + col * 8) = v[j];
                    *reinterpret_cast<u32x4 *>(s + R * BKP + row * BKP + col * 8) = v2[j];
                } else if constexpr (Opnd<T>::PARTS == 2) {
                    const f32x4v x = {__uint_as_float(v[j].x), __uint_as_float(v[j].y),
                                      __uint_as_float(v[j].z), __uint_as_float(v[j].w)};
                    const bf16x4v h = __builtin_convertvector(x, bf16x4v);
                    const f32x4v hf = __builtin_convertvector(h, f32x4v);
                    const bf16x4v l = __builtin_convertvector(x - hf, bf16x4v);
                    uint16_t *p = s + row * BKP + col * 4;
                    *reinterpret_cast<u32x2 *>(p) = __builtin_bit_cast(u32x2, h);
                    *reinterpret_cast<u32x2 *>(p + R * BKP) = __builtin_bit_cast(u32x2, l);
                } else {
                    *reinterpret_cast<u32x4 *>(s + row * BKP + col * 8) = v[j];
                }
            }
        }
    }
};

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <typename TC>
__device__ __forceinline__ void store_out(const GemmArgs &g, int64_t m, int n, f32x4 v) {
    if (n < g.n_split) {
        // n_split is a multiple of 4: the four columns are all on this side
        if constexpr (Opnd<TC>::PARTS == 2) {
            // nontemporal: the product's output is not read again here, and
            // streaming it past L2 keeps the operand panels there
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(static_cast<float *>(g.C0) + m * g.ldc0 + n));
        } else {
            uint2 w;
            w.x = pack_bf16x2(v[0], v[1]);
            w.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(g.C0) + m * g.ldc0 + n) = w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (n + r < g.N) g.C1[m * g.ldc1 + (n + r - g.n_split)] = sigmoid(v[r]);
    }
}

template <typename TA, typename TB, typename TC, int BM, int BN>
__global__ __launch_bounds__(GT) void proj_gemm_kernel(GemmArgs g) {
    constexpr int PA = Opnd<TA>::PARTS, PB = Opnd<TB>::PARTS;
    constexpr int EA = Opnd<TA>::ELEM, EB = Opnd<TB>::ELEM;
    constexpr int WM = BM / 2, WN = BN / 2;            // wavefront tile (tokens x outputs)
    constexpr int TM = WM / 16, TN = WN / 16;
    // the K tiles, and after the K loop the output tile (rows of BN + 4 floats)
    constexpr int SA_BYTES = 2 * PA * BM * BKP * 2, SB_BYTES = 2 * PB * BN * BKP * 2;
    constexpr int SC_BYTES = BM * (BN + 4) * 4;
    constexpr int S_BYTES = SA_BYTES + SB_BYTES > SC_BYTES ? SA_BYTES + SB_BYTES : SC_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S_BYTES];
    auto sA = reinterpret_cast<uint16_t(*)[PA][BM][BKP]>(smem);
    auto sB = reinterpret_cast<uint16_t(*)[PB][BN][BKP]>(smem + SA_BYTES);
    auto sC = reinterpret_cast<float(*)[BN + 4]>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;

    // workgroup -> (split, tile): consecutive workgroups land on different
    // XCDs, so first give each XCD a contiguous range of the tile order;
    // within it, groups of 8 token tiles sweep the weight tiles (the token
    // rows and the weight rows of a group stay in that XCD's L2)
    const int total = g.tiles_m * g.tiles_n * g.splits;
    int bid = blockIdx.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int per_split = g.tiles_m * g.tiles_n;
    const int z = bid / per_split;
    const int t = bid - z * per_split;
    constexpr int GROUP = 8;
    const int group = t / (GROUP * g.tiles_n);
    const int first_m = group * GROUP;
    const int gsize = min(GROUP, g.tiles_m - first_m);
    const int in_group = t - group * GROUP * g.tiles_n;
    const int tm = first_m + in_group % gsize, tn = in_group / gsize;

    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;
    const int rows_a = (int)min((int64_t)BM, g.M - m0);
    const int rows_b = min(BN, g.N - n0);
    // one buffer resource per tile: rows past the end read as zero
    const Rsrc ra = make_rsrc(static_cast<const char *>(g.A) + m0 * g.K * EA, (uint32_t)(rows_a * g.K * EA));
    const Rsrc rb = make_rsrc(static_cast<const char *>(g.B) + (int64_t)n0 * g.K * EB,
                              (uint32_t)(rows_b * g.K * EB));
    // F32P: the low plane follows the high plane's N rows
    const Rsrc rb2 = make_rsrc(static_cast<const char *>(g.B) + ((int64_t)g.N + n0) * g.K * EB,
                               (uint32_t)(rows_b * g.K * EB));
    const int k0 = z * g.k_len;
    const int nst = min(g.k_len, g.K - k0) / BK;

    f32x4 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Tile<TA, BM> la;
    Tile<TB, BN> lb;
    la.issue(ra, tid, g.K * EA, k0 * EA);
    if constexpr (std::is_same<TB, F32P>::value)
        lb.issue2(rb, rb2, tid, g.K * EB, k0 * EB);
    else
        lb.issue(rb, tid, g.K * EB, k0 * EB);
    la.store(&sA[0][0][0][0], tid);
    lb.store(&sB[0][0][0][0], tid);
    __syncthreads();

    const int fr = lane & 15, fk = 8 * (lane >> 4);
#pragma unroll 1
    for (int s = 0; s < nst; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < nst;
        if (more) {
            la.issue(ra, tid, g.K * EA, (k0 + (s + 1) * BK) * EA);
            if constexpr (std::is_same<TB, F32P>::value)
                lb.issue2(rb, rb2, tid, g.K * EB, (k0 + (s + 1) * BK) * EB);
            else
                lb.issue(rb, tid, g.K * EB, (k0 + (s + 1) * BK) * EB);
        }
        u32x4 fw[TN][PB], fx[TM][PA];
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int p = 0; p < PB; ++p)
                fw[i][p] = *reinterpret_cast<const u32x4 *>(&sB[cur][p][wn0 + 16 * i + fr][fk]);
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int p = 0; p < PA; ++p)
                fx[j][p] = *reinterpret_cast<const u32x4 *>(&sA[cur][p][wm0 + 16 * j + fr][fk]);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                if constexpr (PB == 2) acc[i][j] = mfma(fw[i][1], fx[j][0], acc[i][j]);
                if constexpr (PA == 2) acc[i][j] = mfma(fw[i][0], fx[j][1], acc[i][j]);
                acc[i][j] = mfma(fw[i][0], fx[j][0], acc[i][j]);
            }
        if (more) {
            la.store(&sA[cur ^ 1][0][0][0], tid);
            lb.store(&sB[cur ^ 1][0][0][0], tid);
        }
        __syncthreads();
    }

    // accumulator (i, j): token wm0 + 16 j + (lane & 15), outputs
    // wn0 + 16 i + 4 (lane >> 4) .. + 3
    if (g.partial) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int64_t m = m0 + wm0 + 16 * j + fr;
                const int n = n0 + wn0 + 16 * i + 4 * (lane >> 4);
                if (m >= g.M || n >= g.N) continue;
                const f32x4 v = acc[i][j];
                *reinterpret_cast<float4 *>(g.partial + ((int64_t)z * g.M + m) * g.np + n) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        return;
    }
    // through LDS, so that consecutive lanes write consecutive 16-byte pieces
    // of one output row (the K loop ended with a barrier: the tiles are free)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const f32x4 v = acc[i][j];
            *reinterpret_cast<float4 *>(&sC[wm0 + 16 * j + fr][wn0 + 16 * i + 4 * (lane >> 4)]) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
    __syncthreads();
    constexpr int G4 = BN / 4;
    for (int c = tid; c < BM * G4; c += GT) {
        const int row = c / G4, col = (c - row * G4) * 4;
        const int64_t m = m0 + row;
        const int n = n0 + col;
        if (m >= g.M || n >= g.N) continue;
        const float4 v = *reinterpret_cast<const float4 *>(&sC[row][col]);
        store_out<TC>(g, m, n, f32x4{v.x, v.y, v.z, v.w});
    }
}

// ---------------------------------------------------------------------------
// bf16 x bf16 with the K tiles loaded straight into LDS (buffer_load ... lds):
// no registers hold the next stage, so 4 stages are in flight per workgroup
// and the wavefront's registers go to the 128 x 128 accumulator tile.
//
// LDS: per stage and operand, R rows x 32 bf16 (64 bytes), unpadded; the
// 16-byte chunk c of row r is stored at chunk c ^ f(r & 15) with
// f(r) = ((r >> 1) ^ (r >> 3)) & 3: the 16 rows a 16-lane group reads at one
// chunk then fall on distinct 16-byte bank groups both within each 256-byte
// window (16 lanes per clock) and within each 128-byte window (8 lanes per
// clock).  A wavefront's load fills one 1 KiB block (16 rows): lane i lands at
// byte 16 i of the block, so it fetches row i / 4, chunk (i & 3) ^ f(i / 4).
// Each stage and operand has its own LDS array: the compiler then waits, before
// a stage's reads, only for the loads into that array.
typedef __attribute__((address_space(3))) void *lds_ptr;

template <int R>
__device__ __forceinline__ void dma_issue(Rsrc r, uint8_t *stage, int wave, int lane, uint32_t row_bytes,
                                          uint32_t kbyte) {
    const uint32_t rr = lane >> 2;
    const uint32_t c = (lane & 3) ^ (((rr >> 1) ^ (rr >> 3)) & 3);
#pragma unroll
    for (int j = 0; j < R / 64; ++j) {
        const int b = wave + 4 * j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(stage + b * 1024), 16,
                                                 (16 * b + rr) * row_bytes + 16 * c, kbyte, 0, 0);
    }
}

// wait until at most N of this wavefront's global loads are outstanding and
// its LDS reads are complete, then the workgroup barrier (no memory fence:
// that would wait for every load in flight).  The wait is the builtin, which
// the compiler's own wait counting sees; the barrier is asm with a memory
// clobber, so that no LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
    static_assert(N < 64, "vmcnt has 6 bits");
    // s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt 11:8 (0)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    asm volatile("s_barrier" ::: "memory");
}


template <int BM, int BN, int NS, typename TC>
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(DMA_WPE)))
void proj_gemm_dma_kernel(GemmArgs g) {
    static_assert(NS == 3 || NS == 4, "stages in flight");
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int LOADS = (BM + BN) / 64;          // loads per wavefront per stage
    __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * 64], sA1[BM * 64], sA2[BM * 64];
    __shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * 64], sB1[BN * 64], sB2[BN * 64];
    __shared__ __attribute__((aligned(1024))) uint8_t sA3[NS == 4 ? BM * 64 : 16], sB3[NS == 4 ? BN * 64 : 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;

    const int total = g.tiles_m * g.tiles_n * g.splits;
    int bid = blockIdx.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int per_split = g.tiles_m * g.tiles_n;
    const int z = bid / per_split;
    const int t = bid - z * per_split;
    constexpr int GROUP = 8;
    const int group = t / (GROUP * g.tiles_n);
    const int first_m = group * GROUP;
    const int gsize = min(GROUP, g.tiles_m - first_m);
    const int in_group = t - group * GROUP * g.tiles_n;
    const int tm = first_m + in_group % gsize, tn = in_group / gsize;

    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;
    const int rows_a = (int)min((int64_t)BM, g.M - m0);
    const int rows_b = min(BN, g.N - n0);
    const Rsrc ra = make_rsrc(static_cast<const char *>(g.A) + m0 * g.K * 2, (uint32_t)(rows_a * g.K * 2));
    const Rsrc rb = make_rsrc(static_cast<const char *>(g.B) + (int64_t)n0 * g.K * 2, (uint32_t)(rows_b * g.K * 2));
    const uint32_t rowb = (uint32_t)g.K * 2;
    const int k0 = z * g.k_len;
    const int nst = min(g.k_len, g.K - k0) / BK;

    f32x4 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, uint8_t *a, uint8_t *b) {
        const uint32_t kb = (uint32_t)(k0 + s * BK) * 2;
        dma_issue<BM>(ra, a, wave, lane, rowb, kb);
        dma_issue<BN>(rb, b, wave, lane, rowb, kb);
    };
    // fragment of row (base + lane & 15), logical chunk lane >> 4
    const int fr = lane & 15;
    const uint32_t foff = fr * 64 + 16 * ((lane >> 4) ^ (((fr >> 1) ^ (fr >> 3)) & 3));
    auto compute = [&](const uint8_t *a, const uint8_t *b) {
        u32x4 fw[TN];
#pragma unroll
        for (int i = 0; i < TN; ++i) fw[i] = *reinterpret_cast<const u32x4 *>(b + (wn0 + 16 * i) * 64 + foff);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const u32x4 fx = *reinterpret_cast<const u32x4 *>(a + (wm0 + 16 * j) * 64 + foff);
#pragma unroll
            for (int i = 0; i < TN; ++i) acc[i][j] = mfma(fw[i], fx, acc[i][j]);
        }
    };
    // one K stage: its loads done everywhere (and every wavefront's reads of
    // the previous stage complete), the products, then the loads NS - 1
    // stages ahead into the buffer the previous stage used.  (Issued before
    // the products, those loads made the compiler wait for every load in
    // flight before the stage's LDS reads once per loop trip: it cannot tell
    // the stage buffers' loads apart there.)
    auto stage = [&](int s, const uint8_t *a, const uint8_t *b, uint8_t *na, uint8_t *nb) {
        if (s >= nst) return;
        // outstanding after stage s: stages s + 1 .. min(s + NS - 2, nst - 1)
        const int after = min(NS - 2, nst - 1 - s);
        if (NS == 4 && after == 2)
            wait_then_barrier<2 * LOADS>();
        else if (after >= 1)
            wait_then_barrier<LOADS>();
        else
            wait_then_barrier<0>();
        compute(a, b);
        if (s + NS - 1 < nst) issue(s + NS - 1, na, nb);
    };

    issue(0, sA0, sB0);
    if (1 < nst) issue(1, sA1, sB1);
    if (NS == 4 && 2 < nst) issue(2, sA2, sB2);
#pragma unroll 1
    for (int s = 0; s < nst; s += NS) {
        if constexpr (NS == 4) {
            stage(s, sA0, sB0, sA3, sB3);
            stage(s + 1, sA1, sB1, sA0, sB0);
            stage(s + 2, sA2, sB2, sA1, sB1);
            stage(s + 3, sA3, sB3, sA2, sB2);
        } else {
            stage(s, sA0, sB0, sA2, sB2);
            stage(s + 1, sA1, sB1, sA0, sB0);
            stage(s + 2, sA2, sB2, sA1, sB1);
        }
    }

#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int64_t m = m0 + wm0 + 16 * j + fr;
            const int n = n0 + wn0 + 16 * i + 4 * (lane >> 4);
            if (m >= g.M || n >= g.N) continue;
            if (g.partial) {
                const f32x4 v = acc[i][j];
                *reinterpret_cast<float4 *>(g.partial + ((int64_t)z * g.M + m) * g.np + n) =
                    make_float4(v[0], v[1], v[2], v[3]);
            } else {
                store_out<TC>(g, m, n, acc[i][j]);
            }
        }
}

// sum of the split-K partial products, then the epilogue; one thread per
// token and group of four outputs
template <typename TC>
__global__ __launch_bounds__(256) void proj_finalize_kernel(GemmArgs g) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int groups = g.np >> 2;
    const int64_t m = idx / groups;
    if (m >= g.M) return;
    const int n = (int)(idx - m * groups) * 4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < g.splits; ++z) {
        const float4 p = *reinterpret_cast<const float4 *>(g.partial + ((int64_t)z * g.M + m) * g.np + n);
        v[0] += p.x;
        v[1] += p.y;
        v[2] += p.z;
        v[3] += p.w;
    }
    store_out<TC>(g, m, n, v);
}

// tile shapes (tokens x outputs): large for many token rows, small for
// decode-sized batches.  A wavefront's LDS reads per 32 columns of K are
// (WM + WN) rows of 64 bytes for 2 WM WN 32 flops, so bf16 takes 128 x 128
// per wavefront; split fp32 (three products per pair of fragments, two-part
// LDS tiles) stays at 64 x 64, where two workgroups fit a compute unit
// (measured faster than 64 x 128 with one).  bf16 tokens with fp32 weights
// is the low-rank first product, whose r + H outputs (192 at rank 128 and 64
// heads) fill three 64-wide tile columns exactly; 128 x 64 took it from 0.75
// to 0.66 ms over 32768 rows (against 128 x 128, 128 x 192 and 256 x 64)
template <typename TA, typename TB> struct Shapes;
template <> struct Shapes<BF16, BF16> { static constexpr int L_BM = DMA_BM, L_BN = DMA_BN; };
template <> struct Shapes<BF16, F32> { static constexpr int L_BM = 128, L_BN = 64; };
template <> struct Shapes<F32, F32> { static constexpr int L_BM = 128, L_BN = 128; };
template <> struct Shapes<BF16, F32P> : Shapes<BF16, F32> {};
template <> struct Shapes<F32, F32P> : Shapes<F32, F32> {};
constexpr int S_BM = 64, S_BN = 64;
constexpr int64_t LARGE_MIN_M = 512;
constexpr int SPLIT_MIN_K = 256;          // K columns per split at least
constexpr int TARGET_WORKGROUPS = 512;    // two per compute unit

struct Plan {
    bool large;
    int tiles_m, tiles_n, splits, k_len;
};

template <typename TA, typename TB>
Plan plan_typed(const ProjGemm &pg, int64_t scratch_bytes) {
    Plan p;
    p.large = pg.M >= LARGE_MIN_M;
    const int bm = p.large ? Shapes<TA, TB>::L_BM : S_BM, bn = p.large ? Shapes<TA, TB>::L_BN : S_BN;
    p.tiles_m = (int)((pg.M + bm - 1) / bm);
    p.tiles_n = (pg.N + bn - 1) / bn;
    p.splits = 1;
    p.k_len = pg.K;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles < TARGET_WORKGROUPS && pg.K >= 2 * SPLIT_MIN_K) {
        int want = (int)((TARGET_WORKGROUPS + tiles - 1) / tiles);
        want = min(want, pg.K / SPLIT_MIN_K);
        int k_len = (pg.K + want - 1) / want;
        k_len = (k_len + BK - 1) / BK * BK;
        const int splits = (pg.K + k_len - 1) / k_len;
        const int64_t np = (pg.N + 3) / 4 * 4;
        if (splits > 1 && (int64_t)splits * pg.M * np * 4 <= scratch_bytes) {
            p.splits = splits;
            p.k_len = k_len;
        }
    }
    return p;
}

Plan plan_for(const ProjGemm &pg, int64_t scratch_bytes) {
    if (pg.b_presplit) return pg.a_bf16 ? plan_typed<BF16, F32P>(pg, scratch_bytes)
                                        : plan_typed<F32, F32P>(pg, scratch_bytes);
    if (pg.a_bf16 && pg.b_bf16) return plan_typed<BF16, BF16>(pg, scratch_bytes);
    if (pg.a_bf16) return plan_typed<BF16, F32>(pg, scratch_bytes);
    return plan_typed<F32, F32>(pg, scratch_bytes);
}

template <typename TA, typename TB, typename TC>
hipError_t launch_typed(const GemmArgs &a, bool large, hipStream_t stream) {
    const int total = a.tiles_m * a.tiles_n * a.splits;
    constexpr int BM = Shapes<TA, TB>::L_BM, BN = Shapes<TA, TB>::L_BN;
    if (large) {
        if constexpr (Opnd<TA>::PARTS == 1 && Opnd<TB>::PARTS == 1)
            hipLaunchKernelGGL((proj_gemm_dma_kernel<BM, BN, DMA_NS, TC>), dim3(total), dim3(GT), 0, stream, a);
        else
            hipLaunchKernelGGL((proj_gemm_kernel<TA, TB, TC, BM, BN>), dim3(total), dim3(GT), 0, stream, a);
    }
    else
        hipLaunchKernelGGL((proj_gemm_kernel<TA, TB, TC, S_BM, S_BN>), dim3(total), dim3(GT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.partial) return e;
    const int64_t threads = a.M * (a.np / 4);
    hipLaunchKernelGGL((proj_finalize_kernel<TC>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

// fp32 values into two bf16 planes: hi = bf16(x) (RNE) and lo = bf16(x - hi),
// four values per thread
__global__ __launch_bounds__(256) void split_planes_kernel(const float *w, uint16_t *hi, uint16_t *lo, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 x = reinterpret_cast<const float4 *>(w)[i];
    const uint32_t h01 = pack_bf16x2(x.x, x.y), h23 = pack_bf16x2(x.z, x.w);
    uint2 h, l;
    h.x = h01;
    h.y = h23;
    l.x = pack_bf16x2(x.x - __uint_as_float(h01 << 16), x.y - __uint_as_float(h01 & 0xffff0000u));
    l.y = pack_bf16x2(x.z - __uint_as_float(h23 << 16), x.w - __uint_as_float(h23 & 0xffff0000u));
    reinterpret_cast<uint2 *>(hi)[i] = h;
    reinterpret_cast<uint2 *>(lo)[i] = l;
}

}  // namespace

hipError_t launch_split_planes(const float *w, uint16_t *out, int64_t n, hipStream_t stream) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(split_planes_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, w, out,
                       out + n, n4);
    return hipGetLastError();
}

int64_t proj_gemm_scratch_bytes(const ProjGemm &pg) {
    const Plan p = plan_for(pg, INT64_MAX);
    if (p.splits == 1) return 0;
    return (int64_t)p.splits * pg.M * ((pg.N + 3) / 4 * 4) * 4;
}

bool proj_gemm_shape_ok(const ProjGemm &pg) {
    if (pg.M < 0 || pg.N <= 0 || pg.K <= 0 || pg.K % BK != 0) return false;
    if (pg.n_split < 0 || pg.n_split > pg.N || pg.n_split % 4 != 0) return false;
    if (pg.n_split < pg.N && !pg.C1) return false;
    // tile buffer resources: at most 256 rows x K x 4 bytes each
    if ((int64_t)256 * pg.K * 4 > 0xffffffffLL) return false;
    // one-dimensional grid
    const int64_t tm = (pg.M + S_BM - 1) / S_BM, tn = (pg.N + S_BN - 1) / S_BN;
    if (tm * tn > 0x7fffffffLL) return false;
    return true;
}

hipError_t launch_proj_gemm(const ProjGemm &pg, float *scratch, int64_t scratch_bytes, hipStream_t stream) {
    if (pg.M == 0) return hipSuccess;
    const Plan p = plan_for(pg, scratch ? scratch_bytes : 0);
    GemmArgs a;
    a.A = pg.A;
    a.B = pg.B;
    a.M = pg.M;
    a.N = pg.N;
    a.K = pg.K;
    a.k_len = p.k_len;
    a.splits = p.splits;
    a.tiles_m = p.tiles_m;
    a.tiles_n = p.tiles_n;
    a.C0 = pg.C0;
    a.ldc0 = pg.ldc0;
    a.C1 = pg.C1;
    a.ldc1 = pg.ldc1;
    a.n_split = pg.n_split;
    a.np = (pg.N + 3) / 4 * 4;
    a.partial = p.splits > 1 ? scratch : nullptr;
    if (pg.b_presplit) {
        if (pg.b_bf16 || pg.c_bf16) return hipErrorInvalidValue;
        return pg.a_bf16 ? launch_typed<BF16, F32P, F32>(a, p.large, stream)
                         : launch_typed<F32, F32P, F32>(a, p.large, stream);
    }
    if (pg.a_bf16 && pg.b_bf16 && pg.c_bf16) return launch_typed<BF16, BF16, BF16>(a, p.large, stream);
    if (pg.a_bf16 && !pg.b_bf16 && !pg.c_bf16) return launch_typed<BF16, F32, F32>(a, p.large, stream);
    if (!pg.a_bf16 && !pg.b_bf16 && !pg.c_bf16) return launch_typed<F32, F32, F32>(a, p.large, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
