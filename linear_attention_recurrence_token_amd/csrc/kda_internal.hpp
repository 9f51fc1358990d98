// kda_internal.hpp -- parameters shared by the host layer and the kernels of
// libkda (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int DK = 128;        // key channels per head
constexpr int DV = 128;        // value channels per head
constexpr int TAPS = 4;        // causal conv taps
constexpr int PAST = TAPS - 1; // raw rows kept in the conv window
constexpr int CH = 2 * DK + DV; // conv channels per head (q | k | v)

enum GateMode : int32_t { GATE_BOUNDED = 0, GATE_LITERAL = 1, GATE_RAW = 2 };

struct Params {
    const void *q, *k, *v;
    const float *f, *beta;
    const void *g;
    const float *conv_w, *A_log, *dt_bias, *gamma;
    float *state, *win;
    void *y;
    float *o_raw;
    const int32_t *cu_seqlens;   // prefill only; nullptr = dense
    const int32_t *seq_order;    // prefill only; nullptr = natural order
    int64_t total_tokens;
    int32_t num_seqs;
    int32_t H;
    int32_t dense_len;           // tokens per sequence when cu_seqlens is null
    int32_t gate_mode;
    float lb, l2_eps, rms_eps;
    // the low-rank decay form (kda_sequence_lowrank): f = W_fb a formed in the
    // step from a [T, lr_rank] and W_fb [H * 128, lr_rank]; null otherwise
    const float *lr_a, *lr_wfb;
    int32_t lr_rank;
    // the chunk kernel's pair counter (one int32, zeroed by its launcher);
    // null = one (sequence, head) pair per workgroup
    int32_t *tickets;
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_decode(const Params &p, bool bf16, hipStream_t stream);
hipError_t launch_prefill(const Params &p, bool bf16, hipStream_t stream);
// Prefill of short sequences with the decode step's layout and a token loop
// (any gate form); short_supported: the batch's token rows fit its 32-bit
// buffer offsets.
bool short_supported(int64_t total_tokens, int32_t num_heads);
hipError_t launch_short(const Params &p, bool bf16, hipStream_t stream);

// Column-split prefill for workloads with few (sequence, head) pairs, where
// one workgroup per pair would leave most of the GPU idle: each pair's state
// columns are spread over several workgroups, the pre-norm readout goes to
// obuf ([T, H, 128] fp32), and an epilogue kernel applies RMSNorm + gate and
// writes the window.  prefill_split_cols returns the columns per lane (1, 2
// or 4) to use for `units` pairs, or 0 when the fused kernel is the better one.
int prefill_split_cols(int64_t units);

// Chunkwise prefill on the matrix cores (16-token chunks); needs the bounded
// gate with a lower bound of magnitude at most 7.5 so that the in-chunk decay
// factors stay inside fp32 range.
bool prefill_chunk_supported(int32_t gate_mode, float lb, int32_t num_heads);
hipError_t launch_prefill_chunk(const Params &p, bool bf16, hipStream_t stream);
// the chunk kernel with f formed from the low-rank factor (p.lr_a, p.lr_wfb,
// p.lr_rank a multiple of 32 up to LOWRANK_MAX_RANK) instead of read from p.f
constexpr int LOWRANK_MAX_RANK = 128;
hipError_t launch_prefill_chunk_lowrank(const Params &p, bool bf16, hipStream_t stream);
// the chunk form for sequences of a few chunks: no pipeline across chunks, two
// workgroups per compute unit (same gate support as launch_prefill_chunk)
hipError_t launch_prefill_chunk_short(const Params &p, bool bf16, hipStream_t stream);
hipError_t launch_prefill_split(const Params &p, bool bf16, float *obuf, int cols_per_lane,
                                hipStream_t stream);
// RMSNorm + gate from a pre-norm readout buffer ([T, H, 128] fp32) into y, and
// the window out (the column-split path's last two kernels)
hipError_t launch_split_finish(const Params &p, bool bf16, const float *obuf, hipStream_t stream);
// the two parts of launch_split_finish on their own: RMSNorm + gate of token
// rows [row_lo, row_lo + rows) of each of nseq sequences seq_rows rows apart
// (a row is one token of one head), and the window out
hipError_t launch_split_epilogue(const Params &p, bool bf16, const float *obuf, int64_t row_lo, int64_t rows,
                                 int64_t seq_rows, int32_t nseq, hipStream_t stream);
hipError_t launch_split_window(const Params &p, bool bf16, hipStream_t stream);

// Chunkwise prefill in two passes for few (sequence, head) pairs: every
// chunk's input-only operands in parallel into records (prefill_scan_record_bytes
// of them), then the chunks of each pair in order with its state columns over
// eight wavefronts, the readout into obuf, then launch_split_finish.  Same gate
// support as the one-pass chunk kernel.
// side_stream (may be null) lets long calls of few pairs run the operand
// passes of later chunk segments beside the state passes of earlier ones;
// cu_host (may be null) is the host copy of cu_seqlens, which lets ragged
// batches of a few sequences do the same.
int64_t prefill_scan_record_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads);
hipError_t launch_prefill_scan(const Params &p, bool bf16, uint8_t *records, float *obuf, hipStream_t stream,
                               hipStream_t side_stream, const int32_t *cu_host);

// Matrix products on either side of the step (the low-rank decay and beta
// projections, the output-gate and output projections):
//   C[m, n] = sum_k A[m, k] B[n, k],  A [M, K] token rows, B [N, K] weights;
// columns [0, n_split) go to C0 (row stride ldc0, bf16 or fp32), columns
// [n_split, N) through a sigmoid to C1 (fp32, row stride ldc1).
struct ProjGemm {
    const void *A;
    const void *B;
    int64_t M;
    int32_t N, K;
    bool a_bf16, b_bf16, c_bf16;   // supported: all bf16; bf16 A with fp32 B, C; all fp32
    bool b_presplit = false;       // fp32 B given as bf16 parts: the high parts of the N rows
                                   // [N, K], then the low parts [N, K] (launch_split_planes)
    void *C0;
    int64_t ldc0;
    float *C1;
    int64_t ldc1;
    int32_t n_split;
};
// K a multiple of 32, n_split a multiple of 4, sizes within the kernel's
// 32-bit buffer offsets
bool proj_gemm_shape_ok(const ProjGemm &g);
// fp32 scratch with which the product splits K across workgroups (few token
// rows); 0 if it would not split
int64_t proj_gemm_scratch_bytes(const ProjGemm &g);
// scratch may be null or smaller than proj_gemm_scratch_bytes: then K is not split
hipError_t launch_proj_gemm(const ProjGemm &g, float *scratch, int64_t scratch_bytes, hipStream_t stream);
// n fp32 values (a multiple of 4) as bf16 parts: out[0, n) the high parts,
// out[n, 2 n) the remainders (the layout of ProjGemm::b_presplit)
hipError_t launch_split_planes(const float *w, uint16_t *out, int64_t n, hipStream_t stream);

}  // namespace kda
