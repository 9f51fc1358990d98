// kda_api.hip -- the C ABI of libkda: argument validation, device check and
// kernel dispatch.  No compute happens here; a non-OK status means nothing
// was enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = something else
std::atomic<int> g_dev_kind[kMaxDevices];

kda_status device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return KDA_ERR_DEVICE;
    }
    if (dev >= kMaxDevices) return KDA_ERR_DEVICE;
    int kind = g_dev_kind[dev].load(std::memory_order_relaxed);
    if (kind == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return KDA_ERR_DEVICE;
        }
        kind = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_kind[dev].store(kind, std::memory_order_relaxed);
    }
    return kind == 1 ? KDA_OK : KDA_ERR_DEVICE;
}

// The no-allocation entry point's scratch: one array per device, held until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol); it uses the device address
// that hipGetSymbolAddress returns, taken once per device with that device
// current.  Calls that overlap on one device share it and so race; nothing in
// it needs to start at zero (every byte a call reads, the call wrote first).
__device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];
bool g_scratch_tried[kMaxDevices];

// the current device's address of `scratch`, or null if it cannot be had
void *noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_tried[dev]) {
        g_scratch_tried[dev] = true;
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr)
            g_scratch_addr[dev] = ptr;
        else
            (void)hipGetLastError();
    }
    return g_scratch_addr[dev];
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

kda_status check_config(const kda_config *cfg, const kda_tensors *t, int32_t num_seqs) {
    if (!cfg || !t) return KDA_ERR_INVALID_ARG;
    if (cfg->num_heads <= 0 || num_seqs < 0) return KDA_ERR_INVALID_ARG;
    if (cfg->act_dtype != KDA_F32 && cfg->act_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (cfg->gate_mode < KDA_GATE_BOUNDED || cfg->gate_mode > KDA_GATE_RAW) return KDA_ERR_INVALID_ARG;
    if (!(cfg->l2_eps >= 0.0f) || !(cfg->rms_eps >= 0.0f)) return KDA_ERR_INVALID_ARG;
    if (cfg->gate_lower_bound != cfg->gate_lower_bound) return KDA_ERR_INVALID_ARG;
    if (cfg->prefill_path < KDA_PREFILL_AUTO || cfg->prefill_path > KDA_PREFILL_CHUNK_SHORT)
        return KDA_ERR_INVALID_ARG;
    if (cfg->head_dim_k != kda::DK || cfg->head_dim_v != kda::DV || cfg->conv_taps != kda::TAPS)
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

bool chunk_supported(const kda_config *cfg) {
    return kda::prefill_chunk_supported(cfg->gate_mode, cfg->gate_lower_bound, cfg->num_heads);
}

// Sequences shorter than this on average run the short-sequence kernel under
// AUTO (the token-loop kernels' cost grows with the tokens, the chunk
// kernels' barely below a chunk).  Measured at 64 x 32: with the chunk forms'
// gate the token loop is faster up to 3 tokens, level at 4 (fp32) and slower
// from 6 (fp32) or 4 (bf16) on; with the other gates the token loops are the
// only kernels, the short one faster than the fused one below 8 tokens.
constexpr int64_t CHUNK_MIN_AVG_TOKENS = 4;
constexpr int64_t SHORT_MAX_AVG_TOKENS_OTHER_GATES = 8;

bool auto_short(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    const int64_t lim = chunk_supported(cfg) ? CHUNK_MIN_AVG_TOKENS : SHORT_MAX_AVG_TOKENS_OTHER_GATES;
    return total_tokens < lim * (int64_t)num_seqs && kda::short_supported(total_tokens, cfg->num_heads);
}

bool auto_chunk(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    return chunk_supported(cfg) && total_tokens >= CHUNK_MIN_AVG_TOKENS * (int64_t)num_seqs;
}

// The chunk kernel without a pipeline (two workgroups per compute unit, so
// one pair's state round trip overlaps another's arithmetic) against the
// pipelined one, measured: faster up to 16 tokens per sequence at any batch
// (level at 256 pairs), up to 64 tokens from 512 pairs on (64 x 32 fp32: 86
// vs 106 us at 13 tokens, 241 vs 253 at 64, level at 96, slower from 128;
// 16 x 64 bf16: 104 vs 115 us at 64, level at 128; 8 x 32: slower from 32).
constexpr int64_t CHUNK_SHORT_MAX_AVG_TOKENS = 16;
constexpr int64_t CHUNK_SHORT_MAX_AVG_TOKENS_MANY = 64;
constexpr int64_t CHUNK_SHORT_MANY_UNITS = 512;

bool auto_chunk_short(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    const int64_t units = (int64_t)num_seqs * cfg->num_heads;
    const int64_t lim = units >= CHUNK_SHORT_MANY_UNITS ? CHUNK_SHORT_MAX_AVG_TOKENS_MANY : CHUNK_SHORT_MAX_AVG_TOKENS;
    return auto_chunk(cfg, num_seqs, total_tokens) && total_tokens <= lim * (int64_t)num_seqs;
}

// The two-pass chunk path pays for writing and reading every chunk's operands
// once; it wins when the one-pass kernel, one workgroup per (sequence, head),
// would leave most compute units idle.  Measured against the one-pass kernel:
// 2.4x faster at 32 pairs x 8192 tokens, 1.6x at 64 x 4096, 1.15x at 32 x 128;
// 0.88x at 128 pairs x 2048, about 0.5x from 256 pairs on.
constexpr int64_t SCAN_MAX_UNITS = 64;
constexpr int64_t SCAN_MIN_AVG_TOKENS = 128;

bool scan_shape(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    const int64_t units = (int64_t)num_seqs * cfg->num_heads;
    return chunk_supported(cfg) && num_seqs > 0 && units <= SCAN_MAX_UNITS &&
           total_tokens >= SCAN_MIN_AVG_TOKENS * (int64_t)num_seqs;
}

// The one-pass chunk kernel's pair counter: with it the kernel runs one
// workgroup per compute unit, each taking pairs in the scheduling order until
// none are left, which evens out compute units (and chiplets) that run at
// different clocks; its workspace is this one counter.
constexpr int64_t TICKET_BYTES = 256;

// the path kda_sequence takes is the one-pass chunk kernel (given no
// workspace large enough for the two-pass one)
bool chunk_path(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    if (cfg->prefill_path == KDA_PREFILL_CHUNK) return chunk_supported(cfg);
    return cfg->prefill_path == KDA_PREFILL_AUTO && !auto_short(cfg, num_seqs, total_tokens) &&
           !auto_chunk_short(cfg, num_seqs, total_tokens) && auto_chunk(cfg, num_seqs, total_tokens);
}

// the counter's tickets (pairs plus one per workgroup) stay within int32
bool tickets_fit(const kda_config *cfg, int32_t num_seqs) {
    return (int64_t)num_seqs * cfg->num_heads < (int64_t(1) << 30);
}

// workspace of the two-pass path: the chunk records, then (without o_raw)
// the fp32 readout
int64_t scan_record_bytes(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    const int64_t r = kda::prefill_scan_record_bytes(total_tokens, num_seqs, cfg->num_heads);
    return (r + 255) / 256 * 256;
}
int64_t readout_bytes(const kda_config *cfg, int64_t total_tokens) {
    return total_tokens * cfg->num_heads * kda::DV * (int64_t)sizeof(float);
}

// columns per lane of the split prefill for this shape, 0 = another kernel.
// Automatic choice: the short-sequence kernel below the averages above; else
// the chunkwise kernels wherever the gate allows them (they are the fastest
// at every batch size); else the split kernel for few (sequence, head) pairs,
// else the fused kernel.
int split_cols_for(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    const int64_t units = (int64_t)num_seqs * cfg->num_heads;
    if (cfg->prefill_path == KDA_PREFILL_FUSED || cfg->prefill_path == KDA_PREFILL_CHUNK ||
        cfg->prefill_path == KDA_PREFILL_SHORT || cfg->prefill_path == KDA_PREFILL_SCAN ||
        cfg->prefill_path == KDA_PREFILL_CHUNK_SHORT)
        return 0;
    const int c = kda::prefill_split_cols(units);
    if (cfg->prefill_path == KDA_PREFILL_SPLIT) return c ? c : 4;
    if (auto_short(cfg, num_seqs, total_tokens) || auto_chunk(cfg, num_seqs, total_tokens)) return 0;
    return c;
}

kda_status check_tensors(const kda_config *cfg, const kda_tensors *t, int32_t num_seqs) {
    const void *ins[] = {t->q, t->k, t->v, t->f, t->beta, t->g,
                         t->conv_w, t->A_log, t->dt_bias, t->gamma};
    const void *outs[] = {t->state, t->conv_win, t->y};
    // beta is read one float at a time: 4-byte alignment suffices for it
    for (const void *ptr : ins)
        if (!ptr || (ptr == t->beta ? (reinterpret_cast<uintptr_t>(ptr) & 3u) != 0 : !aligned16(ptr)))
            return KDA_ERR_INVALID_ARG;
    for (const void *ptr : outs)
        if (!ptr || !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    if (t->o_raw && !aligned16(t->o_raw)) return KDA_ERR_INVALID_ARG;
    // no output may coincide with an input or with another output
    const void *all_outs[] = {t->state, t->conv_win, t->y, t->o_raw};
    for (int a = 0; a < 4; ++a) {
        if (!all_outs[a]) continue;
        for (const void *in : ins)
            if (in == all_outs[a]) return KDA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 4; ++b)
            if (all_outs[a] == all_outs[b]) return KDA_ERR_INVALID_ARG;
    }
    if ((int64_t)num_seqs * cfg->num_heads > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

constexpr int32_t PROJ_MAX_HEADS = 1 << 16;     // H * 128 outputs stay well inside 32-bit sizes

// the configuration fields the projections use (heads, activation type, and
// the same validity rules as the step)
kda_status check_proj_config(const kda_config *cfg) {
    kda_tensors dummy;
    std::memset(&dummy, 0, sizeof(dummy));
    const kda_status st = check_config(cfg, &dummy, 0);
    if (st != KDA_OK) return st;
    return cfg->num_heads > PROJ_MAX_HEADS ? KDA_ERR_INVALID_ARG : KDA_OK;
}

struct Span {
    const void *p;
    int64_t bytes;
};
bool overlap(Span a, Span b) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}
// every pointer non-null and 16-byte aligned; no output overlaps an input or
// another output
kda_status check_spans(const Span *ins, int n_in, const Span *outs, int n_out) {
    for (int i = 0; i < n_in; ++i)
        if (!ins[i].p || !aligned16(ins[i].p)) return KDA_ERR_INVALID_ARG;
    for (int o = 0; o < n_out; ++o) {
        if (!outs[o].p || !aligned16(outs[o].p)) return KDA_ERR_INVALID_ARG;
        for (int i = 0; i < n_in; ++i)
            if (overlap(outs[o], ins[i])) return KDA_ERR_INVALID_ARG;
        for (int b = o + 1; b < n_out; ++b)
            if (overlap(outs[o], outs[b])) return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

constexpr int32_t PROJ_MAX_HIDDEN = 1 << 20;
constexpr int32_t PROJ_MAX_RANK = 1024;
constexpr int64_t PROJ_MAX_TOKENS = int64_t(1) << 31;
constexpr int64_t WS_ALIGN = 256;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// the two products of the low-rank gates: x -> (a | beta), a -> f
void lowrank_products(const kda_config *cfg, const void *x, const float *w_fa_bp, const float *w_fb,
                      int32_t hidden, int32_t rank, int64_t tokens, float *f, float *beta, float *a,
                      kda::ProjGemm &g1, kda::ProjGemm &g2) {
    const int32_t H = cfg->num_heads;
    g1.A = x; g1.B = w_fa_bp; g1.M = tokens; g1.N = rank + H; g1.K = hidden;
    g1.a_bf16 = cfg->act_dtype == KDA_BF16; g1.b_bf16 = false; g1.c_bf16 = false;
    g1.C0 = a; g1.ldc0 = rank; g1.C1 = beta; g1.ldc1 = H; g1.n_split = rank;
    g2.A = a; g2.B = w_fb; g2.M = tokens; g2.N = H * kda::DK; g2.K = rank;
    g2.a_bf16 = false; g2.b_bf16 = false; g2.c_bf16 = false;
    g2.C0 = f; g2.ldc0 = (int64_t)H * kda::DK; g2.C1 = nullptr; g2.ldc1 = 0; g2.n_split = g2.N;
}

// From this many token rows the first low-rank product reads its fp32 weights
// [W_fa; W_bp] as bf16 parts split once per call into the workspace, instead
// of splitting them again in every K stage of every token tile.
constexpr int64_t LOWRANK_PRESPLIT_MIN_TOKENS = 512;
int64_t lowrank_planes_bytes(int32_t H, int32_t rank, int32_t hidden) {
    return round_up((int64_t)(rank + H) * hidden * 2 * 2, WS_ALIGN);
}

// one product with the activation type on every side
kda::ProjGemm act_product(const kda_config *cfg, const void *A, const void *B, int64_t M, int32_t N,
                          int32_t K, void *C) {
    kda::ProjGemm g;
    const bool bf = cfg->act_dtype == KDA_BF16;
    g.A = A; g.B = B; g.M = M; g.N = N; g.K = K;
    g.a_bf16 = g.b_bf16 = g.c_bf16 = bf;
    g.C0 = C; g.ldc0 = N; g.C1 = nullptr; g.ldc1 = 0; g.n_split = N;
    return g;
}

kda::Params make_params(const kda_config *cfg, const kda_tensors *t, int32_t num_seqs) {
    kda::Params p;
    p.q = t->q; p.k = t->k; p.v = t->v;
    p.f = t->f; p.beta = t->beta; p.g = t->g;
    p.conv_w = t->conv_w; p.A_log = t->A_log; p.dt_bias = t->dt_bias; p.gamma = t->gamma;
    p.state = t->state; p.win = t->conv_win; p.y = t->y; p.o_raw = t->o_raw;
    p.cu_seqlens = nullptr; p.seq_order = nullptr;
    p.total_tokens = 0; p.num_seqs = num_seqs; p.H = cfg->num_heads; p.dense_len = 0;
    p.gate_mode = cfg->gate_mode;
    p.lb = cfg->gate_lower_bound; p.l2_eps = cfg->l2_eps; p.rms_eps = cfg->rms_eps;
    p.lr_a = nullptr; p.lr_wfb = nullptr; p.lr_rank = 0;
    p.tickets = nullptr;
    return p;
}

}  // namespace

extern "C" {

kda_status kda_device_check(void) { return device_ok(); }

int32_t kda_version(void) { return KDA_VERSION; }

const char *kda_status_string(int32_t status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or enum, aliasing)";
        case KDA_ERR_UNSUPPORTED: return "unsupported shape (libkda needs dk = dv = 128 and 4 conv taps)";
        case KDA_ERR_DEVICE: return "no usable device (no current HIP device, or it is not gfx950)";
        case KDA_ERR_LAUNCH: return "kernel launch failed";
        case KDA_ERR_SCRATCH_LIMIT:
            return "the call needs more than the library's static scratch (KDA_NOALLOC_SCRATCH_BYTES); "
                   "use the variant that takes a workspace";
        default: return "unknown status";
    }
}

kda_status kda_token_step(const kda_config *cfg, const kda_tensors *t, int32_t num_seqs, void *stream) {
    kda_status st = check_config(cfg, t, num_seqs);
    if (st != KDA_OK) return st;
    if (num_seqs == 0) return KDA_OK;     // nothing to do; pointers are not inspected
    st = check_tensors(cfg, t, num_seqs);
    if (st != KDA_OK) return st;
    st = device_ok();
    if (st != KDA_OK) return st;
    kda::Params p = make_params(cfg, t, num_seqs);
    p.total_tokens = num_seqs;
    p.dense_len = 1;
    const hipError_t e = kda::launch_decode(p, cfg->act_dtype == KDA_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int64_t kda_sequence_workspace_size(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    kda_tensors dummy;
    std::memset(&dummy, 0, sizeof(dummy));
    const kda_status st = check_config(cfg, &dummy, num_seqs);
    if (st != KDA_OK) return st;
    if (total_tokens < 0) return KDA_ERR_INVALID_ARG;
    if (num_seqs == 0 || total_tokens == 0) return 0;
    if (cfg->prefill_path == KDA_PREFILL_SCAN ||
        (cfg->prefill_path == KDA_PREFILL_AUTO && scan_shape(cfg, num_seqs, total_tokens)))
        return scan_record_bytes(cfg, num_seqs, total_tokens) + readout_bytes(cfg, total_tokens);
    if (split_cols_for(cfg, num_seqs, total_tokens) == 0)
        return chunk_path(cfg, num_seqs, total_tokens) && tickets_fit(cfg, num_seqs) ? TICKET_BYTES : 0;
    return readout_bytes(cfg, total_tokens);
}

}  // extern "C"

namespace {
// the checks kda_sequence and kda_sequence_lowrank share, after the tensors':
// offsets (device alignment, the host copy), the dense length, sizes
kda_status check_packing(const kda_config *cfg, int32_t num_seqs, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, const int32_t *seq_order, int64_t total_tokens,
                         int32_t *dense_len) {
    if ((cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) ||
        (seq_order && (reinterpret_cast<uintptr_t>(seq_order) & 3u)))
        return KDA_ERR_INVALID_ARG;
    // the host copy of the offsets, when given, must describe a valid packing
    if (cu_seqlens_host) {
        if (!cu_seqlens) return KDA_ERR_INVALID_ARG;
        if (cu_seqlens_host[0] != 0 || (int64_t)cu_seqlens_host[num_seqs] != total_tokens) return KDA_ERR_INVALID_ARG;
        for (int32_t n = 0; n < num_seqs; ++n)
            if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return KDA_ERR_INVALID_ARG;
    }
    *dense_len = 0;
    if (!cu_seqlens && num_seqs > 0) {
        if (total_tokens % num_seqs != 0) return KDA_ERR_INVALID_ARG;
        if (total_tokens / num_seqs > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
        *dense_len = (int32_t)(total_tokens / num_seqs);
    }
    // row offsets are formed in 64-bit arithmetic; keep them well inside it
    if (total_tokens > (int64_t(1) << 40) / ((int64_t)cfg->num_heads * kda::DK)) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}
}  // namespace

extern "C" {

kda_status kda_sequence(const kda_config *cfg, const kda_tensors *t, int32_t num_seqs,
                        const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                        const int32_t *seq_order, int64_t total_tokens, void *workspace,
                        int64_t workspace_bytes, void *stream, void *side_stream) {
    kda_status st = check_config(cfg, t, num_seqs);
    if (st != KDA_OK) return st;
    if (total_tokens < 0) return KDA_ERR_INVALID_ARG;
    if (num_seqs == 0 && total_tokens != 0) return KDA_ERR_INVALID_ARG;
    if (total_tokens == 0) return KDA_OK; // every sequence is empty; pointers are not inspected
    st = check_tensors(cfg, t, num_seqs);
    if (st != KDA_OK) return st;
    int32_t dense_len = 0;
    st = check_packing(cfg, num_seqs, cu_seqlens, cu_seqlens_host, seq_order, total_tokens, &dense_len);
    if (st != KDA_OK) return st;
    if (side_stream && side_stream == stream) return KDA_ERR_INVALID_ARG;
    if (workspace_bytes < 0 || (workspace && !aligned16(workspace))) return KDA_ERR_INVALID_ARG;
    // the readout buffer of the split path: o_raw, else a large enough workspace
    const int cols = split_cols_for(cfg, num_seqs, total_tokens);
    float *obuf = nullptr;
    if (cols) {
        const int64_t need = total_tokens * cfg->num_heads * kda::DV * (int64_t)sizeof(float);
        if (t->o_raw)
            obuf = t->o_raw;
        else if (workspace && workspace_bytes >= need)
            obuf = static_cast<float *>(workspace);
        else if (cfg->prefill_path == KDA_PREFILL_SPLIT)
            return KDA_ERR_INVALID_ARG;
    }
    // the two-pass path: records in the workspace, the readout in o_raw or after them
    uint8_t *scan_records = nullptr;
    float *scan_obuf = nullptr;
    if (cfg->prefill_path == KDA_PREFILL_SCAN ||
        (cfg->prefill_path == KDA_PREFILL_AUTO && scan_shape(cfg, num_seqs, total_tokens))) {
        if (cfg->prefill_path == KDA_PREFILL_SCAN && !chunk_supported(cfg)) return KDA_ERR_UNSUPPORTED;
        const int64_t rb = scan_record_bytes(cfg, num_seqs, total_tokens);
        const int64_t need = rb + (t->o_raw ? 0 : readout_bytes(cfg, total_tokens));
        if (workspace && workspace_bytes >= need) {
            scan_records = static_cast<uint8_t *>(workspace);
            scan_obuf = t->o_raw ? t->o_raw : reinterpret_cast<float *>(scan_records + rb);
        } else if (cfg->prefill_path == KDA_PREFILL_SCAN) {
            return KDA_ERR_INVALID_ARG;
        }
    }
    if ((cfg->prefill_path == KDA_PREFILL_CHUNK || cfg->prefill_path == KDA_PREFILL_CHUNK_SHORT) &&
        !chunk_supported(cfg))
        return KDA_ERR_UNSUPPORTED;
    if (cfg->prefill_path == KDA_PREFILL_SHORT && !kda::short_supported(total_tokens, cfg->num_heads))
        return KDA_ERR_UNSUPPORTED;
    st = device_ok();
    if (st != KDA_OK) return st;
    kda::Params p = make_params(cfg, t, num_seqs);
    p.cu_seqlens = cu_seqlens;
    p.seq_order = seq_order;
    p.total_tokens = total_tokens;
    p.dense_len = dense_len;
    const bool bf16 = cfg->act_dtype == KDA_BF16;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (scan_records)
        e = kda::launch_prefill_scan(p, bf16, scan_records, scan_obuf, s, static_cast<hipStream_t>(side_stream),
                                     cu_seqlens_host);
    else if (obuf)
        e = kda::launch_prefill_split(p, bf16, obuf, cols, s);
    else if (cfg->prefill_path == KDA_PREFILL_SHORT ||
             (cfg->prefill_path == KDA_PREFILL_AUTO && auto_short(cfg, num_seqs, total_tokens)))
        e = kda::launch_short(p, bf16, s);
    else if (cfg->prefill_path == KDA_PREFILL_CHUNK_SHORT ||
             (cfg->prefill_path == KDA_PREFILL_AUTO && auto_chunk_short(cfg, num_seqs, total_tokens)))
        e = kda::launch_prefill_chunk_short(p, bf16, s);
    else if (cfg->prefill_path == KDA_PREFILL_CHUNK ||
             (cfg->prefill_path == KDA_PREFILL_AUTO && auto_chunk(cfg, num_seqs, total_tokens))) {
        if (workspace && workspace_bytes >= TICKET_BYTES && tickets_fit(cfg, num_seqs))
            p.tickets = static_cast<int32_t *>(workspace);
        e = kda::launch_prefill_chunk(p, bf16, s);
    }
    else
        e = kda::launch_prefill(p, bf16, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status kda_sequence_lowrank(const kda_config *cfg, const kda_tensors *t, int32_t num_seqs,
                                const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                const int32_t *seq_order, int64_t total_tokens, const float *a,
                                const float *w_fb, int32_t rank, void *stream) {
    kda_status st = check_config(cfg, t, num_seqs);
    if (st != KDA_OK) return st;
    if (total_tokens < 0 || (num_seqs == 0 && total_tokens != 0)) return KDA_ERR_INVALID_ARG;
    if (rank < 32 || rank % 32 != 0) return KDA_ERR_INVALID_ARG;
    if (rank > kda::LOWRANK_MAX_RANK) return KDA_ERR_UNSUPPORTED;
    if (cfg->prefill_path != KDA_PREFILL_AUTO && cfg->prefill_path != KDA_PREFILL_CHUNK) return KDA_ERR_UNSUPPORTED;
    if (!chunk_supported(cfg)) return KDA_ERR_UNSUPPORTED;
    if (total_tokens == 0) return KDA_OK;
    if (t->f) return KDA_ERR_INVALID_ARG;          // f is formed in the step
    // the tensors' checks with a in the place of f, then w_fb like an input
    kda_tensors tt = *t;
    tt.f = a;
    st = check_tensors(cfg, &tt, num_seqs);
    if (st != KDA_OK) return st;
    if (!w_fb || !aligned16(w_fb)) return KDA_ERR_INVALID_ARG;
    for (const void *o : {(const void *)t->state, (const void *)t->conv_win, (const void *)t->y,
                          (const void *)t->o_raw})
        if (o == w_fb) return KDA_ERR_INVALID_ARG;
    int32_t dense_len = 0;
    st = check_packing(cfg, num_seqs, cu_seqlens, cu_seqlens_host, seq_order, total_tokens, &dense_len);
    if (st != KDA_OK) return st;
    st = device_ok();
    if (st != KDA_OK) return st;
    kda::Params p = make_params(cfg, t, num_seqs);
    p.f = nullptr;
    p.cu_seqlens = cu_seqlens;
    p.seq_order = seq_order;
    p.total_tokens = total_tokens;
    p.dense_len = dense_len;
    p.lr_a = a;
    p.lr_wfb = w_fb;
    p.lr_rank = rank;
    const hipError_t e = kda::launch_prefill_chunk_lowrank(p, cfg->act_dtype == KDA_BF16,
                                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int64_t kda_projection_workspace_size(const kda_config *cfg, int32_t which, int32_t hidden,
                                      int32_t rank, int64_t tokens) {
    const kda_status st = check_proj_config(cfg);
    if (st != KDA_OK) return st;
    if (hidden <= 0 || hidden > PROJ_MAX_HIDDEN || tokens < 0 || tokens > PROJ_MAX_TOKENS)
        return KDA_ERR_INVALID_ARG;
    const int32_t HD = cfg->num_heads * kda::DV;
    if (tokens == 0) return 0;
    if (which == KDA_PROJ_LOWRANK_GATES) {
        if (rank < 32 || rank > PROJ_MAX_RANK || rank % 32 != 0 || hidden % 32 != 0) return KDA_ERR_INVALID_ARG;
        kda::ProjGemm g1, g2;
        lowrank_products(cfg, nullptr, nullptr, nullptr, hidden, rank, tokens, nullptr, nullptr, nullptr, g1, g2);
        int64_t planes = 0;
        if (tokens >= LOWRANK_PRESPLIT_MIN_TOKENS) {
            g1.b_presplit = true;
            planes = lowrank_planes_bytes(cfg->num_heads, rank, hidden);
        }
        const int64_t scratch = std::max(kda::proj_gemm_scratch_bytes(g1), kda::proj_gemm_scratch_bytes(g2));
        return round_up(tokens * rank * 4, WS_ALIGN) + planes + scratch;
    }
    if (which == KDA_PROJ_LOWRANK_FACTOR) {
        if (rank < 32 || rank > PROJ_MAX_RANK || rank % 32 != 0 || hidden % 32 != 0) return KDA_ERR_INVALID_ARG;
        kda::ProjGemm g1, g2;
        lowrank_products(cfg, nullptr, nullptr, nullptr, hidden, rank, tokens, nullptr, nullptr, nullptr, g1, g2);
        int64_t planes = 0;
        if (tokens >= LOWRANK_PRESPLIT_MIN_TOKENS) {
            g1.b_presplit = true;
            planes = lowrank_planes_bytes(cfg->num_heads, rank, hidden);
        }
        return planes + kda::proj_gemm_scratch_bytes(g1);
    }
    if (which == KDA_PROJ_GATE) {
        if (hidden % 32 != 0) return KDA_ERR_INVALID_ARG;
        return kda::proj_gemm_scratch_bytes(act_product(cfg, nullptr, nullptr, tokens, HD, hidden, nullptr));
    }
    if (which == KDA_PROJ_OUTPUT) {
        if (hidden % 4 != 0) return KDA_ERR_INVALID_ARG;
        return kda::proj_gemm_scratch_bytes(act_product(cfg, nullptr, nullptr, tokens, hidden, HD, nullptr));
    }
    return KDA_ERR_INVALID_ARG;
}

}  // extern "C"

namespace {

// kda_lowrank_gates with its workspace given (the caller's, or the static
// scratch of the no-allocation variant)
kda_status lowrank_gates_impl(const kda_config *cfg, const void *x, const float *w_fa_bp, const float *w_fb,
                              int32_t hidden, int32_t rank, int64_t tokens, float *f, float *beta,
                              void *workspace, int64_t workspace_bytes, void *stream, bool static_scratch) {
    kda_status st = check_proj_config(cfg);
    if (st != KDA_OK) return st;
    if (hidden <= 0 || hidden > PROJ_MAX_HIDDEN || hidden % 32 != 0) return KDA_ERR_INVALID_ARG;
    if (rank < 32 || rank > PROJ_MAX_RANK || rank % 32 != 0) return KDA_ERR_INVALID_ARG;
    if (tokens < 0 || tokens > PROJ_MAX_TOKENS || workspace_bytes < 0) return KDA_ERR_INVALID_ARG;
    if (tokens == 0) return KDA_OK;       // pointers are not inspected
    const int32_t H = cfg->num_heads;
    const int64_t eb = cfg->act_dtype == KDA_BF16 ? 2 : 4;
    const int64_t a_bytes = round_up(tokens * rank * 4, WS_ALIGN);
    if (static_scratch) {
        if (a_bytes > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH_LIMIT;
    } else if (workspace_bytes < a_bytes) {
        return KDA_ERR_INVALID_ARG;
    }
    const Span ins[] = {{x, tokens * hidden * eb}, {w_fa_bp, (int64_t)(rank + H) * hidden * 4},
                        {w_fb, (int64_t)H * kda::DK * rank * 4}};
    // (the static scratch is the library's own array: no caller buffer can overlap it)
    const Span outs[] = {{f, tokens * H * kda::DK * 4}, {workspace, workspace_bytes}};
    st = check_spans(ins, 3, outs, static_scratch ? 1 : 2);
    if (st != KDA_OK) return st;
    // beta needs word alignment only (it is written one value at a time)
    const Span bs = {beta, tokens * H * 4};
    if (!beta || (reinterpret_cast<uintptr_t>(beta) & 3u)) return KDA_ERR_INVALID_ARG;
    for (const Span &o : ins)
        if (overlap(bs, o)) return KDA_ERR_INVALID_ARG;
    for (int o = 0; o < (static_scratch ? 1 : 2); ++o)
        if (overlap(bs, outs[o])) return KDA_ERR_INVALID_ARG;
    kda::ProjGemm g1, g2;
    lowrank_products(cfg, x, w_fa_bp, w_fb, hidden, rank, tokens, f, beta, nullptr, g1, g2);
    if (!kda::proj_gemm_shape_ok(g1) || !kda::proj_gemm_shape_ok(g2)) return KDA_ERR_INVALID_ARG;
    st = device_ok();
    if (st != KDA_OK) return st;
    if (static_scratch) {
        workspace = noalloc_scratch();
        if (!workspace) return KDA_ERR_DEVICE;
        workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    float *a = static_cast<float *>(workspace);
    g1.C0 = a;
    g2.A = a;
    // the weights' bf16 parts after a, when the workspace holds them
    const int64_t planes = lowrank_planes_bytes(H, rank, hidden);
    uint16_t *wparts = nullptr;
    int64_t used = a_bytes;
    if (tokens >= LOWRANK_PRESPLIT_MIN_TOKENS && workspace_bytes >= a_bytes + planes) {
        wparts = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + a_bytes);
        g1.B = wparts;
        g1.b_presplit = true;
        used += planes;
    }
    float *scratch_f = reinterpret_cast<float *>(static_cast<char *>(workspace) + used);
    const int64_t scratch_bytes = workspace_bytes - used;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (wparts) e = kda::launch_split_planes(w_fa_bp, wparts, (int64_t)(rank + H) * hidden, s);
    if (e == hipSuccess) e = kda::launch_proj_gemm(g1, scratch_bytes > 0 ? scratch_f : nullptr, scratch_bytes, s);
    if (e == hipSuccess) e = kda::launch_proj_gemm(g2, scratch_bytes > 0 ? scratch_f : nullptr, scratch_bytes, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status kda_lowrank_gates(const kda_config *cfg, const void *x, const float *w_fa_bp,
                             const float *w_fb, int32_t hidden, int32_t rank, int64_t tokens,
                             float *f, float *beta, void *workspace, int64_t workspace_bytes,
                             void *stream) {
    return lowrank_gates_impl(cfg, x, w_fa_bp, w_fb, hidden, rank, tokens, f, beta, workspace, workspace_bytes,
                              stream, false);
}

kda_status kda_lowrank_gates_noalloc(const kda_config *cfg, const void *x, const float *w_fa_bp,
                                     const float *w_fb, int32_t hidden, int32_t rank, int64_t tokens,
                                     float *f, float *beta, void *stream) {
    return lowrank_gates_impl(cfg, x, w_fa_bp, w_fb, hidden, rank, tokens, f, beta, nullptr, 0, stream, true);
}

kda_status kda_lowrank_factor(const kda_config *cfg, const void *x, const float *w_fa_bp, int32_t hidden,
                              int32_t rank, int64_t tokens, float *a, float *beta, void *workspace,
                              int64_t workspace_bytes, void *stream) {
    kda_status st = check_proj_config(cfg);
    if (st != KDA_OK) return st;
    if (hidden <= 0 || hidden > PROJ_MAX_HIDDEN || hidden % 32 != 0) return KDA_ERR_INVALID_ARG;
    if (rank < 32 || rank > PROJ_MAX_RANK || rank % 32 != 0) return KDA_ERR_INVALID_ARG;
    if (tokens < 0 || tokens > PROJ_MAX_TOKENS || workspace_bytes < 0) return KDA_ERR_INVALID_ARG;
    if (tokens == 0) return KDA_OK;       // pointers are not inspected
    if (workspace && !aligned16(workspace)) return KDA_ERR_INVALID_ARG;
    const int32_t H = cfg->num_heads;
    const int64_t eb = cfg->act_dtype == KDA_BF16 ? 2 : 4;
    const Span ins[] = {{x, tokens * hidden * eb}, {w_fa_bp, (int64_t)(rank + H) * hidden * 4}};
    const Span outs[] = {{a, tokens * rank * 4}, {workspace, workspace ? workspace_bytes : 0}};
    st = check_spans(ins, 2, outs, workspace ? 2 : 1);
    if (st != KDA_OK) return st;
    const Span bs = {beta, tokens * H * 4};
    if (!beta || (reinterpret_cast<uintptr_t>(beta) & 3u)) return KDA_ERR_INVALID_ARG;
    for (const Span &o : ins)
        if (overlap(bs, o)) return KDA_ERR_INVALID_ARG;
    for (int o = 0; o < (workspace ? 2 : 1); ++o)
        if (overlap(bs, outs[o])) return KDA_ERR_INVALID_ARG;
    kda::ProjGemm g1, g2;
    lowrank_products(cfg, x, w_fa_bp, nullptr, hidden, rank, tokens, nullptr, beta, a, g1, g2);
    if (!kda::proj_gemm_shape_ok(g1)) return KDA_ERR_INVALID_ARG;
    st = device_ok();
    if (st != KDA_OK) return st;
    const int64_t planes = lowrank_planes_bytes(H, rank, hidden);
    uint16_t *wparts = nullptr;
    int64_t used = 0;
    if (tokens >= LOWRANK_PRESPLIT_MIN_TOKENS && workspace && workspace_bytes >= planes) {
        wparts = static_cast<uint16_t *>(workspace);
        g1.B = wparts;
        g1.b_presplit = true;
        used = planes;
    }
    const int64_t scratch_bytes = workspace ? workspace_bytes - used : 0;
    float *scratch_f = scratch_bytes > 0 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + used) : nullptr;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (wparts) e = kda::launch_split_planes(w_fa_bp, wparts, (int64_t)(rank + H) * hidden, s);
    if (e == hipSuccess) e = kda::launch_proj_gemm(g1, scratch_f, scratch_bytes, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

namespace {
kda_status run_act_product(const kda_config *cfg, const kda::ProjGemm &g, int64_t a_bytes, int64_t b_bytes,
                           int64_t c_bytes, void *workspace, int64_t workspace_bytes, void *stream) {
    if (workspace_bytes < 0 || (workspace && !aligned16(workspace))) return KDA_ERR_INVALID_ARG;
    const Span ins[] = {{g.A, a_bytes}, {g.B, b_bytes}};
    const Span outs[] = {{g.C0, c_bytes}, {workspace, workspace ? workspace_bytes : 0}};
    kda_status st = check_spans(ins, 2, outs, workspace ? 2 : 1);
    if (st != KDA_OK) return st;
    if (!kda::proj_gemm_shape_ok(g)) return KDA_ERR_INVALID_ARG;
    st = device_ok();
    if (st != KDA_OK) return st;
    const hipError_t e = kda::launch_proj_gemm(g, static_cast<float *>(workspace), workspace ? workspace_bytes : 0,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}
}  // namespace

kda_status kda_gate_projection(const kda_config *cfg, const void *x, const void *w_g, int32_t hidden,
                               int64_t tokens, void *g, void *workspace, int64_t workspace_bytes,
                               void *stream) {
    const kda_status st = check_proj_config(cfg);
    if (st != KDA_OK) return st;
    if (hidden <= 0 || hidden > PROJ_MAX_HIDDEN || hidden % 32 != 0) return KDA_ERR_INVALID_ARG;
    if (tokens < 0 || tokens > PROJ_MAX_TOKENS) return KDA_ERR_INVALID_ARG;
    if (tokens == 0) return KDA_OK;
    const int32_t HD = cfg->num_heads * kda::DV;
    const int64_t eb = cfg->act_dtype == KDA_BF16 ? 2 : 4;
    return run_act_product(cfg, act_product(cfg, x, w_g, tokens, HD, hidden, g), tokens * hidden * eb,
                           (int64_t)HD * hidden * eb, tokens * HD * eb, workspace, workspace_bytes, stream);
}

kda_status kda_output_projection(const kda_config *cfg, const void *y, const void *w_o, int32_t hidden,
                                 int64_t tokens, void *out, void *workspace, int64_t workspace_bytes,
                                 void *stream) {
    const kda_status st = check_proj_config(cfg);
    if (st != KDA_OK) return st;
    if (hidden <= 0 || hidden > PROJ_MAX_HIDDEN || hidden % 4 != 0) return KDA_ERR_INVALID_ARG;
    if (tokens < 0 || tokens > PROJ_MAX_TOKENS) return KDA_ERR_INVALID_ARG;
    if (tokens == 0) return KDA_OK;
    const int32_t HD = cfg->num_heads * kda::DV;
    const int64_t eb = cfg->act_dtype == KDA_BF16 ? 2 : 4;
    return run_act_product(cfg, act_product(cfg, y, w_o, tokens, hidden, HD, out), tokens * HD * eb,
                           (int64_t)hidden * HD * eb, tokens * hidden * eb, workspace, workspace_bytes, stream);
}

}  // extern "C"
