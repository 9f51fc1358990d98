// kda_device.hpp -- device helpers shared by the libkda kernels: activation
// I/O in fp32 or bf16, the pointwise functions of the pre-step, the decay
// gate, and wavefront reductions built on DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.hpp"

namespace kda {

// ---------------------------------------------------------------- activations

struct F32 {
    using storage = float;
    static __device__ __forceinline__ float load1(const void *p, int64_t i) {
        return static_cast<const float *>(p)[i];
    }
    // two consecutive elements; i must be even
    static __device__ __forceinline__ float2 load2(const void *p, int64_t i) {
        return *reinterpret_cast<const float2 *>(static_cast<const float *>(p) + i);
    }
    static __device__ __forceinline__ void store2(void *p, int64_t i, float2 x) {
        *reinterpret_cast<float2 *>(static_cast<float *>(p) + i) = x;
    }
    static __device__ __forceinline__ void store4(void *p, int64_t i, float4 x) {
        *reinterpret_cast<float4 *>(static_cast<float *>(p) + i) = x;
    }
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// two fp32 -> packed bf16 (v_cvt_pk_bf16_f32: round to nearest even, NaN
// stays NaN); the first value in the low half
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2v x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v));
}

struct BF16 {
    using storage = uint16_t;
    static __device__ __forceinline__ float load1(const void *p, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
    static __device__ __forceinline__ float2 load2(const void *p, int64_t i) {
        uint32_t w = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(p) + i);
        return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    }
    static __device__ __forceinline__ void store2(void *p, int64_t i, float2 x) {
        *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p) + i) = pack_bf16x2(x.x, x.y);
    }
    static __device__ __forceinline__ void store4(void *p, int64_t i, float4 x) {
        uint2 w;
        w.x = pack_bf16x2(x.x, x.y);
        w.y = pack_bf16x2(x.z, x.w);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p) + i) = w;
    }
};

// ------------------------------------------------------------ pointwise math

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + __expf(-x)); }

__device__ __forceinline__ float silu(float x) { return x * sigmoid(x); }

// alpha = exp(gk) for one key channel; expA = exp(A_log) of that channel
__device__ __forceinline__ float decay(float f, float expA, float dtb, int32_t mode, float lb) {
    float gk;
    if (mode == GATE_RAW) {
        gk = f;
    } else {
        const float z = expA * (f + dtb);
        gk = (mode == GATE_BOUNDED) ? lb * sigmoid(z) : lb * z;
    }
    return __expf(gk);
}

// --------------------------------------------------------- lane exchanges

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;   // lane i <-> 15-i within 16 lanes

// sum over each aligned group of 8 lanes, result in every lane of the group
// (identical bits in all 8 lanes: every partial sum is formed symmetrically)
__device__ __forceinline__ float sum8(float x) {
    x += dpp<DPP_QUAD_XOR1>(x);
    x += dpp<DPP_QUAD_XOR2>(x);
    x += dpp<DPP_HALF_MIRROR>(x);
    return x;
}

__device__ __forceinline__ float sum16(float x) {
    x = sum8(x);
    x += dpp<DPP_ROW_MIRROR>(x);
    return x;
}

// Across rows: v_permlane16_swap / v_permlane32_swap exchange rows 2k and
// 2k + 1 / the two halves of the wavefront inside the VALU (no LDS round
// trip).  With both operands equal, the two results hold the two halves of
// every pair in every lane, so the sums below are formed in the same order
// in all lanes.
__device__ __forceinline__ float sum32(float x) {
    x = sum16(x);
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ float sum64(float x) {
    x = sum32(x);
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ---------------------------------------------------------- buffer accesses
// A raw buffer resource lives in scalar registers; each access then needs
// only a 32-bit per-lane byte offset (plus a scalar offset), instead of a
// 64-bit address per load, and reads past num_records return 0.

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int RAW_BUFFER_FLAGS = 0x00020000;   // untyped buffer, word 3 of the descriptor

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             RAW_BUFFER_FLAGS);
}
__device__ __forceinline__ float bld_f32(Rsrc r, uint32_t voff, uint32_t soff = 0) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ float2 bld_f32x2(Rsrc r, uint32_t voff, uint32_t soff = 0) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
}
__device__ __forceinline__ void bst_f32(Rsrc r, float v, uint32_t voff, uint32_t soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}
__device__ __forceinline__ void bst_f32x2(Rsrc r, float2 v, uint32_t voff, uint32_t soff = 0) {
    const u32x2 w = {__float_as_uint(v.x), __float_as_uint(v.y)};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, voff, soff, 0);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 bld_f32x4(Rsrc r, uint32_t voff, uint32_t soff = 0) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                       __uint_as_float(w.w));
}
__device__ __forceinline__ void bst_f32x4(Rsrc r, float4 v, uint32_t voff, uint32_t soff = 0) {
    const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, 0);
}
// A 16-byte store reads its data registers after it issues; an instruction
// that writes one of them right behind it can change what is stored.  The
// compiler puts the needed wait states behind a buffer store whose scalar
// offset is a constant, but not behind one with an SGPR scalar offset (on
// gfx950 that form lost stored data).  This store therefore takes its whole
// offset per lane, through an opaque copy that keeps a constant part from
// being moved back into an SGPR, and the scalar offset 0.
template <int CPOL = 0>
__device__ __forceinline__ void bst_f32x4_at(Rsrc r, float4 v, uint32_t off) {
    const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w)};
    asm volatile("" : "+v"(off));
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, CPOL);
}
// two consecutive activations (element index i, even) through a buffer
template <typename Act> struct BufAct;
// Raw2 / load_raw2 / unpack2 split a load from its conversion, so that a load
// issued ahead of time is not waited for until the value is unpacked.
template <> struct BufAct<F32> {
    static constexpr uint32_t ELEM = 4;
    typedef float2 Raw2;
    static __device__ __forceinline__ float2 load2(Rsrc r, uint32_t i) { return bld_f32x2(r, i * 4); }
    static __device__ __forceinline__ void store2(Rsrc r, uint32_t i, float2 x) { bst_f32x2(r, x, i * 4); }
    static __device__ __forceinline__ Raw2 load_raw2(Rsrc r, uint32_t i) { return bld_f32x2(r, i * 4); }
    static __device__ __forceinline__ float2 unpack2(Raw2 x) { return x; }
};
template <> struct BufAct<BF16> {
    static constexpr uint32_t ELEM = 2;
    typedef uint32_t Raw2;
    static __device__ __forceinline__ Raw2 load_raw2(Rsrc r, uint32_t i) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, i * 2, 0, 0);
    }
    static __device__ __forceinline__ float2 unpack2(Raw2 w) {
        return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    }
    static __device__ __forceinline__ float2 load2(Rsrc r, uint32_t i) {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, i * 2, 0, 0);
        return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    }
    static __device__ __forceinline__ void store2(Rsrc r, uint32_t i, float2 x) {
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(x.x, x.y), r, i * 2, 0, 0);
    }
};

// one activation (element index i) through a buffer
template <typename Act> __device__ __forceinline__ float bld_one(Rsrc r, uint32_t i);
template <> __device__ __forceinline__ float bld_one<F32>(Rsrc r, uint32_t i) { return bld_f32(r, i * 4); }
template <> __device__ __forceinline__ float bld_one<BF16>(Rsrc r, uint32_t i) {
    const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, (i & ~1u) * 2, 0, 0);
    return __uint_as_float((i & 1u) ? (w & 0xffff0000u) : (w << 16));
}

// ------------------------------------------------------------ sequences

struct Range {
    int64_t lo, len;
};

// token range of sequence n: from cu_seqlens (clamped to [0, total_tokens)),
// or the dense layout when cu_seqlens is null
__device__ __forceinline__ Range seq_range(const Params &p, int n) {
    Range r;
    if (p.cu_seqlens) {
        int64_t a = p.cu_seqlens[n], b = p.cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
        b = b < a ? a : (b > p.total_tokens ? p.total_tokens : b);
        r.lo = a;
        r.len = b - a;
    } else {
        r.lo = (int64_t)n * p.dense_len;
        r.len = p.dense_len;
    }
    return r;
}

}  // namespace kda
