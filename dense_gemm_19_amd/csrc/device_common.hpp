// device_common.hpp -- gfx950 device helpers: vector types, output conversion,
// the epilogue store (alpha/beta, bias, activation).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kernels.hpp"

namespace dg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Generic pointer into LDS -> LDS address-space pointer (an addrspacecast).
template <class T>
__device__ __forceinline__ __attribute__((address_space(3))) T *as_lds(const char *p) {
    return (__attribute__((address_space(3))) T *)(const_cast<char *>(p));
}

// FP32 -> output element, round to nearest even (the hardware conversions on
// gfx950 round to nearest even and keep NaN a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    _Float16 h = static_cast<_Float16>(f);
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ float load_out(const char *p, int kind) {
    if (kind == OUT_F32) return *reinterpret_cast<const float *>(p);
    uint16_t b = *reinterpret_cast<const uint16_t *>(p);
    return kind == OUT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

__device__ __forceinline__ void store_out(char *p, int kind, float v) {
    if (kind == OUT_F32) *reinterpret_cast<float *>(p) = v;
    else if (kind == OUT_BF16) *reinterpret_cast<uint16_t *>(p) = f32_to_bf16_bits(v);
    else *reinterpret_cast<uint16_t *>(p) = f32_to_f16_bits(v);
}

// Four adjacent output elements (p 4-element aligned, in the C dtype), as one
// vector access.
__device__ __forceinline__ f32x4 load_out4(const char *p, int kind) {
    if (kind == OUT_F32) return *reinterpret_cast<const f32x4 *>(p);
    const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint16_t b = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        v[e] = kind == OUT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
    }
    return v;
}

__device__ __forceinline__ void store_out4(char *p, int kind, const float (&v)[4]) {
    if (kind == OUT_F32) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
        return;
    }
    u32x2 w;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t lo = kind == OUT_BF16 ? f32_to_bf16_bits(v[2 * h]) : f32_to_f16_bits(v[2 * h]);
        const uint32_t hi = kind == OUT_BF16 ? f32_to_bf16_bits(v[2 * h + 1]) : f32_to_f16_bits(v[2 * h + 1]);
        w[h] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x2 *>(p) = w;
}

// Sum of S split-K partials, ((p0 + p1) + p2) + ... always in this order, with
// the loads issued 8 at a time so that their latencies overlap (a runtime-bounded
// loop would otherwise wait for each load before issuing the next).
// load(q) returns partial q.
template <class Load>
__device__ __forceinline__ float sum_partials(int S, Load load) {
    float s = 0.f;
    for (int q0 = 0; q0 < S; q0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = q0 + j < S ? load(q0 + j) : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (q0 + j < S) s = q0 + j == 0 ? v[j] : s + v[j];
    }
    return s;
}

// Split-K hand-off: the ticket a workgroup takes after publishing its partial
// sums; the workgroup that draws `pieces - 1` is the last and adds them up.
// Ordering rests on gfx950's scoped memory operations, not on a C++
// release/acquire pair:
//  - partials are stored with agent-scope atomic stores, which write through
//    the XCD's L2 to the device coherence point, and the caller waits
//    (s_waitcnt vmcnt(0)) until each wave's stores are acknowledged there,
//    then passes a workgroup barrier, so every partial of this piece is at the
//    coherence point before the ticket is taken;
//  - the ticket is an agent-scope atomic, performed at the coherence point, so
//    exactly one piece of a tile draws `pieces - 1`;
//  - the last piece issues its partial loads only after the ticket has
//    returned (through LDS and a barrier) and loads them with agent-scope
//    atomic loads, which read the coherence point, not a stale L1/L2 line.
// An acquire-release fetch-add gives the same guarantee through the HIP
// memory model, but gfx950 implements it by writing back and invalidating the
// XCD's whole L2; measured on MI355X it slowed the split-K shapes by 9-28 %
// (1 x 14336 x 4096 BF16 21.2 -> 23.2 us, 64 x 4096 x 4096 FP16 15.4 -> 18.3
// us, 8 grouped 1 x 4096 x 512 experts 9.9 -> 12.7 us).
__device__ __forceinline__ bool take_last_ticket(int *counter, int pieces) {
    return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == pieces - 1;
}

// GELU in its tanh form (Hendrycks and Gimpel, "Gaussian Error Linear Units",
// 2016): 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).  Evaluated as
// x * sigmoid(2u), u = sqrt(2/pi) (x + 0.044715 x^3), which is the same
// function (0.5 (1 + tanh u) = 1 / (1 + e^(-2u))) without the cancellation of
// 1 + tanh(u) for negative x.  exp2 and the reciprocal are gfx950's own
// instructions (about 1 ulp each); e^(-2u) = 2^(-2u log2 e).  Large negative x
// gives e = +inf and a zero of x's sign; large positive x gives x.
__device__ __forceinline__ float gelu_tanh(float x) {
    const float u = 0.7978845608028654f * fmaf(0.044715f * x, x * x, x);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// act(v): Act numbering.  ReLU keeps NaN (v < 0 is false for NaN) and -0.
__device__ __forceinline__ float activate(int act, float v) {
    if (act == ACT_RELU) return v < 0.0f ? 0.0f : v;
    if (act == ACT_GELU_TANH) return gelu_tanh(v);
    return v;
}

// bias[n] as FP32 (exact for every bias dtype).  The caller has checked e.bias.
__device__ __forceinline__ float load_bias(const Epilogue &e, int64_t n) {
    return load_out(e.bias + n * e.bias_s, e.bias_kind);
}

// out = act(alpha * acc + beta * C_in + bias[n]) (C_in read only when beta != 0,
// bias only when given), rounded to the C dtype and stored at (m, n).  The
// caller has checked m < M and n < N.
__device__ __forceinline__ void epilogue_store(const Epilogue &e, int64_t m, int64_t n, float acc) {
    char *p = e.C + m * e.c_rs + n * e.c_cs;
    float v = e.alpha * acc;
    if (e.beta != 0.0f) v = fmaf(e.beta, load_out(p, e.out_kind), v);
    if (e.bias) v += load_bias(e, n);
    store_out(p, e.out_kind, activate(e.act, v));
}

}  // namespace dg
