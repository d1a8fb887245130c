// kda_common.hpp -- small device helpers shared by the gfx950 KDA kernels.
//
// Storage-type conversions (bf16 / fp32 inputs, fp16 MFMA operands), the
// gfx950 MFMA 16x16x32 fp16 wrapper and wave reductions.  Everything here is
// plain HIP for CDNA4; there are no other targets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));

// bf16 is stored as the upper 16 bits of an IEEE fp32 value.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct io;

template <> struct io<float> {
    __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float *p, size_t i, float x) { p[i] = x; }
};

template <> struct io<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t *p, size_t i) {
        return bf16_to_f32(p[i].bits);
    }
    __device__ __forceinline__ static void store(bf16_t *p, size_t i, float x) {
        p[i].bits = f32_to_bf16(x);
    }
};

// D = A * B + C for one 16x16 fp32 tile, K = 32 fp16.
// Lane l supplies A row (l % 16), k = 8*(l/16) .. 8*(l/16)+7, B column
// (l % 16) with the same k range; it receives C/D column (l % 16),
// rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two fp32 values -> packed bf16 pair (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Workgroup barrier for LDS traffic only: wait for this wave's LDS operations,
// then meet at s_barrier.  __syncthreads() also carries a global-memory fence,
// which on CDNA waits for every outstanding global load AND store (both are
// counted in vmcnt); that would drain prefetches and output stores at every
// barrier.  Use this where only LDS data is exchanged between the waves.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// log(1 + x) for x >= 0 by D. Goldberg's method ("What Every Computer
// Scientist Should Know About Floating-Point Arithmetic", 1991, Theorem 4):
// with u = fl(1 + x), log1p(x) = log(u) * x / (u - 1), and = x when u == 1.
// The factor x / (u - 1) undoes the rounding of 1 + x, so the result keeps a
// few ulps of relative accuracy even where x is far below 1 (u - 1 is exact).
__device__ __forceinline__ float log1p_nonneg(float x) {
    const float u = 1.f + x;
    return (u == 1.f) ? x : __logf(u) * (x * __builtin_amdgcn_rcpf(u - 1.f));
}

// log(sigmoid(x)) without overflow: min(x, 0) - log(1 + e^{-|x|}).
__device__ __forceinline__ float log_sigmoid(float x) {
    return fminf(x, 0.f) - log1p_nonneg(__expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

__device__ __forceinline__ float fast_exp(float x) {
    // exp(x) = 2^(x * log2(e)) on the hardware exp2 unit.
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

}  // namespace kda
