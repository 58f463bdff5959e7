// la_device.h -- device-side helpers shared by the liblinattn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage tag for bfloat16 tensors (the ABI passes raw 16-bit words).
struct bf16_t {
    uint16_t bits;
};

// ---- bfloat16 <-> float ------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even) packed low/high in one dword.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi)
{
    f32x2 f = {lo, hi};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t to_bf(float x)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// ---- feature map ------------------------------------------------------------------------
// phi(x) = ELU(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise (strictly positive).
// The fast form (the hardware exp2 of x log2 e, relative error about |x| 2^-24) feeds the
// matrix-core kernels, bf16 and float32; the accurate form serves the vector-ALU and decode
// kernels.
__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ float phi_exact(float x) { return x > 0.f ? x + 1.f : expf(x); }
// The feature of one element: phi_exact(x), or x itself when q and k are already features.
__device__ __forceinline__ float feature(float x, bool identity) { return identity ? x : phi_exact(x); }

// ---- decay of the carried state (the retention recurrence) -----------------------------
// The decay gamma of head bh % H as every form reads it: 1 when gamma is null (no decay), NaN
// when the value is negative or NaN (outside the contract; the NaN then reaches every output
// and the state of that head, in the prefill and the decode forms alike -- nothing is clamped).
__device__ __forceinline__ float decay_gamma(const float *gamma, long bh, int H)
{
    if (!gamma)
        return 1.f;
    const float g = gamma[bh % H];
    return g >= 0.f ? g : __builtin_nanf("");
}
// log2 of that decay (0: none), clamped below at -1000 so that gamma = 0 gives gamma^0 = 1 and
// gamma^n = 0 for n > 0 through exp2 without infinities; NaN stays NaN.
__device__ __forceinline__ float decay_log2(const float *gamma, long bh, int H)
{
    const float g = decay_gamma(gamma, bh, H);
    return g != g ? g : fmaxf(log2f(g), -1000.f);
}
__device__ __forceinline__ float decay_pow(float lg, int n) { return exp2f(lg * (float)n); }

// ---- generic element access for the vector-ALU kernels -----------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static float ld(const float *p, size_t i) { return p[i]; }
    __device__ static void st(float *p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<bf16_t> {
    __device__ static float ld(const bf16_t *p, size_t i) { return __uint_as_float(uint32_t(p[i].bits) << 16); }
    __device__ static void st(bf16_t *p, size_t i, float x) { p[i].bits = to_bf(x); }
};

// ---- wave-level reductions (64 lanes) ----------------------------------------------------
__device__ __forceinline__ float wave_sum(float x)
{
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

} // namespace la
