// Device-side building blocks shared by the libgau kernels (gfx950 only):
// element types, the SiLU activation, bf16 rounding and the dynamic-LDS
// attribute helper.  The MFMA tiling lives in gemm_core.h.
//
// Element types: `bf16` (storage of bfloat16 bits; bf16 MFMA with fp32
// accumulation) and `float` (fp32 storage, fp32 MFMA).  The kernels are
// templated on the element type; every MFMA operand fragment is 16 bytes per
// lane along the contraction axis, so LDS tiles are laid out and read the same
// way for both types and only the number of K elements per 16 bytes differs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gau {

struct bf16 {
    uint16_t bits;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ scalars

// fp32 -> bf16, round to nearest, ties to even (finite values): the hardware
// conversion (v_cvt_pk_bf16_f32 on gfx950, which rounds to nearest even in the
// default rounding mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 values as packed bf16 (a in the low half), one conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<bf16> {
    static constexpr int kBytes = 2;
    __device__ static __forceinline__ void put(void* p, float v) { *(uint16_t*)p = f32_to_bf16(v); }
};
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    __device__ static __forceinline__ void put(void* p, float v) { *(float*)p = v; }
};

// SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x)), evaluated in fp32 with the
// hardware exponential and reciprocal (v_exp_f32, v_rcp_f32; about 1 ulp
// each).  For x below about -88, exp(-x) overflows to +inf and the result is
// x * 0 = -0, the correctly rounded limit.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// d SiLU(h) / dh = sigma(h) (1 + h (1 - sigma(h))), fp32 with the hardware
// exponential and reciprocal (as SiLU).
__device__ __forceinline__ float silu_grad(float h) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h));
    return sg * (1.0f + h * (1.0f - sg));
}

// Rotary frequency of pair i of a head of width 2 * half: 10000^(-i / half),
// in fp64 (angles t * theta reach about 10^4 rad).
__device__ __forceinline__ double rope_theta(int i, int half) { return pow(10000.0, -(double)i / (double)half); }

// cos and sin of the rotary angle t * theta: the angle is formed in fp64 and
// reduced to [-pi, pi] there (at t ~ 10^5 an fp32 product would be off by
// 10^-2 rad); only the reduced angle's cosine and sine are fp32 (about 1 ulp).
__device__ __forceinline__ void rope_cos_sin(double t, double theta, float& c, float& s) {
    constexpr double kTwoPi = 6.283185307179586476925287;
    const double a = t * theta;
    const float r = (float)(a - kTwoPi * rint(a / kTwoPi));
    sincosf(r, &s, &c);
}

// Allow kernel `Kernel` more than the default dynamic LDS (the attribute is set
// once per kernel).
template <auto Kernel>
inline hipError_t allow_lds(int bytes) {
    static const hipError_t err =
        hipFuncSetAttribute((const void*)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return err;
}

}  // namespace gau
