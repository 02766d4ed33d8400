// kda_device.hpp -- device-side helpers shared by the KDA kernels (gfx950).
//
// Wavefront size is 64 on CDNA4; every helper below assumes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;
constexpr float kL2Eps = 1e-6f;  // q/k normalisation epsilon of the in-kernel L2 norm

enum GateMode : int { GATE_LOGDECAY = 0, GATE_SAFE = 1, GATE_SOFTPLUS = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {  // bf16 stored as raw bits
    __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) {
        return bf16_bits_to_f32(p[i]);
    }
    __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) {
        p[i] = f32_to_bf16_bits(v);
    }
};

// The hardware reciprocal (1 ulp) instead of an IEEE divide: the divide's
// scale/fixup sequence is about ten instructions per call.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// log(1 + t) for t in [0, 1]: with s = t / (2 + t) in [0, 1/3], log(1 + t) =
// 2 atanh(s) = 2 s sum_n s^(2n) / (2n + 1), summed through n = 7 (the first
// omitted term is below 9^-8 / 17 of the sum, under fp32 rounding).  One
// hardware reciprocal and eight fused multiply-adds instead of the library
// log1pf.
__device__ __forceinline__ float log1p_unit(float t) {
    const float s = t * __builtin_amdgcn_rcpf(2.0f + t);
    const float z = s * s;
    float p = 1.0f / 15.0f;
    p = __builtin_fmaf(p, z, 1.0f / 13.0f);
    p = __builtin_fmaf(p, z, 1.0f / 11.0f);
    p = __builtin_fmaf(p, z, 1.0f / 9.0f);
    p = __builtin_fmaf(p, z, 1.0f / 7.0f);
    p = __builtin_fmaf(p, z, 1.0f / 5.0f);
    p = __builtin_fmaf(p, z, 1.0f / 3.0f);
    p = __builtin_fmaf(p, z, 1.0f);
    return 2.0f * s * p;
}

// log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|).
__device__ __forceinline__ float softplusf_(float x) {
    return fmaxf(x, 0.0f) + log1p_unit(__expf(-fabsf(x)));
}

// softplus(z) and sigmoid(z) from one exponential t = e^-|z|: sigmoid(z) is
// 1 / (1 + t) for z >= 0 and t / (1 + t) below, softplus(z) = max(z, 0) +
// log1p(t) (the softplus gate's chain rule needs both).
__device__ __forceinline__ void softplus_sigmoid(float z, float& sp, float& sg) {
    const float t = __expf(-fabsf(z));
    const float r = __builtin_amdgcn_rcpf(1.0f + t);
    sg = z >= 0.0f ? r : t * r;
    sp = fmaxf(z, 0.0f) + log1p_unit(t);
}

// Per-channel log-decay from the raw gate input (see kda_gate_mode in kda.h).
__device__ __forceinline__ float gate_eff(int mode, float x, float rate, float bias, float lb) {
    if (mode == GATE_LOGDECAY) return x;
    float z = x + bias;
    if (mode == GATE_SAFE) return lb * sigmoidf_(rate * z);
    return -rate * softplusf_(z);
}

typedef uint16_t u16x4_ __attribute__((ext_vector_type(4)));

// Four consecutive elements: Raw is the loaded form (kept until use), f32x4
// the arithmetic form.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    using Raw = f32x4;
    __device__ __forceinline__ static Raw raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ static f32x4 cvt(Raw r) { return r; }
    __device__ __forceinline__ static f32x4 load(const float* p) { return raw(p); }
    __device__ __forceinline__ static void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <> struct Vec4<uint16_t> {
    using Raw = u16x4_;
    __device__ __forceinline__ static Raw raw(const uint16_t* p) { return *reinterpret_cast<const u16x4_*>(p); }
    __device__ __forceinline__ static f32x4 cvt(Raw u) {
        return f32x4{bf16_bits_to_f32(u[0]), bf16_bits_to_f32(u[1]), bf16_bits_to_f32(u[2]), bf16_bits_to_f32(u[3])};
    }
    __device__ __forceinline__ static f32x4 load(const uint16_t* p) { return cvt(raw(p)); }
    __device__ __forceinline__ static void store(uint16_t* p, f32x4 v) {
        const u16x4_ u = {f32_to_bf16_bits(v[0]), f32_to_bf16_bits(v[1]), f32_to_bf16_bits(v[2]), f32_to_bf16_bits(v[3])};
        *reinterpret_cast<u16x4_*>(p) = u;
    }
};

// Sum over each row of 16 lanes, in every lane of the row (DPP row rotations).
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

}  // namespace kda
