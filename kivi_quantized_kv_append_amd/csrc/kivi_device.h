// Device-side helpers: 16-bit formats, the group quantiser's arithmetic, and
// lane-group reductions. gfx950, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kivi {

constexpr int kF16 = 0;
constexpr int kBF16 = 1;

__device__ __forceinline__ float f16_bits_to_f32(uint16_t u) {
    return (float)__builtin_bit_cast(_Float16, u);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
    return __uint_as_float((uint32_t)u << 16);
}
template <int DT>
__device__ __forceinline__ float to_f32(uint16_t u) {
    if constexpr (DT == kBF16) return bf16_bits_to_f32(u);
    else return f16_bits_to_f32(u);
}
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 in the default mode)
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float x) {
    if constexpr (DT == kBF16) return f32_to_bf16_bits(x);
    else return f32_to_f16_bits(x);
}

// -0 is read as +0 so that stored zero-points never depend on reduction order
__device__ __forceinline__ float canon(float x) { return x == 0.0f ? 0.0f : x; }

// Group parameters from the group minimum and maximum (min/max asymmetric
// mapping): scale = (max - min) / (2^b - 1) in IEEE single precision, scale
// and zero-point rounded to fp16; S and Z are the stored values read back.
__device__ __forceinline__ void group_params(float mn, float mx, int qmax, uint16_t& s16,
                                             uint16_t& z16, float& S, float& Z) {
#pragma clang fp contract(off)
    float range = mx - mn;
    float scale32 = range / (float)qmax;  // correctly rounded division
    s16 = f32_to_f16_bits(scale32);
    z16 = f32_to_f16_bits(mn);
    S = f16_bits_to_f32(s16);
    Z = f16_bits_to_f32(z16);
}

// Code of one element against the stored pair: round half to even of
// (x - Z) / S in IEEE single precision, clamped to [0, qmax]; 0 if S == 0.
__device__ __forceinline__ uint32_t group_code(float x, float S, float Z, int qmax) {
#pragma clang fp contract(off)
    if (S == 0.0f) return 0u;
    float diff = x - Z;
    float t = diff / S;
    float r = __builtin_rintf(t);
    r = fminf(fmaxf(r, 0.0f), (float)qmax);
    return (uint32_t)r;
}

// Report device-side argument errors: OR kivi_device_error bits into the
// pool's status word with a vector atomic (the lanes that call it).
__device__ __forceinline__ void report_error(uint32_t* status, uint32_t bits) {
    __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Min / max over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_min(float x, int width) {
    for (int o = 1; o < width; o <<= 1) x = fminf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float group_max(float x, int width) {
    for (int o = 1; o < width; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

}  // namespace kivi
