// Device helpers shared by the bimamba kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bm {

// bfloat16 is carried as raw 16-bit words; conversions round to nearest even.
__device__ __forceinline__ float bf2f(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
// two floats -> packed pair of bf16 (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// dt as the scan uses it when a direction carries its pre-activation:
// softplus(v) = max(v, 0) + log1p(e^{-|v|}) (no overflow, no loss for
// very negative v)
__device__ __forceinline__ float softplus_dt(float v) {
    return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v)));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t *p, size_t i) { return bf2f(p[i]); }
};

}  // namespace bm
