// CDNA4 (gfx950) matrix-core helpers.
//
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16], fp32 accumulate.
// Lane l (0..63), g = l / 16:
//   A: row m = l % 16, k = 8g .. 8g+7  (8 bf16 in 4 VGPRs)
//   B: col n = l % 16, k = 8g .. 8g+7
//   D: col n = l % 16, rows m = 4g .. 4g+3  (4 fp32)
// (layout verified on gfx950 with a host-packed GEMM probe). The k order inside
// one instruction is free as long as A and B agree, which lets a D tile pair
// (rows 4g..4g+3 of two stacked 16x16 tiles) serve directly as the B operand
// of a following product: k-slots 8g..8g+3 <-> tile 0, 8g+4..8g+7 <-> tile 1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_f16: the same lane layouts with fp16 operands.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace bm
