// Gated RMS norm on the scan's output: Mamba-2's output stage, the mixer the
// DiffuMamba pages name, in its default order (gate, then normalize):
//   v = y * silu(z),  out = v / sqrt(mean_group(v^2) + eps) * weight
// over groups of group_size consecutive channels of one token. z is the gate
// branch of the block's input projection (its own dtype, which is also the
// output dtype), y the fp32 sum of the two streams.
//
// One workgroup of four waves per token; lane l of wave w holds channels
// 1024k + 256w + 4l .. +3 of each 1024-channel pass k (16-byte y loads,
// 8- or 16-byte z loads), so each (pass, wave) covers one 256-channel chunk
// and a group (a multiple of 256 channels) is a run of whole chunks. Chunk
// sums of v^2 come from wave shuffles, group sums from the chunks in order.
// HBM-bound: y and z read once, the output written once.
#include "common.hpp"
#include "internal.hpp"

namespace bm {
namespace {

constexpr int kEpiThreads = 256;

typedef __bf16 ebf16x2 __attribute__((ext_vector_type(2)));
typedef float ef32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load4(const float *p, float *o) {
    const float4 v = *(const float4 *)p;
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const uint16_t *p, float *o) {
    const uint2 v = *(const uint2 *)p;
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void store4(float *p, const float *v) {
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
}
// round to nearest even through the hardware conversion
__device__ __forceinline__ void store4(uint16_t *p, const float *v) {
    const ef32x2 a = {v[0], v[1]}, b = {v[2], v[3]};
    uint2 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, ebf16x2));
    o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, ebf16x2));
    *(uint2 *)p = o;
}

__device__ __forceinline__ float silu(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
    return v;
}

template <typename T, int KP>
__global__ __launch_bounds__(kEpiThreads) void k_gated_norm(EpiArgs a) {
    __shared__ float part[KP * 4];
    const size_t row = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int C = a.C;
    const float *y = a.y + row * C;
    const T *z = (const T *)a.z + row * C;
    float v[KP][4];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int c = 1024 * k + 4 * tid;
        float ss = 0.f;
        if (c < C) {
            float yv[4], zv[4];
            load4(y + c, yv);
            load4(z + c, zv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[k][i] = yv[i] * silu(zv[i]);
                ss = fmaf(v[k][i], v[k][i], ss);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[k][i] = 0.f;
        }
        ss = wave_sum(ss);
        if (lane == 0) part[4 * k + wave] = ss;
    }
    __syncthreads();
    T *out = (T *)a.out + row * C;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int c = 1024 * k + 4 * tid;
        if (c < C) {
            const int q0 = (c / a.gs) * (a.gs / 256);     // first chunk of the group
            float ms = 0.f;
            for (int q = 0; q < a.gs / 256; ++q) ms += part[q0 + q];
            const float scale = 1.0f / sqrtf(ms / (float)a.gs + a.eps);
            float w[4], o[4];
            load4(a.w + c, w);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = v[k][i] * scale * w[i];
            store4(out + c, o);
        }
    }
}

template <typename T>
hipError_t launch_t(const EpiArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)a.rows);
    if (a.C <= 1024) BM_LAUNCH("gated_norm", (k_gated_norm<T, 1>), grid, dim3(kEpiThreads), 0, s, a);
    else if (a.C <= 2048) BM_LAUNCH("gated_norm", (k_gated_norm<T, 2>), grid, dim3(kEpiThreads), 0, s, a);
    else if (a.C <= 4096) BM_LAUNCH("gated_norm", (k_gated_norm<T, 4>), grid, dim3(kEpiThreads), 0, s, a);
    else BM_LAUNCH("gated_norm", (k_gated_norm<T, 8>), grid, dim3(kEpiThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_norm(const EpiArgs &a, bool bf16, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    return bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace bm
