// The concatenating merge of the two streams (DiffuMamba blog, "network
// architecture": the block concatenates the forward output and the
// flipped-back reverse output and applies a Linear layer back to one width):
//   out[t] = W [y_fwd[t] ; y_bwd[t]] + bias,   W: cout x (2 cin), bf16
//
// A bf16 matrix-core GEMM (v_mfma_f32_16x16x32_bf16). Workgroup tile 128
// tokens x 128 outputs, four waves of 64 x 64 (4 x 4 MFMA tiles each), K in
// steps of 32. The streams are fp32: each step's 128 x 32 slice is read as
// 16-byte vectors, rounded to bf16 by the hardware conversion and staged in
// LDS next to the weight slice (rows of 32 + 8 halves); the next step's
// slices are loaded into registers while the current one is multiplied
// (double-buffered LDS, one barrier per step). A K step never straddles the
// two streams (cin is a multiple of 32). Workgroups of one token panel are
// placed on one XCD, so the panel is fetched into that XCD's L2 once.
#include "common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace bm {
namespace {

constexpr int kMT = 128, kNT = 128, kKT = 32;
constexpr int kMergeThreads = 256;
constexpr int kRS = kKT + 8;   // LDS row stride in halves (80 bytes)

typedef __bf16 mbf16x2 __attribute__((ext_vector_type(2)));
typedef float mf32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    const mf32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, mbf16x2));
}

__global__ __launch_bounds__(kMergeThreads) void k_merge(MergeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kMT * kRS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kNT * kRS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    // XCD-aware order: consecutive workgroup ids go to different XCDs, so
    // id -> (XCD x = id % 8, k-th on that XCD) is mapped to the k-th tile of
    // the token panels assigned to XCD x
    const int id = blockIdx.x;
    const int xcd = id & 7, k = id >> 3;
    const int per_panel = a.nblk;                 // output blocks per token panel
    const int panel = (k / per_panel) * 8 + xcd;  // token panel of this workgroup
    const int nb = k % per_panel;
    if (panel >= a.mblk) return;
    const int m0 = panel * kMT, n0 = nb * kNT;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int K = 2 * a.cin;
    const uint16_t *W = (const uint16_t *)a.w;

    float4 ra[4];
    uint4 rb[2];
    auto fetch = [&](int k0) {
        const bool first = k0 < a.cin;
        const float *src = first ? a.yf : a.yb;
        const int kk = first ? k0 : k0 - a.cin;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + kMergeThreads * i, r = e >> 3, c4 = e & 7;
            const long long m = (long long)m0 + r;
            ra[i] = m < a.rows ? *(const float4 *)(src + m * a.cin + kk + 4 * c4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid + kMergeThreads * i, r = e >> 2, c8 = e & 3;
            const int n = n0 + r;
            rb[i] = n < a.cout ? *(const uint4 *)(W + (size_t)n * K + k0 + 8 * c8)
                               : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + kMergeThreads * i, r = e >> 3, c4 = e & 7;
            *(uint2 *)&As[buf][r * kRS + 4 * c4] =
                make_uint2(cvt2(ra[i].x, ra[i].y), cvt2(ra[i].z, ra[i].w));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid + kMergeThreads * i, r = e >> 2, c8 = e & 3;
            *(uint4 *)&Bs[buf][r * kRS + 8 * c8] = rb[i];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    fetch(0);
    stash(0);
    __syncthreads();
    const int nk = K / kKT;
    for (int ks = 0; ks < nk; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < nk) fetch((ks + 1) * kKT);
        u32x4 av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = *(const u32x4 *)&As[cur][(wm + 16 * i + l16) * kRS + 8 * g];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = *(const u32x4 *)&Bs[cur][(wn + 16 * j + l16) * kRS + 8 * g];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(av[i], bv[j], acc[i][j]);
        if (ks + 1 < nk) stash(cur ^ 1);
        __syncthreads();
    }
    // out rows m0 + wm + 16 i + 4 g + r, column n0 + wn + 16 j + l16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn + 16 * j + l16;
        if (n >= a.cout) continue;
        const float bn = a.bias ? a.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const long long m = (long long)m0 + wm + 16 * i + 4 * g + r;
                if (m < a.rows) a.out[m * a.cout + n] = acc[i][j][r] + bn;
            }
    }
}

}  // namespace

hipError_t launch_merge(MergeArgs a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    a.mblk = (int)((a.rows + kMT - 1) / kMT);
    a.nblk = (a.cout + kNT - 1) / kNT;
    // whole groups of eight panels, one per XCD
    const long long groups = (a.mblk + 7) / 8;
    const long long blocks = groups * 8 * a.nblk;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    BM_LAUNCH("merge_linear", k_merge, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace bm
