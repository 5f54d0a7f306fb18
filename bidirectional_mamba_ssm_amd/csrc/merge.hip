// The concatenating merge of the two streams (DiffuMamba blog, "network
// architecture": the block concatenates the forward output and the
// flipped-back reverse output and applies a Linear layer back to one width):
//   out[t] = W [y_fwd[t] ; y_bwd[t]] + bias,   W: cout x (2 cin), bf16
//
// A bf16 matrix-core GEMM (v_mfma_f32_16x16x32_bf16), K in steps of 32 or
// 64.
// The streams are fp32: each step's slice is read as 16-byte vectors, rounded to bf16 by the hardware conversion and staged in
// LDS next to the weight slice (rows of K step + 8 halves); the next step's
// slices are loaded into registers while the current one is multiplied
// (double-buffered LDS, one barrier per step). A K step never straddles the
// two streams (cin is a multiple of 32). Workgroups of one token panel are
// placed on one XCD, so the panel is fetched into that XCD's L2 once.
#include "common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace bm {
namespace {


typedef __bf16 mbf16x2 __attribute__((ext_vector_type(2)));
typedef float mf32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    const mf32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, mbf16x2));
}

// Workgroup tile (16 TI WM) x (16 TJ WN): WM x WN waves, each (16 TI) x
// (16 TJ) as TI x TJ MFMA tiles. Large problems take 256 x 256 tiles with
// eight waves of 128 x 64 (two waves per SIMD: one wave alone issues its
// independent products at little more than half the matrix-core rate); per K
// element such a tile fetches 256 x 4 + 256 x 2 bytes for 2 x 256 x 256
// flops. Small ones take 128 x 128 tiles with four waves of 64 x 64, which
// fill the chip.
template <int TI, int TJ, int KT, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void k_merge(MergeArgs a) {
    constexpr int kMergeThreads = 64 * WM * WN;
    constexpr int MT = 16 * TI * WM, NT = 16 * TJ * WN;
    constexpr int kRS = KT + 8;           // LDS row stride in halves
    constexpr int A4 = KT / 4, B8 = KT / 8;  // 16-byte vectors per slice row
    constexpr int AV = MT * A4 / kMergeThreads;  // stream vectors per thread
    constexpr int BV = NT * B8 / kMergeThreads;  // weight vectors per thread
    __shared__ __attribute__((aligned(16))) uint16_t As[2][MT * kRS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][NT * kRS];
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
    const int m0 = panel * MT, n0 = nb * NT;
    const int wm = (wave / WN) * (16 * TI), wn = (wave % WN) * (16 * TJ);
    const int K = 2 * a.cin;
    const uint16_t *W = (const uint16_t *)a.w;

    float4 ra[AV];
    uint4 rb[BV];
    auto fetch = [&](int k0) {
        const bool first = k0 < a.cin;
        const float *src = first ? a.yf : a.yb;
        const int kk = first ? k0 : k0 - a.cin;
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int e = tid + kMergeThreads * i, r = e / A4, c4 = e % A4;
            const long long m = (long long)m0 + r;
            ra[i] = m < a.rows ? *(const float4 *)(src + m * a.cin + kk + 4 * c4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int e = tid + kMergeThreads * i, r = e / B8, c8 = e % B8;
            const int n = n0 + r;
            rb[i] = n < a.cout ? *(const uint4 *)(W + (size_t)n * K + k0 + 8 * c8)
                               : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int e = tid + kMergeThreads * i, r = e / A4, c4 = e % A4;
            *(uint2 *)&As[buf][r * kRS + 4 * c4] =
                make_uint2(cvt2(ra[i].x, ra[i].y), cvt2(ra[i].z, ra[i].w));
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int e = tid + kMergeThreads * i, r = e / B8, c8 = e % B8;
            *(uint4 *)&Bs[buf][r * kRS + 8 * c8] = rb[i];
        }
    };

    f32x4 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = zero4();
    fetch(0);
    stash(0);
    __syncthreads();
    const int nk = K / KT;
    for (int ks = 0; ks < nk; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < nk) fetch((ks + 1) * KT);
#pragma unroll
        for (int kq = 0; kq < KT; kq += 32) {
            // every fragment of the step read at once, so that the reads'
            // latency is paid once and not before each row of products
            u32x4 av[TI], bv[TJ];
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                bv[j] = *(const u32x4 *)&Bs[cur][(wn + 16 * j + l16) * kRS + kq + 8 * g];
#pragma unroll
            for (int i = 0; i < TI; ++i)
                av[i] = *(const u32x4 *)&As[cur][(wm + 16 * i + l16) * kRS + kq + 8 * g];
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16x16x32(av[i], bv[j], acc[i][j]);
        }
        if (ks + 1 < nk) stash(cur ^ 1);
        __syncthreads();
    }
    // The products leave row 4 g + r, column 16 j + l16 of each 16 x 16 tile
    // in a lane; each wave turns its 16 x 64 strips into whole rows through
    // LDS (the operand buffers are free after the last barrier) and writes
    // 16-byte pieces, four rows of 256 bytes per instruction.
    static_assert(TJ == 4, "the row write-out assumes 64-column wave strips");
    constexpr int kSS = 64 + 4;   // staging row stride in floats
    static_assert(sizeof(As) >= (size_t)(kMergeThreads / 64) * 16 * kSS * sizeof(float),
                  "staging does not fit");
    float *stg = reinterpret_cast<float *>(&As[0][0]) + wave * 16 * kSS;
    const int rr = lane >> 4, cc = 4 * (lane & 15);
    const int n = n0 + wn + cc;
    float4 bn = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.bias && n < a.cout) bn = *(const float4 *)(a.bias + n);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) stg[(4 * g + r) * kSS + 16 * j + l16] = acc[i][j][r];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = rr + 4 * q;
            const long long m = (long long)m0 + wm + 16 * i + row;
            const float4 v = *(const float4 *)&stg[row * kSS + cc];
            if (m < a.rows && n < a.cout)
                *(float4 *)(a.out + m * a.cout + n) =
                    make_float4(v.x + bn.x, v.y + bn.y, v.z + bn.z, v.w + bn.w);
        }
        __syncthreads();
    }
}

template <int TI, int TJ, int KT, int WM, int WN>
hipError_t launch_tile(MergeArgs a, hipStream_t s) {
    constexpr int MT = 16 * TI * WM, NT = 16 * TJ * WN;
    a.mblk = (int)((a.rows + MT - 1) / MT);
    a.nblk = (a.cout + NT - 1) / NT;
    // whole groups of eight panels, one per XCD
    const long long groups = (a.mblk + 7) / 8;
    const long long blocks = groups * 8 * a.nblk;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    BM_LAUNCH("merge_linear", (k_merge<TI, TJ, KT, WM, WN>), dim3((unsigned)blocks), dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(MergeArgs a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    // the large tile once it alone gives every CU a workgroup
    const long long big = ((a.rows + 255) / 256) * ((a.cout + 255) / 256);
    if (big >= 256)
        return a.cin % 64 == 0 ? launch_tile<8, 4, 64, 2, 4>(a, s) : launch_tile<8, 4, 32, 2, 4>(a, s);
    // K steps of 64 where they do not straddle the two streams (half the
    // barriers)
    return a.cin % 64 == 0 ? launch_tile<4, 4, 64, 2, 2>(a, s) : launch_tile<4, 4, 32, 2, 2>(a, s);
}

}  // namespace bm
