// Training backward of the bidirectional SSD: gradients of x, dt, A, B, C
// and D of both streams, given dy (the output being the sum of the streams,
// both receive the same dy).
//
// The forward streams are the Mamba-2 recurrence run over the sequence and,
// with the reverse stream's own parameters, over the flipped sequence
// (DiffuMamba blog, "network architecture"); the reverse stream is walked
// here by index arithmetic too: scan position k of the reverse stream is
// token L-1-k. Gradients follow by the chain rule through the block form of
// the recurrence, 64 scan positions per block. With s_i the running sum of
// a_k = dt_k A over the block (up to and including i), G_ij = C_i . B_j,
// L_ij = e^{s_i - s_j} (j <= i), xd_j = dt_j x_j, Hp the state entering the
// block and dHe the gradient of the state leaving it:
//
//   y_i   = sum_j L_ij G_ij xd_j + e^{s_i} C_i^T Hp + D x_i
//   H_end = e^{s_end} Hp + sum_j e^{s_end - s_j} B_j xd_j^T
//
// so that, with dM_ij = dy_i . xd_j and M_ij = L_ij G_ij,
//
//   dxd_j = sum_i M_ij dy_i + e^{s_end - s_j} dHe^T B_j
//   dC_i  = sum_j L_ij dM_ij B_j + e^{s_i} Hp dy_i
//   dB_j  = sum_i L_ij dM_ij C_i + e^{s_end - s_j} dHe xd_j
//   ds_i  = sum_j dM_ij M_ij - sum_k dM_ki M_ki + e^{s_i} (C_i^T Hp) . dy_i
//           - [e^{s_end - s_i} <B_i xd_i^T, dHe>] + [i = end] (e^{s_end} <Hp, dHe>
//           + sum_j e^{s_end - s_j} <B_j xd_j^T, dHe>)
//   da_k  = sum_{i >= k} ds_i,  ddt_k = x_k . dxd_k + A da_k,  dA = sum dt_k da_k
//   dx_k  = D dy_k + dt_k dxd_k,  dD = sum x_k . dy_k
//
// Kernels (products of fp32 values, accumulated in fp32; the running sums s
// in fp64):
//   k_bwd_chain  per (row, stream, head): walks the blocks forward and then
//                backward with the state in the matrix-core accumulators and
//                writes every block's entering state Hp and leaving-state
//                gradient dHe (taken when such units fill the CUs or rows are
//                short); otherwise
//   k_bwd_state  per (row, stream, head, block): the block's own state
//                S = sum_j e^{s_end - s_j} dt_j B_j x_j^T, its output-gradient
//                feed R = sum_i e^{s_i} C_i dy_i^T and s_end, and
//   k_bwd_pass   per (row, stream, head, state element): Hp (forward over
//                blocks) and dHe (backward over blocks), written over S and R.
//   k_bwd_grad[_heads][_mx]  per (row, stream, block) and head, or walking the
//                heads of a group: everything above; dB and dC per head into
//                the workspace, or summed over the group's heads in registers;
//                dA and dD per block. The _mx form (bf16 inputs, headdim 64,
//                d_state 128) runs every product on the bf16 matrix cores
//                with fp32 operands as exact sums of three bf16 parts, the
//                other on the fp32 matrix cores.
//   k_bwd_sum_bc / k_bwd_sum_ad: sums over the heads of a group and over the
//                blocks, in a fixed order (deterministic results).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace bm {
namespace {

constexpr int kQ = 64;          // scan positions per block
constexpr int kStateThreads = 256;
constexpr int kGradThreads = 1024;   // 16 waves: one workgroup fills a CU (LDS)

struct BwdArgs {
    DirPtrs fwd, bwd;
    GradPtrs gfwd, gbwd;
    const float *dy;
    int batch, L, H, G, ndir, nc;
    float *S;      // [batch][ndir][H][nc][N x P]: block states, then entering states
    float *R;      // [batch][ndir][H][nc][N x P]: output-gradient feeds, then dHe
    double *lg;    // [batch][ndir][H][nc]: s_end of each block
    float *dBp;    // [batch][ndir][H][L][N]
    float *dCp;    // [batch][ndir][H][L][N]
    float *dAp;    // [batch][ndir][H][nc]
    float *dDp;    // [batch][ndir][H][nc]
    int head_loop; // the gradient kernel walks each group's heads (no dBp, dCp)
    int chain;     // Hp and dHe by k_bwd_chain (else k_bwd_state + k_bwd_pass)
};

__device__ __forceinline__ int tok_of(int k, int L, bool rev) { return rev ? L - 1 - k : k; }

// An N x P state in the workspace, in the matrix cores' result layout: 16 x
// 16 tiles (n-tile major), each as the 64 lanes' 4-vectors of a 16x16
// product's result (lane l: column l % 16, rows 4 (l / 16) .. +3), so that a
// wave writes a tile as one contiguous kilobyte. Element (n, p) is at
//   ((n / 16) (P / 16) + p / 16) 256 + 4 (16 ((n % 16) / 4) + p % 16) + n % 4;
// tile_pos gives the start of lane's 4-vector in tile (nt, pt).
template <int P>
__device__ __forceinline__ int tile_pos(int nt, int pt, int lane) {
    return (nt * (P / 16) + pt) * 256 + lane * 4;
}

// threadIdx.x; with LT behind an empty asm statement, a fresh value wherever
// it is read, so that the compiler recomputes lane addresses inside the loop
// over heads instead of hoisting them all out of it and running out of
// registers (elsewhere the plain value lets it share them).
template <bool LT>
__device__ __forceinline__ int lane_tid() {
    int t = threadIdx.x;
    if (LT) asm volatile("" : "+v"(t));
    return t;
}

// dt of the block's positions into dtv (zero past len) and the running sums
// of a = dt*A into sv (fp64): one lane per position in wave 0 (a block is
// one wave wide), a shuffle scan. Ends with a workgroup barrier.
template <typename T, bool LT = false>
__device__ void block_scan(const BwdArgs &a, const DirPtrs &d, size_t rowt, int h, int k0,
                           int len, bool rev, double *sv, float *dtv) {
    static_assert(kQ == 64, "one wave per block");
    const int tid = lane_tid<LT>();
    if (tid < kQ) {
        const float dtr = tid < len
            ? Elem<T>::load((const T *)d.dt, (rowt + tok_of(k0 + tid, a.L, rev)) * a.H + h)
            : 0.f;
        dtv[tid] = dtr;
        double v = (double)dtr * (double)d.A[h];
        for (int off = 1; off < kQ; off <<= 1) {
            const double u = __shfl_up(v, off);
            if (tid >= off) v += u;
        }
        sv[tid] = v;
    }
    __syncthreads();
}

// Sum over the G lanes of an aligned group (the same value in all of them).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = 1; off < G; off <<= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
    return v;
}

// Inclusive running sum over the 64 lanes of a wave (lane order), fp64.
__device__ __forceinline__ double wave_scan(double v, int lane) {
    for (int off = 1; off < 64; off <<= 1) {
        const double u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    return v;
}

// Four consecutive elements as floats (8-byte bf16 or 16-byte fp32 loads).
__device__ __forceinline__ void ld4(const float *p, float *o) {
    const float4 v = *(const float4 *)p;
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void ld4(const uint16_t *p, float *o) {
    const uint2 v = *(const uint2 *)p;
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// A block's rows of a per-token array (row r is token tok_of(k0 + r); W
// columns from element off of each token's stride), held in registers:
// thread t owns 4-vectors t, t + NT, ... All loads are issued before any
// is used.
template <int W, int NT>
struct Rows {
    static constexpr int NV = kQ * W / 4, VPT = (NV + NT - 1) / NT;
    float v[VPT][4];
};

template <typename T, bool LT = false, int W, int NT>
__device__ __forceinline__ void fetch_rows(Rows<W, NT> &rw, const void *src, size_t rowt,
                                           size_t stride, size_t off, int k0, int len, int L,
                                           bool rev) {
#pragma unroll
    for (int k = 0; k < Rows<W, NT>::VPT; ++k) {
        const int e4 = lane_tid<LT>() + k * NT;
        const int r = e4 * 4 / W, c = e4 * 4 % W;
        if (e4 < Rows<W, NT>::NV && r < len) {
            ld4((const T *)src + (rowt + tok_of(k0 + r, L, rev)) * stride + off + c, rw.v[k]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) rw.v[k][i] = 0.f;
        }
    }
}

// Stores held rows into an LDS array [kQ][S], each row scaled by scale(r).
template <bool LT = false, int W, int NT, int S, class F>
__device__ __forceinline__ void store_rows(const Rows<W, NT> &rw, float (*dst)[S], F scale) {
#pragma unroll
    for (int k = 0; k < Rows<W, NT>::VPT; ++k) {
        const int e4 = lane_tid<LT>() + k * NT;
        if (e4 < Rows<W, NT>::NV) {
            const int r = e4 * 4 / W, c = e4 * 4 % W;
            const float sc = scale(r);
            *(float4 *)&dst[r][c] = make_float4(rw.v[k][0] * sc, rw.v[k][1] * sc,
                                                rw.v[k][2] * sc, rw.v[k][3] * sc);
        }
    }
}

// An N x P state (flat, 16-byte aligned) in registers, and into LDS [N][S].
template <int NP, int NT>
struct Flat {
    static constexpr int VPT = (NP / 4 + NT - 1) / NT;
    float v[VPT][4];
};

template <bool LT = false, int NP, int NT>
__device__ __forceinline__ void fetch_flat(Flat<NP, NT> &f, const float *src) {
#pragma unroll
    for (int k = 0; k < Flat<NP, NT>::VPT; ++k) {
        const int e4 = lane_tid<LT>() + k * NT;
        if (e4 < NP / 4) {
            ld4(src + 4 * e4, f.v[k]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) f.v[k][i] = 0.f;
        }
    }
}

// A state held as loaded (the tile layout of tile_pos) into LDS [N][S]:
// 4-vector e4 is lane e4 % 64 of tile e4 / 64, rows 4 (lane / 16) .. +3 of
// column lane % 16.
template <int NP, int NT, int P, bool LT = false, int S>
__device__ __forceinline__ void store_flat(const Flat<NP, NT> &f, float (*dst)[S]) {
#pragma unroll
    for (int k = 0; k < Flat<NP, NT>::VPT; ++k) {
        const int e4 = lane_tid<LT>() + k * NT;
        if (e4 < NP / 4) {
            const int tile = e4 >> 6, ln = e4 & 63;
            const int n0 = (tile / (P / 16)) * 16 + 4 * (ln >> 4), p = (tile % (P / 16)) * 16 + (ln & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[n0 + i][p] = f.v[k][i];
        }
    }
}

// One 16x16 output tile of a product on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32; lane l, g = l / 16, m = l % 16: A supplies
// A[m][k + g], B supplies B[k + g][m], the result holds rows 4g .. 4g+3 of
// column m). a(m, k) and b(k, m) read the operands (from LDS).
template <bool LT = false, class FA, class FB>
__device__ __forceinline__ f32x4 mm(FA a, FB b, int k0, int k1, f32x4 acc) {
    const int l = lane_tid<LT>() & 63, g = l >> 4, m = l & 15;
    for (int k = k0; k < k1; k += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(m, k + g), b(k + g, m), acc, 0, 0, 0);
    return acc;
}

template <typename T, int P, int N>
__global__ __launch_bounds__(kStateThreads) void k_bwd_state(BwdArgs a) {
    constexpr int NT = kStateThreads, NW = NT / 64;
    constexpr int TN = N / 16, TP = P / 16, TILES = TN * TP, TPW = (TILES + NW - 1) / NW;
    constexpr int SW = N + 4, SV = P + 4;     // padded LDS rows
    __shared__ __attribute__((aligned(16))) float Wm[kQ][SW];
    __shared__ __attribute__((aligned(16))) float Vm[kQ][SV];
    static_assert(SW % 4 == 0 && SV % 4 == 0, "16-byte LDS rows");
    __shared__ double sv[kQ];
    __shared__ float dtv[kQ];
    const int c = blockIdx.x, h = blockIdx.y;
    const int dir = (int)(blockIdx.z % (unsigned)a.ndir), b = (int)(blockIdx.z / (unsigned)a.ndir);
    const bool rev = dir == 1;
    const DirPtrs d = rev ? a.bwd : a.fwd;
    const int g = h / (a.H / a.G);
    const int k0 = c * kQ;
    const int len = min(kQ, a.L - k0);
    const size_t rowt = (size_t)b * a.L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t unit = ((size_t)b * a.ndir + dir) * a.H + h;
    const size_t so = (unit * a.nc + c) * (size_t)(N * P);

    // the first pass's rows are in flight during the scan of dt
    const size_t sgn = (size_t)a.G * N, hp = (size_t)a.H * P;
    Rows<N, NT> rb;
    Rows<P, NT> rx;
    fetch_rows<T>(rb, d.B, rowt, sgn, (size_t)g * N, k0, len, a.L, rev);
    fetch_rows<T>(rx, d.x, rowt, hp, (size_t)h * P, k0, len, a.L, rev);
    block_scan<T>(a, d, rowt, h, k0, len, rev, sv, dtv);
    const double send = sv[len - 1];
    for (int pass = 0; pass < 2; ++pass) {
        // pass 0: S = sum_j (e^{s_end - s_j} dt_j B_j) x_j^T
        // pass 1: R = sum_i (e^{s_i} C_i) dy_i^T
        if (pass == 0) {
            store_rows(rb, Wm, [&](int r) { return r < len ? expf((float)(send - sv[r])) * dtv[r] : 0.f; });
            store_rows(rx, Vm, [&](int) { return 1.f; });
            // the second pass's rows, in flight during the first pass's products
            fetch_rows<T>(rb, d.C, rowt, sgn, (size_t)g * N, k0, len, a.L, rev);
            fetch_rows<float>(rx, a.dy, rowt, hp, (size_t)h * P, k0, len, a.L, rev);
        } else {
            store_rows(rb, Wm, [&](int r) { return r < len ? expf((float)sv[r]) : 0.f; });
            store_rows(rx, Vm, [&](int) { return 1.f; });
        }
        __syncthreads();
        float *out = pass == 0 ? a.S : a.R;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wave + u * NW;
            if (t < TILES) {
                const int nt = t / TP, pt = t % TP;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mm([&](int mm_, int k) { return Wm[k][nt * 16 + mm_]; },
                         [&](int k, int mm_) { return Vm[k][pt * 16 + mm_]; }, 0, kQ, acc);
                *(f32x4 *)&out[so + tile_pos<P>(nt, pt, lane)] = acc;
            }
        }
        __syncthreads();
    }
    if (tid == 0) a.lg[unit * a.nc + c] = send;
}

// Entering states forward over the blocks, leaving-state gradients backward.
__global__ __launch_bounds__(256) void k_bwd_pass(BwdArgs a, int np) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= np) return;
    const int h = blockIdx.y;
    const int dir = (int)(blockIdx.z % (unsigned)a.ndir), b = (int)(blockIdx.z / (unsigned)a.ndir);
    const size_t unit = ((size_t)b * a.ndir + dir) * a.H + h;
    // eight blocks' values are loaded before any is overwritten, so that
    // their loads are in flight together (the in-place stores would
    // otherwise hold each load back until the previous store)
    constexpr int kB = 8;
    const size_t base = unit * a.nc * (size_t)np + e;
    float carry = 0.f;
    for (int c0 = 0; c0 < a.nc; c0 += kB) {
        float v[kB];
#pragma unroll
        for (int k = 0; k < kB; ++k)
            v[k] = c0 + k < a.nc ? a.S[base + (size_t)(c0 + k) * np] : 0.f;
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            if (c0 + k >= a.nc) break;
            a.S[base + (size_t)(c0 + k) * np] = carry;
            carry = fmaf(expf((float)a.lg[unit * a.nc + c0 + k]), carry, v[k]);
        }
    }
    carry = 0.f;
    for (int c0 = a.nc - 1; c0 >= 0; c0 -= kB) {
        float v[kB];
#pragma unroll
        for (int k = 0; k < kB; ++k)
            v[k] = c0 - k >= 0 ? a.R[base + (size_t)(c0 - k) * np] : 0.f;
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            if (c0 - k < 0) break;
            a.R[base + (size_t)(c0 - k) * np] = carry;
            carry = fmaf(expf((float)a.lg[unit * a.nc + c0 - k]), carry, v[k]);
        }
    }
}

// ---- the chained form of the two kernels above, for many (row, stream,
// head) units: one workgroup per unit walks its blocks forward, then
// backward, the state in the matrix-core accumulators, and writes each
// block's entering state Hp_c (over S) and leaving-state gradient dHe_c (over
// R) before folding the block in:
//   Hp_{c+1}   = e^{s_end} Hp_c   + sum_j B_j (e^{s_end - s_j} dt_j x_j)^T
//   dHe_{c-1}  = e^{s_end} dHe_c  + sum_i C_i (e^{s_i} dy_i)^T
// (the block's own S and R of k_bwd_state never leave the CU). Products on
// the bf16 matrix cores (v_mfma_f32_16x16x32_bf16): an fp32 operand enters as
// the exact sum of three bf16 parts, bf16 inputs B and C as they are, so the
// products are those of fp32 operands, accumulated in fp32.

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef short v4i16_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_v lds_v4i16_v;

__device__ __forceinline__ uint32_t bf_pair(float v0, float v1) {
    const bf16x2_v h = {(__bf16)v0, (__bf16)v1};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float bf_low(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_high(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// v = p[0] + p[1] + p[2] exactly (each part bf16, rounded to nearest; the
// residues v - p[0] and v - p[0] - p[1] are exact in fp32), for a pair.
__device__ __forceinline__ void split3(float v0, float v1, uint32_t (&p)[3]) {
    p[0] = bf_pair(v0, v1);
    const float r0 = v0 - bf_low(p[0]), r1 = v1 - bf_high(p[0]);
    p[1] = bf_pair(r0, r1);
    p[2] = bf_pair(r0 - bf_low(p[1]), r1 - bf_high(p[1]));
}

// Matrix-core operand (A or B of v_mfma_f32_16x16x32_bf16) for the 16
// columns c0 .. c0+15 of a row-major [t][c] bf16 tile in LDS (row stride rs
// elements), k over its 32 rows t32 .. t32+31, by two transposing LDS reads
// (ds_read_b64_tr_b16: within 16 lanes, lane s points at row t + s/4,
// column c0 + 4 (s%4), and lane i receives column c0 + i of those 4 rows).
// Lane group g holds k slots 0..3 = rows t32 + 4g + (0..3) and 4..7 = rows
// t32 + 16 + 4g + (0..3); both operands of a product read this way agree.
__device__ __forceinline__ u32x4 tr_op(const uint16_t *base, int rs, int t32, int c0) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, s = lane & 15;
    const uint16_t *p = base + (t32 + 4 * g4 + (s >> 2)) * rs + c0 + 4 * (s & 3);
    const v4i16_v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_v *)p);
    const v4i16_v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_v *)(p + 16 * rs));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

constexpr int kChainThreads = 256;

// A block's rows of a per-token array as loaded (bf16 bits or fp32), for
// loads that stay in flight across a loop iteration: every load is issued
// (rows past the block's end re-read its last row, and are zeroed where
// used) and nothing reads the registers until then, so no wait falls between
// the loads and the work they overlap.
template <typename T, int W, int NT>
struct RawRows {
    static constexpr int NV = kQ * W / 4, VPT = NV / NT;
    static_assert(NV % NT == 0, "whole 4-vectors per thread");
    using V = typename std::conditional<sizeof(T) == 2, u32x2, f32x4>::type;
    V v[VPT];
    __device__ __forceinline__ void fetch(const void *src, size_t rowt, size_t stride, size_t off,
                                          int k0, int len, int L, bool rev) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int e4 = (int)threadIdx.x + k * NT;
            const int r = min(e4 * 4 / W, len - 1), c = e4 * 4 % W;
            v[k] = *(const V *)((const T *)src + (rowt + tok_of(k0 + r, L, rev)) * stride + off + c);
        }
    }
    // the four values of vector k as floats
    __device__ __forceinline__ void get(int k, float *o) const {
        if constexpr (sizeof(T) == 2) {
            o[0] = __uint_as_float(v[k][0] << 16);
            o[1] = __uint_as_float(v[k][0] & 0xffff0000u);
            o[2] = __uint_as_float(v[k][1] << 16);
            o[3] = __uint_as_float(v[k][1] & 0xffff0000u);
        } else {
            o[0] = v[k][0]; o[1] = v[k][1]; o[2] = v[k][2]; o[3] = v[k][3];
        }
    }
};

template <int P, int N, bool EXACT>
struct ChainSmem {
    static constexpr int NA = EXACT ? 1 : 3;
    static constexpr int RA = N + 8, RB = P + 8;   // bf16 row strides (8-byte aligned reads)
    uint16_t a[NA][kQ][RA];   // B (forward sweep) or C (backward sweep) rows, [t][n]
    uint16_t b[3][kQ][RB];    // weighted x or dy rows, [t][p], three parts
    float w[kQ];
    float gamma;
};

// One sweep: SW 0 walks blocks forward (B, x; Hp over S), SW 1 backward (C,
// dy; dHe over R).
template <typename T, int P, int N, int SW>
__device__ __forceinline__ void chain_sweep(const BwdArgs &a, ChainSmem<P, N, sizeof(T) == 2> &sm,
                                            int h, int dir, int b) {
    constexpr bool EXACT = sizeof(T) == 2;
    using Sm = ChainSmem<P, N, EXACT>;
    constexpr int NT = kChainThreads, NW = NT / 64;
    constexpr int TN = N / 16, TP = P / 16, TILES = TN * TP, TPW = (TILES + NW - 1) / NW;
    static_assert(NW % TP == 0, "a wave's tiles share their columns p");
    using XT = typename std::conditional<SW == 0, T, float>::type;
    const bool rev = dir == 1;
    const DirPtrs d = rev ? a.bwd : a.fwd;
    const int g = h / (a.H / a.G);
    const size_t rowt = (size_t)b * a.L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t unit = ((size_t)b * a.ndir + dir) * a.H + h;
    const size_t sgn = (size_t)a.G * N, hp = (size_t)a.H * P;
    const void *asrc = SW == 0 ? d.B : d.C;
    const void *bsrc = SW == 0 ? d.x : (const void *)a.dy;
    float *out = SW == 0 ? a.S : a.R;
    const float A = d.A[h];
    const int pt = wave % TP;

    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = zero4();

    RawRows<T, N, NT> ra;
    RawRows<XT, P, NT> rb;
    T dtn = 0;   // (as loaded; lanes of wave 0, one position each)
    auto fetch = [&](int c) {
        const int k0 = c * kQ, len = min(kQ, a.L - k0);
        ra.fetch(asrc, rowt, sgn, (size_t)g * N, k0, len, a.L, rev);
        rb.fetch(bsrc, rowt, hp, (size_t)h * P, k0, len, a.L, rev);
        if (tid < kQ) dtn = ((const T *)d.dt)[(rowt + tok_of(k0 + min(tid, len - 1), a.L, rev)) * a.H + h];
    };
    fetch(SW == 0 ? 0 : a.nc - 1);
    for (int step = 0; step < a.nc; ++step) {
        const int c = SW == 0 ? step : a.nc - 1 - step;
        const int k0 = c * kQ, len = min(kQ, a.L - k0);
        // running sums of dt A over the block (fp64, one lane per position),
        // the weights and the block's decay
        if (tid < kQ) {
            const float dtf = tid < len ? Elem<T>::load(&dtn, 0) : 0.f;
            const double s = wave_scan((double)dtf * (double)A, tid);
            const double send = __shfl(s, len - 1);
            sm.w[tid] = tid >= len ? 0.f : SW == 0 ? expf((float)(send - s)) * dtf : expf((float)s);
            if (tid == 0) sm.gamma = expf((float)send);
        }
        __syncthreads();   // (also: the previous block's products are done with the tiles)
        // the block's rows into LDS: B or C as bf16 (exact for bf16 inputs,
        // else three parts), x or dy times the weight of its row in three
        // parts; rows past the block's end as zeros
#pragma unroll
        for (int k = 0; k < RawRows<T, N, NT>::VPT; ++k) {
            const int e4 = tid + k * NT;
            const int r = e4 * 4 / N, cc = e4 * 4 % N;
            float v[4];
            ra.get(k, v);
            if constexpr (EXACT) {
                *(u32x2 *)&sm.a[0][r][cc] = u32x2{bf_pair(r < len ? v[0] : 0.f, r < len ? v[1] : 0.f),
                                                  bf_pair(r < len ? v[2] : 0.f, r < len ? v[3] : 0.f)};
            } else {
                uint32_t p01[3], p23[3];
                split3(r < len ? v[0] : 0.f, r < len ? v[1] : 0.f, p01);
                split3(r < len ? v[2] : 0.f, r < len ? v[3] : 0.f, p23);
#pragma unroll
                for (int q = 0; q < Sm::NA; ++q) *(u32x2 *)&sm.a[q][r][cc] = u32x2{p01[q], p23[q]};
            }
        }
#pragma unroll
        for (int k = 0; k < RawRows<XT, P, NT>::VPT; ++k) {
            const int e4 = tid + k * NT;
            const int r = e4 * 4 / P, cc = e4 * 4 % P;
            const float wr = sm.w[r];
            float v[4];
            rb.get(k, v);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = r < len ? v[i] * wr : 0.f;
            uint32_t p01[3], p23[3];
            split3(v[0], v[1], p01);
            split3(v[2], v[3], p23);
#pragma unroll
            for (int q = 0; q < 3; ++q) *(u32x2 *)&sm.b[q][r][cc] = u32x2{p01[q], p23[q]};
        }
        const float gmm = sm.gamma;
        // the next block's rows are in flight during this block's products
        // (the last block loads its own again: no branch around the loads)
        fetch(SW == 0 ? min(c + 1, a.nc - 1) : max(c - 1, 0));
        __syncthreads();
        // the state before the block, then the update
        const size_t so = (unit * a.nc + c) * (size_t)(N * P);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wave + u * NW;
            if (t < TILES) {
                const int nt = t / TP;
                *(f32x4 *)&out[so + tile_pos<P>(nt, pt, lane)] = acc[u];
                // a block whose decay is exactly 0 starts from nothing
                // (assigned: 0 times a non-finite state is not 0)
                acc[u] = gmm == 0.f ? zero4() : acc[u] * gmm;
            }
        }
#pragma unroll
        for (int ks = 0; ks < kQ / 32; ++ks) {
            u32x4 bo[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) bo[q] = tr_op(&sm.b[q][0][0], Sm::RB, 32 * ks, pt * 16);
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int t = wave + u * NW;
                if (t < TILES) {
                    const int nt = t / TP;
                    // result rows n (the A operand's columns), columns p
                    const u32x4 a0 = tr_op(&sm.a[0][0][0], Sm::RA, 32 * ks, nt * 16);
                    if constexpr (EXACT) {
                        acc[u] = mfma16x16x32(a0, bo[2], acc[u]);
                        acc[u] = mfma16x16x32(a0, bo[1], acc[u]);
                        acc[u] = mfma16x16x32(a0, bo[0], acc[u]);
                    } else {
                        const u32x4 a1 = tr_op(&sm.a[1][0][0], Sm::RA, 32 * ks, nt * 16);
                        const u32x4 a2 = tr_op(&sm.a[2][0][0], Sm::RA, 32 * ks, nt * 16);
                        // the six products down to 2^-16 x 2^-16 of the leading one
                        acc[u] = mfma16x16x32(a1, bo[1], acc[u]);
                        acc[u] = mfma16x16x32(a2, bo[0], acc[u]);
                        acc[u] = mfma16x16x32(a0, bo[2], acc[u]);
                        acc[u] = mfma16x16x32(a1, bo[0], acc[u]);
                        acc[u] = mfma16x16x32(a0, bo[1], acc[u]);
                        acc[u] = mfma16x16x32(a0, bo[0], acc[u]);
                    }
                }
            }
        }
    }
}

template <typename T, int P, int N>
__global__ __launch_bounds__(kChainThreads) void k_bwd_chain(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) ChainSmem<P, N, sizeof(T) == 2> sm;
    const int h = blockIdx.x;
    const int dir = (int)(blockIdx.y % (unsigned)a.ndir), b = (int)(blockIdx.y / (unsigned)a.ndir);
    chain_sweep<T, P, N, 0>(a, sm, h, dir, b);
    __syncthreads();
    chain_sweep<T, P, N, 1>(a, sm, h, dir, b);
}

template <int P, int N>
struct GradSmem {
    static constexpr int SN = N + 4, SP = P + 4, SQ = kQ + 4;   // padded rows, 16-byte aligned
    float Bs[kQ][SN];
    float Cs[kQ][SN];
    float Xs[kQ][SP];
    float Ys[kQ][SP];
    union {
        struct {
            float Ms[kQ][SQ];   // M = L o G
            float Gs[kQ][SQ];   // L o dM
            float Zs[kQ][SQ];   // dM o M
        } q;
        struct {
            float Hs[N][SP];    // entering state, then leaving-state gradient
            float Tq[kQ][SP];   // per-position products summed over p
        } st;
        float Dx[kQ][SP];       // dxd, at the end
    } u;
    double sv[kQ];
    float dtv[kQ], es[kQ], wv[kQ], dsi[kQ], dso[kQ], dss[kQ];
    float red[kGradThreads];
};

// The gradients of one (row, stream, head, block). HSUM: the head's dB and
// dC fragments are added to accb / accc (registers of the caller, which
// walks the heads of the group in order: the same fp32 sums as the
// separate head-sum kernel); else they go to the workspace.
template <typename T, int P, int N, bool HSUM>
__device__ __forceinline__ void grad_block(const BwdArgs &a, GradSmem<P, N> &sm, const int c,
                                           const int h, const int dir, const int b, const bool first,
                                           f32x4 *accb, f32x4 *accc) {
    constexpr int NT = kGradThreads, NW = NT / 64, NP = N * P;
    constexpr int LPR = NT / kQ;                              // lanes per position
    constexpr int TQ = kQ / 16, TN = N / 16, TP = P / 16;
    constexpr int XT = TQ * TP, XPW = (XT + NW - 1) / NW;     // (position, p) tiles
    constexpr int CT = TQ * TN, CPW = (CT + NW - 1) / NW;     // (position, n) tiles
    constexpr int LT = TQ * (TQ + 1) / 2;                     // lower (i, j) tiles
    const bool rev = dir == 1;
    const DirPtrs d = rev ? a.bwd : a.fwd;
    const GradPtrs gr = rev ? a.gbwd : a.gfwd;
    const int g = h / (a.H / a.G);
    const int k0 = c * kQ;
    const int len = min(kQ, a.L - k0);
    const size_t rowt = (size_t)b * a.L;
    const int tid = lane_tid<HSUM>(), wave = tid >> 6, lane = tid & 63;
    const int gq = lane >> 4, lm = lane & 15;     // result rows 4gq .. 4gq+3, column lm
    const size_t unit = ((size_t)b * a.ndir + dir) * a.H + h;
    const size_t so = (unit * a.nc + c) * (size_t)NP;

    // ---- inputs of the block; the entering state and the leaving-state
    // gradient are fetched now too and held until their phases
    const size_t sgn = (size_t)a.G * N, hp = (size_t)a.H * P;
    // (walking the heads of a group, B and C of the block stay in LDS from
    // the first head on: nothing else writes those rows then)
    const bool bc = !HSUM || first;
    {
        Rows<N, NT> rb, rc;
        Rows<P, NT> rx, ry;
        if (bc) {
            fetch_rows<T, HSUM>(rb, d.B, rowt, sgn, (size_t)g * N, k0, len, a.L, rev);
            fetch_rows<T, HSUM>(rc, d.C, rowt, sgn, (size_t)g * N, k0, len, a.L, rev);
        }
        fetch_rows<T, HSUM>(rx, d.x, rowt, hp, (size_t)h * P, k0, len, a.L, rev);
        fetch_rows<float, HSUM>(ry, a.dy, rowt, hp, (size_t)h * P, k0, len, a.L, rev);
        block_scan<T, HSUM>(a, d, rowt, h, k0, len, rev, sm.sv, sm.dtv);
        if (bc) {
            store_rows<HSUM>(rb, sm.Bs, [](int) { return 1.f; });
            store_rows<HSUM>(rc, sm.Cs, [](int) { return 1.f; });
        }
        store_rows<HSUM>(rx, sm.Xs, [](int) { return 1.f; });
        store_rows<HSUM>(ry, sm.Ys, [](int) { return 1.f; });
    }
    Flat<NP, NT> fhp, fdh;
    fetch_flat<HSUM>(fhp, a.S + so);
    fetch_flat<HSUM>(fdh, a.R + so);
    __syncthreads();
    const double send = sm.sv[len - 1];
    if (tid < kQ) {
        const int r = tid;
        sm.es[r] = r < len ? expf((float)sm.sv[r]) : 0.f;
        sm.wv[r] = r < len ? expf((float)(send - sm.sv[r])) : 0.f;
    }
    __syncthreads();

    // ---- the block's quadratic form: M = L o G, L o dM and dM o M, lower
    // tiles on the matrix cores, upper tiles zero
    for (int t = wave; t < TQ * TQ; t += NW) {
        const int it = t / TQ, jt = t % TQ;
        f32x4 G = {0.f, 0.f, 0.f, 0.f}, D = {0.f, 0.f, 0.f, 0.f};
        if (jt <= it) {
            G = mm<HSUM>([&](int m, int k) { return sm.Cs[it * 16 + m][k]; },
                   [&](int k, int m) { return sm.Bs[jt * 16 + m][k]; }, 0, N, G);
            D = mm<HSUM>([&](int m, int k) { return sm.Ys[it * 16 + m][k]; },
                   [&](int k, int m) { return sm.Xs[jt * 16 + m][k]; }, 0, P, D);
        }
        const int j = jt * 16 + lm;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = it * 16 + 4 * gq + r;
            float M = 0.f, dG = 0.f, Z = 0.f;
            if (j <= i && i < len) {
                const float dm = D[r] * sm.dtv[j];
                const float Lij = expf((float)(sm.sv[i] - sm.sv[j]));
                M = Lij * G[r];
                dG = Lij * dm;
                Z = dm * M;
            }
            sm.u.q.Ms[i][j] = M;
            sm.u.q.Gs[i][j] = dG;
            sm.u.q.Zs[i][j] = Z;
        }
    }
    (void)LT;
    __syncthreads();

    // ---- quadratic-form gradients
    // the block's share of da_k = sum_{i >= k} ds_i. Summed over i >= k,
    // (row i of Z minus column i of Z) leaves the rectangle R(k) =
    // sum_{i >= k > j} Z_ij (the pairs with both ends >= k cancel); it is
    // built without that cancellation as R(k+1) = R(k) + sum_{i > k} Z_ik -
    // sum_{j < k} Z_kj. Here: those two sums per k, 8 lanes per k.
    {
        const int k = tid / LPR, part = tid % LPR;
        float cs = 0.f, rp = 0.f;
        for (int i = part; i < kQ; i += LPR) {
            if (i > k) cs += sm.u.q.Zs[i][k];
            if (i < k) rp += sm.u.q.Zs[k][i];
        }
        cs = group_sum<LPR>(cs);
        rp = group_sum<LPR>(rp);
        if (part == 0) sm.dsi[k] = cs - rp;
    }
    f32x4 dxd[XPW], dcv[CPW], dbv[CPW];
#pragma unroll
    for (int u = 0; u < XPW; ++u) {
        const int t = wave + u * NW;
        dxd[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < XT) {
            const int jt = t / TP, pt = t % TP;
            // dxd_j = sum_{i >= j} M_ij dy_i
            dxd[u] = mm<HSUM>([&](int m, int k) { return sm.u.q.Ms[k][jt * 16 + m]; },
                        [&](int k, int m) { return sm.Ys[k][pt * 16 + m]; }, jt * 16, kQ, dxd[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int t = wave + u * NW;
        dcv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        dbv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < CT) {
            const int rt = t / TN, nt = t % TN;
            // dC_i = sum_{j <= i} (L o dM)_ij B_j
            dcv[u] = mm<HSUM>([&](int m, int k) { return sm.u.q.Gs[rt * 16 + m][k]; },
                        [&](int k, int m) { return sm.Bs[k][nt * 16 + m]; }, 0, rt * 16 + 16, dcv[u]);
            // dB_j = sum_{i >= j} (L o dM)_ij C_i
            dbv[u] = mm<HSUM>([&](int m, int k) { return sm.u.q.Gs[k][rt * 16 + m]; },
                        [&](int k, int m) { return sm.Cs[k][nt * 16 + m]; }, rt * 16, kQ, dbv[u]);
        }
    }
    __syncthreads();

    // ---- terms of the entering state Hp
    store_flat<NP, NT, P, HSUM>(fhp, sm.u.st.Hs);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int t = wave + u * NW;
        if (t < CT) {
            const int rt = t / TN, nt = t % TN;
            // dC_i += e^{s_i} Hp dy_i
            f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
            tmp = mm<HSUM>([&](int m, int k) { return sm.Ys[rt * 16 + m][k]; },
                     [&](int k, int m) { return sm.u.st.Hs[nt * 16 + m][k]; }, 0, P, tmp);
#pragma unroll
            for (int r = 0; r < 4; ++r) dcv[u][r] = fmaf(sm.es[rt * 16 + 4 * gq + r], tmp[r], dcv[u][r]);
        }
    }
#pragma unroll
    for (int u = 0; u < XPW; ++u) {
        const int t = wave + u * NW;
        if (t < XT) {
            const int it = t / TP, pt = t % TP;
            // (C_i^T Hp)[p] dy_i[p], summed over p below
            f32x4 ch = {0.f, 0.f, 0.f, 0.f};
            ch = mm<HSUM>([&](int m, int k) { return sm.Cs[it * 16 + m][k]; },
                    [&](int k, int m) { return sm.u.st.Hs[k][pt * 16 + m]; }, 0, N, ch);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = it * 16 + 4 * gq + r, p = pt * 16 + lm;
                sm.u.st.Tq[i][p] = ch[r] * sm.Ys[i][p];
            }
        }
    }
    // <Hp, dHe> over the whole state (block tree, fixed order)
    float hd = 0.f;
#pragma unroll
    for (int k = 0; k < Flat<NP, NT>::VPT; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) hd = fmaf(fhp.v[k][i], fdh.v[k][i], hd);
    hd = wave_sum(hd);
    if (lane == 0) sm.red[wave] = hd;
    __syncthreads();
    float hp_dhe = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) hp_dhe += sm.red[w];
    {
        const int r = tid / LPR, part = tid % LPR;
        float acc = 0.f;
        for (int p = part; p < P; p += LPR) acc += sm.u.st.Tq[r][p];
        acc = group_sum<LPR>(acc);
        if (part == 0) sm.dso[r] = r < len ? sm.es[r] * acc : 0.f;
    }
    __syncthreads();

    // ---- terms of the leaving-state gradient dHe
    store_flat<NP, NT, P, HSUM>(fdh, sm.u.st.Hs);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < XPW; ++u) {
        const int t = wave + u * NW;
        if (t < XT) {
            const int jt = t / TP, pt = t % TP;
            // (B_j^T dHe)[p]: dxd_j += e^{s_end - s_j} B_j^T dHe
            f32x4 bdh = {0.f, 0.f, 0.f, 0.f};
            bdh = mm<HSUM>([&](int m, int k) { return sm.Bs[jt * 16 + m][k]; },
                     [&](int k, int m) { return sm.u.st.Hs[k][pt * 16 + m]; }, 0, N, bdh);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = jt * 16 + 4 * gq + r, p = pt * 16 + lm;
                dxd[u][r] = fmaf(sm.wv[j], bdh[r], dxd[u][r]);
                sm.u.st.Tq[j][p] = sm.Xs[j][p] * bdh[r];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int t = wave + u * NW;
        if (t < CT) {
            const int rt = t / TN, nt = t % TN;
            // dB_j += e^{s_end - s_j} dt_j dHe x_j
            f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
            tmp = mm<HSUM>([&](int m, int k) { return sm.Xs[rt * 16 + m][k]; },
                     [&](int k, int m) { return sm.u.st.Hs[nt * 16 + m][k]; }, 0, P, tmp);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = rt * 16 + 4 * gq + r;
                dbv[u][r] = fmaf(sm.wv[j] * sm.dtv[j], tmp[r], dbv[u][r]);
            }
        }
    }
    __syncthreads();
    {
        const int r = tid / LPR, part = tid % LPR;
        float acc = 0.f;
        for (int p = part; p < P; p += LPR) acc += sm.u.st.Tq[r][p];
        acc = group_sum<LPR>(acc);
        if (part == 0) sm.dss[r] = -sm.wv[r] * sm.dtv[r] * acc;
    }

    // ---- per-head dB, dC into the workspace (staged in LDS over B and C,
    // which are no longer read, then written a row at a time), or summed
    // over the heads in registers; dxd into LDS
    if (HSUM) {
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            accb[u] = first ? dbv[u] : accb[u] + dbv[u];
            accc[u] = first ? dcv[u] : accc[u] + dcv[u];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int t = wave + u * NW;
        if (!HSUM && t < CT) {
            const int rt = t / TN, nt = t % TN;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sm.Bs[rt * 16 + 4 * gq + r][nt * 16 + lm] = dbv[u][r];
                sm.Cs[rt * 16 + 4 * gq + r][nt * 16 + lm] = dcv[u][r];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < XPW; ++u) {
        const int t = wave + u * NW;
        if (t < XT) {
            const int jt = t / TP, pt = t % TP;
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.u.Dx[jt * 16 + 4 * gq + r][pt * 16 + lm] = dxd[u][r];
        }
    }
    __syncthreads();
    if (!HSUM) {
        const size_t pb = unit * (size_t)a.L * N;
        for (int e4 = tid; e4 < len * (N / 4); e4 += NT) {
            const int row = e4 / (N / 4), cc = (e4 % (N / 4)) * 4;
            const size_t o = pb + (size_t)tok_of(k0 + row, a.L, rev) * N + cc;
            *(float4 *)(a.dBp + o) = *(const float4 *)&sm.Bs[row][cc];
            *(float4 *)(a.dCp + o) = *(const float4 *)&sm.Cs[row][cc];
        }
    }

    // ---- per-position sums x . dxd and x . dy, 8 lanes per position
    {
        const int r = tid / LPR, part = tid % LPR;
        float xd = 0.f, xy = 0.f;
        for (int p = part; p < P; p += LPR) {
            xd = fmaf(sm.Xs[r][p], sm.u.Dx[r][p], xd);
            xy = fmaf(sm.Xs[r][p], sm.Ys[r][p], xy);
        }
        xd = group_sum<LPR>(xd);
        xy = group_sum<LPR>(xy);
        if (part == 0) {
            sm.red[r] = xd;
            sm.red[kQ + r] = xy;
        }
    }
    __syncthreads();

    // ---- da_k = sum_{i >= k} ds_i, each part summed without cancellation:
    // the quadratic form's rectangle R(k) (an exclusive running sum of the
    // per-k terms above), the carried-state terms over i >= k, and the
    // leaving-state terms, whose sum over i >= k is e^{s_end} <Hp, dHe>
    // minus their sum over j < k. One lane per position, fp64 scans.
    const float A = d.A[h];
    const float Dh = d.D ? d.D[h] : 0.f;
    if (tid < kQ) {
        const int r = tid;
        const double q = sm.dsi[r];
        const double rect = wave_scan(q, r) - q;
        const double so_rev = wave_scan((double)sm.dso[kQ - 1 - r], r);   // suffix sums, reversed
        const double so_suf = __shfl(so_rev, kQ - 1 - r);
        const double ss = sm.dss[r];
        const double ss_pre = wave_scan(ss, r) - ss;
        const double da = r < len ? rect + so_suf + (double)sm.es[len - 1] * hp_dhe - ss_pre : 0.0;
        if (r < len) gr.ddt[(rowt + tok_of(k0 + r, a.L, rev)) * a.H + h] = sm.red[r] + A * (float)da;
        const float sa = wave_sum(r < len ? sm.dtv[r] * (float)da : 0.f);
        const float sd = wave_sum(sm.red[kQ + r]);
        if (r == 0) {
            a.dDp[unit * a.nc + c] = sd;
            a.dAp[unit * a.nc + c] = sa;
        }
    }
    for (int e = tid; e < len * P; e += NT) {
        const int r = e / P, p = e % P;
        gr.dx[((rowt + tok_of(k0 + r, a.L, rev)) * a.H + h) * P + p] =
            fmaf(Dh, sm.Ys[r][p], sm.dtv[r] * sm.u.Dx[r][p]);
    }
}

// One workgroup per (block, head, row and stream); dB, dC per head.
template <typename T, int P, int N>
__global__ __launch_bounds__(kGradThreads) void k_bwd_grad(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) GradSmem<P, N> sm;
    const int dir = (int)(blockIdx.z % (unsigned)a.ndir), b = (int)(blockIdx.z / (unsigned)a.ndir);
    grad_block<T, P, N, false>(a, sm, blockIdx.x, blockIdx.y, dir, b, false, nullptr, nullptr);
}

// One workgroup per (block, group, row and stream), walking the group's
// heads in order; dB, dC summed over them in place.
template <typename T, int P, int N>
__global__ __launch_bounds__(kGradThreads) void k_bwd_grad_heads(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) GradSmem<P, N> sm;
    const int dir = (int)(blockIdx.z % (unsigned)a.ndir), b = (int)(blockIdx.z / (unsigned)a.ndir);
    constexpr int NT = kGradThreads, NW = NT / 64, TQ = kQ / 16, TN = N / 16;
    constexpr int CT = TQ * TN, CPW = (CT + NW - 1) / NW;
    const int hg = a.H / a.G, g = blockIdx.y, h0 = g * hg, c = blockIdx.x;
    f32x4 accb[CPW], accc[CPW];
    for (int k = 0; k < hg; ++k) {
        if (k) __syncthreads();   // the previous head's last phase reads the LDS rows
        grad_block<T, P, N, true>(a, sm, c, h0 + k, dir, b, k == 0, accb, accc);
    }
    // the group's dB, dC of the block: staged over B and C in LDS, then
    // written a row at a time
    const bool rev = dir == 1;
    const GradPtrs gr = rev ? a.gbwd : a.gfwd;
    const int k0 = c * kQ, len = min(kQ, a.L - k0);
    const size_t rowt = (size_t)b * a.L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, lm = lane & 15;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int t = wave + u * NW;
        if (t < CT) {
            const int rt = t / TN, nt = t % TN;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sm.Bs[rt * 16 + 4 * gq + r][nt * 16 + lm] = accb[u][r];
                sm.Cs[rt * 16 + 4 * gq + r][nt * 16 + lm] = accc[u][r];
            }
        }
    }
    __syncthreads();
    for (int e4 = tid; e4 < len * (N / 4); e4 += NT) {
        const int row = e4 / (N / 4), cc = (e4 % (N / 4)) * 4;
        const size_t o = ((rowt + tok_of(k0 + row, a.L, rev)) * a.G + g) * N + cc;
        *(float4 *)(gr.dB + o) = *(const float4 *)&sm.Bs[row][cc];
        *(float4 *)(gr.dC + o) = *(const float4 *)&sm.Cs[row][cc];
    }
}

// ---- the gradient block on the bf16 matrix cores (bf16 inputs, headdim
// 64, d_state 128): the same terms as grad_block, every product a sum of
// bf16 products with fp32 accumulation. B, C and x enter as given (exact);
// the fp32 operands (dy, M = L o G, L o dM, Hp, dHe) as the exact sum of
// three bf16 parts. Operands are read so that both of a product agree on the
// order of k inside an instruction: lane group g holds k32 + 4g + (0..3) and
// k32 + 16 + 4g + (0..3), read along a row (dir_op) or down the rows of a
// row-major tile (tr_ops).

// The bf16 tiles of this kernel are row-major [row][col] arrays padded by
// 16 elements a row (so that consecutive rows start 4 bank pairs apart, of
// 16 pairs of 4-byte banks), with bits 2..3 of the column index XORed with
// (row / 4) % 4: the 16 lanes that one LDS cycle serves then fall on 16
// different bank pairs both when they read one 4-column group of 16
// consecutive rows (dir_op, and the row-wise writes) and when they read 4
// groups of 4 consecutive rows (tr_ops). The XOR touches only the bits that
// vary between a wave's lanes, so an operand's address is a per-lane base
// plus an offset fixed where it is read.
__device__ __forceinline__ int swz_x(int r) { return ((r >> 2) & 3) << 2; }
template <int RS>
__device__ __forceinline__ int swz(int r, int col) { return r * RS + (col ^ swz_x(r)); }

// Matrix-core operand from rows m0 + (lane % 16) of a swizzled tile (row
// stride RS; m0 a multiple of 16), k along the row from k32.
template <int RS>
__device__ __forceinline__ u32x4 dir_op(const uint16_t *base, int m0, int k32) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, m = lane & 15;
    const uint16_t *p = base + (m0 + m) * RS + k32 + ((4 * g4) ^ swz_x(m));
    const u32x2 x0 = *(const u32x2 *)p, x1 = *(const u32x2 *)(p + 16);
    return u32x4{x0[0], x0[1], x1[0], x1[1]};
}

// Matrix-core operand for the 16 columns c0 .. c0+15 (c0 a multiple of 16)
// of a swizzled tile, k down its rows t32 .. t32+31 (t32 a multiple of 32),
// by two transposing LDS reads (ds_read_b64_tr_b16: lane s of a 16-lane
// group points at row t + s/4, columns c0 + 4 (s%4) .. +3, and lane i
// receives column c0 + i of those 4 rows; here (row / 4) % 4 is the lane
// group g, so the XOR is (s%4) ^ g).
template <int RS>
__device__ __forceinline__ u32x4 tr_ops(const uint16_t *base, int t32, int c0) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, s = lane & 15;
    const uint16_t *p = base + (t32 + 4 * g4 + (s >> 2)) * RS + c0 + 4 * ((s & 3) ^ g4);
    const v4i16_v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_v *)p);
    const v4i16_v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_v *)(p + 16 * RS));
    const u32x2 ua = __builtin_bit_cast(u32x2, x0), ub = __builtin_bit_cast(u32x2, x1);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// acc += A B with both operands in three parts, the six products down to
// the second parts' product (the rest is below 2^-24 of the leading one)
__device__ __forceinline__ f32x4 mfma_split6(const u32x4 (&x)[3], const u32x4 (&y)[3], f32x4 acc) {
    acc = mfma16x16x32(x[1], y[1], acc);
    acc = mfma16x16x32(x[2], y[0], acc);
    acc = mfma16x16x32(x[0], y[2], acc);
    acc = mfma16x16x32(x[1], y[0], acc);
    acc = mfma16x16x32(x[0], y[1], acc);
    return mfma16x16x32(x[0], y[0], acc);
}

// the value an element of a three-part array holds (the parts' exact sum)
__device__ __forceinline__ float part_sum(const uint16_t *p0, size_t stride) {
    return (bf2f(p0[2 * stride]) + bf2f(p0[stride])) + bf2f(p0[0]);
}

// four values (rows of one column) as three parts, into [col][row0 .. row0+3]
// of three [.][rs] arrays spaced by stride elements
__device__ __forceinline__ void put_split4(uint16_t *dst, size_t stride, const float *v) {
    uint32_t p01[3], p23[3];
    split3(v[0], v[1], p01);
    split3(v[2], v[3], p23);
#pragma unroll
    for (int q = 0; q < 3; ++q) *(u32x2 *)(dst + q * stride) = u32x2{p01[q], p23[q]};
}

// Cross-lane sums by DPP (data-parallel primitives: a VALU operand read from
// another lane of the same 16-lane row, row_shr:n = 0x110 + n, or the last
// lane of a row broadcast to the next rows, row_bcast:15 = 0x142 and
// row_bcast:31 = 0x143), instead of LDS permutes. Lanes whose source falls
// outside the row, or whose row is masked off, add 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, true));
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ double dpp_d(double v) {
    const long long u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)u, CTRL, ROWS, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, ROWS, 0xf, true);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Sum over each 16-lane row of the wave, in the row's last lane (lane % 16
// == 15; the other lanes hold partial sums).
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f<0x111>(v);
    v += dpp_f<0x112>(v);
    v += dpp_f<0x114>(v);
    v += dpp_f<0x118>(v);
    return v;
}

// Inclusive running sum over the 64 lanes (lane order), fp64: within rows,
// then each row adds the totals of the rows before it.
__device__ __forceinline__ double wave_scan_dpp(double v) {
    v += dpp_d<0x111>(v);
    v += dpp_d<0x112>(v);
    v += dpp_d<0x114>(v);
    v += dpp_d<0x118>(v);
    v += dpp_d<0x142, 0xa>(v);
    v += dpp_d<0x143, 0xc>(v);
    return v;
}

// Sum over the wave (in every lane).
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f<0x111>(v);
    v += dpp_f<0x112>(v);
    v += dpp_f<0x114>(v);
    v += dpp_f<0x118>(v);
    v += dpp_f<0x142, 0xa>(v);
    v += dpp_f<0x143, 0xc>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

constexpr int kMxThreads = 1024;   // 16 waves: one per 16 x 16 tile of the block's square

struct GradMxSmem {
    static constexpr int P = 64, N = 128;
    static constexpr int RN = N + 16, RP = P + 16, RQ = kQ + 16;   // bf16 row strides
    uint16_t bx[kQ * RN];      // B rows [t][n]
    uint16_t cx[kQ * RN];      // C rows [t][n]
    uint16_t xx[kQ * RP];      // x rows [t][p]
    uint16_t y3[3][kQ * RP];   // dy rows [t][p], three parts
    union {
        struct {
            uint16_t mt[3][kQ * RQ];   // M^T [j][i], three parts
            uint16_t gt[3][kQ * RQ];   // (L o dM)^T [j][i], three parts
        } q;
        uint16_t ht[3][P * RN];        // Hp^T, then dHe^T: [p][n], three parts
    } u;
    float colz[4][kQ];   // sums of the strictly lower Z over each tile row of i, per column
    float rowz[4][kQ];   // ... over each tile column of j, per row
    float dsop[4][kQ];   // per position, sums over each 16 p of (C^T Hp) o dy
    float dssp[4][kQ];   // ... of x o (B^T dHe)
    float xdp[4][kQ];    // ... of x o dxd
    float xyr[kQ];       // per position, x . dy
    double sv[kQ];
    float dtv[kQ], es[kQ], wv[kQ];
    float red[16];
};

// G holds the wave's tile of the block's Gram C B^T: the same for every head
// of a group, so computed with the first head only when walking them (HSUM).
template <bool HSUM>
__device__ __forceinline__ void grad_mx(const BwdArgs &a, GradMxSmem &sm, const int c, const int h,
                                        const int dir, const int b, const bool first,
                                        f32x4 (&accb)[2], f32x4 (&accc)[2], f32x4 &G) {
    using Sm = GradMxSmem;
    constexpr int P = Sm::P, N = Sm::N, RN = Sm::RN, RP = Sm::RP, RQ = Sm::RQ;
    constexpr size_t YS = (size_t)kQ * RP, QS = (size_t)kQ * RQ, HS = (size_t)P * RN;   // part strides
    const bool rev = dir == 1;
    const DirPtrs d = rev ? a.bwd : a.fwd;
    const GradPtrs gr = rev ? a.gbwd : a.gfwd;
    const int g = h / (a.H / a.G);
    const int k0 = c * kQ;
    const int len = min(kQ, a.L - k0);
    const size_t rowt = (size_t)b * a.L;
    const int tid = lane_tid<HSUM>(), wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const size_t unit = ((size_t)b * a.ndir + dir) * a.H + h;
    const size_t so = (unit * a.nc + c) * (size_t)(N * P);
    const size_t sgn = (size_t)a.G * N, hp = (size_t)a.H * P;

    // ---- loads, all issued before any is used (rows past the block's end
    // re-read its last row and are zeroed when staged): B and C rows (two
    // 4-vectors per thread), x and dy rows (one), dt (wave 0), and Hp, dHe
    // (two 4-vectors each, held until their phases)
    const bool bc = !HSUM || first;
    u32x2 rbv[2], rcv[2], rxv;
    f32x4 ryv, fhp[2], fdh[2];
    uint16_t dtr = 0;
    if (bc) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e4 = tid + k * kMxThreads, r = min(e4 >> 5, len - 1), cc = (e4 & 31) * 4;
            const size_t o = (rowt + tok_of(k0 + r, a.L, rev)) * sgn + (size_t)g * N + cc;
            rbv[k] = *(const u32x2 *)((const uint16_t *)d.B + o);
            rcv[k] = *(const u32x2 *)((const uint16_t *)d.C + o);
        }
    }
    {
        const int r = min(tid >> 4, len - 1), cc = (tid & 15) * 4;
        const size_t o = (rowt + tok_of(k0 + r, a.L, rev)) * hp + (size_t)h * P + cc;
        rxv = *(const u32x2 *)((const uint16_t *)d.x + o);
        ryv = *(const f32x4 *)(a.dy + o);
    }
    if (tid < kQ) dtr = ((const uint16_t *)d.dt)[(rowt + tok_of(k0 + min(tid, len - 1), a.L, rev)) * a.H + h];

    // ---- the block's running sums of dt A (fp64), weights; the rows into LDS
    if (tid < kQ) {
        const float dtf = tid < len ? bf2f(dtr) : 0.f;
        const double s = wave_scan_dpp((double)dtf * (double)d.A[h]);
        const long long su = __double_as_longlong(s);
        const double send = __longlong_as_double(
            ((long long)__builtin_amdgcn_readlane((int)(su >> 32), len - 1) << 32) |
            (unsigned)__builtin_amdgcn_readlane((int)su, len - 1));
        sm.sv[tid] = s;
        sm.dtv[tid] = dtf;
        sm.es[tid] = tid < len ? expf((float)s) : 0.f;
        sm.wv[tid] = tid < len ? expf((float)(send - s)) : 0.f;
    }
    if (bc) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e4 = tid + k * kMxThreads, r = e4 >> 5, cc = (e4 & 31) * 4;
            const bool ok = r < len;
            *(u32x2 *)&sm.bx[swz<RN>(r, cc)] = u32x2{ok ? rbv[k][0] : 0u, ok ? rbv[k][1] : 0u};
            *(u32x2 *)&sm.cx[swz<RN>(r, cc)] = u32x2{ok ? rcv[k][0] : 0u, ok ? rcv[k][1] : 0u};
        }
    }
    {
        const int r = tid >> 4, cc = (tid & 15) * 4;
        const bool ok = r < len;
        const u32x2 xv = u32x2{ok ? rxv[0] : 0u, ok ? rxv[1] : 0u};
        *(u32x2 *)&sm.xx[swz<RP>(r, cc)] = xv;
        float yv[4] = {ok ? ryv[0] : 0.f, ok ? ryv[1] : 0.f, ok ? ryv[2] : 0.f, ok ? ryv[3] : 0.f};
        put_split4(&sm.y3[0][swz<RP>(r, cc)], YS, yv);
        // x . dy of the position (the thread's four p, then the row's 16 lanes)
        float xy = bf_low(xv[0]) * yv[0];
        xy = fmaf(bf_high(xv[0]), yv[1], xy);
        xy = fmaf(bf_low(xv[1]), yv[2], xy);
        xy = fmaf(bf_high(xv[1]), yv[3], xy);
        xy = sum16(xy);
        if ((tid & 15) == 15) sm.xyr[r] = xy;
    }
    __syncthreads();
    // Hp and dHe (needed after the quadratic form) go out after the first
    // barrier, which waits for every load in flight: the staging then waits
    // only for the rows it stores
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        fhp[k] = *(const f32x4 *)(a.S + so + 4 * (tid + k * kMxThreads));
        fdh[k] = *(const f32x4 *)(a.R + so + 4 * (tid + k * kMxThreads));
    }

    // ---- the block's quadratic form, one 16 x 16 tile (it, jt) per wave:
    // G = C B^T, dM = dy x^T dt_j; M = L o G, L o dM into LDS (transposed,
    // three parts; zeros above the diagonal), and the strictly lower Z = dM o
    // M summed over the tile's rows and columns
    const int it = wave >> 2, jt = wave & 3;
    {
        float M[4] = {0.f, 0.f, 0.f, 0.f}, dG[4] = {0.f, 0.f, 0.f, 0.f}, zs[4] = {0.f, 0.f, 0.f, 0.f};
        const int j = jt * 16 + l16;
        if (jt <= it) {
            f32x4 D = zero4();
            if (!HSUM || first) {
                G = zero4();
#pragma unroll
                for (int kc = 0; kc < N / 32; ++kc)
                    G = mfma16x16x32(dir_op<RN>(sm.cx, it * 16, 32 * kc), dir_op<RN>(sm.bx, jt * 16, 32 * kc), G);
            }
#pragma unroll
            for (int kc = 0; kc < P / 32; ++kc) {
                const u32x4 xo = dir_op<RP>(sm.xx, jt * 16, 32 * kc);
#pragma unroll
                for (int q = 2; q >= 0; --q) D = mfma16x16x32(dir_op<RP>(sm.y3[q], it * 16, 32 * kc), xo, D);
            }
            const float dtj = sm.dtv[j];
            const double svj = sm.sv[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = it * 16 + 4 * g4 + r;
                if (j <= i && i < len) {
                    const float dm = D[r] * dtj;
                    const float Lij = expf((float)(sm.sv[i] - svj));
                    M[r] = Lij * G[r];
                    dG[r] = Lij * dm;
                    zs[r] = j < i ? dm * M[r] : 0.f;
                }
            }
        }
        put_split4(&sm.u.q.mt[0][swz<RQ>(j, it * 16 + 4 * g4)], QS, M);
        put_split4(&sm.u.q.gt[0][swz<RQ>(j, it * 16 + 4 * g4)], QS, dG);
        float cz = (zs[0] + zs[1]) + (zs[2] + zs[3]);
        cz += __shfl_xor(cz, 16);
        cz += __shfl_xor(cz, 32);
        if (g4 == 0) sm.colz[it][j] = cz;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float rz = sum16(zs[r]);
            if (l16 == 15) sm.rowz[jt][it * 16 + 4 * g4 + r] = rz;
        }
    }
    __syncthreads();

    // ---- the quadratic form's gradients: dxd (tile (jt, pt) = (it, jt) of
    // the wave), dC and dB (two tiles each: t = wave, wave + 16 of 4 x 8)
    f32x4 dxd = zero4(), dcv[2], dbv[2];
    {
        const int jr = it, pt = jt;   // dxd_j = sum_{i >= j} M_ij dy_i
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            if (kc == 0 && jr > 1) continue;
            u32x4 x3[3], y3[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                x3[q] = dir_op<RQ>(sm.u.q.mt[q], jr * 16, 32 * kc);
                y3[q] = tr_ops<RP>(sm.y3[q], 32 * kc, pt * 16);
            }
            dxd = mfma_split6(x3, y3, dxd);
        }
    }
    // (the wave's two tiles t = wave, wave + 16 of the 4 x 8 (row, n) tiles
    // share their columns n: rows rt0 = wave / 8 and rt0 + 2)
    const int rt0 = wave >> 3, ntw = wave & 7;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        dcv[u] = zero4();
        dbv[u] = zero4();
    }
    // dC_i = sum_{j <= i} (L o dM)_ij B_j (j chunk 1 only for rows 32 ..)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const u32x4 bo = tr_ops<RN>(sm.bx, 32 * kc, ntw * 16);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (kc == 1 && u == 0) continue;
#pragma unroll
            for (int q = 2; q >= 0; --q)
                dcv[u] = mfma16x16x32(tr_ops<RQ>(sm.u.q.gt[q], 32 * kc, (rt0 + 2 * u) * 16), bo, dcv[u]);
        }
    }
    // dB_j = sum_{i >= j} (L o dM)_ij C_i (i chunk 0 only for rows .. 31)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const u32x4 co = tr_ops<RN>(sm.cx, 32 * kc, ntw * 16);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (kc == 0 && u == 1) continue;
#pragma unroll
            for (int q = 2; q >= 0; --q)
                dbv[u] = mfma16x16x32(dir_op<RQ>(sm.u.q.gt[q], (rt0 + 2 * u) * 16, 32 * kc), co, dbv[u]);
        }
    }
    __syncthreads();

    // ---- terms of the entering state Hp (staged transposed, three parts)
    float hd = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e4 = tid + k * kMxThreads, tile = e4 >> 6, ln = e4 & 63;
        const int n0 = (tile >> 2) * 16 + 4 * (ln >> 4), p = (tile & 3) * 16 + (ln & 15);
        const float v[4] = {fhp[k][0], fhp[k][1], fhp[k][2], fhp[k][3]};
        put_split4(&sm.u.ht[0][swz<RN>(p, n0)], HS, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) hd = fmaf(fhp[k][i], fdh[k][i], hd);
    }
    hd = wave_sum_dpp(hd);
    if (lane == 0) sm.red[wave] = hd;
    __syncthreads();
    {
        // dC_i += e^{s_i} Hp dy_i (Hp's operand shared by the two tiles)
        f32x4 tmp[2] = {zero4(), zero4()};
#pragma unroll
        for (int kc = 0; kc < P / 32; ++kc) {
            u32x4 h3[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) h3[q] = tr_ops<RN>(sm.u.ht[q], 32 * kc, ntw * 16);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                u32x4 x3[3];
#pragma unroll
                for (int q = 0; q < 3; ++q) x3[q] = dir_op<RP>(sm.y3[q], (rt0 + 2 * u) * 16, 32 * kc);
                tmp[u] = mfma_split6(x3, h3, tmp[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dcv[u][r] = fmaf(sm.es[(rt0 + 2 * u) * 16 + 4 * g4 + r], tmp[u][r], dcv[u][r]);
    }
    {
        // (C_i^T Hp)[p] dy_i[p], summed over p: tile (i, p) = (it, jt)
        f32x4 ch = zero4();
#pragma unroll
        for (int kc = 0; kc < N / 32; ++kc) {
            const u32x4 co = dir_op<RN>(sm.cx, it * 16, 32 * kc);
#pragma unroll
            for (int q = 2; q >= 0; --q) ch = mfma16x16x32(co, dir_op<RN>(sm.u.ht[q], jt * 16, 32 * kc), ch);
        }
        const int p = jt * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = it * 16 + 4 * g4 + r;
            const float v = sum16(ch[r] * part_sum(&sm.y3[0][swz<RP>(i, p)], YS));
            if (l16 == 15) sm.dsop[jt][i] = v;
        }
    }
    __syncthreads();

    // ---- terms of the leaving-state gradient dHe (over Hp in LDS)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e4 = tid + k * kMxThreads, tile = e4 >> 6, ln = e4 & 63;
        const int n0 = (tile >> 2) * 16 + 4 * (ln >> 4), p = (tile & 3) * 16 + (ln & 15);
        const float v[4] = {fdh[k][0], fdh[k][1], fdh[k][2], fdh[k][3]};
        put_split4(&sm.u.ht[0][swz<RN>(p, n0)], HS, v);
    }
    __syncthreads();
    {
        // (B_j^T dHe)[p]: dxd_j += e^{s_end - s_j} B_j^T dHe; x_j . (B_j^T dHe)
        f32x4 bdh = zero4();
#pragma unroll
        for (int kc = 0; kc < N / 32; ++kc) {
            const u32x4 bo = dir_op<RN>(sm.bx, it * 16, 32 * kc);
#pragma unroll
            for (int q = 2; q >= 0; --q) bdh = mfma16x16x32(bo, dir_op<RN>(sm.u.ht[q], jt * 16, 32 * kc), bdh);
        }
        const int p = jt * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = it * 16 + 4 * g4 + r;
            dxd[r] = fmaf(sm.wv[j], bdh[r], dxd[r]);
            const float v = sum16(bf2f(sm.xx[swz<RP>(j, p)]) * bdh[r]);
            if (l16 == 15) sm.dssp[jt][j] = v;
        }
    }
    {
        // dB_j += e^{s_end - s_j} dt_j dHe x_j (dHe's operand shared)
        f32x4 tmp[2] = {zero4(), zero4()};
#pragma unroll
        for (int kc = 0; kc < P / 32; ++kc) {
            u32x4 h3[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) h3[q] = tr_ops<RN>(sm.u.ht[q], 32 * kc, ntw * 16);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const u32x4 xo = dir_op<RP>(sm.xx, (rt0 + 2 * u) * 16, 32 * kc);
#pragma unroll
                for (int q = 2; q >= 0; --q) tmp[u] = mfma16x16x32(xo, h3[q], tmp[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = (rt0 + 2 * u) * 16 + 4 * g4 + r;
                dbv[u][r] = fmaf(sm.wv[j] * sm.dtv[j], tmp[u][r], dbv[u][r]);
            }
    }

    // ---- dB, dC: summed over the heads in registers, or per head into the
    // workspace; x . dxd per position; dx
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (HSUM) {
            accb[u] = first ? dbv[u] : accb[u] + dbv[u];
            accc[u] = first ? dcv[u] : accc[u] + dcv[u];
        } else {
            const int rt = rt0 + 2 * u, nt = ntw;
            const size_t pb = unit * (size_t)a.L * N;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rt * 16 + 4 * g4 + r;
                if (row < len) {
                    const size_t o = pb + (size_t)tok_of(k0 + row, a.L, rev) * N + nt * 16 + l16;
                    a.dBp[o] = dbv[u][r];
                    a.dCp[o] = dcv[u][r];
                }
            }
        }
    }
    const float A = d.A[h];
    const float Dh = d.D ? d.D[h] : 0.f;
    {
        const int p = jt * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = it * 16 + 4 * g4 + r;
            const float v = sum16(bf2f(sm.xx[swz<RP>(j, p)]) * dxd[r]);
            if (l16 == 15) sm.xdp[jt][j] = v;
            if (j < len)
                gr.dx[((rowt + tok_of(k0 + j, a.L, rev)) * a.H + h) * P + p] =
                    fmaf(Dh, part_sum(&sm.y3[0][swz<RP>(j, p)], YS), sm.dtv[j] * dxd[r]);
        }
    }
    __syncthreads();

    // ---- da_k = sum_{i >= k} ds_i as in grad_block; ddt, and the block's
    // shares of dA and dD. One lane per position, fp64 scans.
    if (tid < kQ) {
        const int r = tid;
        const float dsi = ((sm.colz[0][r] + sm.colz[1][r]) + (sm.colz[2][r] + sm.colz[3][r])) -
                          ((sm.rowz[0][r] + sm.rowz[1][r]) + (sm.rowz[2][r] + sm.rowz[3][r]));
        const float dso = r < len ? sm.es[r] * ((sm.dsop[0][r] + sm.dsop[1][r]) + (sm.dsop[2][r] + sm.dsop[3][r]))
                                  : 0.f;
        const float dss = -sm.wv[r] * sm.dtv[r] * ((sm.dssp[0][r] + sm.dssp[1][r]) + (sm.dssp[2][r] + sm.dssp[3][r]));
        const float xd = (sm.xdp[0][r] + sm.xdp[1][r]) + (sm.xdp[2][r] + sm.xdp[3][r]);
        float hp_dhe = 0.f;
#pragma unroll
        for (int w = 0; w < 16; ++w) hp_dhe += sm.red[w];
        const double q = dsi;
        const double rect = wave_scan_dpp(q) - q;
        const double so_rev = wave_scan_dpp((double)__shfl(dso, kQ - 1 - r));   // suffix sums, reversed
        const double so_suf = __shfl(so_rev, kQ - 1 - r);
        const double ss = dss;
        const double ss_pre = wave_scan_dpp(ss) - ss;
        const double da = r < len ? rect + so_suf + (double)sm.es[len - 1] * hp_dhe - ss_pre : 0.0;
        if (r < len) gr.ddt[(rowt + tok_of(k0 + r, a.L, rev)) * a.H + h] = xd + A * (float)da;
        const float sa = wave_sum_dpp(r < len ? sm.dtv[r] * (float)da : 0.f);
        const float sd = wave_sum_dpp(sm.xyr[r]);
        if (r == 0) {
            a.dDp[unit * a.nc + c] = sd;
            a.dAp[unit * a.nc + c] = sa;
        }
    }
}

// One workgroup per (block, head, row and stream); dB, dC per head.
__global__ __launch_bounds__(kMxThreads) void k_bwd_grad_mx(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) GradMxSmem sm;
    const int dir = (int)(blockIdx.z % (unsigned)a.ndir), b = (int)(blockIdx.z / (unsigned)a.ndir);
    f32x4 accb[2], accc[2], G;
    grad_mx<false>(a, sm, blockIdx.x, blockIdx.y, dir, b, false, accb, accc, G);
}

// One workgroup per (block, group, row and stream), walking the group's
// heads in order; dB, dC summed over them in registers.
__global__ __launch_bounds__(kMxThreads) void k_bwd_grad_heads_mx(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) GradMxSmem sm;
    constexpr int N = GradMxSmem::N;
    const int dir = (int)(blockIdx.z % (unsigned)a.ndir), b = (int)(blockIdx.z / (unsigned)a.ndir);
    const int hg = a.H / a.G, g = blockIdx.y, h0 = g * hg, c = blockIdx.x;
    f32x4 accb[2], accc[2], G = zero4();
    for (int k = 0; k < hg; ++k) {
        if (k) __syncthreads();   // the previous head's last phase reads the LDS rows
        grad_mx<true>(a, sm, c, h0 + k, dir, b, k == 0, accb, accc, G);
    }
    const bool rev = dir == 1;
    const GradPtrs gr = rev ? a.gbwd : a.gfwd;
    const int k0 = c * kQ, len = min(kQ, a.L - k0);
    const size_t rowt = (size_t)b * a.L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = wave + 16 * u, rt = t >> 3, nt = t & 7;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rt * 16 + 4 * g4 + r;
            if (row < len) {
                const size_t o = ((rowt + tok_of(k0 + row, a.L, rev)) * a.G + g) * N + nt * 16 + l16;
                gr.dB[o] = accb[u][r];
                gr.dC[o] = accc[u][r];
            }
        }
    }
}

// dB, dC of one stream: sums over the heads of each group, in head order.
__global__ __launch_bounds__(256) void k_bwd_sum_bc(BwdArgs a, int N, size_t total) {
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int dir = blockIdx.y;
    if (e >= total) return;
    // e indexes [batch][L][G][N]
    const int n = (int)(e % N);
    const int g = (int)((e / N) % a.G);
    const size_t bt = e / ((size_t)N * a.G);       // b * L + t
    const int b = (int)(bt / a.L), t = (int)(bt % a.L);
    const int hg = a.H / a.G;
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < hg; ++k) {
        const int h = g * hg + k;
        const size_t o = ((((size_t)b * a.ndir + dir) * a.H + h) * a.L + t) * N + n;
        sb += a.dBp[o];
        sc += a.dCp[o];
    }
    const GradPtrs gr = dir ? a.gbwd : a.gfwd;
    gr.dB[e] = sb;
    gr.dC[e] = sc;
}

// dA, dD of one stream: sums over rows and blocks, in order.
__global__ __launch_bounds__(64) void k_bwd_sum_ad(BwdArgs a) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    const int dir = blockIdx.y;
    if (h >= a.H) return;
    float sa = 0.f, sd = 0.f;
    for (int b = 0; b < a.batch; ++b)
        for (int c = 0; c < a.nc; ++c) {
            const size_t o = (((size_t)b * a.ndir + dir) * a.H + h) * a.nc + c;
            sa += a.dAp[o];
            sd += a.dDp[o];
        }
    const GradPtrs gr = dir ? a.gbwd : a.gfwd;
    gr.dA[h] = sa;
    if (gr.dD) gr.dD[h] = sd;
}

template <typename T, int P, int N>
hipError_t launch_pn(BwdArgs &a, hipStream_t s) {
    if (a.L > 0) {
        const dim3 grid(a.nc, a.H, a.batch * a.ndir);
        if (a.chain) {
            BM_LAUNCH("bwd_chain", (k_bwd_chain<T, P, N>), dim3(a.H, a.batch * a.ndir),
                      dim3(kChainThreads), 0, s, a);
        } else {
            BM_LAUNCH("bwd_state", (k_bwd_state<T, P, N>), grid, dim3(kStateThreads), 0, s, a);
            const dim3 pgrid((N * P + 255) / 256, a.H, a.batch * a.ndir);
            BM_LAUNCH("bwd_pass", k_bwd_pass, pgrid, dim3(256), 0, s, a, N * P);
        }
        // bf16 inputs at headdim 64, d_state 128: the gradient block on the
        // bf16 matrix cores
        constexpr bool MX = sizeof(T) == 2 && P == GradMxSmem::P && N == GradMxSmem::N;
        if (a.head_loop) {
            const dim3 ggrid(a.nc, a.G, a.batch * a.ndir);
            if (MX)
                BM_LAUNCH("bwd_grad", k_bwd_grad_heads_mx, ggrid, dim3(kMxThreads), 0, s, a);
            else
                BM_LAUNCH("bwd_grad", (k_bwd_grad_heads<T, P, N>), ggrid, dim3(kGradThreads), 0, s, a);
        } else {
            if (MX)
                BM_LAUNCH("bwd_grad", k_bwd_grad_mx, grid, dim3(kMxThreads), 0, s, a);
            else
                BM_LAUNCH("bwd_grad", (k_bwd_grad<T, P, N>), grid, dim3(kGradThreads), 0, s, a);
            const size_t total = (size_t)a.batch * a.L * a.G * N;
            const dim3 sgrid((unsigned)((total + 255) / 256), a.ndir);
            BM_LAUNCH("bwd_sum_bc", k_bwd_sum_bc, sgrid, dim3(256), 0, s, a, N, total);
        }
    }
    BM_LAUNCH("bwd_sum_ad", k_bwd_sum_ad, dim3((a.H + 63) / 64, a.ndir), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(BwdArgs &a, int P, int N, hipStream_t s) {
    if (P == 64 && N == 128) return launch_pn<T, 64, 128>(a, s);
    if (P == 64 && N == 16) return launch_pn<T, 64, 16>(a, s);
    if (P == 16 && N == 128) return launch_pn<T, 16, 128>(a, s);
    if (P == 16 && N == 16) return launch_pn<T, 16, 16>(a, s);
    return hipErrorInvalidValue;
}

struct BwdLayout {
    size_t S, R, lg, dBp, dCp, dAp, dDp, total;
};

size_t al(size_t n) { return (n + 255) & ~(size_t)255; }

// Whether the gradient kernel walks the heads of each group: once the
// (block, row, stream) workgroups alone cover the CUs (one gradient
// workgroup fits per CU), walking the heads costs no parallelism and removes
// the per-head dB, dC arrays and their sum.
bool head_loop(int batch, int L, int ndir) {
    const long long nc = (L + kQ - 1) / kQ;
    return nc * batch * ndir >= 256;
}

// Whether the entering states and leaving-state gradients come from the
// chained kernel: it walks a unit's blocks one after another, so it needs
// units to fill the CUs (two or more chains per CU) or few blocks per chain;
// otherwise the block-parallel state kernel and the element-parallel pass
// over its output take less time despite their traffic.
bool use_chain(int batch, int L, int H, int ndir) {
    const long long nc = (L + kQ - 1) / kQ, units = (long long)batch * ndir * H;
    return units >= 512 || nc <= 16;
}

BwdLayout layout(int batch, int L, int H, int P, int N, int ndir) {
    const size_t nc = (size_t)(L + kQ - 1) / kQ;
    const size_t units = (size_t)batch * ndir * H;
    const size_t per_head = head_loop(batch, L, ndir) ? 0 : units * (size_t)L * N * sizeof(float);
    BwdLayout w;
    size_t off = 0;
    w.S = off; off += al(units * nc * N * P * sizeof(float));
    w.R = off; off += al(units * nc * N * P * sizeof(float));
    w.lg = off; off += al(units * nc * sizeof(double));
    w.dBp = off; off += al(per_head);
    w.dCp = off; off += al(per_head);
    w.dAp = off; off += al(units * nc * sizeof(float));
    w.dDp = off; off += al(units * nc * sizeof(float));
    w.total = off;
    return w;
}

}  // namespace

bool bwd_supported(int P, int N) { return (P == 16 || P == 64) && (N == 16 || N == 128); }

size_t bwd_workspace(int batch, int L, int H, int P, int N, int ndir) {
    return layout(batch, L, H, P, N, ndir).total;
}

hipError_t launch_bwd(const BwdProblem &p, void *ws, hipStream_t s) {
    BwdArgs a;
    a.fwd = p.dir[0];
    a.bwd = p.dir[1];
    a.gfwd = p.grad[0];
    a.gbwd = p.grad[1];
    a.dy = p.dy;
    a.batch = p.batch;
    a.L = p.L;
    a.H = p.H;
    a.G = p.G;
    a.ndir = p.has_bwd ? 2 : 1;
    a.nc = (p.L + kQ - 1) / kQ;
    a.head_loop = head_loop(p.batch, p.L, a.ndir);
    a.chain = use_chain(p.batch, p.L, p.H, a.ndir);
    const BwdLayout w = layout(p.batch, p.L, p.H, p.P, p.N, a.ndir);
    char *base = (char *)ws;
    a.S = (float *)(base + w.S);
    a.R = (float *)(base + w.R);
    a.lg = (double *)(base + w.lg);
    a.dBp = (float *)(base + w.dBp);
    a.dCp = (float *)(base + w.dCp);
    a.dAp = (float *)(base + w.dAp);
    a.dDp = (float *)(base + w.dDp);
    return p.bf16 ? launch_t<uint16_t>(a, p.P, p.N, s) : launch_t<float>(a, p.P, p.N, s);
}

}  // namespace bm
