// Chunked bidirectional SSD on the matrix cores (bf16 inputs, fp32
// accumulation), headdim 64, d_state 128.
//
// The sequence is cut into chunks of Q tokens (the SSD block decomposition of
// Mamba-2, the mixer the DiffuMamba pages name). With a_t = dt_t*A_h, per
// chunk and direction:
//   forward : cs_i = sum_{k=c0..i} a_k             (inclusive prefix)
//             y_i  = sum_{j<=i} G_ij e^{cs_i-cs_j} dt_j x_j   (intra-chunk)
//                  + e^{cs_i} C_i . H_in                    (carried state)
//             H_out = e^{sum a} H_in + sum_j e^{sum_{k>j} a_k} dt_j B_j x_j^T
//   reverse : the mirror image (flip / scan / flip-back of the DiffuMamba
//             blog's bidirectional block) done by index arithmetic:
//             cs_i = sum_{k=i..c1} a_k, mask j >= i, the state enters from
//             the right and leaves at the chunk's first token.
// with G = C B^T. The two directions' outputs are added (gist.science/ja
// DiffuMamba summary, Sec. 2). Kernels:
//   k_gram        G per (row, direction, chunk, group), bf16 MFMA
//   k_chunk_state H_out of each chunk from a zero state, bf16 MFMA, and the
//                 chunk's carry factor gamma
//   k_state_scan  H_in(c) of every chunk by a sequential pass over chunks
//   k_chunk_out   intra-chunk + carried-state + skip terms of both
//                 directions, summed, y written once
// Packed sequences: a per-token sequence index masks every term that would
// cross a sequence boundary; the carry factor of a chunk that contains a
// boundary (in the walking direction) is zero.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace bm {

namespace {

constexpr int kP = 64;        // headdim handled by this path
constexpr int kN = 128;       // d_state handled by this path
constexpr int kThreads = 256; // 4 waves; wave w owns headdim columns 16w..16w+15

struct ChunkArgs {
    DirPtrs dir[2];
    int ndir, batch, L, H, G, nC;
    const int32_t *seq;       // per-token sequence index (packed) or nullptr
    float *S;                 // [batch][2][nC][H][P][N]: chunk states, then H_in
    float *gamma;             // [batch][2][nC][H]
    float *Gm;                // [batch][2][nC][G][Q][Q]
    const float *init_state;  // [batch][H][P][N] or nullptr
    float *final_state;       // [batch][H][P][N] or nullptr
    float *y;                 // [batch][L][H][P]
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Inclusive prefix sum over the 256 threads of the block in thread order.
// `tmp` holds 4 floats of LDS. Returns the thread's inclusive value; *total
// receives the sum of all 256 inputs.
__device__ float block_scan_incl(float v, float *tmp, float *total) {
    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float n = __shfl_up(v, off, 64);
        if (lane >= off) v += n;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    float add = 0.f, tot = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float t = tmp[k];
        if (k < w) add += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return v + add;
}

__device__ __forceinline__ size_t tok_off(int b, int L, int t) { return (size_t)b * L + t; }

__device__ __forceinline__ float ld_bf(const uint16_t *p, size_t i) { return bf2f(p[i]); }

// 8 bf16 at p (16-byte aligned) as an MFMA operand
__device__ __forceinline__ u32x4 ld8(const uint16_t *p) { return *(const u32x4 *)p; }
// 4 bf16 at p (8-byte aligned)
__device__ __forceinline__ u32x2 ld4(const uint16_t *p) { return *(const u32x2 *)p; }

__device__ __forceinline__ uint32_t bf_scale2(uint32_t pair, float s0, float s1) {
    return pack2bf(bf2f((uint16_t)(pair & 0xffffu)) * s0, bf2f((uint16_t)(pair >> 16)) * s1);
}

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi): the pair carries about
// 16 significant bits, so a product on the matrix cores loses ~2^-17
// relative instead of bf16's 2^-9. Stores two packed pairs.
__device__ __forceinline__ void split_store(uint32_t *hi, uint32_t *lo, int o, float v0, float v1) {
    const uint16_t h0 = f2bf(v0), h1 = f2bf(v1);
    hi[o] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[o] = pack2bf(v0 - bf2f(h0), v1 - bf2f(h1));
}

__device__ __forceinline__ void split4(const f32x4 v, uint32_t &h01, uint32_t &h23, uint32_t &l01,
                                       uint32_t &l23) {
    const uint16_t a = f2bf(v[0]), b = f2bf(v[1]), c = f2bf(v[2]), d = f2bf(v[3]);
    h01 = (uint32_t)a | ((uint32_t)b << 16);
    h23 = (uint32_t)c | ((uint32_t)d << 16);
    l01 = pack2bf(v[0] - bf2f(a), v[1] - bf2f(b));
    l23 = pack2bf(v[2] - bf2f(c), v[3] - bf2f(d));
}

// ---------------------------------------------------------------- k_gram
template <int Q>
__global__ void __launch_bounds__(kThreads) k_gram(const ChunkArgs a) {
    const int c = blockIdx.x, d = blockIdx.y;
    const int b = blockIdx.z / a.G, grp = blockIdx.z % a.G;
    const int c0 = c * Q;
    const int len = min(Q, a.L - c0);
    const int lane = lane_id(), w = wave_id(), g4 = lane >> 4, l16 = lane & 15;
    const uint16_t *Bm = (const uint16_t *)a.dir[d].B;
    const uint16_t *Cm = (const uint16_t *)a.dir[d].C;
    float *Gout = a.Gm + ((((size_t)b * 2 + d) * a.nC + c) * a.G + grp) * Q * Q;
    constexpr int T = Q / 16;
    int counter = 0;
    for (int ti = 0; ti < T; ++ti) {
        for (int tj = 0; tj < T; ++tj) {
            const bool need = d == 0 ? tj <= ti : tj >= ti;
            if (!need) continue;
            if ((counter++ & 3) != w) continue;
            const int i = 16 * ti + l16, j = 16 * tj + l16;
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < kN / 32; ++ks) {
                u32x4 av = {0u, 0u, 0u, 0u}, bv = {0u, 0u, 0u, 0u};
                if (i < len) av = ld8(Cm + (tok_off(b, a.L, c0 + i) * a.G + grp) * kN + 32 * ks + 8 * g4);
                if (j < len) bv = ld8(Bm + (tok_off(b, a.L, c0 + j) * a.G + grp) * kN + 32 * ks + 8 * g4);
                acc = mfma16x16x32(av, bv, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Gout[(size_t)(16 * ti + 4 * g4 + r) * Q + 16 * tj + l16] = acc[r];
        }
    }
}

// --------------------------------------------------------- k_chunk_state
constexpr int kSub = 64;            // tokens per LDS sub-block
constexpr int kRS = kSub + 8;       // LDS row stride (bf16) of transposed tiles

template <int Q>
__global__ void __launch_bounds__(kThreads) k_chunk_state(const ChunkArgs a) {
    const int c = blockIdx.x, d = blockIdx.y;
    const int b = blockIdx.z / a.H, h = blockIdx.z % a.H;
    const int grp = h / (a.H / a.G);
    const int c0 = c * Q;
    const int len = min(Q, a.L - c0);
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int g4 = lane >> 4, l16 = lane & 15;
    const DirPtrs dp = a.dir[d];
    const uint16_t *X = (const uint16_t *)dp.x;
    const uint16_t *DT = (const uint16_t *)dp.dt;
    const uint16_t *Bm = (const uint16_t *)dp.B;
    const float Ah = dp.A[h];

    __shared__ __attribute__((aligned(16))) float s_w[Q];
    __shared__ __attribute__((aligned(16))) float s_tmp[4];
    __shared__ __attribute__((aligned(16))) uint32_t s_bt[kN * kRS / 2];   // B^T  [n][t] bf16
    __shared__ __attribute__((aligned(16))) uint32_t s_xt[kP * kRS / 2];   // (w x)^T [p][t], bf16 high part
    __shared__ __attribute__((aligned(16))) uint32_t s_xl[kP * kRS / 2];   // (w x)^T [p][t], bf16 residual

    // weights w_t = exp(sum of a between t and the outgoing edge, exclusive) * dt_t
    // forward: edge = last token (suffix sums); reverse: edge = first token.
    const int idx = d == 0 ? (Q - 1 - tid) : tid;   // scan runs toward the edge
    float at = 0.f, dtt = 0.f;
    if (tid < Q && idx < len) {
        dtt = ld_bf(DT, tok_off(b, a.L, c0 + idx) * a.H + h);
        at = dtt * Ah;
    }
    float total;
    const float incl = block_scan_incl(tid < Q ? at : 0.f, s_tmp, &total);
    if (tid < Q) {
        float wt = 0.f;
        if (idx < len) {
            bool keep = true;
            if (a.seq) {
                const int edge = d == 0 ? c0 + len - 1 : c0;
                keep = a.seq[tok_off(b, a.L, c0 + idx)] == a.seq[tok_off(b, a.L, edge)];
            }
            if (keep) wt = expf(incl - at) * dtt;
        }
        s_w[idx] = wt;
    }
    if (tid == 0) {
        bool carry = true;
        if (a.seq) {
            if (d == 0 && c0 > 0)
                carry = a.seq[tok_off(b, a.L, c0 - 1)] == a.seq[tok_off(b, a.L, c0 + len - 1)];
            if (d == 1 && c0 + len < a.L)
                carry = a.seq[tok_off(b, a.L, c0 + len)] == a.seq[tok_off(b, a.L, c0)];
        }
        a.gamma[(((size_t)b * 2 + d) * a.nC + c) * a.H + h] = carry ? expf(total) : 0.f;
    }
    __syncthreads();

    f32x4 acc[kN / 16];
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt) acc[nt] = zero4();

    for (int sb = 0; sb < Q / kSub; ++sb) {
        const int tb = sb * kSub;
        // B^T: 32 row pairs x 16 column groups of 8
        for (int item = tid; item < 32 * (kN / 8); item += kThreads) {
            const int rp = item & 31, cg = item >> 5;
            const int t0 = tb + 2 * rp;
            u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = {0u, 0u, 0u, 0u};
            if (t0 < len) r0 = ld8(Bm + (tok_off(b, a.L, c0 + t0) * a.G + grp) * kN + 8 * cg);
            if (t0 + 1 < len) r1 = ld8(Bm + (tok_off(b, a.L, c0 + t0 + 1) * a.G + grp) * kN + 8 * cg);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo0 = r0[q] & 0xffffu, hi0 = r0[q] >> 16;
                const uint32_t lo1 = r1[q] & 0xffffu, hi1 = r1[q] >> 16;
                s_bt[((8 * cg + 2 * q) * kRS) / 2 + rp] = lo0 | (lo1 << 16);
                s_bt[((8 * cg + 2 * q + 1) * kRS) / 2 + rp] = hi0 | (hi1 << 16);
            }
        }
        // (w x)^T: 32 row pairs x 8 column groups of 8
        for (int item = tid; item < 32 * (kP / 8); item += kThreads) {
            const int rp = item & 31, cg = item >> 5;
            const int t0 = tb + 2 * rp;
            u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = {0u, 0u, 0u, 0u};
            if (t0 < len) r0 = ld8(X + (tok_off(b, a.L, c0 + t0) * a.H + h) * kP + 8 * cg);
            if (t0 + 1 < len) r1 = ld8(X + (tok_off(b, a.L, c0 + t0 + 1) * a.H + h) * kP + 8 * cg);
            const float w0 = s_w[t0], w1 = s_w[t0 + 1];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x00 = bf2f((uint16_t)(r0[q] & 0xffffu)) * w0;
                const float x01 = bf2f((uint16_t)(r0[q] >> 16)) * w0;
                const float x10 = bf2f((uint16_t)(r1[q] & 0xffffu)) * w1;
                const float x11 = bf2f((uint16_t)(r1[q] >> 16)) * w1;
                const int o0 = ((8 * cg + 2 * q) * kRS) / 2 + rp;
                const int o1 = ((8 * cg + 2 * q + 1) * kRS) / 2 + rp;
                split_store(s_xt, s_xl, o0, x00, x10);
                split_store(s_xt, s_xl, o1, x01, x11);
            }
        }
        __syncthreads();
        const uint16_t *bt = (const uint16_t *)s_bt;
        const uint16_t *xt = (const uint16_t *)s_xt;
        const uint16_t *xl = (const uint16_t *)s_xl;
#pragma unroll
        for (int ks = 0; ks < kSub / 32; ++ks) {
            const u32x4 bhi = *(const u32x4 *)(xt + (16 * w + l16) * kRS + 32 * ks + 8 * g4);
            const u32x4 blo = *(const u32x4 *)(xl + (16 * w + l16) * kRS + 32 * ks + 8 * g4);
#pragma unroll
            for (int nt = 0; nt < kN / 16; ++nt) {
                const u32x4 aop = *(const u32x4 *)(bt + (16 * nt + l16) * kRS + 32 * ks + 8 * g4);
                acc[nt] = mfma16x16x32(aop, bhi, acc[nt]);
                acc[nt] = mfma16x16x32(aop, blo, acc[nt]);
            }
        }
        __syncthreads();
    }
    // S[p][n]: lane holds n = 16nt + 4g4 + r, p = 16w + l16
    float *Sout = a.S + ((((size_t)b * 2 + d) * a.nC + c) * a.H + h) * (size_t)(kP * kN);
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt)
        *(f32x4 *)(Sout + (16 * w + l16) * kN + 16 * nt + 4 * g4) = acc[nt];
}

// ---------------------------------------------------------- k_state_scan
__global__ void __launch_bounds__(256) k_state_scan(const ChunkArgs a) {
    const int e = blockIdx.x * 256 + threadIdx.x;   // element p*N + n
    const int h = blockIdx.y;
    const int b = blockIdx.z / a.ndir, d = blockIdx.z % a.ndir;
    const size_t PN = (size_t)kP * kN;
    float hv = 0.f;
    if (d == 0 && a.init_state) hv = a.init_state[((size_t)b * a.H + h) * PN + e];
    for (int step = 0; step < a.nC; ++step) {
        const int c = d == 0 ? step : a.nC - 1 - step;
        const size_t ci = (((size_t)b * 2 + d) * a.nC + c) * a.H + h;
        float *slot = a.S + ci * PN + e;
        const float s = *slot;
        const float gm = a.gamma[ci];
        *slot = hv;                 // state entering chunk c
        hv = fmaf(gm, hv, s);       // state leaving chunk c
    }
    if (d == 0 && a.final_state) a.final_state[((size_t)b * a.H + h) * PN + e] = hv;
}

// ----------------------------------------------------------- k_chunk_out
template <int Q>
__global__ void __launch_bounds__(kThreads) k_chunk_out(const ChunkArgs a) {
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int grp = h / (a.H / a.G);
    const int c0 = c * Q;
    const int len = min(Q, a.L - c0);
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int g4 = lane >> 4, l16 = lane & 15;
    constexpr int XRS = Q + 8;   // row stride (bf16) of X^T and M tiles

    __shared__ __attribute__((aligned(16))) float s_cs[Q];
    __shared__ __attribute__((aligned(16))) float s_dt[Q];
    __shared__ __attribute__((aligned(16))) float s_u[Q];
    __shared__ __attribute__((aligned(16))) int s_seq[Q];
    __shared__ __attribute__((aligned(16))) float s_tmp[4];
    __shared__ __attribute__((aligned(16))) uint32_t s_xt[kP * XRS / 2];   // X^T [p][t] bf16
    __shared__ __attribute__((aligned(16))) uint32_t s_m[64 * XRS / 2];    // 64 rows of M [i][j], bf16 high part
    __shared__ __attribute__((aligned(16))) uint32_t s_ml[64 * XRS / 2];   // bf16 residual of M

    f32x4 acc[Q / 16];
#pragma unroll
    for (int it = 0; it < Q / 16; ++it) acc[it] = zero4();

    for (int d = 0; d < a.ndir; ++d) {
        const DirPtrs dp = a.dir[d];
        const uint16_t *X = (const uint16_t *)dp.x;
        const uint16_t *DT = (const uint16_t *)dp.dt;
        const uint16_t *Cm = (const uint16_t *)dp.C;
        const float Ah = dp.A[h];
        const float Dh = dp.D ? dp.D[h] : 0.f;

        // inclusive scan in the walking direction
        const int idx = d == 0 ? tid : (Q - 1 - tid);
        float at = 0.f, dtt = 0.f;
        if (tid < Q && idx < len) {
            dtt = ld_bf(DT, tok_off(b, a.L, c0 + idx) * a.H + h);
            at = dtt * Ah;
        }
        float total;
        const float cs = block_scan_incl(tid < Q ? at : 0.f, s_tmp, &total);
        if (tid < Q) {
            s_cs[idx] = cs;
            s_dt[idx] = dtt;
            int sq = 0;
            bool off_ok = idx < len;
            if (a.seq && idx < len) {
                sq = a.seq[tok_off(b, a.L, c0 + idx)];
                const int nb = d == 0 ? c0 - 1 : c0 + len;
                const bool has_nb = d == 0 ? c0 > 0 : c0 + len < a.L;
                off_ok = has_nb && a.seq[tok_off(b, a.L, nb)] == sq;
            }
            s_seq[idx] = sq;
            s_u[idx] = off_ok ? expf(cs) : 0.f;
        }
        // X^T for the whole chunk: Q/2 row pairs x 8 column groups
        for (int item = tid; item < (Q / 2) * (kP / 8); item += kThreads) {
            const int rp = item % (Q / 2), cg = item / (Q / 2);
            const int t0 = 2 * rp;
            u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = {0u, 0u, 0u, 0u};
            if (t0 < len) r0 = ld8(X + (tok_off(b, a.L, c0 + t0) * a.H + h) * kP + 8 * cg);
            if (t0 + 1 < len) r1 = ld8(X + (tok_off(b, a.L, c0 + t0 + 1) * a.H + h) * kP + 8 * cg);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo0 = r0[q] & 0xffffu, hi0 = r0[q] >> 16;
                const uint32_t lo1 = r1[q] & 0xffffu, hi1 = r1[q] >> 16;
                s_xt[((8 * cg + 2 * q) * XRS) / 2 + rp] = lo0 | (lo1 << 16);
                s_xt[((8 * cg + 2 * q + 1) * XRS) / 2 + rp] = hi0 | (hi1 << 16);
            }
        }
        __syncthreads();

        // carried state: acc[i][p] += u_i * sum_n C[i][n] H_in[n][p]; C enters the
        // matrix cores exactly, H_in as a hi+lo bf16 pair, u_i in fp32 on the output
        {
            const float *Hin = a.S + ((((size_t)b * 2 + d) * a.nC + c) * a.H + h) * (size_t)(kP * kN);
            u32x4 hhi[kN / 32], hlo[kN / 32];
#pragma unroll
            for (int ks = 0; ks < kN / 32; ++ks) {
                const float *hp = Hin + (16 * w + l16) * kN + 32 * ks + 4 * g4;
                uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
                split4(*(const f32x4 *)hp, a0, a1, b0, b1);
                split4(*(const f32x4 *)(hp + 16), a2, a3, b2, b3);
                hhi[ks] = u32x4{a0, a1, a2, a3};
                hlo[ks] = u32x4{b0, b1, b2, b3};
            }
            for (int it = 0; it < Q / 16; ++it) {
                const int i = 16 * it + l16;
                const uint16_t *crow = Cm + (tok_off(b, a.L, c0 + min(i, len - 1)) * a.G + grp) * kN;
                f32x4 t = zero4();
#pragma unroll
                for (int ks = 0; ks < kN / 32; ++ks) {
                    u32x4 aop = {0u, 0u, 0u, 0u};
                    if (i < len) {
                        const u32x2 p0 = ld4(crow + 32 * ks + 4 * g4);
                        const u32x2 p1 = ld4(crow + 32 * ks + 16 + 4 * g4);
                        aop = u32x4{p0[0], p0[1], p1[0], p1[1]};
                    }
                    t = mfma16x16x32(aop, hhi[ks], t);
                    t = mfma16x16x32(aop, hlo[ks], t);
                }
                const f32x4 uu = *(const f32x4 *)(s_u + 16 * it + 4 * g4);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[it][r] = fmaf(uu[r], t[r], acc[it][r]);
            }
        }

        // intra-chunk: 64-row blocks of M = G o exp(cs_i - cs_j) dt_j (masked)
        const float *Gin = a.Gm + ((((size_t)b * 2 + d) * a.nC + c) * a.G + grp) * Q * Q;
        const uint16_t *xt = (const uint16_t *)s_xt;
        for (int ib = 0; ib < Q / 64; ++ib) {
            // fwd needs j < 64(ib+1); rev needs j >= 64 ib
            const int jlo = d == 0 ? 0 : 64 * ib;
            const int jhi = d == 0 ? 64 * (ib + 1) : Q;
            const int ncols = jhi - jlo;
            __syncthreads();   // previous block's M reads are done
            for (int e = tid; e < 64 * (ncols / 2); e += kThreads) {
                const int r = e / (ncols / 2), cp = e % (ncols / 2);
                const int i = 64 * ib + r, j = jlo + 2 * cp;
                float v[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int jj = j + q;
                    bool ok = i < len && jj < len && (d == 0 ? jj <= i : jj >= i);
                    if (ok && a.seq) ok = s_seq[i] == s_seq[jj];
                    v[q] = ok ? Gin[(size_t)i * Q + jj] * expf(s_cs[i] - s_cs[jj]) * s_dt[jj] : 0.f;
                }
                split_store(s_m, s_ml, (r * XRS) / 2 + (j >> 1), v[0], v[1]);
            }
            __syncthreads();
            const uint16_t *mm = (const uint16_t *)s_m;
            const uint16_t *ml = (const uint16_t *)s_ml;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const int it = 4 * ib + t4;
                const int rowl = 16 * t4 + l16;     // row within the 64-row block
                // k-steps holding the terms within 16 tokens of the diagonal, where
                // nothing has decayed yet, take M as hi + lo
                const int kd = it >> 1;
                const int knb = d == 0 ? kd - 1 : kd + 1;
                f32x4 ac = acc[it];
                for (int ks = jlo / 32; ks < jhi / 32; ++ks) {
                    const u32x4 bop = *(const u32x4 *)(xt + (16 * w + l16) * XRS + 32 * ks + 8 * g4);
                    const u32x4 aop = *(const u32x4 *)(mm + rowl * XRS + 32 * ks + 8 * g4);
                    ac = mfma16x16x32(aop, bop, ac);
                    if (ks == kd || ks == knb) {
                        const u32x4 alo = *(const u32x4 *)(ml + rowl * XRS + 32 * ks + 8 * g4);
                        ac = mfma16x16x32(alo, bop, ac);
                    }
                }
                acc[it] = ac;
            }
        }

        // skip term D x (exact fp32 product of bf16 x)
#pragma unroll
        for (int it = 0; it < Q / 16; ++it) {
            const int i0 = 16 * it + 4 * g4;
            const u32x2 xv = *(const u32x2 *)(xt + (16 * w + l16) * XRS + i0);
            acc[it][0] += Dh * bf2f((uint16_t)(xv[0] & 0xffffu));
            acc[it][1] += Dh * bf2f((uint16_t)(xv[0] >> 16));
            acc[it][2] += Dh * bf2f((uint16_t)(xv[1] & 0xffffu));
            acc[it][3] += Dh * bf2f((uint16_t)(xv[1] >> 16));
        }
        __syncthreads();   // LDS is reused by the next direction
    }

    // y[token][h][p]: lane holds rows i = 16it + 4g4 + r, column p = 16w + l16
#pragma unroll
    for (int it = 0; it < Q / 16; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * it + 4 * g4 + r;
            if (i < len) a.y[(tok_off(b, a.L, c0 + i) * a.H + h) * kP + 16 * w + l16] = acc[it][r];
        }
    }
}

template <int Q>
hipError_t launch_q(const ChunkArgs &a, hipStream_t s) {
    const int nd = a.ndir;
    BM_LAUNCH("ssd_gram", k_gram<Q>, dim3(a.nC, nd, a.batch * a.G), dim3(kThreads), 0, s, a);
    BM_LAUNCH("ssd_chunk_state", k_chunk_state<Q>, dim3(a.nC, nd, a.batch * a.H), dim3(kThreads), 0, s, a);
    BM_LAUNCH("ssd_state_scan", k_state_scan, dim3(kP * kN / 256, a.H, a.batch * nd), dim3(256), 0, s, a);
    BM_LAUNCH("ssd_chunk_out", k_chunk_out<Q>, dim3(a.nC, a.H, a.batch), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool chunked_supported(const Problem &p) {
    return p.bf16 && p.P == kP && p.N == kN && p.L > 0 &&
           (p.Q == 64 || p.Q == 128 || p.Q == 256);
}

size_t chunked_workspace(int batch, int L, int H, int G, int Q) {
    const size_t nC = (size_t)(L + Q - 1) / Q;
    auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
    return al(batch * 2 * nC * H * (size_t)(kP * kN) * 4) + al(batch * 2 * nC * H * 4) +
           al(batch * 2 * nC * G * (size_t)Q * Q * 4);
}

hipError_t launch_chunked(const Problem &p, void *ws, hipStream_t s) {
    ChunkArgs a;
    a.dir[0] = p.dir[0];
    a.dir[1] = p.dir[1];
    a.ndir = p.has_bwd ? 2 : 1;
    a.batch = p.batch; a.L = p.L; a.H = p.H; a.G = p.G;
    a.nC = (p.L + p.Q - 1) / p.Q;
    a.seq = p.seq_idx;
    const size_t nC = a.nC;
    auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
    char *w = (char *)ws;
    a.S = (float *)w;
    w += al(p.batch * 2 * nC * p.H * (size_t)(kP * kN) * 4);
    a.gamma = (float *)w;
    w += al(p.batch * 2 * nC * p.H * 4);
    a.Gm = (float *)w;
    a.init_state = p.init_state;
    a.final_state = p.final_state;
    a.y = p.y;
    switch (p.Q) {
        case 64: return launch_q<64>(a, s);
        case 128: return launch_q<128>(a, s);
        case 256: return launch_q<256>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace bm
