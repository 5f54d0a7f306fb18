// Chunked bidirectional SSD on the matrix cores (bf16 inputs, fp32
// accumulation and output), headdim 64, d_state 128.
//
// Operator (per head h, a_t = dt_t * A_h): the Mamba-2 selective recurrence
// (the mixer the DiffuMamba pages name), run forward and, with its own
// parameters, over the time-reversed sequence (the flip / scan / flip-back of
// the DiffuMamba blog's bidirectional block, done here by index arithmetic);
// the two outputs are added (gist.science/ja DiffuMamba summary, Sec. 2).
//
// Block decomposition with chunks of Q tokens. Inside a chunk, for the
// forward direction (the reverse one is its mirror image):
//   cs_i  = sum_{k=c0..i} a_k
//   y_i   = sum_{j<=i} G_ij e^{cs_i-cs_j} dt_j x_j        G = C B^T (intra)
//         + e^{cs_i} C_i . H                               (carried state)
//         + D x_i
//   H    <- e^{cs_end} H + sum_j e^{sum_{k>j} a_k} dt_j B_j x_j^T
//
// Work split (one WG = 4 waves):
//   k_seg_state  each segment's (Ts tokens) outgoing state from a zero state,
//                walking away from the outgoing edge and stopping where every
//                remaining weight is exactly 0.0f in fp32 (e^x underflows)
//   k_seg_scan   incoming state of each segment where a chain carries over;
//                where a segment's carry factor is 0 the next segment's
//                incoming state is just the previous segment's local state
//   k_seg_out    per (row, segment, head): the reverse direction walks the
//                segment's chunks right to left writing its part of y, the
//                forward direction walks left to right and adds its part.
//                Per chunk, B and x are staged once in LDS; for each 64-row
//                block C is staged and wave w computes rows 16w..16w+15: the
//                Gram tiles G^T = B C^T on the matrix cores (their accumulator
//                layout is already the A operand of the following M.x product),
//                the masked decay, M.x, the carried-state term and D x. The
//                state update runs with wave w owning state columns
//                16w..16w+15, kept in registers as MFMA accumulators.
//
// Operands enter the matrix cores as fp16 (v_mfma_f32_16x16x32_f16), each
// tile scaled by a power of two chosen from a bound on its magnitude so that
// it stays inside fp16's range; the fp32 results are scaled back exactly.
// bf16 inputs (8 significant bits) are exact in fp16 after scaling; the
// operands that must be rounded (the masked decayed Gram matrix, the carried
// state, the dt-weighted inputs) keep 11 bits instead of bf16's 8, and the
// Gram-matrix terms within 16 tokens of the diagonal (undecayed, the largest)
// enter as an fp16 hi + lo pair.
//
// Packed sequences: a per-token sequence index masks every term that would
// cross a sequence boundary, and a chunk or segment holding a boundary (in
// the walking direction) does not carry the incoming state through.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace bm {

namespace {

constexpr int kP = 64;         // headdim handled here
constexpr int kN = 128;        // d_state handled here
constexpr int kThreads = 256;  // 4 waves
constexpr int kSub = 64;       // tokens per staged sub-block
constexpr int kRS = kSub + 8;  // LDS row stride (16-bit elements) of 64-wide tiles
constexpr float kDead = -110.f;  // expf(x) is exactly 0.0f for every x < kDead
// magnitude targets (log2) of the scaled fp16 operands
constexpr int kTop = 14;       // generic operand: |v| < 2^14 (fp16 max 65504)
constexpr int kTopX = 10;      // x, multiplied later by weights < 2^4

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_h(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float h_lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
}
__device__ __forceinline__ float h_hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}
__device__ __forceinline__ float b_lo(uint32_t u) { return bf2f((uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float b_hi(uint32_t u) { return bf2f((uint16_t)(u >> 16)); }

// smallest e with m < 2^e for finite m >= 0 (e = -126 for m == 0), clamped
__device__ __forceinline__ int exp_bound(float m) {
    if (!(m > 0.f)) return -126;
    int e;
    (void)frexpf(m, &e);
    return e;
}
__device__ __forceinline__ int clamp_scale(int s) { return s < -60 ? -60 : (s > 60 ? 60 : s); }

struct SegArgs {
    DirPtrs dir[2];
    int ndir, batch, L, H, G, nC, Ts, nseg;
    const int32_t *seq;       // per-token sequence index (packed) or nullptr
    float *S;                 // [batch][2][nseg][H][P*N] segment-local outgoing states
    float *Hs;                // [batch][2][nseg][H][P*N] incoming states of carried chains
    float *gam;               // [batch][2][nseg][H]      segment carry factors
    const float *init_state;  // [batch][H][P][N] or nullptr
    float *final_state;       // [batch][H][P][N] or nullptr
    float *y;                 // [batch][L][H][P]
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ size_t tok(const SegArgs &a, int b, int t) { return (size_t)b * a.L + t; }
__device__ __forceinline__ u32x4 ld8(const uint16_t *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ u32x2 ld4(const uint16_t *p) { return *(const u32x2 *)p; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
// max over the block's 256 threads; tmp is 4 floats of LDS; two barriers
__device__ float block_max(float v, float *tmp) {
    v = wave_max(v);
    if (lane_id() == 0) tmp[wave_id()] = v;
    __syncthreads();
    const float m = fmaxf(fmaxf(tmp[0], tmp[1]), fmaxf(tmp[2], tmp[3]));
    __syncthreads();
    return m;
}
// inclusive prefix sum over the block's 256 threads; *total = sum; two barriers
__device__ float block_scan(float v, float *tmp, float *total) {
    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float n = __shfl_up(v, off, 64);
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
__device__ __forceinline__ float wave_scan(float v) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float n = __shfl_up(v, off, 64);
        if (lane >= off) v += n;
    }
    return v;
}
__device__ __forceinline__ float absmax8(u32x4 r) {
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(fabsf(b_lo(r[q])), fabsf(b_hi(r[q]))));
    return m;
}

// --------------------------------------------------------- staging helpers
// B^T of the 64 tokens [t0, t0+64) (rows row0 + t, valid for t < tlimit) into
// bt[n][t] as fp16 scaled by 2^s, s chosen from the tokens' largest |B|;
// returns s; the tile is visible to the whole block on return. Three barriers.
__device__ int stage_bt16(const SegArgs &a, const uint16_t *Bm, int b, int grp, int row0, int t0,
                          int tlimit, uint32_t *bt, float *tmp) {
    constexpr int PER = 32 * (kN / 8) / kThreads;   // 2
    u32x4 r0[PER], r1[PER];
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int item = threadIdx.x + kThreads * k;
        const int rp = item >> 4, cg = item & 15;
        const int t = t0 + 2 * rp;
        r0[k] = u32x4{0u, 0u, 0u, 0u};
        r1[k] = u32x4{0u, 0u, 0u, 0u};
        if (t < tlimit) r0[k] = ld8(Bm + (tok(a, b, row0 + t) * a.G + grp) * kN + 8 * cg);
        if (t + 1 < tlimit) r1[k] = ld8(Bm + (tok(a, b, row0 + t + 1) * a.G + grp) * kN + 8 * cg);
        m = fmaxf(m, fmaxf(absmax8(r0[k]), absmax8(r1[k])));
    }
    const int sc = clamp_scale(kTop - exp_bound(block_max(m, tmp)));
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int item = threadIdx.x + kThreads * k;
        const int rp = item >> 4, cg = item & 15;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bt[((8 * cg + 2 * q) * kRS) / 2 + rp] =
                pack2h(ldexpf(b_lo(r0[k][q]), sc), ldexpf(b_lo(r1[k][q]), sc));
            bt[((8 * cg + 2 * q + 1) * kRS) / 2 + rp] =
                pack2h(ldexpf(b_hi(r0[k][q]), sc), ldexpf(b_hi(r1[k][q]), sc));
        }
    }
    __syncthreads();   // every wave reads rows other waves wrote
    return sc;
}

// x of COUNT tokens (rows row0 + t, valid for t < tlimit) of head h into
// xt[p][t] (row stride xrs) as fp16 scaled by 2^sx, sx chosen from the tile's
// largest |x|. Returns sx (the same in every thread); the tile is visible to
// the whole block on return. Three barriers.
template <int COUNT>
__device__ int stage_x16(const SegArgs &a, const uint16_t *X, int b, int h, int row0, int tlimit,
                         uint32_t *xt, int xrs, float *tmp) {
    constexpr int PAIRS = COUNT / 2;
    constexpr int ITEMS = PAIRS * (kP / 8);
    constexpr int PER = (ITEMS + kThreads - 1) / kThreads;
    u32x4 r0[PER], r1[PER];
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int item = threadIdx.x + kThreads * k;
        r0[k] = u32x4{0u, 0u, 0u, 0u};
        r1[k] = u32x4{0u, 0u, 0u, 0u};
        if (item < ITEMS) {
            const int rp = item / (kP / 8), cg = item % (kP / 8);
            const int t = 2 * rp;
            if (t < tlimit) r0[k] = ld8(X + (tok(a, b, row0 + t) * a.H + h) * kP + 8 * cg);
            if (t + 1 < tlimit) r1[k] = ld8(X + (tok(a, b, row0 + t + 1) * a.H + h) * kP + 8 * cg);
            m = fmaxf(m, fmaxf(absmax8(r0[k]), absmax8(r1[k])));
        }
    }
    const int sx = clamp_scale(kTopX - exp_bound(block_max(m, tmp)));
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int item = threadIdx.x + kThreads * k;
        if (item < ITEMS) {
            const int rp = item / (kP / 8), cg = item % (kP / 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xt[((8 * cg + 2 * q) * xrs) / 2 + rp] =
                    pack2h(ldexpf(b_lo(r0[k][q]), sx), ldexpf(b_lo(r1[k][q]), sx));
                xt[((8 * cg + 2 * q + 1) * xrs) / 2 + rp] =
                    pack2h(ldexpf(b_hi(r0[k][q]), sx), ldexpf(b_hi(r1[k][q]), sx));
            }
        }
    }
    __syncthreads();   // every wave reads rows other waves wrote
    return sx;
}

// T[n][p-block w] = sum_t B^T[n][t] (w_t x_t[p]) over one staged 64-token
// sub-block (scaled domain). xt: X^T[p][t] fp16 (row stride xrs, column
// offset xoff); wv: 64 scaled weights.
__device__ __forceinline__ void state_mfma(f32x4 (&T)[kN / 16], const uint32_t *bt,
                                           const uint16_t *xt, int xrs, int xoff, const float *wv) {
    const int lane = lane_id(), w = wave_id(), g4 = lane >> 4, l16 = lane & 15;
    const uint16_t *btp = (const uint16_t *)bt;
#pragma unroll
    for (int ks = 0; ks < kSub / 32; ++ks) {
        const int tk = 32 * ks + 8 * g4;
        const u32x4 xv = *(const u32x4 *)(xt + (16 * w + l16) * xrs + xoff + tk);
        const f32x4 w0 = *(const f32x4 *)(wv + tk);
        const f32x4 w1 = *(const f32x4 *)(wv + tk + 4);
        const u32x4 bop = {pack2h(h_lo(xv[0]) * w0[0], h_hi(xv[0]) * w0[1]),
                           pack2h(h_lo(xv[1]) * w0[2], h_hi(xv[1]) * w0[3]),
                           pack2h(h_lo(xv[2]) * w1[0], h_hi(xv[2]) * w1[1]),
                           pack2h(h_lo(xv[3]) * w1[2], h_hi(xv[3]) * w1[3])};
#pragma unroll
        for (int nt = 0; nt < kN / 16; ++nt) {
            const u32x4 aop = *(const u32x4 *)(btp + (16 * nt + l16) * kRS + tk);
            T[nt] = mfma_h(aop, bop, T[nt]);
        }
    }
}

// ----------------------------------------------------------- k_seg_state
struct StateSmem {
    float w[kSub];
    float tmp[4];
    uint32_t bt[kN * kRS / 2];
    uint32_t xt[kP * kRS / 2];
    float run[2];   // running sum of a from the outgoing edge, by step parity
    int sw;         // weight scale of the current sub-block
};

__global__ void __launch_bounds__(kThreads) k_seg_state(const SegArgs a) {
    const int seg = blockIdx.x, d = blockIdx.y;
    const int b = blockIdx.z / a.H, h = blockIdx.z % a.H;
    const int grp = h / (a.H / a.G);
    const int t0 = seg * a.Ts, t1 = min(t0 + a.Ts, a.L);
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), g4 = lane >> 4, l16 = lane & 15;
    const DirPtrs dp = a.dir[d];
    const uint16_t *X = (const uint16_t *)dp.x;
    const uint16_t *DT = (const uint16_t *)dp.dt;
    const uint16_t *Bm = (const uint16_t *)dp.B;
    const float Ah = dp.A[h];
    __shared__ __attribute__((aligned(16))) StateSmem sm;

    const int edge = d == 0 ? t1 - 1 : t0;
    const int edge_seq = a.seq ? a.seq[tok(a, b, edge)] : 0;
    if (tid == 0) sm.run[0] = 0.f;
    f32x4 Hacc[kN / 16];
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt) Hacc[nt] = zero4();
    __syncthreads();

    const int nsub = (t1 - t0 + kSub - 1) / kSub;
    int step = 0;
    for (; step < nsub; ++step) {
        // sub-block [s0, s1), the step-th counted away from the outgoing edge
        const int s0 = d == 0 ? max(t0, t1 - kSub * (step + 1)) : t0 + kSub * step;
        const int s1 = d == 0 ? t1 - kSub * step : min(t1, s0 + kSub);
        const int n = s1 - s0;
        // every remaining weight is e^{<= run} * dt == 0.0f exactly, or every
        // remaining token belongs to another sequence: nothing left to add
        const float run = sm.run[step & 1];
        if (run < kDead) break;
        if (a.seq && a.seq[tok(a, b, d == 0 ? s1 - 1 : s0)] != edge_seq) break;
        if (w == 0) {
            // lane 0 is the token nearest the outgoing edge
            const bool in = lane < n;
            const int pos = d == 0 ? n - 1 - lane : lane;
            float at = 0.f, dtt = 0.f;
            if (in) {
                dtt = bf2f(DT[tok(a, b, s0 + pos) * a.H + h]);
                at = dtt * Ah;
            }
            const float incl = wave_scan(at);
            const int sw = clamp_scale(4 - exp_bound(wave_max(dtt)));
            float wt = 0.f;
            if (in && (!a.seq || a.seq[tok(a, b, s0 + pos)] == edge_seq))
                wt = ldexpf(expf(run + incl - at) * dtt, sw);
            if (in) sm.w[pos] = wt;
            else sm.w[lane] = 0.f;
            const float tot = __shfl(incl, 63, 64);
            if (lane == 0) {
                sm.run[(step + 1) & 1] = run + tot;
                sm.sw = sw;
            }
        }
        const int sB = stage_bt16(a, Bm, b, grp, 0, s0, s1, sm.bt, sm.tmp);
        const int sx = stage_x16<kSub>(a, X, b, h, s0, n, sm.xt, kRS, sm.tmp);
        f32x4 T[kN / 16];
#pragma unroll
        for (int nt = 0; nt < kN / 16; ++nt) T[nt] = zero4();
        state_mfma(T, sm.bt, (const uint16_t *)sm.xt, kRS, 0, sm.w);
        const int unscale = -(sB + sm.sw + sx);
#pragma unroll
        for (int nt = 0; nt < kN / 16; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) Hacc[nt][r] += ldexpf(T[nt][r], unscale);
        __syncthreads();
    }
    const size_t si = (((size_t)b * 2 + d) * a.nseg + seg) * a.H + h;
    float *Sout = a.S + si * (size_t)(kP * kN);
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt)
        *(f32x4 *)(Sout + (16 * w + l16) * kN + 16 * nt + 4 * g4) = Hacc[nt];
    if (tid == 0) {
        // the incoming state passes through iff the whole segment was walked
        // (its total decay did not underflow), and no sequence boundary lies
        // between the segment's incoming side and its edge
        bool carry = step == nsub;
        if (carry && a.seq) {
            if (d == 0 && t0 > 0) carry = a.seq[tok(a, b, t0 - 1)] == edge_seq;
            if (d == 1 && t1 < a.L) carry = a.seq[tok(a, b, t1)] == edge_seq;
        }
        a.gam[si] = carry ? expf(sm.run[nsub & 1]) : 0.f;
    }
}

// ------------------------------------------------------------ k_seg_scan
__global__ void __launch_bounds__(256) k_seg_scan(const SegArgs a) {
    const int e = blockIdx.x * 256 + threadIdx.x;   // element p*N + n
    const int h = blockIdx.y;
    const int b = blockIdx.z / a.ndir, d = blockIdx.z % a.ndir;
    const size_t PN = (size_t)kP * kN;
    auto slot = [&](int k) { return (((size_t)b * 2 + d) * a.nseg + k) * a.H + h; };
    const int ns = a.nseg;
    // walk in the direction of travel; `hv` holds the incoming state of the
    // segment about to be left when `have` is set
    float hv = 0.f;
    bool have = true;
    if (d == 0 && a.init_state) hv = a.init_state[((size_t)b * a.H + h) * PN + e];
    for (int s = 0; s + 1 < ns; ++s) {
        const int k = d == 0 ? s : ns - 1 - s;           // segment being left
        const int kn = d == 0 ? k + 1 : k - 1;           // segment being entered
        const float g = a.gam[slot(k)];
        if (g == 0.f) { have = false; continue; }        // entered state == S(k)
        if (!have) {
            const int kp = d == 0 ? k - 1 : k + 1;       // incoming state of k is S(kp)
            hv = a.S[slot(kp) * PN + e];
        }
        hv = fmaf(g, hv, a.S[slot(k) * PN + e]);
        a.Hs[slot(kn) * PN + e] = hv;
        have = true;
    }
}

// ------------------------------------------------------------- k_seg_out
constexpr int kNRS = kN + 8;   // LDS row stride (16-bit elements) of [t][n] / [p][n] tiles
constexpr int kTileU32 = (kN * kRS > 64 * kNRS ? kN * kRS : 64 * kNRS) / 2;

template <int Q>
struct OutSmem {
    float cs[Q], w[Q], u[Q], dt[Q], a[Q];
    int sq[Q];
    float tmp[4];
    int utile[Q / 16];     // any nonzero e^{cs} in the 16-row tile
    int wsub[Q / kSub];    // any nonzero weight in the 64-token sub-block
    int sB[Q / kSub];      // fp16 scale exponent of each staged B sub-block
    int eBmax;             // bound (log2) of |B| over the chunk
    int sH[4];             // fp16 scale exponent of each 16-column block of H^T
    float gamma;
    int sx, sw, edt;       // x scale, weight scale, dt bound of the chunk
    uint32_t xt[kP * (Q + 8) / 2];   // X^T [p][t], fp16 scaled by 2^sx
    uint32_t bn[Q * kNRS / 2];       // B [t][n] of the chunk, fp16 scaled per sub-block
    uint32_t tile[kTileU32];         // C tile [64][n] (rows) or B^T [n][64] (state update)
    uint32_t ht[kP * kNRS / 2];      // H^T [p][n], fp16 scaled per column block
};

// 64 rows [t0, t0+64) (valid below tlimit) of a [t][G][N] bf16 tensor into
// dst[row][n] (row stride kNRS) as fp16 scaled by 2^s, s chosen from the
// rows' largest |value|; returns s, *e gets the bound. Two barriers.
__device__ int stage_rows16(const SegArgs &a, const uint16_t *M, int b, int grp, int row0, int t0,
                            int tlimit, uint32_t *dst, float *tmp, int *e) {
    constexpr int PER = 64 * (kN / 8) / kThreads;   // 4
    u32x4 r[PER];
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int item = threadIdx.x + kThreads * k;
        const int row = item >> 4, cg = item & 15;
        const int t = t0 + row;
        r[k] = u32x4{0u, 0u, 0u, 0u};
        if (t < tlimit) r[k] = ld8(M + (tok(a, b, row0 + t) * a.G + grp) * kN + 8 * cg);
        m = fmaxf(m, absmax8(r[k]));
    }
    const int eb = exp_bound(block_max(m, tmp));
    const int sc = clamp_scale(kTop - eb);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int item = threadIdx.x + kThreads * k;
        const int row = item >> 4, cg = item & 15;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack2h(ldexpf(b_lo(r[k][q]), sc), ldexpf(b_hi(r[k][q]), sc));
        *(u32x4 *)(dst + (row * kNRS + 8 * cg) / 2) = o;
    }
    *e = eb;
    return sc;
}

// One chunk [c0, c0+len) of direction d: scans, weights, masks, X^T, B.
template <int Q>
__device__ void chunk_prep(const SegArgs &a, OutSmem<Q> &sm, int d, int b, int h, int grp, int c0,
                           int len) {
    const int tid = threadIdx.x;
    const DirPtrs &dp = a.dir[d];
    const uint16_t *DT = (const uint16_t *)dp.dt;
    const float Ah = dp.A[h];
    // (1) inclusive scan in the walking direction
    const int iw = d == 0 ? tid : Q - 1 - tid;
    float at = 0.f, dtt = 0.f;
    if (tid < Q && iw < len) {
        dtt = bf2f(DT[tok(a, b, c0 + iw) * a.H + h]);
        at = dtt * Ah;
    }
    float total;
    const float cs = block_scan(tid < Q ? at : 0.f, sm.tmp, &total);
    const int edt = exp_bound(block_max(dtt, sm.tmp));
    const int sw = clamp_scale(4 - edt);
    int sq = 0;
    if (tid < Q) {
        sm.cs[iw] = cs;
        sm.dt[iw] = dtt;
        sm.a[iw] = at;
        if (a.seq && iw < len) sq = a.seq[tok(a, b, c0 + iw)];
        sm.sq[iw] = sq;
        bool off_ok = iw < len;
        if (a.seq && iw < len) {
            const int nb = d == 0 ? c0 - 1 : c0 + len;
            const bool has_nb = d == 0 ? c0 > 0 : c0 + len < a.L;
            off_ok = has_nb && a.seq[tok(a, b, nb)] == sq;
        }
        sm.u[iw] = off_ok ? expf(cs) : 0.f;
    }
    __syncthreads();
    // (2) exclusive sums toward the outgoing edge -> state weights (scaled)
    const int ie = d == 0 ? Q - 1 - tid : tid;
    const float ae = (tid < Q && ie < len) ? sm.a[ie] : 0.f;
    float tot2;
    const float incl = block_scan(tid < Q ? ae : 0.f, sm.tmp, &tot2);
    if (tid < Q) {
        float wt = 0.f;
        if (ie < len) {
            const int edge = d == 0 ? len - 1 : 0;
            if (!a.seq || sm.sq[ie] == sm.sq[edge]) wt = ldexpf(expf(incl - ae) * sm.dt[ie], sw);
        }
        sm.w[ie] = wt;
    }
    if (tid == 0) {
        bool carry = true;
        if (a.seq) {
            if (d == 0 && c0 > 0) carry = a.seq[tok(a, b, c0 - 1)] == a.seq[tok(a, b, c0 + len - 1)];
            if (d == 1 && c0 + len < a.L) carry = a.seq[tok(a, b, c0 + len)] == a.seq[tok(a, b, c0)];
        }
        sm.gamma = carry ? expf(total) : 0.f;
        sm.sw = sw;
        sm.edt = edt;
    }
    const int sx = stage_x16<Q>(a, (const uint16_t *)dp.x, b, h, c0, len, sm.xt, Q + 8, sm.tmp);
    // B of the chunk, natural layout, one scale per 64-token sub-block
    int ebmax = -126;
    for (int sb = 0; sb < Q / kSub; ++sb) {
        int eb = -126;
        const int sc = kSub * sb < len
            ? stage_rows16(a, (const uint16_t *)dp.B, b, grp, c0, kSub * sb, len,
                           sm.bn + (kSub * sb * kNRS) / 2, sm.tmp, &eb)
            : 0;
        if (tid == 0) sm.sB[sb] = sc;
        ebmax = max(ebmax, eb);
    }
    if (tid == 0) { sm.sx = sx; sm.eBmax = ebmax; }
    if (tid < Q / 16) {
        int any = 0;
        for (int r = 0; r < 16; ++r) any |= sm.u[16 * tid + r] != 0.f;
        sm.utile[tid] = any;
    }
    if (tid >= 64 && tid < 64 + Q / kSub) {
        const int sb = tid - 64;
        int any = 0;
        for (int r = 0; r < kSub; ++r) any |= sm.w[kSub * sb + r] != 0.f;
        sm.wsub[sb] = any;
    }
    __syncthreads();
}

// Writes H (the wave's 16 columns, fp32 accumulators) into sm.ht as fp16,
// scaled by a per-wave power of two.
template <int Q>
__device__ void publish_state(OutSmem<Q> &sm, const f32x4 (&Hacc)[kN / 16]) {
    const int lane = lane_id(), w = wave_id(), g4 = lane >> 4, l16 = lane & 15;
    float hm = 0.f;
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hm = fmaxf(hm, fabsf(Hacc[nt][r]));
    const int sH = clamp_scale(kTop - exp_bound(wave_max(hm)));
    uint16_t *ht = (uint16_t *)sm.ht;
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt) {
        const u32x2 v = {pack2h(ldexpf(Hacc[nt][0], sH), ldexpf(Hacc[nt][1], sH)),
                         pack2h(ldexpf(Hacc[nt][2], sH), ldexpf(Hacc[nt][3], sH))};
        *(u32x2 *)(ht + (16 * w + l16) * kNRS + 16 * nt + 4 * g4) = v;
    }
    if (lane == 0) sm.sH[w] = sH;
}

// Row block I (64 rows) of the chunk: intra-chunk form, carried state, skip
// term, output. Wave w owns rows 64I + 16w .. +15 and all 64 columns.
template <int Q>
__device__ void row_block(const SegArgs &a, OutSmem<Q> &sm, int d, int b, int h, int grp,
                          int c0, int len, int I, bool has_state, float Dh, bool add) {
    const int lane = lane_id(), w = wave_id(), g4 = lane >> 4, l16 = lane & 15;
    const DirPtrs &dp = a.dir[d];
    int eC;
    const int sC = stage_rows16(a, (const uint16_t *)dp.C, b, grp, c0, 64 * I, len, sm.tile, sm.tmp, &eC);
    // C is now in sm.tile (natural rows)
    __syncthreads();
    const uint16_t *ct = (const uint16_t *)sm.tile;
    const uint16_t *bn = (const uint16_t *)sm.bn;
    const uint16_t *xt = (const uint16_t *)sm.xt;
    constexpr int XRS = Q + 8;
    const int it = 4 * I + w;               // this wave's 16-row tile
    const int i = 16 * it + l16;            // this lane's row (A operand / G^T column)
    const bool row_ok = i < len;
    const float csi = sm.cs[i];
    const int sqi = sm.sq[i];
    const int sM = clamp_scale(kTop - (sm.eBmax + eC + 7 + sm.edt));
    f32x4 acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = zero4();

    // ---- intra-chunk: sum over column blocks J of M[i][j] x_j
    const int Jlo = d == 0 ? 0 : I, Jhi = d == 0 ? I : Q / 64 - 1;
    if (16 * it < len) {
        for (int J = Jlo; J <= Jhi; ++J) {
            if (64 * J >= len) break;
            if (J != I) {
                const float near = d == 0 ? sm.cs[64 * I] - sm.cs[64 * J + 63]
                                          : sm.cs[64 * I + 63] - sm.cs[64 * J];
                if (near < kDead) continue;
            }
            const int gexp = sM - sm.sB[J] - sC;   // G (scaled) -> M scaled by 2^sM
            const int ref = d == 0 ? 64 * J + 63 : 64 * J;
            const float ui = J != I ? expf(csi - sm.cs[ref]) : 0.f;
            // terms within 16 tokens of the diagonal carry no decay and are the
            // largest: they enter as an fp16 hi + lo pair
            u32x4 mop[2], mlo[2];
            bool near_diag[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int jk = 64 * J + 32 * kk, ik = 16 * it;
                near_diag[kk] = jk <= ik + 30 && jk + 31 >= ik - 15;
                uint32_t pk[4], pl[4];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int jt = 2 * kk + half;
                    const int j0 = 64 * J + 16 * jt;
                    // whole 16-column tile on the masked side of the diagonal
                    const bool dead = J == I && (d == 0 ? jt > w : jt < w);
                    float mv[4] = {0.f, 0.f, 0.f, 0.f};
                    if (!dead) {
                        f32x4 g = zero4();
#pragma unroll
                        for (int ks = 0; ks < kN / 32; ++ks) {
                            const u32x4 aop = *(const u32x4 *)(bn + (j0 + l16) * kNRS + 32 * ks + 8 * g4);
                            const u32x4 bop = *(const u32x4 *)(ct + (16 * w + l16) * kNRS + 32 * ks + 8 * g4);
                            g = mfma_h(aop, bop, g);
                        }
                        // g[r] = G[i][j] (scaled), j = j0 + 4 g4 + r
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = j0 + 4 * g4 + r;
                            bool ok = row_ok && j < len;
                            if (J == I) ok = ok && (d == 0 ? j <= i : j >= i);
                            if (a.seq) ok = ok && sm.sq[j] == sqi;
                            float dec;
                            if (J == I) dec = expf(csi - sm.cs[j]);
                            else dec = ui * expf(sm.cs[ref] - sm.cs[j]);
                            mv[r] = ok ? ldexpf(g[r], gexp) * dec * sm.dt[j] : 0.f;
                        }
                    }
                    pk[2 * half] = pack2h(mv[0], mv[1]);
                    pk[2 * half + 1] = pack2h(mv[2], mv[3]);
                    pl[2 * half] = pack2h(mv[0] - h_lo(pk[2 * half]), mv[1] - h_hi(pk[2 * half]));
                    pl[2 * half + 1] = pack2h(mv[2] - h_lo(pk[2 * half + 1]), mv[3] - h_hi(pk[2 * half + 1]));
                }
                mop[kk] = u32x4{pk[0], pk[1], pk[2], pk[3]};
                mlo[kk] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            }
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int jb = 64 * J + 32 * kk + 4 * g4;
                    const uint16_t *xr = xt + (16 * pt + l16) * XRS;
                    const u32x2 x0 = *(const u32x2 *)(xr + jb);
                    const u32x2 x1 = *(const u32x2 *)(xr + jb + 16);
                    const u32x4 xo = {x0[0], x0[1], x1[0], x1[1]};
                    acc[pt] = mfma_h(mop[kk], xo, acc[pt]);
                    if (near_diag[kk]) acc[pt] = mfma_h(mlo[kk], xo, acc[pt]);
                }
            }
        }
    }
    const int un = -(sM + sm.sx);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[pt][r] = ldexpf(acc[pt][r], un);

    // ---- carried state: u_i * C_i . H (rows with u == 0 skipped: exact)
    if (has_state && sm.utile[it]) {
        const uint16_t *ht = (const uint16_t *)sm.ht;
        f32x4 t[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) t[pt] = zero4();
#pragma unroll
        for (int ks = 0; ks < kN / 32; ++ks) {
            const u32x4 aop = *(const u32x4 *)(ct + (16 * w + l16) * kNRS + 32 * ks + 8 * g4);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const u32x4 bop = *(const u32x4 *)(ht + (16 * pt + l16) * kNRS + 32 * ks + 8 * g4);
                t[pt] = mfma_h(aop, bop, t[pt]);
            }
        }
        const f32x4 uu = *(const f32x4 *)(sm.u + 16 * it + 4 * g4);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int unh = -(sC + sm.sH[pt]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] = fmaf(uu[r], ldexpf(t[pt][r], unh), acc[pt][r]);
        }
    }

    // ---- skip term (x exact) and output rows 16it + 4g4 + r
    const int sxn = -sm.sx;
    const int i0 = 16 * it + 4 * g4;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
        const u32x2 xv = *(const u32x2 *)(xt + (16 * pt + l16) * XRS + i0);
        acc[pt][0] = fmaf(Dh, ldexpf(h_lo(xv[0]), sxn), acc[pt][0]);
        acc[pt][1] = fmaf(Dh, ldexpf(h_hi(xv[0]), sxn), acc[pt][1]);
        acc[pt][2] = fmaf(Dh, ldexpf(h_lo(xv[1]), sxn), acc[pt][2]);
        acc[pt][3] = fmaf(Dh, ldexpf(h_hi(xv[1]), sxn), acc[pt][3]);
    }
    float *yrow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        yrow[r] = a.y + (tok(a, b, c0 + min(i0 + r, len - 1)) * a.H + h) * kP + l16;
    if (add) {
        // the reverse pass wrote these rows: fetch all 16 values before any
        // store so the loads overlap instead of forming a chain
        float prev[4][4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                prev[pt][r] = yrow[r][16 * pt];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] += prev[pt][r];
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (i0 + r < len) yrow[r][16 * pt] = acc[pt][r];
    __syncthreads();   // the C tile is reused
}

// H <- gamma H + sum over the chunk's tokens of w_t B_t x_t^T (the wave's
// 16 columns), B^T transposed inside LDS from the staged B.
template <int Q>
__device__ void chunk_state_update(OutSmem<Q> &sm, f32x4 (&Hacc)[kN / 16], int len) {
    const float gmm = sm.gamma;
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt) Hacc[nt] *= gmm;
    const uint16_t *bn = (const uint16_t *)sm.bn;
    for (int sb = 0; sb < Q / kSub; ++sb) {
        if (kSub * sb >= len) break;
        if (!sm.wsub[sb]) continue;    // every weight is exactly 0
        for (int item = threadIdx.x; item < 32 * (kN / 8); item += kThreads) {
            const int rp = item & 31, cg = item >> 5;
            const int t = kSub * sb + 2 * rp;
            const u32x4 r0 = *(const u32x4 *)(bn + t * kNRS + 8 * cg);
            const u32x4 r1 = *(const u32x4 *)(bn + (t + 1) * kNRS + 8 * cg);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sm.tile[((8 * cg + 2 * q) * kRS) / 2 + rp] = (r0[q] & 0xffffu) | (r1[q] << 16);
                sm.tile[((8 * cg + 2 * q + 1) * kRS) / 2 + rp] = (r0[q] >> 16) | (r1[q] & 0xffff0000u);
            }
        }
        __syncthreads();
        f32x4 T[kN / 16];
#pragma unroll
        for (int nt = 0; nt < kN / 16; ++nt) T[nt] = zero4();
        state_mfma(T, sm.tile, (const uint16_t *)sm.xt, Q + 8, kSub * sb, sm.w + kSub * sb);
        const int un = -(sm.sB[sb] + sm.sw + sm.sx);
#pragma unroll
        for (int nt = 0; nt < kN / 16; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) Hacc[nt][r] += ldexpf(T[nt][r], un);
        __syncthreads();
    }
}

template <int Q>
__global__ void __launch_bounds__(kThreads) k_seg_out(const SegArgs a) {
    // XCD-aware order: consecutive workgroups go to different XCDs
    // (round-robin by 8), so the 8 streams of work that share one XCD's L2 are
    // made to hold the same (row, segment) and share its B and C.
    const int id = blockIdx.x;
    const int xcd = id & 7, r8 = id >> 3;
    const int h = r8 % a.H;
    const int rs = (r8 / a.H) * 8 + xcd;        // (row, segment) index
    if (rs >= a.batch * a.nseg) return;
    const int b = rs / a.nseg, seg = rs % a.nseg;
    const int grp = h / (a.H / a.G);
    const int t0 = seg * a.Ts, t1 = min(t0 + a.Ts, a.L);
    const int cfirst = t0 / Q, clast = (t1 - 1) / Q;
    const int lane = lane_id(), w = wave_id(), g4 = lane >> 4, l16 = lane & 15;
    __shared__ __attribute__((aligned(16))) OutSmem<Q> sm;
    const size_t PN = (size_t)kP * kN;
    auto slot = [&](int d, int k) { return (((size_t)b * 2 + d) * a.nseg + k) * a.H + h; };

    for (int pass = 0; pass < a.ndir; ++pass) {
        const int d = a.ndir == 2 ? 1 - pass : 0;   // reverse first, then forward adds
        const DirPtrs &dp = a.dir[d];
        const float Dh = dp.D ? dp.D[h] : 0.f;
        // incoming state of this segment in the walking direction
        f32x4 Hacc[kN / 16];
        const float *src = nullptr;
        if (d == 0) {
            if (seg == 0) src = a.init_state ? a.init_state + ((size_t)b * a.H + h) * PN : nullptr;
            else src = a.gam[slot(0, seg - 1)] == 0.f ? a.S + slot(0, seg - 1) * PN : a.Hs + slot(0, seg) * PN;
        } else {
            if (seg == a.nseg - 1) src = nullptr;
            else src = a.gam[slot(1, seg + 1)] == 0.f ? a.S + slot(1, seg + 1) * PN : a.Hs + slot(1, seg) * PN;
        }
#pragma unroll
        for (int nt = 0; nt < kN / 16; ++nt)
            Hacc[nt] = src ? *(const f32x4 *)(src + (16 * w + l16) * kN + 16 * nt + 4 * g4) : zero4();
        bool has_state = src != nullptr;
        if (has_state) publish_state<Q>(sm, Hacc);

        const int nch = clast - cfirst + 1;
        for (int s = 0; s < nch; ++s) {
            const int c = d == 0 ? cfirst + s : clast - s;
            const int c0 = c * Q;
            const int len = min(Q, a.L - c0);
            chunk_prep<Q>(a, sm, d, b, h, grp, c0, len);
            for (int I = 0; I < Q / 64; ++I) {
                if (64 * I >= len) break;
                row_block<Q>(a, sm, d, b, h, grp, c0, len, I, has_state, Dh, d == 0 && a.ndir == 2);
            }
            const bool last = s == nch - 1;
            const bool want_final = d == 0 && seg == a.nseg - 1 && a.final_state;
            if (!last || want_final) {
                chunk_state_update<Q>(sm, Hacc, len);
                if (!last) {
                    publish_state<Q>(sm, Hacc);
                    has_state = true;
                }
            }
            __syncthreads();
        }
        if (d == 0 && seg == a.nseg - 1 && a.final_state) {
            float *fs = a.final_state + ((size_t)b * a.H + h) * PN;
#pragma unroll
            for (int nt = 0; nt < kN / 16; ++nt)
                *(f32x4 *)(fs + (16 * w + l16) * kN + 16 * nt + 4 * g4) = Hacc[nt];
        }
    }
}

int pick_ts(int batch, int L, int H, int Q) {
    int ts = 2048;
    while (ts > Q && (long)batch * ((L + ts - 1) / ts) * H < 512) ts /= 2;
    return ts < Q ? Q : ts;
}

template <int Q>
hipError_t launch_q(const SegArgs &a, hipStream_t s) {
    const int nd = a.ndir;
    if (a.nseg > 1) {
        BM_LAUNCH("ssd_seg_state", k_seg_state, dim3(a.nseg, nd, a.batch * a.H), dim3(kThreads), 0,
                  s, a);
        BM_LAUNCH("ssd_seg_scan", k_seg_scan, dim3(kP * kN / 256, a.H, a.batch * nd), dim3(256), 0,
                  s, a);
    }
    const int groups = (a.batch * a.nseg + 7) / 8;
    BM_LAUNCH("ssd_seg_out", k_seg_out<Q>, dim3(groups * 8 * a.H), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

bool chunked_supported(const Problem &p) {
    return p.bf16 && p.P == kP && p.N == kN && p.L > 0 &&
           (p.Q == 64 || p.Q == 128 || p.Q == 256);
}

size_t chunked_workspace(int batch, int L, int H, int G, int Q) {
    const int ts = pick_ts(batch, L, H, Q);
    const size_t nseg = (size_t)(L + ts - 1) / ts;
    const size_t nC = (size_t)(L + Q - 1) / Q;
    (void)nC; (void)G;
    if (nseg == 1) return 0;   // one segment per row: no segment states
    const size_t st = batch * 2 * nseg * H * (size_t)(kP * kN) * 4;
    return al256(st) * 2 + al256(batch * 2 * nseg * H * 4);
}

hipError_t launch_chunked(const Problem &p, void *ws, hipStream_t s) {
    SegArgs a;
    a.dir[0] = p.dir[0];
    a.dir[1] = p.dir[1];
    a.ndir = p.has_bwd ? 2 : 1;
    a.batch = p.batch; a.L = p.L; a.H = p.H; a.G = p.G;
    a.nC = (p.L + p.Q - 1) / p.Q;
    a.Ts = pick_ts(p.batch, p.L, p.H, p.Q);
    a.nseg = (p.L + a.Ts - 1) / a.Ts;
    a.seq = p.seq_idx;
    const size_t nseg = a.nseg;
    a.S = a.Hs = a.gam = nullptr;   // only read when a row has several segments
    if (nseg > 1) {
        const size_t st = p.batch * 2 * nseg * p.H * (size_t)(kP * kN) * 4;
        char *w = (char *)ws;
        a.S = (float *)w;
        w += al256(st);
        a.Hs = (float *)w;
        w += al256(st);
        a.gam = (float *)w;
    }
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
