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
// Kernels:
//   k_seg_state  (4 waves) each segment's (Ts tokens) outgoing state from a
//                zero state, walking away from the outgoing edge and stopping
//                where every remaining weight is exactly 0.0f in fp32; the
//                next sub-block's rows are fetched during the current one's
//                products
//   k_seg_scan   incoming state of each segment where a chain carries over;
//                where a segment's carry factor is 0 the next segment's
//                incoming state is just the previous segment's local state
//   k_pair_out   the output kernel wherever a group's heads pair up (8 waves,
//                two heads per workgroup, 64-token chunks, fp16 products with
//                a range guard; described at its definition below)
//   k_seg_out    (8 waves, two per SIMD) per (row, segment, head): the reverse
//                direction walks the segment's chunks right to left writing
//                its part of y, the forward direction walks left to right and
//                adds its part. Per chunk, x and B are staged raw in LDS; each
//                wave then owns whole 16-row tiles with C in registers: Gram
//                tiles G^T = B C^T (whose accumulator layout is directly the A
//                operand of the next product), the masked decay, M.x, the
//                carried-state term and D x, with no barrier. The state update
//                runs with each wave owning a 16 x 64 block of H as MFMA
//                accumulators. (4 waves and two workgroups per CU for
//                64-token chunks.)
//   k_dual_out   rows of at most one 64-token chunk (the block-decode step):
//                both directions at once, waves 0-3 the reverse one and
//                waves 4-7 the forward one, the reverse sums handed over
//                through LDS.
//
// k_seg_state, k_seg_out and k_dual_out run on v_mfma_f32_16x16x32_bf16 (and
// k_pair_out on its fp16 form, see there). x, B, C are bf16 already and
// enter exactly. An operand that has to be rounded (the masked decayed Gram
// matrix M, the carried state H, the dt-weighted inputs w x) is split into
// hi = bf16(v) and lo = bf16(v - hi) and multiplied twice: ~16 significant
// bits, fp32's exponent range, no scaling. Where every decay factor of such a
// block is at most 2^-8, one rounding gives the same error bound relative to
// the undecayed product (kOneRound).
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
constexpr int kThreads = 256;  // k_seg_state: 4 waves
constexpr int kSub = 64;       // tokens per state-update sub-block
constexpr int kNRS = kN + 8;   // LDS row stride (16-bit elements) of H^T [p][n]
// Staged B [t][n] tiles: row stride kBS, rows in odd groups of 8 shifted by 8
// elements. A 16-byte row read by 16 lanes (the Gram operand, rows r..r+15)
// and a transposing read by 32 lanes (the state-update operand, rows r..r+7,
// 32 bytes each) both land on 64 distinct 4-byte banks.
constexpr int kBS = kN + 16;
__device__ __forceinline__ int bn_row(int t) { return t * kBS + ((t >> 3) & 1) * 8; }
// bn_row(r + l) - r * kBS for a multiple r of 16 and l < 16
__device__ __forceinline__ int bn_lane(int l) { return l * kBS + (l >> 3) * 8; }
constexpr int bn_elems(int rows) { return rows * kBS; }
constexpr int kXS = kP + 16;   // LDS row stride (16-bit elements) of x [t][p] tiles
constexpr float kDead = -110.f;  // expf(x) is exactly 0.0f for every x < kDead
constexpr float kLog2e = 1.4426950408889634f;
// Where every decay factor of a block of products is at most 2^kOneRound,
// its decayed operand is rounded once to bf16 instead of split into hi + lo:
// the rounding error, at most 2^-9 of an entry, is then at most 2^-17 of the
// undecayed product, the bound the hi/lo pair gives where the factor is 1.
constexpr float kOneRound = -8.f;   // log2 of the factor


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// v = hi + lo, hi = bf16(v), lo = bf16(v - hi), packed per pair of values
__device__ __forceinline__ void split2(float v0, float v1, uint32_t &hi, uint32_t &lo) {
    const bf16x2_t h = {(__bf16)v0, (__bf16)v1};
    hi = __builtin_bit_cast(uint32_t, h);
    const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
    const bf16x2_t l = {(__bf16)(v0 - h0), (__bf16)(v1 - h1)};
    lo = __builtin_bit_cast(uint32_t, l);
}
// bf16(v0), bf16(v1) packed (one rounding, no residual)
__device__ __forceinline__ uint32_t pack2(float v0, float v1) {
    const bf16x2_t h = {(__bf16)v0, (__bf16)v1};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float b_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float b_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Matrix-core operand (A or B of v_mfma_f32_16x16x32_bf16) for the 16
// columns c0..c0+15 of a row-major [t][c] bf16 tile in LDS (row stride rs),
// with k running over the 32 rows t32..t32+31, read by two transposing LDS
// loads (ds_read_b64_tr_b16). Within each group of 16 lanes such a load hands
// lane i the 4 values that the group's lanes 4q + i/4 (q < 4) point at, at
// element i%4; so lane s points at row t0 + s/4, column c0 + 4(s%4), and lane
// i receives column c0 + i of rows t0..t0+3. Lane group g4 thus holds k slots
//   0..3 -> rows t32 + 4 g4 + (0..3),   4..7 -> rows t32 + 16 + 4 g4 + (0..3),
// the k order in which a pair of Gram accumulator tiles feeds the next
// product.
__device__ __forceinline__ u32x2 ld_tr(const uint16_t *p) {
    const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)p);
    return __builtin_bit_cast(u32x2, r);
}
__device__ __forceinline__ u32x4 tr_operand(const uint16_t *base, int rs, int t32, int c0) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, s = lane & 15;
    const uint16_t *p = base + (t32 + 4 * g4 + (s >> 2)) * rs + c0 + 4 * (s & 3);
    const u32x2 a = ld_tr(p), b = ld_tr(p + 16 * rs);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// tr_operand for a staged B tile (bn_row layout); t32 is a multiple of 8, so
// rows t and t + 16 share their shift.
__device__ __forceinline__ u32x4 tr_operand_bn(const uint16_t *bn, int t32, int c0) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, s = lane & 15;
    const uint16_t *p = bn + t32 * kBS + bn_lane(4 * g4 + (s >> 2)) + c0 + 4 * (s & 3);
    const u32x2 a = ld_tr(p), b = ld_tr(p + 16 * kBS);
    return u32x4{a[0], a[1], b[0], b[1]};
}

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
    const float *dt_bias[2];  // with the softplus step size: [H] per direction or nullptr
    float *y2;                // streams kept apart: the forward stream's output
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ size_t tok(const SegArgs &a, int b, int t) { return (size_t)b * a.L + t; }
__device__ __forceinline__ u32x4 ld8(const uint16_t *p) { return *(const u32x4 *)p; }

// Workgroup barrier that orders LDS only: global loads in flight (the next
// chunk's prefetch) stay in flight across it. Workgroups here exchange data
// through LDS alone; each y element is read back only by the lane that wrote
// it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// fp64 value moved across lanes by a DPP control (both 32-bit halves);
// lanes without a source (or outside ROWMASK) read 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_d(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    int lo = (int)(unsigned)(u & 0xffffffffull), hi = (int)(unsigned)(u >> 32);
    lo = __builtin_amdgcn_update_dpp(0, lo, CTRL, ROWMASK, 0xf, true);
    hi = __builtin_amdgcn_update_dpp(0, hi, CTRL, ROWMASK, 0xf, true);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Inclusive fp64 scan over the wave's 64 lanes with DPP lane moves (no LDS
// round trips): shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the
// row totals broadcast into the following rows.
__device__ __forceinline__ double wave_scan_d(double v) {
    v += dpp_d<0x111, 0xf>(v);   // row_shr:1
    v += dpp_d<0x112, 0xf>(v);   // row_shr:2
    v += dpp_d<0x114, 0xf>(v);   // row_shr:4
    v += dpp_d<0x118, 0xf>(v);   // row_shr:8
    v += dpp_d<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_d<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return v;
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

// --------------------------------------------------------- staging helpers
// ROWS rows of COLS bf16 each (m0 = the first row, rstride elements between
// rows in memory), raw, into dst (row stride RS). All global loads are issued
// before the first LDS write so that they overlap; rows at or past `tlimit`
// are loaded clamped and stored as zeros.
template <int ROWS, int COLS, int RS, int NT, bool BROWS = false, int WB = 0>
struct RowStage {
    static constexpr int CG = COLS / 8;
    static constexpr int ITEMS = ROWS * CG;
    static constexpr int PER = (ITEMS + NT - 1) / NT;
    u32x4 v[PER];
    // items k0 <= k < k1 of this thread (the loads can be spread over a loop)
    __device__ __forceinline__ void load_part(const uint16_t *m0, uint32_t rstride, int tlimit,
                                              int k0, int k1) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            if (k < k0 || k >= k1) continue;
            const int item = (int)threadIdx.x - 64 * WB + k * NT;
            if (ITEMS % NT == 0 || item < ITEMS) {
                const int row = item / CG, cg = item % CG;
                v[k] = ld8(m0 + (uint32_t)min(row, tlimit - 1) * rstride + 8 * cg);
            }
        }
    }
    __device__ __forceinline__ void load(const uint16_t *m0, uint32_t rstride, int tlimit) {
        load_part(m0, rstride, tlimit, 0, PER);
    }
    __device__ __forceinline__ void store(int tlimit, uint16_t *dst) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int item = (int)threadIdx.x - 64 * WB + k * NT;
            if (ITEMS % NT == 0 || item < ITEMS) {
                const int row = item / CG, cg = item % CG;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const int ro = BROWS ? bn_row(row) : row * RS;
                *(u32x4 *)(dst + ro + 8 * cg) = row < tlimit ? v[k] : z;
            }
        }
    }
};

// B operand of the state update for the 32 tokens t32..t32+31 and the 16
// columns p0..p0+15: (w_t x_t[p]) split into bf16 hi / lo. xs: x [t][p]
// (row stride kXS); wv: the weights, natural token order.
// With !lo (every weight factor at most 2^kOneRound) only bhi, rounded once.
__device__ __forceinline__ void wx_operand(const uint16_t *xs, int t32, int p0, const float *wv,
                                           u32x4 &bhi, u32x4 &blo, bool lo = true) {
    const int g4 = (threadIdx.x & 63) >> 4;
    const u32x4 xv = tr_operand(xs, kXS, t32, p0);
    const f32x4 w0 = *(const f32x4 *)(wv + t32 + 4 * g4);        // k slots 0..3
    const f32x4 w1 = *(const f32x4 *)(wv + t32 + 16 + 4 * g4);   // k slots 4..7
    const float v[8] = {b_lo(xv[0]) * w0[0], b_hi(xv[0]) * w0[1], b_lo(xv[1]) * w0[2],
                        b_hi(xv[1]) * w0[3], b_lo(xv[2]) * w1[0], b_hi(xv[2]) * w1[1],
                        b_lo(xv[3]) * w1[2], b_hi(xv[3]) * w1[3]};
    if (lo) {
        uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
        split2(v[0], v[1], h0, l0);
        split2(v[2], v[3], h1, l1);
        split2(v[4], v[5], h2, l2);
        split2(v[6], v[7], h3, l3);
        bhi = u32x4{h0, h1, h2, h3};
        blo = u32x4{l0, l1, l2, l3};
    } else {
        bhi = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
        blo = u32x4{0u, 0u, 0u, 0u};
    }
}

// ----------------------------------------------------------- k_seg_state
struct StateSmem {
    float w[kSub];
    alignas(16) uint16_t bn[bn_elems(kSub)];   // B [t][n], bn_row layout
    alignas(16) uint16_t xs[kSub * kXS];    // x [t][p]
    float run[2];   // running sum of a from the outgoing edge, by step parity
    int stop[2];    // the previous sub-block reached another sequence
};

// SP: dt holds the step size's pre-activation (softplus(dt + bias) is used).
// The sub-blocks are walked one after another; each one's rows (B, x, and on
// wave 0 its step sizes and sequence indices) are fetched into registers
// while the one before is multiplied, so a step costs about one of the two
// rather than their sum.
template <bool SP>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) k_seg_state(const SegArgs a) {
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
    const float dtb = SP && a.dt_bias[d] ? a.dt_bias[d][h] : 0.f;
    __shared__ __attribute__((aligned(16))) StateSmem sm;

    const int edge = d == 0 ? t1 - 1 : t0;
    const int edge_seq = a.seq ? a.seq[tok(a, b, edge)] : 0;
    if (tid == 0) {
        sm.run[0] = 0.f;
        sm.stop[0] = 0;
    }
    // wave w owns state columns p = 16w..16w+15 for all n
    f32x4 Hacc[kN / 16];
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt) Hacc[nt] = zero4();

    const int nsub = (t1 - t0 + kSub - 1) / kSub;
    // sub-block k = [s0, s0 + n), the k-th counted away from the outgoing edge
    auto sub0 = [&](int k) { return d == 0 ? max(t0, t1 - kSub * (k + 1)) : t0 + kSub * k; };
    auto subn = [&](int k) { return d == 0 ? t1 - kSub * k - sub0(k) : min(t1, t0 + kSub * (k + 1)) - sub0(k); };
    RowStage<kSub, kN, kBS, kThreads, true> sb;
    RowStage<kSub, kP, kXS, kThreads> sx;
    uint16_t dtr = 0;     // wave 0: raw step size of the lane's token
    int sqr = edge_seq;   // wave 0: its sequence index
    // a whole sub-block (every one but a segment's last, in walking order)
    // is read without clamping: this thread's pieces sit at fixed offsets
    // from the sub-block's first row (RowStage's item order: B item
    // tid + 256 q is row tid / 16 + 16 q, x item tid + 256 q row tid / 8 + 32 q)
    const uint32_t bstride = (uint32_t)(a.G * kN), xstride = (uint32_t)(a.H * kP);
    const uint32_t boff = (uint32_t)(tid >> 4) * bstride + 8 * (tid & 15);
    const uint32_t xoff = (uint32_t)(tid >> 3) * xstride + 8 * (tid & 7);
    auto fetch = [&](int k) {
        const int s0 = sub0(k), n = subn(k);
        const uint16_t *bb = Bm + (tok(a, b, s0) * a.G + grp) * kN;
        const uint16_t *xb = X + (tok(a, b, s0) * a.H + h) * kP;
        if (n == kSub) {
#pragma unroll
            for (int q = 0; q < 4; ++q) sb.v[q] = ld8(bb + boff + (uint32_t)q * 16 * bstride);
#pragma unroll
            for (int q = 0; q < 2; ++q) sx.v[q] = ld8(xb + xoff + (uint32_t)q * 32 * xstride);
        } else {
            sb.load(bb, bstride, n);
            sx.load(xb, xstride, n);
        }
        if (w == 0) {
            // lane 0 is the token nearest the outgoing edge; lanes past the
            // sub-block re-read its last token (not used)
            const int pos = min(d == 0 ? n - 1 - lane : lane, n - 1);
            const size_t ti = tok(a, b, s0 + max(pos, 0));
            dtr = DT[ti * a.H + h];
            if (a.seq) sqr = a.seq[ti];
        }
    };
    fetch(0);
    __syncthreads();

    int step = 0;
    for (; step < nsub; ++step) {
        const int n = subn(step);
        // every remaining weight is e^{<= run} * dt == 0.0f exactly, or every
        // remaining token belongs to another sequence: nothing left to add
        const float run = sm.run[step & 1];
        if (run < kDead || sm.stop[step & 1]) break;
        if (w == 0) {
            const bool in = lane < n;
            const int pos = d == 0 ? n - 1 - lane : lane;
            float at = 0.f, dtt = 0.f;
            if (in) {
                dtt = bf2f(dtr);
                if (SP) dtt = softplus_dt(dtt + dtb);
                at = dtt * Ah;
            }
            const float incl = wave_scan(at);
            float wt = 0.f;
            if (in && (!a.seq || sqr == edge_seq)) wt = expf(run + incl - at) * dtt;
            if (in) sm.w[pos] = wt;
            else sm.w[lane] = 0.f;
            const float tot = __shfl(incl, 63, 64);
            // the sub-block's token farthest from the edge (lane n - 1): once
            // it lies in another sequence, so does everything past it
            const int far_seq = __shfl(sqr, n - 1, 64);
            if (lane == 0) {
                sm.run[(step + 1) & 1] = run + tot;
                sm.stop[(step + 1) & 1] = a.seq && far_seq != edge_seq;
            }
        }
        if (n == kSub) {   // (no row past the end to zero)
            sb.store(kSub, sm.bn);
            sx.store(kSub, sm.xs);
        } else {
            sb.store(n, sm.bn);
            sx.store(n, sm.xs);
        }
        lds_barrier();
        if (step + 1 < nsub) fetch(step + 1);
        // H[n][p] += sum_t B^T[n][t] (w_t x_t[p]): A = B^T rows, B = w x
#pragma unroll
        for (int ks = 0; ks < kSub / 32; ++ks) {
            u32x4 bhi, blo;
            wx_operand(sm.xs, 32 * ks, 16 * w, sm.w, bhi, blo);
#pragma unroll
            for (int nt = 0; nt < kN / 16; ++nt) {
                const u32x4 aop = tr_operand_bn(sm.bn, 32 * ks, 16 * nt);
                Hacc[nt] = mfma16x16x32(aop, bhi, Hacc[nt]);
                Hacc[nt] = mfma16x16x32(aop, blo, Hacc[nt]);
            }
        }
        lds_barrier();
    }
    // Hacc[nt][r] = H[n = 16nt + 4g4 + r][p = 16w + l16]
    const size_t si = (((size_t)b * 2 + d) * a.nseg + seg) * a.H + h;
    float *Sout = a.S + si * (size_t)(kP * kN);
#pragma unroll
    for (int nt = 0; nt < kN / 16; ++nt)
        *(f32x4 *)(Sout + (16 * w + l16) * kN + 16 * nt + 4 * g4) = Hacc[nt];
    if (tid == 0) {
        // the incoming state passes through iff the whole segment was walked
        // (its total decay did not underflow), and no sequence boundary lies
        // between the segment's incoming side and its edge
        bool carry = step == nsub && !sm.stop[nsub & 1];
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
    if (d == 0 && a.init_state) {
        hv = a.init_state[((size_t)b * a.H + h) * PN + e];
        // the first segment's copy of the caller's incoming state (its slot of
        // Hs is otherwise unused): the output kernel reads this copy, so no
        // workgroup of it reads init_state while the last segment's workgroup
        // writes final_state (which may be the same array)
        a.Hs[slot(0) * PN + e] = hv;
    }
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
// Waves per workgroup: 8 (two per SIMD, so one wave's VALU and LDS work
// overlaps another's matrix-core work and waits); with 64-token chunks, which
// have only 4 row tiles and need 64 KB of LDS, 4 waves and two workgroups per
// CU. Wave w owns state block (p-tile w%4, n-tiles NQ*(w/4) .. +NQ-1).
template <int Q>
struct Cfg {
    static constexpr int NW = Q == 64 ? 4 : 8;
    static constexpr int NT = 64 * NW;
    static constexpr int NQ = 32 / NW;   // 16x16 state tiles per wave
    // single rounding where every decay factor is at most 2^kOneRound (off
    // for 128-token chunks, where the extra branches measured slower)
    static constexpr bool ONE_ROUND = Q != 128;
};

// The wave's index within its group of Cfg<Q>::NW waves: the workgroup, or
// (WB = 4) the upper half of the two-direction workgroup of k_dual_out.
template <int WB>
__device__ __forceinline__ int wave_in() { return wave_id() - WB; }

template <int Q>
struct OutSmem {
    float cs2[Q];          // inclusive scan of a in the walking direction, times log2(e)
    float rl2[Q];          // the same scan restarted at the token's 64-block (walking order), times log2(e)
    float w[Q];            // state-update weights
    float v16[Q];          // e^{cs(edge of the token's 16-tile) - cs} dt
    float v64[Q];          // e^{cs(edge of the token's 64-block) - cs} dt
    float dt[Q];
    int sq[Q];             // sequence index (packed) of each token
    int utile[Q / 16];     // the carried state reaches some row of the 16-row tile
    int wsub[Q / kSub];    // some weight of the 64-token sub-block is nonzero
    int wbig[Q / kSub];    // some weight factor of the sub-block exceeds 2^kOneRound
    float gamma;           // decay of the whole chunk (0: the state does not pass)
    float bt2[Q / 64][Q / 64];  // [I][J] (walking order, J < I): sum of a over the blocks strictly between, times log2(e)
    int sq_nb;             // sequence index of the token the carried state comes from
    alignas(16) uint16_t xs[Q * kXS];       // x [t][p], raw bf16
    alignas(16) uint16_t bn[bn_elems(Q)];   // B [t][n], raw bf16, bn_row layout
    alignas(16) uint16_t hs[2 * kP * kNRS]; // H^T [p][n]: bf16 high part, then bf16 residual
};

// A row tile's inputs from global memory, fetched one phase ahead of the
// tile so that their latency is hidden: C of its 16 rows in the layout that
// is both the B operand of the Gram tiles and the A operand of the
// carried-state product, and, for the forward pass, the tile's rows of y as
// the reverse pass left them (read by the same lane that wrote them).
struct TileIn {
    u32x4 cr[kN / 32];
    float prev[4][4];
};

template <int D>
__device__ __forceinline__ void tile_fetch(TileIn &t, const SegArgs &a, int b, int h, int grp,
                                           int c0, int len, int it, bool add) {
    if (it < 0) return;   // the wave has no such tile
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    const int i = 16 * it + l16, i0 = 16 * it + 4 * g4;
    const uint16_t *cp = (const uint16_t *)a.dir[D].C + (tok(a, b, c0) * a.G + grp) * kN +
                         (uint32_t)(min(i, len - 1) * a.G * kN) + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < kN / 32; ++ks) t.cr[ks] = ld8(cp + 32 * ks);
    if (add) {
        const float *ybase = a.y + (tok(a, b, c0) * a.H + h) * kP + l16;
        const uint32_t ystride = (uint32_t)(a.H * kP);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t yo = (uint32_t)min(i0 + r, len - 1) * ystride;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) t.prev[pt][r] = ybase[yo + 16 * pt];
        }
    }
}

// Position in a chunk of Q tokens of the i-th of the Q/64 tokens that lane
// `lane` of a scanning wave holds: walking order for wave 0, from the
// outgoing edge for wave 1.
template <int Q>
__device__ __forceinline__ int scan_pos(int d, int wv, int lane, int i) {
    const int k = lane * (Q / 64) + i;
    return (wv == 0) == (d == 0) ? k : Q - 1 - k;
}

// Loads of one chunk [c0, c0+len) of direction D, issued ahead of use (the
// next chunk's are issued before the current chunk's state update, so their
// latency overlaps it): x and B for every thread, and for waves 0 and 1 the
// dt (and sequence index) of the chunk's tokens, Q/64 per lane, in walking
// order (wave 0) or from the outgoing edge (wave 1).
template <int Q, bool PACKED, int WB = 0>
struct ChunkLoads {
    static constexpr int TPL = Q / 64;   // tokens per lane of the scanning waves
    RowStage<Q, kP, kXS, Cfg<Q>::NT, false, WB> sx;
    RowStage<Q, kN, kBS, Cfg<Q>::NT, true, WB> sb;
    uint16_t dtv[TPL];   // raw bf16 bits: no use (and no wait) until the scan
    int sqv[TPL];
    TileIn tin;          // the wave's first row tile

    __device__ static __forceinline__ int pos_of(int d, int wv, int lane, int i) {
        return scan_pos<Q>(d, wv, lane, i);
    }

    const uint16_t *x0, *b0;
    uint32_t xstride, bstride;
    int tl;

    // dt (waves 0, 1) now; x and B in `parts` slices through part()
    __device__ __forceinline__ void begin(const SegArgs &a, int d, int b, int h, int grp, int c0,
                                          int len) {
        const DirPtrs &dp = a.dir[d];
        const int wv = wave_in<WB>(), lane = lane_id();
        if (wv < 2) {
            const uint16_t *DT = (const uint16_t *)dp.dt;
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                // clamped, unconditional: positions past the end are masked
                // where the values are used
                const int pos = min(pos_of(d, wv, lane, i), len - 1);
                dtv[i] = DT[tok(a, b, c0 + pos) * a.H + h];
                sqv[i] = PACKED ? a.seq[tok(a, b, c0 + pos)] : 0;
            }
        }
        x0 = (const uint16_t *)dp.x + (tok(a, b, c0) * a.H + h) * kP;
        b0 = (const uint16_t *)dp.B + (tok(a, b, c0) * a.G + grp) * kN;
        xstride = (uint32_t)(a.H * kP);
        bstride = (uint32_t)(a.G * kN);
        tl = len;
    }
    // the s-th of n equal slices of the x and B loads
    __device__ __forceinline__ void part(int s, int n) {
        sx.load_part(x0, xstride, tl, s * sx.PER / n, (s + 1) * sx.PER / n);
        sb.load_part(b0, bstride, tl, s * sb.PER / n, (s + 1) * sb.PER / n);
    }
    __device__ __forceinline__ void issue(const SegArgs &a, int d, int b, int h, int grp, int c0,
                                          int len) {
        begin(a, d, b, h, grp, c0, len);
        part(0, 1);
    }
};

// Stores the T values a scanning lane holds for its consecutive tokens
// (walking order k = lane*T + i) into a per-token array: ascending positions
// when `asc`, else descending (pos = Q-1-k); one vector store.
template <int Q, int T, typename V>
__device__ __forceinline__ void store_run(V *dst, bool asc, int lane, const V (&v)[T]) {
    const int base = asc ? lane * T : Q - (lane + 1) * T;
    V o[T];
#pragma unroll
    for (int i = 0; i < T; ++i) o[i] = asc ? v[i] : v[T - 1 - i];
    if constexpr (T == 4) {
        typedef V v4 __attribute__((ext_vector_type(4)));
        *(v4 *)(dst + base) = v4{o[0], o[1], o[2], o[3]};
    } else if constexpr (T == 2) {
        typedef V v2 __attribute__((ext_vector_type(2)));
        *(v2 *)(dst + base) = v2{o[0], o[1]};
    } else {
        dst[base] = o[0];
    }
}

// The scans of one chunk [c0, c0+len) of direction d for head h, by the two
// scanning waves (wv 0 and 1) of the group of waves that serves the head:
// wave 0 scans a over the chunk in the walking direction (the decay factors,
// the 16-tiles the carried state reaches, the chunk's decay), wave 1 toward
// the outgoing edge (the state-update weights); Q/64 tokens per lane, the
// tile-edge values from lane shuffles. dtv / sqv: the raw step sizes (and
// sequence indices) of the lane's tokens (scan_pos order). SM is any shared
// layout with the per-token arrays and flags used below.
template <int Q, bool PACKED, bool SP, typename SM>
__device__ __forceinline__ void chunk_scans(const SegArgs &a, SM &sm, int wv,
                                            const uint16_t (&dtv)[Q / 64], const int (&sqv)[Q / 64],
                                            int d, int b, int h, int c0, int len) {
    constexpr int TPL = Q / 64;
    const int lane = lane_id();
    const float Ah = a.dir[d].A[h];
    const float dtb = SP && a.dt_bias[d] ? a.dt_bias[d][h] : 0.f;
    int sq_nb = 0, sq_edge = 0;
    bool has_nb = true;
    if (PACKED) {
        const int nb = d == 0 ? c0 - 1 : c0 + len;
        has_nb = d == 0 ? c0 > 0 : c0 + len < a.L;
        sq_nb = has_nb ? a.seq[tok(a, b, nb)] : -1;
        sq_edge = a.seq[tok(a, b, d == 0 ? c0 + len - 1 : c0)];
    }
    // inclusive scan over the lane's tokens, then across lanes, in fp64:
    // every exponent below is a difference of these sums, formed in fp64
    // and rounded once, so none is the difference of two large fp32 values
    float at[TPL], dtf[TPL];
    double cs[TPL];
    double run = 0.0;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        dtf[i] = scan_pos<Q>(d, wv, lane, i) < len ? bf2f(dtv[i]) : 0.f;
        if (SP) dtf[i] = scan_pos<Q>(d, wv, lane, i) < len ? softplus_dt(dtf[i] + dtb) : 0.f;
        at[i] = dtf[i] * Ah;
        run += (double)at[i];
        cs[i] = run;
    }
    const double incl = wave_scan_d(run);
    const double excl = incl - run;
#pragma unroll
    for (int i = 0; i < TPL; ++i) cs[i] += excl;
    if (wv == 0) {
        // in walking order a token's 16-tile (64-block) ends at the last
        // token of lane (lane | (16/TPL - 1)) (resp. lane | (64/TPL - 1));
        // its 64-block starts after the last token of lane
        // (lane & ~(64/TPL - 1)) - 1
        const double last = cs[TPL - 1];
        const double e16 = __shfl(last, lane | (16 / TPL - 1), 64);
        const double e64 = __shfl(last, lane | (64 / TPL - 1), 64);
        const int sl = (lane & ~(64 / TPL - 1)) - 1;
        const double b64 = __shfl(last, sl < 0 ? 0 : sl, 64);
        const double start = sl < 0 ? 0.0 : b64;
        bool reach = false;
        float c2v[TPL], rlv[TPL], v16v[TPL], v64v[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int pos = scan_pos<Q>(d, 0, lane, i);
            c2v[i] = (float)(cs[i] * kLog2e);
            rlv[i] = (float)((cs[i] - start) * kLog2e);
            v16v[i] = exp2_((float)((e16 - cs[i]) * kLog2e)) * dtf[i];
            v64v[i] = exp2_((float)((e64 - cs[i]) * kLog2e)) * dtf[i];
            reach |= pos < len && (!PACKED || sqv[i] == sq_nb) && cs[i] >= kDead;
        }
        const bool asc = d == 0;   // wave 0 walks ascending positions forward
        store_run<Q, TPL>(sm.cs2, asc, lane, c2v);
        store_run<Q, TPL>(sm.rl2, asc, lane, rlv);
        store_run<Q, TPL>(sm.dt, asc, lane, dtf);
        store_run<Q, TPL>(sm.sq, asc, lane, sqv);
        store_run<Q, TPL>(sm.v16, asc, lane, v16v);
        store_run<Q, TPL>(sm.v64, asc, lane, v64v);
        // block table: the last token of walking block K is lane
        // 64/TPL*(K+1) - 1; bt2[I][J] = cs(end of I-1) - cs(end of J)
        {
            const bool tl = lane < (Q / 64) * (Q / 64);
            const int I = tl ? lane / (Q / 64) : 0, J = tl ? lane % (Q / 64) : 0;
            const double eI = __shfl(last, (64 / TPL) * (I > 0 ? I : 1) - 1, 64);
            const double eJ = __shfl(last, (64 / TPL) * (J + 1) - 1, 64);
            if (tl) sm.bt2[I][J] = J < I ? (float)((eI - eJ) * kLog2e) : 0.f;
        }
        // 16-tiles (walking order m) the carried state reaches
        const unsigned long long m = __ballot(reach);
        if (lane < Q / 16) {
            constexpr int LPT = 16 / TPL;   // lanes per 16-tile
            const bool any = ((m >> (lane * LPT)) & ((1ull << LPT) - 1)) != 0;
            sm.utile[d == 0 ? lane : Q / 16 - 1 - lane] = any;
        }
        if (lane == 63) {
            bool carry = true;
            if (PACKED) carry = has_nb && sq_nb == sq_edge;
            sm.gamma = carry ? expf((float)last) : 0.f;
            sm.sq_nb = PACKED ? sq_nb : 0;
        }
    } else {
        // exclusive sums toward the outgoing edge -> weight of each token
        // in the state leaving the chunk
        bool nz = false, big = false;
        float wv_[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int pos = scan_pos<Q>(d, 1, lane, i);
            float wt = 0.f;
            if (pos < len && (!PACKED || sqv[i] == sq_edge)) {
                const double lf = cs[i] - (double)at[i];   // log of the weight factor
                wt = expf((float)lf) * dtf[i];
                if (Cfg<Q>::ONE_ROUND) big |= lf * (double)kLog2e > (double)kOneRound;
            }
            wv_[i] = wt;
            nz |= wt != 0.f;
        }
        store_run<Q, TPL>(sm.w, d != 0, lane, wv_);   // wave 1 walks from the edge
        const unsigned long long m = __ballot(nz);
        const unsigned long long mb = Cfg<Q>::ONE_ROUND ? __ballot(big) : 0ull;
        if (lane < Q / 64) {
            constexpr int LPS = 64 / TPL;   // lanes per 64-token sub-block
            constexpr unsigned long long lm = LPS == 64 ? ~0ull : (1ull << (LPS & 63)) - 1;
            const int sb = d == 0 ? Q / 64 - 1 - lane : lane;
            sm.wsub[sb] = ((m >> ((lane * LPS) & 63)) & lm) != 0;
            if (Cfg<Q>::ONE_ROUND) sm.wbig[sb] = ((mb >> ((lane * LPS) & 63)) & lm) != 0;
        }
    }
}

// One chunk [c0, c0+len) of direction d: staged x and B, the scans
// (chunk_scans); one barrier.
template <int Q, bool PACKED, int WB = 0, bool SP = false>
__device__ void chunk_prep(const SegArgs &a, OutSmem<Q> &sm, ChunkLoads<Q, PACKED, WB> &ld,
                           int d, int b, int h, int c0, int len) {
    const int wv = wave_in<WB>();
    ld.sx.store(len, sm.xs);
    ld.sb.store(len, sm.bn);
    if (wv < 2) chunk_scans<Q, PACKED, SP>(a, sm, wv, ld.dtv, ld.sqv, d, b, h, c0, len);
    lds_barrier();
}

// The wave's state block (p-tile w%4, n-half w/4; fp32 accumulators) into
// H^T hi / lo.
template <int Q, int WB = 0>
__device__ void publish_state(OutSmem<Q> &sm, const f32x4 (&Hacc)[Cfg<Q>::NQ]) {
    constexpr int NQ = Cfg<Q>::NQ;
    const int lane = lane_id(), w = wave_in<WB>(), g4 = lane >> 4, l16 = lane & 15;
    const int pq = w & 3, nbase = NQ * (w >> 2);
    uint16_t *hh = sm.hs;
    uint16_t *hl = hh + kP * kNRS;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        uint32_t a0, a1, b0, b1;
        split2(Hacc[q][0], Hacc[q][1], a0, b0);
        split2(Hacc[q][2], Hacc[q][3], a1, b1);
        const int o = (16 * pq + l16) * kNRS + 16 * (nbase + q) + 4 * g4;
        *(u32x2 *)(hh + o) = u32x2{a0, a1};
        *(u32x2 *)(hl + o) = u32x2{b0, b1};
    }
}

// One 16x16x32 matrix-core product: bf16 operands, or fp16 ones with F16.
template <bool F16>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (F16) return mfma16x16x32_f16(a, b, c);
    else return mfma16x16x32(a, b, c);
}

// G^T tile rows j0..j0+15 x this lane group's 16 rows i: gg[r] = G[i][j0 + 4g4 + r]
template <bool F16 = false>
__device__ __forceinline__ f32x4 gram_tile(const uint16_t *bn, int j0, const u32x4 (&cr)[kN / 32]) {
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    f32x4 g = zero4();
#pragma unroll
    for (int ks = 0; ks < kN / 32; ++ks)
        g = mma<F16>(*(const u32x4 *)(bn + j0 * kBS + bn_lane(l16) + 32 * ks + 8 * g4), cr[ks], g);
    return g;
}

// acc[pt] += M x over the 32 columns j32..j32+31; M given as a hi / lo pair
// in the k order of a Gram accumulator pair, which is the order in which the
// transposing reads deliver x. An operand's registers read the same as A
// (row = lane % 16) or as B (column = lane % 16), so with TR the product is
// taken as x^T M^T: acc then holds (M x)^T, lane (g4, l16) the entries
// [row l16][columns 16 pt + 4 g4 + r].
template <bool F16 = false, bool TR = false>
__device__ __forceinline__ void mx_step(f32x4 (&acc)[4], const uint16_t *xs, int j32, u32x4 mhi,
                                        u32x4 mlo, bool lo = true) {
    u32x4 xo[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xo[pt] = tr_operand(xs, kXS, j32, 16 * pt);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = TR ? mma<F16>(xo[pt], mhi, acc[pt]) : mma<F16>(mhi, xo[pt], acc[pt]);
    if (lo) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = TR ? mma<F16>(xo[pt], mlo, acc[pt]) : mma<F16>(mlo, xo[pt], acc[pt]);
    }
}

// Two G^T tiles (rows j0a.., j0b..) at once: all operand loads first, then
// the two MFMA chains interleaved.
template <bool F16 = false>
__device__ __forceinline__ void gram_pair(const uint16_t *bn, int j0a, int j0b,
                                          const u32x4 (&cr)[kN / 32], f32x4 &ga, f32x4 &gb) {
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    u32x4 oa[kN / 32], ob[kN / 32];
#pragma unroll
    for (int ks = 0; ks < kN / 32; ++ks) {
        oa[ks] = *(const u32x4 *)(bn + j0a * kBS + bn_lane(l16) + 32 * ks + 8 * g4);
        ob[ks] = *(const u32x4 *)(bn + j0b * kBS + bn_lane(l16) + 32 * ks + 8 * g4);
    }
    ga = zero4();
    gb = zero4();
#pragma unroll
    for (int ks = 0; ks < kN / 32; ++ks) {
        ga = mma<F16>(oa[ks], cr[ks], ga);
        gb = mma<F16>(ob[ks], cr[ks], gb);
    }
}

// Zero the entries of columns jb..jb+3 that belong to another sequence.
template <int Q, bool PACKED, typename SM>
__device__ __forceinline__ void seq_mask(float (&mv)[4], const SM &sm, int jb, int sqi) {
    if (PACKED) {
        const int4 s4 = *(const int4 *)(sm.sq + jb);
        mv[0] = s4.x == sqi ? mv[0] : 0.f;
        mv[1] = s4.y == sqi ? mv[1] : 0.f;
        mv[2] = s4.z == sqi ? mv[2] : 0.f;
        mv[3] = s4.w == sqi ? mv[3] : 0.f;
    }
}

// The diagonal 64-column block of a row tile at position WQ in its 64-row
// block: 16-tiles on the far side of the diagonal are 0; the others factor
// the decay through their edge nearest the diagonal; the diagonal tile
// itself takes one exponential per entry.
template <int Q, bool PACKED, int D, int WQ>
__device__ __forceinline__ void diag_block(f32x4 (&acc)[4], const OutSmem<Q> &sm,
                                           const u32x4 (&cr)[kN / 32], int I, int i, float rli,
                                           int sqi) {
    const int g4 = lane_id() >> 4;
    const uint16_t *bn = sm.bn;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        if (D == 0 ? 2 * kk > WQ : 2 * kk + 1 < WQ) continue;   // both tiles dead
        uint32_t ph[4], pl[4];
        const bool live0 = D == 0 ? 2 * kk <= WQ : 2 * kk >= WQ;
        const bool live1 = D == 0 ? 2 * kk + 1 <= WQ : 2 * kk + 1 >= WQ;
        f32x4 gp[2];
        if (live0 && live1) {
            gram_pair(bn, 64 * I + 32 * kk, 64 * I + 32 * kk + 16, cr, gp[0], gp[1]);
        } else {
            gp[0] = live0 ? gram_tile(bn, 64 * I + 32 * kk, cr) : zero4();
            gp[1] = live1 ? gram_tile(bn, 64 * I + 32 * kk + 16, cr) : zero4();
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int jt = 2 * kk + half;
            const int j0 = 64 * I + 16 * jt;
            float mv[4] = {0.f, 0.f, 0.f, 0.f};
            if (D == 0 ? jt <= WQ : jt >= WQ) {
                const f32x4 gg = gp[half];
                const int jb = j0 + 4 * g4;
                if (jt != WQ) {
                    // the J-tile's edge is in this 64-block: both exponents
                    // are relative to the block's start
                    const float u16 = exp2_(rli - sm.rl2[D == 0 ? j0 + 15 : j0]);
                    const f32x4 vv = *(const f32x4 *)(sm.v16 + jb);
#pragma unroll
                    for (int r = 0; r < 4; ++r) mv[r] = gg[r] * (u16 * vv[r]);
                } else {
                    const f32x4 c4 = *(const f32x4 *)(sm.rl2 + jb);
                    const f32x4 d4 = *(const f32x4 *)(sm.dt + jb);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = jb + r;
                        const bool tri = D == 0 ? j <= i : j >= i;
                        const float e = exp2_(rli - c4[r]);
                        mv[r] = tri ? gg[r] * (e * d4[r]) : 0.f;
                    }
                }
                seq_mask<Q, PACKED>(mv, sm, jb, sqi);
            }
            split2(mv[0], mv[1], ph[2 * half], pl[2 * half]);
            split2(mv[2], mv[3], ph[2 * half + 1], pl[2 * half + 1]);
        }
        mx_step(acc, sm.xs, 64 * I + 32 * kk, u32x4{ph[0], ph[1], ph[2], ph[3]},
                   u32x4{pl[0], pl[1], pl[2], pl[3]});
    }
}

// Row tile `it` (16 rows) of the chunk: intra-chunk form, carried state, skip
// term, output, by one wave alone (no barrier). C of the tile lives in
// registers in the layout that serves both as the B operand of the Gram tiles
// and as the A operand of the carried-state product.
//
// Rows and columns past the chunk's end need no mask: their x and B were
// staged as zeros and their dt is 0, so every such entry is a finite value
// times 0, and a row past the end only reaches its own (unstored) output.
// STORE: adds the reverse pass's rows (add) and writes y; otherwise hands
// this direction's sums for the tile back in `out`.
// Y2: the forward stream's output goes to y2 (streams kept apart)
template <int Q, bool PACKED, int D, bool STORE = true, bool Y2 = false>
__device__ void row_tile(const SegArgs &a, const OutSmem<Q> &sm, int b, int h, int c0, int len,
                         int it, bool has_state, float Dh, bool add, const TileIn &tin,
                         f32x4 *out = nullptr) {
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    const uint16_t *bn = sm.bn;
    const int I = it >> 2, wq = it & 3;   // 64-row block, tile inside it
    const int i = 16 * it + l16;          // this lane's row (G^T column)
    const int i0 = 16 * it + 4 * g4;      // first of this lane's output rows
    const bool full = 16 * it + 16 <= len;
    const u32x4 (&cr)[kN / 32] = tin.cr;
    const float rli = sm.rl2[i];
    const int sqi = PACKED ? sm.sq[i] : 0;
    f32x4 acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = zero4();

    // ---- 64-column blocks off the diagonal: M = G e^{cs_i - cs_r} v64_j,
    // r the block's edge nearest the diagonal (its last token in walking
    // order)
    const int nJ = D == 0 ? I : (len + 63) / 64 - 1 - I;
    const int Iw = D == 0 ? I : Q / 64 - 1 - I;   // walking-order block of the rows
    for (int q = 0; q < nJ; ++q) {
        const int J = D == 0 ? q : I + 1 + q;
        const int Jw = D == 0 ? J : Q / 64 - 1 - J;
        // e^{cs_i - cs_r} = e^{rl_i} e^{(sum of a over the blocks between)}, r
        // the column block's edge; every entry is at most e^{bt2}
        const float between = sm.bt2[Iw][Jw];
        if (between < kDead * kLog2e) continue;   // every entry is exactly 0
        const float u64 = exp2_(rli + between);
        const bool lo = !Cfg<Q>::ONE_ROUND || between > kOneRound;   // else one rounding suffices
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            uint32_t ph[4], pl[4] = {0u, 0u, 0u, 0u};
            f32x4 gp[2];
            gram_pair(bn, 64 * J + 32 * kk, 64 * J + 32 * kk + 16, cr, gp[0], gp[1]);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j0 = 64 * J + 32 * kk + 16 * half;
                const f32x4 gg = gp[half];
                const int jb = j0 + 4 * g4;
                const f32x4 vv = *(const f32x4 *)(sm.v64 + jb);
                float mv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) mv[r] = gg[r] * (u64 * vv[r]);
                seq_mask<Q, PACKED>(mv, sm, jb, sqi);
                if (lo) {
                    split2(mv[0], mv[1], ph[2 * half], pl[2 * half]);
                    split2(mv[2], mv[3], ph[2 * half + 1], pl[2 * half + 1]);
                } else {
                    ph[2 * half] = pack2(mv[0], mv[1]);
                    ph[2 * half + 1] = pack2(mv[2], mv[3]);
                }
            }
            mx_step(acc, sm.xs, 64 * J + 32 * kk, u32x4{ph[0], ph[1], ph[2], ph[3]},
                    u32x4{pl[0], pl[1], pl[2], pl[3]}, lo);
        }
    }
    switch (wq) {
        case 0: diag_block<Q, PACKED, D, 0>(acc, sm, cr, I, i, rli, sqi); break;
        case 1: diag_block<Q, PACKED, D, 1>(acc, sm, cr, I, i, rli, sqi); break;
        case 2: diag_block<Q, PACKED, D, 2>(acc, sm, cr, I, i, rli, sqi); break;
        default: diag_block<Q, PACKED, D, 3>(acc, sm, cr, I, i, rli, sqi); break;
    }


    // ---- carried state: e^{cs_i} C_i . H (tiles it does not reach: skipped, exact)
    if (has_state && sm.utile[it]) {
        const uint16_t *hh = sm.hs;
        const uint16_t *hl = hh + kP * kNRS;
        // the tile's largest factor is that of its first row in walking order
        const bool lo = !Cfg<Q>::ONE_ROUND || sm.cs2[D == 0 ? 16 * it : 16 * it + 15] > kOneRound;
        f32x4 tt[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) tt[pt] = zero4();
        if (lo) {
#pragma unroll
            for (int ks = 0; ks < kN / 32; ++ks) {
                u32x4 oh[4], ol[4];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int o = (16 * pt + l16) * kNRS + 32 * ks + 8 * g4;
                    oh[pt] = *(const u32x4 *)(hh + o);
                    ol[pt] = *(const u32x4 *)(hl + o);
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) tt[pt] = mfma16x16x32(cr[ks], oh[pt], tt[pt]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) tt[pt] = mfma16x16x32(cr[ks], ol[pt], tt[pt]);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < kN / 32; ++ks) {
                u32x4 oh[4];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    oh[pt] = *(const u32x4 *)(hh + (16 * pt + l16) * kNRS + 32 * ks + 8 * g4);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) tt[pt] = mfma16x16x32(cr[ks], oh[pt], tt[pt]);
            }
        }
        const f32x4 c4 = *(const f32x4 *)(sm.cs2 + i0);
        float uu[4];
        if (PACKED) {
            const int4 s4 = *(const int4 *)(sm.sq + i0);
            const int nb = sm.sq_nb;
            uu[0] = s4.x == nb ? exp2_(c4[0]) : 0.f;
            uu[1] = s4.y == nb ? exp2_(c4[1]) : 0.f;
            uu[2] = s4.z == nb ? exp2_(c4[2]) : 0.f;
            uu[3] = s4.w == nb ? exp2_(c4[3]) : 0.f;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) uu[r] = exp2_(c4[r]);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] = fmaf(uu[r], tt[pt][r], acc[pt][r]);
    }

    // ---- skip term (x exact) and output rows i0 + r
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
        // x of rows i0..i0+3, column 16 pt + l16 (one transposing read)
        const u32x2 xv = ld_tr(sm.xs + (i0 + (l16 >> 2)) * kXS + 16 * pt + 4 * (l16 & 3));
        acc[pt][0] = fmaf(Dh, b_lo(xv[0]), acc[pt][0]);
        acc[pt][1] = fmaf(Dh, b_hi(xv[0]), acc[pt][1]);
        acc[pt][2] = fmaf(Dh, b_lo(xv[1]), acc[pt][2]);
        acc[pt][3] = fmaf(Dh, b_hi(xv[1]), acc[pt][3]);
    }
    if constexpr (!STORE) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) out[pt] = acc[pt];
        return;
    }
    if (add) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] += tin.prev[pt][r];
    }
    float *ybase = (Y2 ? a.y2 : a.y) + (tok(a, b, c0) * a.H + h) * kP + l16;
    const uint32_t ystride = (uint32_t)(a.H * kP);
    uint32_t yoff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) yoff[r] = (uint32_t)min(i0 + r, len - 1) * ystride;
    if (full) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) ybase[yoff[r] + 16 * pt] = acc[pt][r];
    } else {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (i0 + r < len) ybase[yoff[r] + 16 * pt] = acc[pt][r];
    }
}

// Row tiles of wave w: pairs whose column counts add up to the same total,
// and the two waves of a SIMD (w, w+4) get equal shares.
template <int Q>
__device__ __forceinline__ int tile_of(int w, int k) {
    if (Q == 256) return k == 0 ? 15 - w : w;
    if (Q == 128) return k == 0 ? (w < 4 ? w : 11 - w) : -1;
    return k == 0 && w < 4 ? w : -1;
}

// H <- gamma H + sum over the chunk's tokens of w_t B_t x_t^T (the wave's
// block of the state). B^T and x come straight from the staged natural tiles
// through transposing reads: no barrier.
template <int Q, bool PACKED, bool PF = true, int WB = 0>
__device__ void chunk_state_update(const OutSmem<Q> &sm, f32x4 (&Hacc)[Cfg<Q>::NQ], int len,
                                   bool math, ChunkLoads<Q, PACKED, WB> &nxt) {
    constexpr int NQ = Cfg<Q>::NQ;
    const int w = wave_in<WB>();
    const int pq = w & 3, nbase = NQ * (w >> 2);
    if (math) {
        const float gmm = sm.gamma;
#pragma unroll
        for (int q = 0; q < NQ; ++q) Hacc[q] *= gmm;
    }
#pragma unroll
    for (int sb = 0; sb < Q / kSub; ++sb) {
        // a slice of the next chunk's loads per sub-block, so the memory
        // pipeline works beside the matrix cores
        if (PF) nxt.part(sb, Q / kSub);
        if (!math || kSub * sb >= len || !sm.wsub[sb]) continue;   // every weight is exactly 0
        // both 32-token halves' operands first, then their products
        u32x4 aop[kSub / 32][NQ], bhi[kSub / 32], blo[kSub / 32];
#pragma unroll
        for (int ks = 0; ks < kSub / 32; ++ks)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                aop[ks][q] = tr_operand_bn(sm.bn, kSub * sb + 32 * ks, 16 * (nbase + q));
        const bool lo = !Cfg<Q>::ONE_ROUND || sm.wbig[sb];   // else one rounding suffices
#pragma unroll
        for (int ks = 0; ks < kSub / 32; ++ks)
            wx_operand(sm.xs, kSub * sb + 32 * ks, 16 * pq, sm.w, bhi[ks], blo[ks], lo);
#pragma unroll
        for (int ks = 0; ks < kSub / 32; ++ks) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) Hacc[q] = mfma16x16x32(aop[ks][q], bhi[ks], Hacc[q]);
            if (lo) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) Hacc[q] = mfma16x16x32(aop[ks][q], blo[ks], Hacc[q]);
            }
        }
    }
}

// One direction's walk over the segment's chunks (by the Cfg<Q>::NW waves
// starting at wave WB).
template <int Q, bool PACKED, int D, bool SP, bool Y2 = false, int WB = 0>
__device__ void seg_pass(const SegArgs &a, OutSmem<Q> &sm, int b, int seg, int h, int grp, bool add) {
    constexpr int NQ = Cfg<Q>::NQ;
    const int lane = lane_id(), w = wave_in<WB>(), g4 = lane >> 4, l16 = lane & 15;
    const int pq = w & 3, nbase = NQ * (w >> 2);
    const int t0 = seg * a.Ts, t1 = min(t0 + a.Ts, a.L);
    const int cfirst = t0 / Q, clast = (t1 - 1) / Q;
    const size_t PN = (size_t)kP * kN;
    auto slot = [&](int d, int k) { return (((size_t)b * 2 + d) * a.nseg + k) * a.H + h; };
    const int hoff = (16 * pq + l16) * kN + 16 * nbase + 4 * g4;   // + 16 q: this lane's state entries
    const DirPtrs &dp = a.dir[D];
    const float Dh = dp.D ? dp.D[h] : 0.f;
    // incoming state of this segment in the walking direction
    const float *src = nullptr;
    if (D == 0) {
        // several segments: the first one reads the copy k_seg_scan made of
        // the incoming state (final_state may alias init_state, and the last
        // segment's workgroup writes it during this launch)
        if (seg == 0) src = a.init_state ? (a.nseg > 1 ? a.Hs + slot(0, 0) * PN
                                                        : a.init_state + ((size_t)b * a.H + h) * PN)
                                         : nullptr;
        else src = a.gam[slot(0, seg - 1)] == 0.f ? a.S + slot(0, seg - 1) * PN : a.Hs + slot(0, seg) * PN;
    } else {
        if (seg == a.nseg - 1) src = nullptr;
        else src = a.gam[slot(1, seg + 1)] == 0.f ? a.S + slot(1, seg + 1) * PN : a.Hs + slot(1, seg) * PN;
    }
    const int nch = clast - cfirst + 1;
    const bool want_final = D == 0 && seg == a.nseg - 1 && a.final_state;
    auto chunk_at = [&](int s, int &c0, int &len) {
        const int c = D == 0 ? cfirst + s : clast - s;
        c0 = c * Q;
        len = min(Q, a.L - c0);
    };
    // the first chunk's loads go out before the incoming state is read, so
    // the two round trips overlap
    ChunkLoads<Q, PACKED, WB> ld;
    {
        int c0, len;
        chunk_at(0, c0, len);
        ld.issue(a, D, b, h, grp, c0, len);
        if (Q != 256) tile_fetch<D>(ld.tin, a, b, h, grp, c0, len, tile_of<Q>(w, 0), add);
    }
    f32x4 Hacc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) Hacc[q] = src ? *(const f32x4 *)(src + hoff + 16 * q) : zero4();
    bool has_state = src != nullptr;
    if (has_state) publish_state<Q, WB>(sm, Hacc);
    for (int s = 0; s < nch; ++s) {
        int c0, len;
        chunk_at(s, c0, len);
        chunk_prep<Q, PACKED, WB, SP>(a, sm, ld, D, b, h, c0, len);
        if (Q == 256) {
            // two tiles per wave: each fetches its own inputs (holding them
            // through the state update would cost spills)
#pragma unroll 1
            for (int k = 0; k < 2; ++k) {
                const int it = tile_of<Q>(w, k);
                TileIn t;
                tile_fetch<D>(t, a, b, h, grp, c0, len, it, add);
                if (16 * it < len) row_tile<Q, PACKED, D, true, Y2>(a, sm, b, h, c0, len, it, has_state, Dh, add, t);
            }
        } else {
            const int it = tile_of<Q>(w, 0);
            if (it >= 0 && 16 * it < len)
                row_tile<Q, PACKED, D, true, Y2>(a, sm, b, h, c0, len, it, has_state, Dh, add, ld.tin);
        }
        const bool last = s == nch - 1;
        {
            // next chunk's loads, spread over the state update (the last chunk
            // re-reads its own: the loads stay unconditional, so the registers
            // they fill are dead across the row tiles)
            int c0n, lenn;
            chunk_at(last ? s : s + 1, c0n, lenn);
            ld.begin(a, D, b, h, grp, c0n, lenn);
            if (Q != 256) tile_fetch<D>(ld.tin, a, b, h, grp, c0n, lenn, tile_of<Q>(w, 0), add);
        }
        chunk_state_update<Q, PACKED, true, WB>(sm, Hacc, len, !last || want_final, ld);
        // every wave is done with this chunk's tiles and the published state
        lds_barrier();
        if (!last) {
            publish_state<Q, WB>(sm, Hacc);
            has_state = true;
        }
    }
    if (want_final) {
        float *fs = a.final_state + ((size_t)b * a.H + h) * PN;
#pragma unroll
        for (int q = 0; q < NQ; ++q) *(f32x4 *)(fs + hoff + 16 * q) = Hacc[q];
    }
}

template <int Q, bool PACKED, bool SP, bool SPLIT = false>
__global__ void __launch_bounds__(Cfg<Q>::NT) __attribute__((amdgpu_waves_per_eu(2)))
k_seg_out(const SegArgs a) {
    // XCD-aware order: consecutive workgroup ids go round-robin over the 8
    // XCDs, so XCD x runs ids x, x+8, x+16, ... It is given the contiguous
    // range [x*per, (x+1)*per) of the (row-segment, head) pairs in
    // head-fastest order: every XCD gets the same share, and the workgroups
    // that share one XCD's L2 mostly hold the same (row, segment), so its B
    // and C are read from HBM once.
    const int id = blockIdx.x;
    const int total = a.batch * a.nseg * a.H;
    const int per = (total + 7) / 8;
    const int lin = (id & 7) * per + (id >> 3);
    if (lin >= total) return;
    const int rs = lin / a.H, h = lin % a.H;     // (row, segment) index, head
    const int b = rs / a.nseg, seg = rs % a.nseg;
    const int grp = h / (a.H / a.G);
    __shared__ __attribute__((aligned(16))) OutSmem<Q> sm;
    if (a.ndir == 2) {
        // reverse first, then the forward pass adds its part
        seg_pass<Q, PACKED, 1, SP>(a, sm, b, seg, h, grp, false);
        if (SPLIT)
            seg_pass<Q, PACKED, 0, SP, true>(a, sm, b, seg, h, grp, false);
        else
            seg_pass<Q, PACKED, 0, SP>(a, sm, b, seg, h, grp, true);
    } else {
        seg_pass<Q, PACKED, 0, SP>(a, sm, b, seg, h, grp, false);
    }
}

// ------------------------------------------------------------ k_dual_out
// Rows of at most one 64-token chunk (the block-decode step), both
// directions at once: waves 0-3 run the reverse direction and waves 4-7 the
// forward one, each half with its own staged tiles, so that the two passes
// (and their memory latencies) overlap instead of running back to back. The
// reverse half leaves its tile sums in LDS; the forward half adds them and
// writes y. Both halves pass the same two workgroup barriers.
constexpr int kEX = kP + 4;   // row stride (floats) of the exchanged tile sums

struct DualSmem {
    OutSmem<64> half[2];   // [0] reverse, [1] forward
    alignas(16) float ex[64 * kEX];
};

// Output rows of row tile `it` (this lane: rows 16 it + 4 g4 + r, column
// 16 pt + l16): acc[pt][r].
__device__ __forceinline__ void store_tile(const SegArgs &a, int b, int h, int len, int it,
                                           const f32x4 (&acc)[4]) {
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    const int i0 = 16 * it + 4 * g4;
    float *ybase = a.y + (tok(a, b, 0) * a.H + h) * kP + l16;
    const uint32_t ystride = (uint32_t)(a.H * kP);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (i0 + r >= len) continue;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) ybase[(uint32_t)(i0 + r) * ystride + 16 * pt] = acc[pt][r];
    }
}

// D: the half's direction; WB: its first wave (0 for D = 1, 4 for D = 0)
template <int D, int WB, bool SP>
__device__ void dual_half(const SegArgs &a, OutSmem<64> &sm, float *ex, int b, int h, int grp) {
    constexpr int Q = 64, NQ = Cfg<Q>::NQ;
    const int lane = lane_id(), w = wave_in<WB>(), g4 = lane >> 4, l16 = lane & 15;
    const int len = a.L;
    const DirPtrs &dp = a.dir[D];
    const float Dh = dp.D ? dp.D[h] : 0.f;
    const size_t PN = (size_t)kP * kN;
    const int hoff = (16 * w + l16) * kN + 4 * g4;   // + 16 q: this lane's state entries
    // the carried state (the largest piece, needed first) goes out first
    f32x4 Hacc[NQ];
    const float *src = D == 0 && a.init_state ? a.init_state + ((size_t)b * a.H + h) * PN : nullptr;
#pragma unroll
    for (int q = 0; q < NQ; ++q) Hacc[q] = src ? *(const f32x4 *)(src + hoff + 16 * q) : zero4();
    ChunkLoads<Q, false, WB> ld;
    ld.issue(a, D, b, h, grp, 0, len);
    TileIn tin;
    tile_fetch<D>(tin, a, b, h, grp, 0, len, w, false);
    if (src) publish_state<Q, WB>(sm, Hacc);
    chunk_prep<Q, false, WB, SP>(a, sm, ld, D, b, h, 0, len);   // barrier 1
    f32x4 acc[4];
    const bool mine = 16 * w < len;
    if (mine)
        row_tile<Q, false, D, false>(a, sm, b, h, 0, len, w, src != nullptr, Dh, false, tin, acc);
    if (D == 1 && mine) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) ex[(16 * w + 4 * g4 + r) * kEX + 16 * pt + l16] = acc[pt][r];
    }
    lds_barrier();   // barrier 2: the reverse sums are in LDS
    if (D == 0) {
        // the committed state is updated and stored before the y stores: the
        // waits that the compiler places before reusing a store's registers
        // count every store in flight (one counter covers loads and stores),
        // so work after the y stores would first wait for them to land
        if (a.final_state) {
            chunk_state_update<Q, false, false, WB>(sm, Hacc, len, true, ld);
            float *fs = a.final_state + ((size_t)b * a.H + h) * PN;
#pragma unroll
            for (int q = 0; q < NQ; ++q) *(f32x4 *)(fs + hoff + 16 * q) = Hacc[q];
        }
        if (mine) {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pt][r] += ex[(16 * w + 4 * g4 + r) * kEX + 16 * pt + l16];
            store_tile(a, b, h, len, w, acc);
        }
    }
}

template <bool SP>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
k_dual_out(const SegArgs a) {
    // XCD-aware order as in k_seg_out
    const int id = blockIdx.x;
    const int total = a.batch * a.H;
    const int per = (total + 7) / 8;
    const int lin = (id & 7) * per + (id >> 3);
    if (lin >= total) return;
    const int b = lin / a.H, h = lin % a.H;
    const int grp = h / (a.H / a.G);
    __shared__ __attribute__((aligned(16))) DualSmem sm;
    if (wave_id() < 4) dual_half<1, 0, SP>(a, sm.half[0], sm.ex, b, h, grp);
    else dual_half<0, 4, SP>(a, sm.half[1], sm.ex, b, h, grp);
}

// ------------------------------------------------------------ k_pair_out
// The output kernel in fp16 matrix-core form: 64-token chunks, two heads of
// one group per workgroup of 8 waves (waves 0-3 serve the first head, 4-7
// the second), the reverse pass writing y and the forward pass adding its
// part, as in k_seg_out.
//
// Every product runs on v_mfma_f32_16x16x32_f16 with fp32 accumulation. x, B
// and C arrive as bf16 and are converted to fp16 as they are staged in LDS
// (exact for magnitudes in fp16's normal range); B and C are staged once for
// both heads. The operands computed on the way are rounded once to fp16 (11
// significant bits against bf16's 8): the decay-masked Gram matrix M, the
// carried state H and the weighted inputs w x -- except the 32 columns of M
// that hold the diagonal 16-tile, which the rows' own terms dominate: they
// are split into fp16 hi + lo. The skip term D x rides on the diagonal of M.
//
// Range: fp16 overflows at 65504. Each fp16 operand reaches an output or the
// state, so an operand that overflowed leaves a non-finite value in y or in
// the final state: the last pass sums its outputs per lane, and if a sum is
// not finite anywhere in the workgroup, the workgroup recomputes its segment
// for both heads with the split-bf16 path (seg_pass with 64-token chunks,
// fp32's range), which overwrites every output. final_state is written only
// after that check. Magnitudes below fp16's normal range (2^-14) keep an
// absolute error of at most 2^-25 per rounded value.
//
// Packed sequences: every product is masked by the tokens' sequence indices,
// except that a chunk whose tokens, and the token its carried state comes
// from, are all of one sequence (all but the few chunks holding a boundary)
// builds M with the unmasked code: every mask would pass there.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_h(float a, float b) {
    const f16x2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}
// v = hi + lo, both fp16, per pair of values
__device__ __forceinline__ void split_h(float v0, float v1, uint32_t &hi, uint32_t &lo) {
    const f16x2_t h = {(_Float16)v0, (_Float16)v1};
    hi = __builtin_bit_cast(uint32_t, h);
    const f16x2_t l = {(_Float16)(v0 - (float)h[0]), (_Float16)(v1 - (float)h[1])};
    lo = __builtin_bit_cast(uint32_t, l);
}
// a pair of bf16 (raw bits) as a pair of fp16
__device__ __forceinline__ uint32_t bf2h(uint32_t u) {
    return pk_h(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
__device__ __forceinline__ u32x4 bf2h4(u32x4 v) {
    return u32x4{bf2h(v[0]), bf2h(v[1]), bf2h(v[2]), bf2h(v[3])};
}
__device__ __forceinline__ uint32_t mul_h(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) * __builtin_bit_cast(f16x2_t, b));
}

// One chunk's scan results for one head.
struct PairScan {
    float cs2[64];         // inclusive scan of a in the walking direction, times log2(e)
    float w[64];           // state-update weights
    float v16[64];         // e^{cs(edge of the token's 16-tile) - cs} dt
    float dt[64];
    int sq[64];            // sequence index (packed)
    int utile[4];          // the carried state reaches some row of the 16-row tile
    int wsub;              // some weight of the chunk is nonzero
    float gamma;           // decay of the whole chunk (0: the state does not pass)
    int sq_nb;             // sequence index of the token the carried state comes from
    int uni;               // (packed) the chunk's tokens and that token are of one sequence
};

// fp32 value moved across lanes by a DPP control; lanes without a source (or
// outside ROWMASK) read 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xf, true));
}
// Inclusive fp32 scan over the wave's 64 lanes (as wave_scan_d).
__device__ __forceinline__ float wave_scan_f(float v) {
    v += dpp_f<0x111, 0xf>(v);   // row_shr:1
    v += dpp_f<0x112, 0xf>(v);   // row_shr:2
    v += dpp_f<0x114, 0xf>(v);   // row_shr:4
    v += dpp_f<0x118, 0xf>(v);   // row_shr:8
    v += dpp_f<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}
__device__ __forceinline__ float lane_f(float v, int src) {
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), src));
}

// The scans of one 64-token chunk [c0, c0+len) of direction d for head h by
// one wave; lane k holds the k-th token in walking order (position k forward,
// 63 - k reverse; positions past the end carry dt = 0). The sums of
// a = dt A are taken in log2 units in fp32: within 64 tokens every exponent
// used is a difference of two such sums whose error is a few ulps of at most
// 64 |a|, and where |a| is large enough for that to matter the only factors
// that survive have an exponent of exactly 0 (a token's own). A token's
// state-update weight is 2^(the sum of a after it) dt, that sum being the
// chunk's total minus the token's walking sum.
// A2: A_h log2(e); dtb: the step-size bias (with SP), both read once per pass.
template <bool PACKED, bool SP>
// With PACKED, sqv is the sequence index of the lane's token and sqn that of
// the token the carried state comes from (-1: none), both loaded with the
// step sizes.
__device__ __forceinline__ void pair_scans(const SegArgs &a, PairScan &sm, uint16_t dtv, int sqv,
                                           int sqn, float A2, float dtb, int d, int b, int c0,
                                           int len) {
    const int lane = lane_id();
    const int pos = d == 0 ? lane : 63 - lane;
    int sq_nb = 0, sq_edge = 0;
    bool has_nb = true;
    if (PACKED) {
        sq_nb = __builtin_amdgcn_readfirstlane(sqn);
        has_nb = sq_nb >= 0;
        // the chunk's outgoing edge: position len - 1 forward (lane len - 1),
        // position 0 backward (lane 63)
        sq_edge = __builtin_amdgcn_readlane(sqv, d == 0 ? len - 1 : 63);
    }
    const bool in = pos < len;
    float dtf = in ? bf2f(dtv) : 0.f;
    if (SP) dtf = in ? softplus_dt(dtf + dtb) : 0.f;
    const float cs = wave_scan_f(dtf * A2);
    const float total = lane_f(cs, 63);
    // the walking sum at the end of the lane's 16-tile (lane | 15)
    const float t0 = lane_f(cs, 15), t1 = lane_f(cs, 31), t2 = lane_f(cs, 47);
    const int row = lane >> 4;
    const float e16 = row == 0 ? t0 : row == 1 ? t1 : row == 2 ? t2 : total;
    sm.cs2[pos] = cs;
    sm.dt[pos] = dtf;
    if (PACKED) sm.sq[pos] = sqv;
    sm.v16[pos] = exp2_(e16 - cs) * dtf;
    const bool reach = in && (!PACKED || sqv == sq_nb) && cs >= kDead * kLog2e;
    const unsigned long long m = __ballot(reach);
    if (lane < 4) sm.utile[d == 0 ? lane : 3 - lane] = ((m >> (16 * lane)) & 0xffffull) != 0;
    float wt = 0.f;
    if (in && (!PACKED || sqv == sq_edge)) wt = exp2_(total - cs) * dtf;
    sm.w[pos] = wt;
    const bool nz = __ballot(wt != 0.f) != 0ull;
    // every token of the chunk in the sequence of its outgoing edge, and the
    // carried state (if any) from that sequence too: then every sequence mask
    // of the chunk's products passes, and the unmasked products give the
    // same values
    const bool uni = !PACKED || (__ballot(in && sqv != sq_edge) == 0ull && (!has_nb || sq_nb == sq_edge));
    if (lane == 0) {
        bool carry = true;
        if (PACKED) carry = has_nb && sq_nb == sq_edge;
        sm.gamma = carry ? exp2_(total) : 0.f;
        sm.sq_nb = PACKED ? sq_nb : 0;
        sm.wsub = nz;
        sm.uni = uni;
    }
}
// One chunk's staged inputs (fp16): B and C of the group, x of each head.
// Two of them alternate, so the next chunk is staged while this one is in use.
struct PairStage {
    alignas(16) uint16_t bn[bn_elems(64)];   // B [t][n], bn_row layout
    alignas(16) uint16_t cn[bn_elems(64)];   // C [t][n], bn_row layout
    alignas(16) uint16_t xs[2][64 * kXS];    // x [t][p] of each head
};
// The decay-masked Gram matrix M of each head as matrix-core operands: per
// 16-row tile, the fp16 images that its lanes hand to the product, for the
// 32-column pairs 0 and 1 (hi) and the residual (lo) of the pair holding the
// diagonal tile.
struct PairM {
    u32x4 op[4][3][64];   // [row tile][pair 0 hi, pair 1 hi, band lo][lane]
};
struct PairSmem {
    PairStage st[2];
    PairScan sc[2][2];    // [head][chunk parity]
    PairM m[2];           // [head]
    int bad[8];           // per wave: a non-finite output or state
};
union PairShared {
    PairSmem fast;
    OutSmem<64> slow[2];   // the split-bf16 recomputation, one per head
};

// Loads of one 64-token chunk, issued ahead of use: x of the half's head (two
// 16-byte pieces per thread of the half), B and C (two pieces each per thread
// of the workgroup), and for the half's scanning wave the step size (and
// sequence index) of the lane's token.
template <bool PACKED>
struct PairLoads {
    u32x4 xv[2], bv[2], cv[2];
    uint16_t dtv[1];
    int sqv[1], sqn[1];
    uint32_t ox[2], ob[2];   // element offsets of this thread's pieces in a whole chunk

    __device__ __forceinline__ void init(const SegArgs &a) {
        const int th = threadIdx.x & 255, tid = threadIdx.x;
        const uint32_t xstride = (uint32_t)(a.H * kP), bstride = (uint32_t)(a.G * kN);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = th + 256 * k;
            ox[k] = (uint32_t)(item >> 3) * xstride + 8 * (item & 7);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = tid + 512 * k;
            ob[k] = (uint32_t)(item >> 4) * bstride + 8 * (item & 15);
        }
    }
    // the step size (and sequence index) of the scanning wave's token; dt and
    // sq point at the chunk's first token (dt of the head). Every wave loads
    // (no branch for the compiler to move); a wave that does not scan (own
    // false) reads the first token in every lane, one cache line.
    __device__ __forceinline__ void issue_dt(const uint16_t *dt, const int32_t *sq, uint32_t dstride,
                                             int d, int len, bool own, bool has_nb) {
        const int pos = own ? min(d == 0 ? lane_id() : 63 - lane_id(), len - 1) : 0;
        dtv[0] = dt[(uint32_t)pos * dstride];
        if (PACKED) {
            sqv[0] = sq[pos];
            // the token the carried state comes from: before the chunk
            // forward, after it backward
            sqn[0] = has_nb ? sq[d == 0 ? -1 : len] : -1;
        } else {
            sqv[0] = sqn[0] = 0;
        }
    }
    // X: the chunk's first row of x for the half's head; Bm, Cm: of B and C
    // for the group
    // the same loads in two parts: x, and B with C (a partial chunk's rows
    // read clamped), so that a chunk's loads can go out at two points of the
    // previous chunk's work
    __device__ __forceinline__ void issue_x(const SegArgs &a, const uint16_t *X, int len) {
        const int th = threadIdx.x & 255;
        const uint32_t xstride = (uint32_t)(a.H * kP);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = th + 256 * k, row = item >> 3, cg = item & 7;
            xv[k] = len == 64 ? ld8(X + ox[k]) : ld8(X + (uint32_t)min(row, len - 1) * xstride + 8 * cg);
        }
    }
    __device__ __forceinline__ void issue_bc(const SegArgs &a, const uint16_t *Bm, const uint16_t *Cm, int len) {
        const int tid = threadIdx.x;
        const uint32_t bstride = (uint32_t)(a.G * kN);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = tid + 512 * k, row = item >> 4, cg = item & 15;
            const uint32_t o = len == 64 ? ob[k] : (uint32_t)min(row, len - 1) * bstride + 8 * cg;
            bv[k] = ld8(Bm + o);
            cv[k] = ld8(Cm + o);
        }
    }
    __device__ __forceinline__ void issue(const SegArgs &a, const uint16_t *X, const uint16_t *Bm,
                                          const uint16_t *Cm, int len) {
        const int th = threadIdx.x & 255, tid = threadIdx.x;
        if (len == 64) {
#pragma unroll
            for (int k = 0; k < 2; ++k) xv[k] = ld8(X + ox[k]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                bv[k] = ld8(Bm + ob[k]);
                cv[k] = ld8(Cm + ob[k]);
            }
            return;
        }
        // a partial chunk: rows past its end are read clamped (and staged as 0)
        const uint32_t xstride = (uint32_t)(a.H * kP), bstride = (uint32_t)(a.G * kN);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = th + 256 * k, row = item >> 3, cg = item & 7;
            xv[k] = ld8(X + (uint32_t)min(row, len - 1) * xstride + 8 * cg);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = tid + 512 * k, row = item >> 4, cg = item & 15;
            const uint32_t o = (uint32_t)min(row, len - 1) * bstride + 8 * cg;
            bv[k] = ld8(Bm + o);
            cv[k] = ld8(Cm + o);
        }
    }
    // converted to fp16 into the stage (x into the half's head); in a
    // partial chunk, rows at or past len as zeros, masked rather than
    // branched per row so that every lane passes the same waits (a whole
    // chunk, the uniform common case, is stored unmasked)
    __device__ __forceinline__ void store(PairStage &st, int half, int len) const {
        const int th = threadIdx.x & 255, tid = threadIdx.x;
        if (len == 64) {   // a whole chunk (a uniform branch): no row to zero
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int item = th + 256 * k, row = item >> 3, cg = item & 7;
                *(u32x4 *)(st.xs[half] + row * kXS + 8 * cg) = bf2h4(xv[k]);
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int item = tid + 512 * k, row = item >> 4, cg = item & 15;
                *(u32x4 *)(st.bn + bn_row(row) + 8 * cg) = bf2h4(bv[k]);
                *(u32x4 *)(st.cn + bn_row(row) + 8 * cg) = bf2h4(cv[k]);
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = th + 256 * k, row = item >> 3, cg = item & 7;
            *(u32x4 *)(st.xs[half] + row * kXS + 8 * cg) = bf2h4(xv[k]) & (row < len ? ~0u : 0u);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = tid + 512 * k, row = item >> 4, cg = item & 15;
            const uint32_t m = row < len ? ~0u : 0u;
            *(u32x4 *)(st.bn + bn_row(row) + 8 * cg) = bf2h4(bv[k]) & m;
            *(u32x4 *)(st.cn + bn_row(row) + 8 * cg) = bf2h4(cv[k]) & m;
        }
    }
};

// One unit of M: the 32-column pair KK of row tile WQ (16 rows) for both heads
// of the workgroup, from one Gram computation (B and C are the group's, shared
// by its heads); written to pm[e].op as matrix-core operands. 16-tiles on the
// far side of the diagonal are 0 (not written; their readers skip them); the
// others factor the decay through their edge nearest the diagonal; the
// diagonal tile takes one exponential per entry and D on its diagonal. The
// pair holding the diagonal tile is split into fp16 hi + lo, the other pair
// rounded once.
template <bool PACKED, int D, int WQ, int KK>
__device__ __forceinline__ void pair_munit(PairM (&pm)[2], const PairStage &st, const PairScan &s0,
                                           const PairScan &s1, const u32x4 (&cr)[kN / 32], int i,
                                           float td, float Dh0, float Dh1) {
    if constexpr (D == 0 ? 2 * KK > WQ : 2 * KK + 1 < WQ) {
        return;   // both tiles dead
    } else {
        const int lane = lane_id(), g4 = lane >> 4;
        constexpr bool live0 = D == 0 ? 2 * KK <= WQ : 2 * KK >= WQ;
        constexpr bool live1 = D == 0 ? 2 * KK + 1 <= WQ : 2 * KK + 1 >= WQ;
        constexpr bool band = KK == WQ / 2;
        f32x4 gp[2];
        if (live0 && live1) {
            gram_pair<true>(st.bn, 32 * KK, 32 * KK + 16, cr, gp[0], gp[1]);
        } else {
            gp[0] = live0 ? gram_tile<true>(st.bn, 32 * KK, cr) : zero4();
            gp[1] = live1 ? gram_tile<true>(st.bn, 32 * KK + 16, cr) : zero4();
        }
        // the sequence index is the token's, the same for both heads
        const int sqi = PACKED ? s0.sq[i] : 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const PairScan &sc = e == 0 ? s0 : s1;
            const float Dh = e == 0 ? Dh0 : Dh1;
            const float rli = sc.cs2[i];
            uint32_t ph[4], pl[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jt = 2 * KK + half;
                const int j0 = 16 * jt;
                float mv[4] = {0.f, 0.f, 0.f, 0.f};
                if (D == 0 ? jt <= WQ : jt >= WQ) {
                    const f32x4 gg = gp[half];
                    const int jb = j0 + 4 * g4;
                    if (jt != WQ) {
                        const float u16 = exp2_(rli - sc.cs2[D == 0 ? j0 + 15 : j0]);
                        const f32x4 vv = *(const f32x4 *)(sc.v16 + jb);
#pragma unroll
                        for (int r = 0; r < 4; ++r) mv[r] = gg[r] * (u16 * vv[r]);
                    } else {
                        // td = l16 - 4 g4 (row minus column of entry r = 0): the
                        // far side of the diagonal gets an exponent below -2^98
                        // (exactly 0 after exp2), the diagonal itself adds D
                        const f32x4 c4 = *(const f32x4 *)(sc.cs2 + jb);
                        const f32x4 d4 = *(const f32x4 *)(sc.dt + jb);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float off = D == 0 ? td - (float)r : (float)r - td;
                            const float far = fminf(off + 0.5f, 0.f) * 1e30f;
                            const float dg = fmaxf(1.f - fabsf(off), 0.f) * Dh;
                            mv[r] = fmaf(gg[r], exp2_((rli + far) - c4[r]) * d4[r], dg);
                        }
                    }
                    seq_mask<64, PACKED>(mv, sc, jb, sqi);
                }
                if (band) {
                    split_h(mv[0], mv[1], ph[2 * half], pl[2 * half]);
                    split_h(mv[2], mv[3], ph[2 * half + 1], pl[2 * half + 1]);
                } else {
                    ph[2 * half] = pk_h(mv[0], mv[1]);
                    ph[2 * half + 1] = pk_h(mv[2], mv[3]);
                }
            }
            pm[e].op[WQ][KK][lane] = u32x4{ph[0], ph[1], ph[2], ph[3]};
            if (band) pm[e].op[WQ][2][lane] = u32x4{pl[0], pl[1], pl[2], pl[3]};
        }
    }
}

// The wave's unit of M (row tile rt, column pair kk) into LDS for both heads.
template <bool PACKED, int D>
__device__ __forceinline__ void pair_mrows(PairM (&pm)[2], const PairStage &st, const PairScan &s0,
                                           const PairScan &s1, int rt, int kk, float Dh0, float Dh1) {
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    u32x4 cr[kN / 32];
#pragma unroll
    for (int ks = 0; ks < kN / 32; ++ks)
        cr[ks] = *(const u32x4 *)(st.cn + 16 * rt * kBS + bn_lane(l16) + 32 * ks + 8 * g4);
    const int i = 16 * rt + l16;
    const float td = (float)(l16 - 4 * g4);
    switch (2 * rt + kk) {
        case 0: pair_munit<PACKED, D, 0, 0>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
        case 1: pair_munit<PACKED, D, 0, 1>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
        case 2: pair_munit<PACKED, D, 1, 0>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
        case 3: pair_munit<PACKED, D, 1, 1>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
        case 4: pair_munit<PACKED, D, 2, 0>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
        case 5: pair_munit<PACKED, D, 2, 1>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
        case 6: pair_munit<PACKED, D, 3, 0>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
        default: pair_munit<PACKED, D, 3, 1>(pm, st, s0, s1, cr, i, td, Dh0, Dh1); break;
    }
}

// The wave's 16 columns p = 16 v .. 16 v + 15 of the outputs, for all four
// row tiles, are held transposed: acc[rt] lane (g4, l16) has row 16 rt + l16,
// columns 16 v + 4 g4 .. + 3, four consecutive floats of y. In memory the
// four 16-byte pieces of a row are taken by four consecutive lanes (one
// 64-byte run per lane quad, which the memory pipeline moves at full rate):
// lane (g4, 4 a + b) moves row 16 rt + 4 a + g4, columns 16 v + 4 b .. + 3,
// the piece that lane (b, 4 a + g4) holds -- the lane index with its bits
// 0-1 and 4-5 exchanged, a permutation that is its own inverse.
__device__ __forceinline__ f32x4 quad_swap(f32x4 x) {
    const int l = lane_id();
    const int src = 4 * ((l & 12) | ((l & 3) << 4) | ((l >> 4) & 3));
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x[r])));
    return y;
}
// the row of y that this lane moves for row tile rt
__device__ __forceinline__ int pair_mem_row(int rt) {
    const int l = lane_id();
    return 16 * rt + (l & 12) + (l >> 4);
}
// yb points at the chunk's first row of y for the head. The reverse pass's
// rows are read back (rows past the chunk's end read its last row).
__device__ __forceinline__ void pair_prev(f32x4 (&prev)[4], const float *yb, uint32_t ystride,
                                          int len, int v) {
    const int lane = lane_id();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int row = min(pair_mem_row(rt), len - 1);
        prev[rt] = *(const f32x4 *)(yb + (uint32_t)row * ystride + 16 * v + 4 * (lane & 3));
    }
}
// prev as loaded into the register layout of acc. The reverse pass leaves a
// whole chunk's rows unpermuted (each lane's pieces in the places that it
// moves: y between the passes is the kernel's own), so only a partial
// chunk's rows are permuted.
__device__ __forceinline__ void pair_prev_regs(f32x4 (&acc)[4], int len) {
    if (len < 64) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = quad_swap(acc[rt]);
    }
}

// acc += M x for the wave's columns: M from the operand images in LDS, x^T
// through transposing reads (the k order of the images). Every operand is
// read first (rows past the chunk's end included: computed, not stored).
template <int D>
__device__ __forceinline__ void pair_mx(f32x4 (&acc)[4], const PairM &pm, const uint16_t *xs, int v) {
    const int lane = lane_id();
    u32x4 xo[2], mo[4][3];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) xo[kk] = tr_operand(xs, kXS, 32 * kk, 16 * v);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const bool live = q == 2 || (D == 0 ? 2 * q <= rt : 2 * q + 1 >= rt);
            mo[rt][q] = live ? pm.op[rt][q][lane] : u32x4{0u, 0u, 0u, 0u};
        }
    // products grouped by operand, the row tiles' chains interleaved
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (q < 2 && (D == 0 ? 2 * q > rt : 2 * q + 1 < rt)) continue;
            acc[rt] = mfma16x16x32_f16(xo[q < 2 ? q : rt / 2], mo[rt][q], acc[rt]);
        }
}

// The state's part of the outputs for the wave's columns: acc[rt] +=
// e^{cs_i} C_i . H, H held in registers (Hacc; see pair_state_update) and
// handed to the matrix cores as fp16: lane group g4 holds n = 32 ks + 8 g4 ..
// + 7, the order of a plain C row read. Row tiles the state does not reach
// (u = 0) are computed and dropped.
template <bool PACKED>
__device__ __forceinline__ void pair_state_out(f32x4 (&acc)[4], const PairStage &st, const PairScan &sc,
                                               const f32x4 (&Hacc)[8]) {
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    u32x4 ho[kN / 32];
#pragma unroll
    for (int ks = 0; ks < kN / 32; ++ks) {
        const f32x4 h0 = Hacc[2 * ks], h1 = Hacc[2 * ks + 1];
        ho[ks] = u32x4{pk_h(h0[0], h0[1]), pk_h(h0[2], h0[3]), pk_h(h1[0], h1[1]), pk_h(h1[2], h1[3])};
    }
    // k steps outer, the four row tiles' chains interleaved (independent
    // products back to back); a k step's C operands are read a step ahead
    const uint16_t *cb = st.cn + bn_lane(l16) + 8 * g4;
    u32x4 co[2][4];
    f32x4 tt[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        co[0][rt] = *(const u32x4 *)(cb + 16 * rt * kBS);
        tt[rt] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < kN / 32; ++ks) {
        if (ks + 1 < kN / 32) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                co[(ks + 1) & 1][rt] = *(const u32x4 *)(cb + 16 * rt * kBS + 32 * (ks + 1));
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) tt[rt] = mfma16x16x32_f16(ho[ks], co[ks & 1][rt], tt[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int t = 16 * rt + l16;
        const float u = (!PACKED || sc.sq[t] == sc.sq_nb) ? exp2_(sc.cs2[t]) : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rt][r] = fmaf(u, tt[rt][r], acc[rt][r]);
    }
}

// The outputs (rows below len) into y; with `check`, their sum joins chk (a
// non-finite output makes it non-finite).
// With perm false (a whole chunk of the reverse pass, read back by the
// forward pass), the pieces are written unpermuted.
__device__ __forceinline__ void pair_store(float *yb, uint32_t ystride, const f32x4 (&out)[4], int len,
                                           int v, float &chk, bool check, bool perm) {
    const int lane = lane_id();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int row = pair_mem_row(rt);
        const f32x4 o = perm ? quad_swap(out[rt]) : out[rt];
        if (row < len) *(f32x4 *)(yb + (uint32_t)row * ystride + 16 * v + 4 * (lane & 3)) = o;
    }
    if (check) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            s0 += out[rt][0] + out[rt][1];
            s1 += out[rt][2] + out[rt][3];
        }
        chk += s0 + s1;
    }
}

// B^T as the A operand of the state update, rows n in the state's order: for
// tile nt = 2 ks + e, row m = 4 g + r is n = 32 ks + 8 g + 4 e + r (so that a
// lane group of the product holds 8 consecutive n of each 32). As
// tr_operand_bn with the lanes' column pointers spread accordingly.
__device__ __forceinline__ u32x4 tr_operand_bt(const uint16_t *bn, int t32, int nt) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, s = lane & 15;
    const uint16_t *p = bn + t32 * kBS + bn_lane(4 * g4 + (s >> 2)) + 32 * (nt >> 1) + 8 * (s & 3) +
                        4 * (nt & 1);
    const u32x2 a = ld_tr(p), b = ld_tr(p + 16 * kBS);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// H <- gamma H + sum over the chunk's tokens of w_t B_t x_t^T for the wave's
// columns p = 16 v .. 16 v + 15, all n: Hacc[nt][r] = H[n][p = 16 v + l16]
// with n = 32 (nt / 2) + 8 g4 + 4 (nt % 2) + r. B^T and x come from the stage
// through transposing reads, w x as packed fp16 products.
__device__ __forceinline__ void pair_state_update(const PairStage &st, int half, const PairScan &sc,
                                                  f32x4 (&Hacc)[8], int v) {
    // (uniform values, read as scalars)
    const float gmm = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(sc.gamma)));
    // a chunk whose decay is exactly 0 starts the new state from nothing
    // (assigned, not scaled: 0 times a non-finite state is not 0)
    if (gmm == 0.f) {
#pragma unroll
        for (int q = 0; q < 8; ++q) Hacc[q] = zero4();
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) Hacc[q] *= gmm;
    }
    if (!__builtin_amdgcn_readfirstlane(sc.wsub)) return;   // every weight is exactly 0
    const int g4 = lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const f32x4 w0 = *(const f32x4 *)(sc.w + 32 * ks + 4 * g4);        // k slots 0..3
        const f32x4 w1 = *(const f32x4 *)(sc.w + 32 * ks + 16 + 4 * g4);   // k slots 4..7
        const u32x4 wp = {pk_h(w0[0], w0[1]), pk_h(w0[2], w0[3]), pk_h(w1[0], w1[1]), pk_h(w1[2], w1[3])};
        const u32x4 xv = tr_operand(st.xs[half], kXS, 32 * ks, 16 * v);
        const u32x4 bx = {mul_h(xv[0], wp[0]), mul_h(xv[1], wp[1]), mul_h(xv[2], wp[2]), mul_h(xv[3], wp[3])};
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const u32x4 aop = tr_operand_bt(st.bn, 32 * ks, nt);
            Hacc[nt] = mfma16x16x32_f16(aop, bx, Hacc[nt]);
        }
    }
}

// Offset in a [p][n] state of this lane's entries of Hacc[nt] (4 consecutive n).
__device__ __forceinline__ int pair_hoff(int v, int nt) {
    const int lane = lane_id(), g4 = lane >> 4, l16 = lane & 15;
    return (16 * v + l16) * kN + 32 * (nt >> 1) + 8 * g4 + 4 * (nt & 1);
}

// One direction's walk over the segment's chunks for the half's head. Wave v
// of the half owns the 16 columns p = 16 v .. + 15 (of the outputs and of the
// state, which stays in its registers) and row tile rt of M, which it shares
// through LDS. Per chunk, between the two barriers: M's row tile, the state's
// part of the outputs and the state update (all from the stage and the
// registers); after the second: M x, the outputs, the next chunk's stage and
// scans. Returns the outgoing state in Hacc.
template <bool PACKED, int D, bool SP, bool ADD, bool Y2 = false>
__device__ __forceinline__ void pair_pass(const SegArgs &a, PairSmem &sm, int b, int seg, int h,
                                          int grp, int half, int v, f32x4 (&Hacc)[8],
                                          float &chk, bool check) {
    constexpr int Q = 64;
    // row tiles mirrored in the second half: the two waves of a SIMD (v and
    // v + 4) then carry 16-row tiles of complementary causal length
    const int rt = half == 0 ? v : 3 - v;
    const int t0 = seg * a.Ts, t1 = min(t0 + a.Ts, a.L);
    const int cfirst = t0 / Q, clast = (t1 - 1) / Q;
    const size_t PN = (size_t)kP * kN;
    auto slot = [&](int d, int k) { return (((size_t)b * 2 + d) * a.nseg + k) * a.H + h; };
    const DirPtrs &dp = a.dir[D];
    // D of the workgroup's two heads (2 hp, 2 hp + 1)
    const float Dh0 = dp.D ? dp.D[h & ~1] : 0.f, Dh1 = dp.D ? dp.D[h | 1] : 0.f;
    // the wave's unit of M: the first half takes the column pair every row
    // tile has, the second half the other pair of the mirrored row tile
    // (absent for two of its waves)
    const int kk = half == 0 ? (D == 0 ? 0 : 1) : (D == 0 ? 1 : 0);
    // incoming state of this segment in the walking direction (as seg_pass)
    const float *src = nullptr;
    if (D == 0) {
        if (seg == 0) src = a.init_state ? (a.nseg > 1 ? a.Hs + slot(0, 0) * PN
                                                        : a.init_state + ((size_t)b * a.H + h) * PN)
                                         : nullptr;
        else src = a.gam[slot(0, seg - 1)] == 0.f ? a.S + slot(0, seg - 1) * PN : a.Hs + slot(0, seg) * PN;
    } else {
        if (seg == a.nseg - 1) src = nullptr;
        else src = a.gam[slot(1, seg + 1)] == 0.f ? a.S + slot(1, seg + 1) * PN : a.Hs + slot(1, seg) * PN;
    }
    const int nch = clast - cfirst + 1;
    auto chunk_at = [&](int s, int &c0, int &len) {
        const int c = D == 0 ? cfirst + s : clast - s;
        c0 = c * Q;
        len = min(Q, a.L - c0);
    };
    PairLoads<PACKED> ld;
    ld.init(a);
    // the row's first token of x, dt, y for the head, of B, C for the group
    const size_t row0 = tok(a, b, 0);
    const uint32_t xstride = (uint32_t)(a.H * kP), bstride = (uint32_t)(a.G * kN);
    const uint16_t *xrow = (const uint16_t *)dp.x + (row0 * a.H + h) * kP;
    const uint16_t *brow = (const uint16_t *)dp.B + (row0 * a.G + grp) * kN;
    const uint16_t *crow = (const uint16_t *)dp.C + (row0 * a.G + grp) * kN;
    const uint16_t *dtrow = (const uint16_t *)dp.dt + row0 * a.H + h;
    const int32_t *sqrow = PACKED ? a.seq + row0 : nullptr;
    // (streams kept apart: the forward pass writes y2)
    float *yrow = ((Y2 && D == 0) ? a.y2 : a.y) + (row0 * a.H + h) * kP;
    auto issue = [&](int c0, int len) {
        ld.issue(a, xrow + (size_t)c0 * xstride, brow + (size_t)c0 * bstride,
                 crow + (size_t)c0 * bstride, len);
    };
    // the scans run on the wave with the shortest row tile
    const bool scanner = rt == 0;
    auto issue_dt = [&](int c0, int len) {
        ld.issue_dt(dtrow + (size_t)c0 * a.H, PACKED ? sqrow + c0 : nullptr, (uint32_t)a.H, D, len, scanner,
                    D == 0 ? c0 > 0 : c0 + len < a.L);
    };
    const float A2 = dp.A[h] * kLog2e;
    const float dtb = SP && a.dt_bias[D] ? a.dt_bias[D][h] : 0.f;
    f32x4 acc[4];   // the outputs of the wave's columns (pair_prev's layout)
    {
        int c0, len;
        chunk_at(0, c0, len);
        issue(c0, len);
        issue_dt(c0, len);
        if (ADD) pair_prev(acc, yrow + (size_t)c0 * xstride, xstride, len, v);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) Hacc[q] = src ? *(const f32x4 *)(src + pair_hoff(v, q)) : zero4();
    for (int s = 0; s < nch; ++s) {
        int c0, len;
        chunk_at(s, c0, len);
        PairStage &st = sm.st[s & 1];
        PairScan &sc = sm.sc[half][s & 1];
        // stage and scans of chunk s: the buffers were last read two chunks
        // ago, before the previous chunk's first barrier
        ld.store(st, half, len);
        if (scanner) pair_scans<PACKED, SP>(a, sc, ld.dtv[0], ld.sqv[0], ld.sqn[0], A2, dtb, D, b, c0, len);
        const bool last = s == nch - 1;
        int c0n, lenn;
        chunk_at(last ? s : s + 1, c0n, lenn);
        lds_barrier();   // chunk s staged and scanned
        // the next chunk's loads (the last chunk re-reads its own) land during
        // this chunk's work: x and the step sizes now, B and C after the
        // carried state's term (all eight waves issuing all of them at once
        // after the barrier held every wave up in the memory pipeline)
        ld.issue_x(a, xrow + (size_t)c0n * xstride, lenn);
        issue_dt(c0n, lenn);
        if (ADD) {
            pair_prev_regs(acc, len);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = zero4();
        }
        // straight-line code, so that the scheduler can interleave the three:
        // a row tile past the chunk's end is computed (not read), the state's
        // part is taken with a zero state before the first update, and the
        // last chunk's update is kept (its result unused unless final)
        // (packed rows: a chunk inside one sequence builds M unmasked)
        if (!PACKED || __builtin_amdgcn_readfirstlane(sm.sc[0][s & 1].uni))
            pair_mrows<false, D>(sm.m, st, sm.sc[0][s & 1], sm.sc[1][s & 1], rt, kk, Dh0, Dh1);
        else
            pair_mrows<PACKED, D>(sm.m, st, sm.sc[0][s & 1], sm.sc[1][s & 1], rt, kk, Dh0, Dh1);
        pair_state_out<PACKED>(acc, st, sc, Hacc);
        ld.issue_bc(a, brow + (size_t)c0n * bstride, crow + (size_t)c0n * bstride, lenn);
        pair_state_update(st, half, sc, Hacc, v);
        lds_barrier();   // every row tile of M written
        pair_mx<D>(acc, sm.m[half], st.xs[half], v);
        // the reverse pass of two writes y for the forward pass to read back
        // (in the lanes' own order; a final output in memory order)
        pair_store(yrow + (size_t)c0 * xstride, xstride, acc, len, v, chk, check, D == 0 || Y2 || len < 64);
        if (ADD) pair_prev(acc, yrow + (size_t)c0n * xstride, xstride, lenn, v);
    }
}

// The split-bf16 recomputation of one head's segment by the four waves from
// WB. Kept out of line (it runs only after an fp16 overflow, and inlined its
// registers would crowd the fast path's), with the arguments copied: a
// reference to the kernel's arguments would move them to private memory for
// the fast path too.
template <bool PACKED, bool SP, int WB, bool Y2 = false>
__device__ __attribute__((noinline)) void pair_exact(const SegArgs a, OutSmem<64> &sm, int b, int seg, int h, int grp) {
    if (a.ndir == 2) {
        seg_pass<64, PACKED, 1, SP, false, WB>(a, sm, b, seg, h, grp, false);
        seg_pass<64, PACKED, 0, SP, Y2, WB>(a, sm, b, seg, h, grp, !Y2);
    } else {
        seg_pass<64, PACKED, 0, SP, false, WB>(a, sm, b, seg, h, grp, false);
    }
}

// Both passes of the fp16 form (NDIR directions); returns the forward
// direction's outgoing state in Hacc and the check sum of the last pass in chk
// (of both passes with the streams kept apart, Y2: each is an output then).
template <bool PACKED, bool SP, int NDIR, bool Y2 = false>
__device__ __forceinline__ void pair_fast(const SegArgs &a, PairSmem &sm, int b, int seg, int h,
                                          int grp, int half, int v, f32x4 (&Hacc)[8], float &chk) {
    if (NDIR == 2) {
        pair_pass<PACKED, 1, SP, false, Y2>(a, sm, b, seg, h, grp, half, v, Hacc, chk, Y2);
        pair_pass<PACKED, 0, SP, !Y2, Y2>(a, sm, b, seg, h, grp, half, v, Hacc, chk, true);
    } else {
        pair_pass<PACKED, 0, SP, false>(a, sm, b, seg, h, grp, half, v, Hacc, chk, true);
    }
}

// NDIR (the number of directions, a.ndir) is a template argument: with it a
// run-time branch, both passes share live ranges across it and the
// register allocator spills the state.
template <bool PACKED, bool SP, int NDIR, bool Y2 = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
k_pair_out(const SegArgs a) {
    // XCD-aware order as in k_seg_out, over (row-segment, head pair)
    const int id = blockIdx.x;
    const int HP = a.H / 2;
    const int total = a.batch * a.nseg * HP;
    const int per = (total + 7) / 8;
    const int lin = (id & 7) * per + (id >> 3);
    if (lin >= total) return;
    const int rs = lin / HP, hp = lin % HP;
    const int b = rs / a.nseg, seg = rs % a.nseg;
    // the wave index as a scalar: head, row tile and roles are then uniform
    // to the compiler (scalar loads of the per-head parameters, scalar branches)
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    const int half = wave >> 2, v = wave & 3;
    const int h = 2 * hp + half;
    // the wave with the shorter row tile of each SIMD's pair issues first
    // (it carries the scans and runs on the critical path between barriers)
    if ((half == 0 ? v : 3 - v) < 2) __builtin_amdgcn_s_setprio(1);
    const int grp = (2 * hp) / (a.H / a.G);
    __shared__ __attribute__((aligned(16))) PairShared sh;
    f32x4 Hacc[8];
    float chk = 0.f;
    pair_fast<PACKED, SP, NDIR, Y2>(a, sh.fast, b, seg, h, grp, half, v, Hacc, chk);
    const bool want_final = seg == a.nseg - 1 && a.final_state;
    if (want_final) {
#pragma unroll
        for (int q = 0; q < 8; ++q) chk += (Hacc[q][0] + Hacc[q][1]) + (Hacc[q][2] + Hacc[q][3]);
    }
    const unsigned long long bad = __ballot(!__builtin_isfinite(chk));
    if (lane_id() == 0) sh.fast.bad[wave] = bad != 0ull;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) any |= sh.fast.bad[w];
    if (!any) {
        if (want_final) {
            float *fs = a.final_state + ((size_t)b * a.H + h) * (kP * kN);
#pragma unroll
            for (int q = 0; q < 8; ++q) *(f32x4 *)(fs + pair_hoff(v, q)) = Hacc[q];
        }
        return;
    }
    // an fp16 operand overflowed: recompute the segment of both heads exactly
    lds_barrier();   // every wave has read the flags before the memory is reused
    if (half == 0) pair_exact<PACKED, SP, 0, Y2>(a, sh.slow[0], b, seg, h, grp);
    else pair_exact<PACKED, SP, 4, Y2>(a, sh.slow[1], b, seg, h, grp);
}

size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of segment length ts: the segment states S, Hs and the carry
// factors when a row has more than one segment.
size_t seg_workspace(int batch, int L, int H, long ts) {
    const size_t nseg = (size_t)((L + ts - 1) / ts);
    if (nseg <= 1) return 0;   // one segment per row: no segment states
    const size_t st = (size_t)batch * 2 * nseg * H * (size_t)(kP * kN) * 4;
    return al256(st) * 2 + al256((size_t)batch * 2 * nseg * H * 4);
}

// Segment length: a multiple of the chunk chosen for the output kernel's
// time, estimated as (rounds of 256 workgroups, one per CU) x (the segment's
// tokens + 256 tokens' worth of per-workgroup overhead), ties to the longer
// segment: long segments mean fewer segment states to write, scan and read,
// and the segment pass stops reading a segment once its decay has
// underflowed, but a partial last round of workgroups costs as much as a
// full one. The candidates are, for each segment count n, the shortest
// multiple of the chunk that cuts a row into n segments (so a row whose
// length is not a power of two can still fill whole rounds); counts are
// tried until they would need eight rounds. With a workspace limit, the
// length is then doubled until the segment states fit in it (a whole row is
// one segment and needs none).
int pick_ts(int batch, int L, int H, int Q, size_t limit) {
    const long pairs = (long)batch * ((H + 1) / 2);
    const long nmax = ((long)L + Q - 1) / Q;
    long ts = Q, best_cost = -1;
    for (long n = 1; n <= nmax && (n == 1 || pairs * n <= 8L * 256); ++n) {
        long t = ((long)L + n - 1) / n;
        t = (t + Q - 1) / Q * Q;
        const long segs = ((long)L + t - 1) / t;
        if (segs != n) continue;   // the same length as a smaller count
        const long rounds = (pairs * segs + 255) / 256;
        const long cost = rounds * (t + 256);
        if (best_cost < 0 || cost < best_cost || (cost == best_cost && t > ts)) {
            ts = t;
            best_cost = cost;
        }
    }
    while (ts < L && seg_workspace(batch, L, H, ts) > limit) ts *= 2;
    return (int)(ts < L ? ts : (L > Q ? L : Q));
}

// The pair kernel serves two heads of one group per workgroup.
bool pair_ok(const SegArgs &a) { return a.H % 2 == 0 && (a.H / a.G) % 2 == 0; }

template <bool SP, bool Y2 = false>
hipError_t launch_pair(const SegArgs &a, hipStream_t s) {
    if (a.nseg > 1) {
        BM_LAUNCH("ssd_seg_state", k_seg_state<SP>, dim3(a.nseg, a.ndir, a.batch * a.H), dim3(kThreads), 0,
                  s, a);
        BM_LAUNCH("ssd_seg_scan", k_seg_scan, dim3(kP * kN / 256, a.H, a.batch * a.ndir), dim3(256), 0,
                  s, a);
    }
    const int per_xcd = (a.batch * a.nseg * (a.H / 2) + 7) / 8;
    const dim3 grid(per_xcd * 8), block(512);
    if (Y2) {   // (both directions)
        if (a.seq) BM_LAUNCH("ssd_pair_out", (k_pair_out<true, SP, 2, true>), grid, block, 0, s, a);
        else BM_LAUNCH("ssd_pair_out", (k_pair_out<false, SP, 2, true>), grid, block, 0, s, a);
    } else if (a.seq) {
        if (a.ndir == 2) BM_LAUNCH("ssd_pair_out", (k_pair_out<true, SP, 2>), grid, block, 0, s, a);
        else BM_LAUNCH("ssd_pair_out", (k_pair_out<true, SP, 1>), grid, block, 0, s, a);
    } else {
        if (a.ndir == 2) BM_LAUNCH("ssd_pair_out", (k_pair_out<false, SP, 2>), grid, block, 0, s, a);
        else BM_LAUNCH("ssd_pair_out", (k_pair_out<false, SP, 1>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <int Q, bool SP, bool SPLIT = false>
hipError_t launch_q(const SegArgs &a, hipStream_t s) {
    const int nd = a.ndir;
    if (a.nseg > 1) {
        BM_LAUNCH("ssd_seg_state", k_seg_state<SP>, dim3(a.nseg, nd, a.batch * a.H), dim3(kThreads), 0,
                  s, a);
        BM_LAUNCH("ssd_seg_scan", k_seg_scan, dim3(kP * kN / 256, a.H, a.batch * nd), dim3(256), 0,
                  s, a);
    }
    const int per_xcd = (a.batch * a.nseg * a.H + 7) / 8;
    // one chunk per row: both directions at once, except for committing
    // steps over many (row, head) pairs, where the segment kernel (both
    // directions in turn, two workgroups per CU) measured 3-7 % faster
    const bool many_commit = a.final_state && (long)a.batch * a.H >= 320;
    if (Q == 64 && a.ndir == 2 && !a.seq && a.L <= 64 && !SPLIT && !many_commit) {
        BM_LAUNCH("ssd_dual_out", k_dual_out<SP>, dim3(per_xcd * 8), dim3(512), 0, s, a);
        return hipGetLastError();
    }
    if (a.seq)
        BM_LAUNCH("ssd_seg_out", (k_seg_out<Q, true, SP, SPLIT>), dim3(per_xcd * 8), dim3(Cfg<Q>::NT), 0, s, a);
    else
        BM_LAUNCH("ssd_seg_out", (k_seg_out<Q, false, SP, SPLIT>), dim3(per_xcd * 8), dim3(Cfg<Q>::NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool chunked_supported(const Problem &p) {
    return p.bf16 && p.P == kP && p.N == kN && p.L > 0 &&
           (p.Q == 64 || p.Q == 128 || p.Q == 256);
}

size_t chunked_workspace(int batch, int L, int H, int G, int Q, size_t limit) {
    (void)G;
    return seg_workspace(batch, L, H, pick_ts(batch, L, H, Q, limit));
}

hipError_t launch_chunked(const Problem &p, void *ws, size_t limit, hipStream_t s) {
    SegArgs a;
    a.dir[0] = p.dir[0];
    a.dir[1] = p.dir[1];
    a.ndir = p.has_bwd ? 2 : 1;
    a.batch = p.batch; a.L = p.L; a.H = p.H; a.G = p.G;
    a.nC = (p.L + p.Q - 1) / p.Q;
    a.Ts = pick_ts(p.batch, p.L, p.H, p.Q, limit);
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
    a.dt_bias[0] = p.dt_bias[0];
    a.dt_bias[1] = p.dt_bias[1];
    a.y2 = p.y2;
    const bool sp = p.dt_softplus;
    // the fp16 pair kernel, except for rows of one 64-token chunk with both
    // directions (the block step), which k_dual_out serves in one pass
    const bool dual = p.Q == 64 && a.ndir == 2 && !a.seq && a.L <= 64;
    // streams kept apart (no softplus step size in that mode): the pair
    // kernel as for the summed output, else the exact kernels
    if (p.y2) {
        if (sp || a.ndir != 2) return hipErrorInvalidValue;
        if (pair_ok(a) && !dual) return launch_pair<false, true>(a, s);
        switch (p.Q) {
            case 64: return launch_q<64, false, true>(a, s);
            case 128: return launch_q<128, false, true>(a, s);
            case 256: return launch_q<256, false, true>(a, s);
        }
        return hipErrorInvalidValue;
    }
    if (pair_ok(a) && !dual) return sp ? launch_pair<true>(a, s) : launch_pair<false>(a, s);
    switch (p.Q) {
        case 64: return sp ? launch_q<64, true>(a, s) : launch_q<64, false>(a, s);
        case 128: return sp ? launch_q<128, true>(a, s) : launch_q<128, false>(a, s);
        case 256: return sp ? launch_q<256, true>(a, s) : launch_q<256, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace bm
