// Token-sequential bidirectional SSD scan.
//
// One workgroup per (sequence or segment, head), LPP lanes per headdim column
// p (LPP = 4 for headdim <= 16, 2 for <= 32, else 1, so that a wave's lanes
// are used); the LPP lanes of column p keep its d_state entries in registers,
// N / LPP each, and apply the Mamba-2 recurrence one token at a time:
//   h <- exp(dt_t*A_h) h + dt_t B_t x_t[p],   y_t[p] = C_t . h + D_h x_t[p]
// forward over the sequence, then backward over it with the reverse stream's
// parameters: the flip of the DiffuMamba blog's bidirectional block ("network
// architecture") done by walking the indices downwards. Inputs are staged
// through LDS a tile of tokens at a time.
//
// This is the fp32 path (exact fp32 arithmetic, no chunking, so no cumsum
// cancellation) and the path for shapes the matrix-core kernels do not cover.
//
// Long rows with few (row, head) pairs are cut into segments so that the GPU
// has enough workgroups: k_seq_seg_state runs each segment from a zero state
// and keeps its outgoing state and total decay, k_seq_seg_scan chains those
// into each segment's incoming state, and k_seq_seg_out reruns every segment
// from its incoming state, writing y. The chaining is the same linear
// recurrence applied a segment at a time (h_out = e^{sum a} h_in + S).
#include "common.hpp"
#include "internal.hpp"

namespace bm {

constexpr int kSeqTile = 32;   // tokens staged per LDS tile
constexpr int kMaxP = 128;

struct SeqArgs {
    DirPtrs dir[2];
    int ndir;
    int batch, L, H, P, G;
    int seg_len, nseg;        // segments of each row (nseg == 1: whole rows)
    const int32_t *cu;        // packed offsets (device) or nullptr
    const float *init_state;
    float *final_state;
    float *y;
    float *S;                 // [batch][2][nseg][H][P][N] segment states from zero
    float *Hin;               // [batch][2][nseg][H][P][N] segment incoming states
    float *tot;               // [batch][2][nseg][H] e^{total of a over the segment}
    int dt_softplus;          // dt holds the pre-activation: softplus(dt + bias)
    const float *dt_bias[2];  // [H] per direction, or nullptr (zero)
    float *y2;                // streams kept apart: the forward stream's output
};

// A tile's inputs and outputs for headdim up to PM (small heads leave room
// for more workgroups per CU).
template <int N, int PM>
struct SeqSmem {
    // (16-byte aligned rows: a lane's run of state entries is one wide read)
    alignas(16) float B[kSeqTile][N];
    alignas(16) float C[kSeqTile][N];
    alignas(16) float x[kSeqTile][PM];
    alignas(16) float y[kSeqTile][PM];
    float dt[kSeqTile];
    float at[kSeqTile];    // dt * A
    float dec[kSeqTile];   // exp(dt * A)
};

// The headdim bound PM a launch is compiled for (16, 32, 64 or 128: the
// tiles' width), and its lanes per headdim column.
inline int seq_pm(int P) { return P <= 16 ? 16 : P <= 32 ? 32 : P <= 64 ? 64 : kMaxP; }
template <int PM>
struct SeqLPP {
    static constexpr int value = PM <= 16 ? 4 : PM <= 32 ? 2 : 1;
};

// Sum over the LPP consecutive lanes of a column, in its last lane (DPP row
// shifts within a 16-lane row; LPP divides 16, so a column's lanes share a
// row; the other lanes hold partial sums).
template <int LPP>
__device__ __forceinline__ float col_sum(float v) {
    if (LPP >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    if (LPP >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    return v;
}

// Whether a walk prefetches the next tile into registers: one-wave
// workgroups (headdim bound up to 64) whose prefetch registers (B, and C, x,
// and the old y as the mode needs them) number at most 80 per lane.
template <int N, int PM, int MODE>
constexpr bool pf_fits() {
    return PM <= 64 && (kSeqTile * N / 64) * (MODE != 0 ? 2 : 1) + (kSeqTile * PM / 64) * (MODE == 2 ? 2 : 1) <= 80;
}

template <typename T, int N, int PM, int MODE>
__device__ float walk_pf(const SeqArgs &a, SeqSmem<N, PM> &sm, int d, size_t row_tok, int h, int g,
                         int t0, int t1, float (&st)[N / SeqLPP<PM>::value]);

// Walks tokens [t0, t1) of one direction (upwards for d == 0, downwards for
// d == 1) from the state in st and returns the sum of dt*A over them.
// MODE 0: state only; MODE 1: writes y; MODE 2: adds into y. y goes through
// LDS a tile at a time (the old values of a MODE 2 tile are read with the
// inputs), so no token waits on a global load.
template <typename T, int N, int PM, int MODE>
__device__ float walk(const SeqArgs &a, SeqSmem<N, PM> &sm, int d, size_t row_tok, int h, int g,
                      int t0, int t1, float (&st)[N / SeqLPP<PM>::value]) {
    // one-wave workgroups with small states fetch the next tile during this one
    if constexpr (pf_fits<N, PM, MODE>()) return walk_pf<T, N, PM, MODE>(a, sm, d, row_tok, h, g, t0, t1, st);
    constexpr int LPP = SeqLPP<PM>::value;
    constexpr int NL = N / LPP;            // state entries per lane
    constexpr int NA = NL >= 16 ? 4 : NL >= 8 ? 2 : 1;   // independent partial sums of y
    // the output this direction writes (or adds into)
    float *Y = (a.y2 && d == 0) ? a.y2 : a.y;
    const int H = a.H, P = a.P, G = a.G;
    // column p, entries q NL .. q NL + NL - 1 (lanes past the last column
    // compute on column P - 1 and write nothing)
    const int p = (int)threadIdx.x / LPP, q = (int)threadIdx.x % LPP;
    const int pc = min(p, P - 1);
    const bool own = p < P && q == LPP - 1;
    const DirPtrs &dp = a.dir[d];
    const T *X = (const T *)dp.x;
    const T *DT = (const T *)dp.dt;
    const T *Bm = (const T *)dp.B;
    const T *Cm = (const T *)dp.C;
    const float Ah = dp.A[h];
    const float Dh = dp.D ? dp.D[h] : 0.f;
    const int len = t1 - t0;
    if (len <= 0) return 0.f;
    // the first token walked and the element strides of one token in the
    // walking direction (x and y are staged on the PM-column grid, so that
    // an element's token and column come from shifts)
    const size_t tfirst = row_tok + (d == 0 ? t0 : t1 - 1);
    const int sgn = d == 0 ? 1 : -1;
    const long stepB = (long)sgn * G * N, stepX = (long)sgn * H * P;
    const T *pB = Bm + (tfirst * G + g) * N;
    const T *pC = Cm + (tfirst * G + g) * N;
    const T *pX = X + (tfirst * H + h) * P;
    float *pY = Y + (tfirst * H + h) * P;
    float asum = 0.f;
    for (int base = 0; base < len; base += kSeqTile) {
        const int nsteps = len - base < kSeqTile ? len - base : kSeqTile;
        __syncthreads();
        for (int i = threadIdx.x; i < nsteps * N; i += blockDim.x) {
            const int s = i / N, n = i % N;
            const long o = (long)(base + s) * stepB + n;
            sm.B[s][n] = Elem<T>::load(pB + o, 0);
            if (MODE != 0) sm.C[s][n] = Elem<T>::load(pC + o, 0);
        }
        for (int i = threadIdx.x; i < nsteps * PM; i += blockDim.x) {
            const int s = i / PM, pp = i % PM;
            if (pp >= P) continue;
            const long o = (long)(base + s) * stepX + pp;
            sm.x[s][pp] = Elem<T>::load(pX + o, 0);
            if (MODE == 2) sm.y[s][pp] = pY[o];
        }
        // the step sizes and decays of the tile, in parallel (off the
        // token-to-token chain)
        for (int i = threadIdx.x; i < nsteps; i += blockDim.x) {
            const int t = d == 0 ? t0 + base + i : t1 - 1 - base - i;
            float dtv = Elem<T>::load(DT, (row_tok + t) * H + h);
            if (a.dt_softplus) dtv = softplus_dt(dtv + (a.dt_bias[d] ? a.dt_bias[d][h] : 0.f));
            sm.dt[i] = dtv;
            const float at = dtv * Ah;
            sm.at[i] = at;
            sm.dec[i] = expf(at);
        }
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
            // the token's operands first (reads in flight together), then
            // the arithmetic
            float bv[NL], cv[NL];
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                bv[i] = sm.B[s][q * NL + i];
                cv[i] = MODE != 0 ? sm.C[s][q * NL + i] : 0.f;
            }
            const float decay = sm.dec[s];
            asum += sm.at[s];
            const float xv = sm.x[s][pc];
            const float dx = sm.dt[s] * xv;
            float acc[NA];
#pragma unroll
            for (int k = 0; k < NA; ++k) acc[k] = 0.f;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                st[i] = fmaf(decay, st[i], dx * bv[i]);
                if (MODE != 0) acc[i % NA] = fmaf(cv[i], st[i], acc[i % NA]);
            }
            if (MODE != 0) {
                float yv = acc[0];
#pragma unroll
                for (int k = 1; k < NA; ++k) yv += acc[k];
                yv = col_sum<LPP>(yv);
                if (own) {
                    if (MODE == 1) sm.y[s][p] = fmaf(Dh, xv, yv);
                    if (MODE == 2) sm.y[s][p] += fmaf(Dh, xv, yv);
                }
            }
        }
        if (MODE != 0) {
            __syncthreads();
            for (int i = threadIdx.x; i < nsteps * PM; i += blockDim.x) {
                const int s = i / PM, pp = i % PM;
                if (pp < P) pY[(long)(base + s) * stepX + pp] = sm.y[s][pp];
            }
        }
    }
    return asum;
}

// walk for headdim bounds up to 64 (one wave of 64 lanes: PM columns of LPP
// lanes) when the prefetch registers fit (pf_fits): the same arithmetic, with
// the next tile's inputs (B, C, x, dt, and the old y when adding) loaded into
// registers while this tile's tokens are walked, so that a tile does not
// start with a round trip to memory. Each lane keeps elements of token rows
// (B, C: element lane + 64 k of the tile's rows; x, y: column lane % PM of
// token lane / PM) and reaches the k-th token it handles by a stride from
// its first one; token indices past the tile's end are clamped onto its last
// token, so every load is in bounds and unconditional, and the LDS rows (or
// columns past headdim) they fill are never read.
template <typename T, int N, int PM, int MODE>
__device__ float walk_pf(const SeqArgs &a, SeqSmem<N, PM> &sm, int d, size_t row_tok, int h, int g,
                         int t0, int t1, float (&st)[N / SeqLPP<PM>::value]) {
    static_assert(PM * SeqLPP<PM>::value == 64 && pf_fits<N, PM, MODE>(), "one-wave tiles");
    constexpr int LPP = SeqLPP<PM>::value;
    constexpr int NL = N / LPP;
    constexpr int NA = NL >= 16 ? 4 : NL >= 8 ? 2 : 1;
    constexpr int KB = kSeqTile * N / 64;              // B, C: elements per lane
    constexpr int RX = 64 / PM, KX = kSeqTile / RX;    // x, y: tokens per pass, passes
    float *Y = (a.y2 && d == 0) ? a.y2 : a.y;
    const int H = a.H, P = a.P, G = a.G;
    const int lane = (int)threadIdx.x;
    const int p = lane / LPP, q = lane % LPP;
    const int pc = min(p, P - 1);
    const bool own = p < P && q == LPP - 1;
    const DirPtrs &dp = a.dir[d];
    const float Ah = dp.A[h];
    const float Dh = dp.D ? dp.D[h] : 0.f;
    const float dtb = a.dt_softplus && a.dt_bias[d] ? a.dt_bias[d][h] : 0.f;
    const int len = t1 - t0;
    if (len <= 0) return 0.f;
    // the first token walked and the element strides of one token in the
    // walking direction
    const size_t tfirst = row_tok + (d == 0 ? t0 : t1 - 1);
    const int sgn = d == 0 ? 1 : -1;
    const int sx = lane / PM, cx = lane % PM, px = min(cx, P - 1);
    const long stepB = (long)sgn * G * N, stepX = (long)sgn * H * P, stepD = (long)sgn * H;
    const T *pB = (const T *)dp.B + (tfirst * G + g) * N;
    const T *pC = (const T *)dp.C + (tfirst * G + g) * N;
    const T *pX = (const T *)dp.x + (tfirst * H + h) * P + px;
    const float *pY = Y + (tfirst * H + h) * P + px;
    const T *pD = (const T *)dp.dt + tfirst * H + h;
    float rb[KB], rc[KB], rx[KX], ry[KX], rdt;
    auto fetch = [&](int base) {
        const int last = min(len - base, kSeqTile) - 1;
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            // element lane + 64 k: token (lane + 64 k) / N, entry (lane + 64 k) % N
            const int i = lane + 64 * k;
            const long o = (long)(base + min(i / N, last)) * stepB + i % N;
            rb[k] = Elem<T>::load(pB + o, 0);
            if (MODE != 0) rc[k] = Elem<T>::load(pC + o, 0);
        }
#pragma unroll
        for (int k = 0; k < KX; ++k) {
            const long o = (long)(base + min(sx + RX * k, last)) * stepX;
            rx[k] = Elem<T>::load(pX + o, 0);
            if (MODE == 2) ry[k] = pY[o];
        }
        rdt = Elem<T>::load(pD + (long)(base + min(lane, last)) * stepD, 0);
    };
    float asum = 0.f;
    // (adding: the rows of y the other direction wrote, by other lanes, are
    // read after a barrier)
    __syncthreads();
    fetch(0);
    for (int base = 0; base < len; base += kSeqTile) {
        const int nsteps = min(len - base, kSeqTile);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int i = lane + 64 * k;
            sm.B[i / N][i % N] = rb[k];
            if (MODE != 0) sm.C[i / N][i % N] = rc[k];
        }
#pragma unroll
        for (int k = 0; k < KX; ++k) {
            sm.x[sx + RX * k][cx] = rx[k];
            if (MODE == 2) sm.y[sx + RX * k][cx] = ry[k];
        }
        if (lane < kSeqTile) {
            float dtv = rdt;
            if (a.dt_softplus) dtv = softplus_dt(dtv + dtb);
            sm.dt[lane] = dtv;
            const float at = dtv * Ah;
            sm.at[lane] = at;
            sm.dec[lane] = expf(at);
        }
        __syncthreads();
        if (base + kSeqTile < len) fetch(base + kSeqTile);
        for (int s = 0; s < nsteps; ++s) {
            float bv[NL], cv[NL];
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                bv[i] = sm.B[s][q * NL + i];
                cv[i] = MODE != 0 ? sm.C[s][q * NL + i] : 0.f;
            }
            const float decay = sm.dec[s];
            asum += sm.at[s];
            const float xv = sm.x[s][pc];
            const float dx = sm.dt[s] * xv;
            float acc[NA];
#pragma unroll
            for (int k = 0; k < NA; ++k) acc[k] = 0.f;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                st[i] = fmaf(decay, st[i], dx * bv[i]);
                if (MODE != 0) acc[i % NA] = fmaf(cv[i], st[i], acc[i % NA]);
            }
            if (MODE != 0) {
                float yv = acc[0];
#pragma unroll
                for (int k = 1; k < NA; ++k) yv += acc[k];
                yv = col_sum<LPP>(yv);
                if (own) {
                    if (MODE == 1) sm.y[s][p] = fmaf(Dh, xv, yv);
                    if (MODE == 2) sm.y[s][p] += fmaf(Dh, xv, yv);
                }
            }
        }
        if (MODE != 0) {
            __syncthreads();
            float *Yt = Y + (tfirst * H + h) * P + cx;
#pragma unroll
            for (int k = 0; k < KX; ++k) {
                const int s = sx + RX * k;
                if (cx < P && s < nsteps) Yt[(long)(base + s) * stepX] = sm.y[s][cx];
            }
        }
    }
    return asum;
}

// The lane's state entries: column p, entries q NL .. q NL + NL - 1 of the
// [P][N] state at base (lanes past the last column hold zeros, write nothing).
template <int N, int LPP>
__device__ __forceinline__ void state_load(float (&st)[N / LPP], const float *base, int P) {
    constexpr int NL = N / LPP;
    const int p = (int)threadIdx.x / LPP, q = (int)threadIdx.x % LPP;
#pragma unroll
    for (int i = 0; i < NL; ++i) st[i] = (base && p < P) ? base[(size_t)p * N + q * NL + i] : 0.f;
}
template <int N, int LPP>
__device__ __forceinline__ void state_store(const float (&st)[N / LPP], float *base, int P) {
    constexpr int NL = N / LPP;
    const int p = (int)threadIdx.x / LPP, q = (int)threadIdx.x % LPP;
    if (p < P) {
#pragma unroll
        for (int i = 0; i < NL; ++i) base[(size_t)p * N + q * NL + i] = st[i];
    }
}

// Whole rows or packed sequences: one workgroup per (unit, head).
template <typename T, int N, int PM>
__global__ void __launch_bounds__(kMaxP) k_scan_seq(const SeqArgs a) {
    __shared__ SeqSmem<N, PM> sm;
    constexpr int LPP = SeqLPP<PM>::value;
    const int unit = blockIdx.x;
    const int h = blockIdx.y;
    const int g = h / (a.H / a.G);
    int row, t0, t1;
    if (a.cu) { row = 0; t0 = a.cu[unit]; t1 = a.cu[unit + 1]; }
    else      { row = unit; t0 = 0; t1 = a.L; }
    const size_t row_tok = (size_t)row * a.L;
    const size_t state_off = ((size_t)unit * a.H + h) * a.P * N;
    float st[N / LPP];
    state_load<N, LPP>(st, a.init_state ? a.init_state + state_off : nullptr, a.P);
    walk<T, N, PM, 1>(a, sm, 0, row_tok, h, g, t0, t1, st);
    if (a.final_state) state_store<N, LPP>(st, a.final_state + state_off, a.P);
    if (a.ndir == 2) {
#pragma unroll
        for (int i = 0; i < N / LPP; ++i) st[i] = 0.f;
        if (a.y2) walk<T, N, PM, 1>(a, sm, 1, row_tok, h, g, t0, t1, st);
        else walk<T, N, PM, 2>(a, sm, 1, row_tok, h, g, t0, t1, st);
    }
}

__device__ __forceinline__ size_t seg_slot(const SeqArgs &a, int row, int d, int seg, int h) {
    return (((size_t)row * 2 + d) * a.nseg + seg) * a.H + h;
}

// Pass 1: every segment from a zero state; its outgoing state and decay
// (e to the sum of a).
template <typename T, int N, int PM>
__global__ void __launch_bounds__(kMaxP) k_seq_seg_state(const SeqArgs a) {
    __shared__ SeqSmem<N, PM> sm;
    constexpr int LPP = SeqLPP<PM>::value;
    const int seg = blockIdx.x, h = blockIdx.y;
    const int row = blockIdx.z / a.ndir, d = blockIdx.z % a.ndir;
    const int g = h / (a.H / a.G);
    const int t0 = seg * a.seg_len, t1 = min(t0 + a.seg_len, a.L);
    float st[N / LPP];
#pragma unroll
    for (int i = 0; i < N / LPP; ++i) st[i] = 0.f;
    const float asum = walk<T, N, PM, 0>(a, sm, d, (size_t)row * a.L, h, g, t0, t1, st);
    const size_t slot = seg_slot(a, row, d, seg, h);
    state_store<N, LPP>(st, a.S + slot * a.P * N, a.P);
    if (threadIdx.x == 0) a.tot[slot] = expf(asum);
}

// Pass 2: incoming state of every segment, one lane per state element and a
// run of consecutive segments (in the walking direction) per wave (one wave
// per 4 segments, at most kScanWaves; the launch's width): each wave
// folds its run from a zero state into the run's decay product and outgoing
// state, the runs' incoming states are chained through LDS (the same linear
// recurrence, a run at a time), and each wave reruns its segments from its
// run's incoming state, storing every segment's. Up to 32 segments' values
// are loaded before any is used, so that their loads are in flight together;
// their decays, the same in every lane, come one per lane (at clamped
// indices) and are read out lane by lane.
constexpr int kScanWaves = 16;

template <int N>
__global__ void __launch_bounds__(64 * kScanWaves) k_seq_seg_scan(const SeqArgs a) {
    constexpr int kB = 32;
    __shared__ float run_s[kScanWaves][64];
    __shared__ float run_t[kScanWaves];
    const int lane = (int)threadIdx.x & 63, w = (int)threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;   // p * N + n
    const int h = blockIdx.y;
    const int row = blockIdx.z / a.ndir, d = blockIdx.z % a.ndir;
    const int PN = a.P * N;
    // lanes past the last element work on a clamped one and store nothing
    const bool live = e < PN;
    const int ec = live ? e : PN - 1;
    const int nw = (int)blockDim.x >> 6;
    const int per = (a.nseg + nw - 1) / nw;
    const int s_begin = min(w * per, a.nseg), s_end = min(s_begin + per, a.nseg);
    auto slot_of = [&](int s) { return seg_slot(a, row, d, d == 0 ? s : a.nseg - 1 - s, h); };
    // walks the run from hv; stores each segment's incoming state if asked;
    // returns the product of the run's decays
    auto walk_run = [&](float &hv, bool store) {
        float tp = 1.f;
        for (int s0 = s_begin; s0 < s_end; s0 += kB) {
            float sv[kB];
#pragma unroll
            for (int k = 0; k < kB; ++k)
                if (s0 + k < s_end) sv[k] = a.S[slot_of(s0 + k) * PN + ec];
            const float tl = a.tot[slot_of(min(s0 + (lane & (kB - 1)), s_end - 1))];
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                if (s0 + k >= s_end) break;
                const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tl), k));
                if (store && live) a.Hin[slot_of(s0 + k) * PN + e] = hv;
                hv = fmaf(tv, hv, sv[k]);
                tp *= tv;
            }
        }
        return tp;
    };
    float hv = 0.f;
    const float tp = walk_run(hv, false);
    run_s[w][lane] = hv;
    if (lane == 0) run_t[w] = tp;
    __syncthreads();
    hv = d == 0 && a.init_state ? a.init_state[((size_t)row * a.H + h) * PN + ec] : 0.f;
    for (int v = 0; v < w; ++v) hv = fmaf(run_t[v], hv, run_s[v][lane]);
    walk_run(hv, true);
    if (live && d == 0 && a.final_state && s_begin < s_end && s_end == a.nseg)
        a.final_state[((size_t)row * a.H + h) * PN + e] = hv;
}

// Pass 3: every segment from its incoming state, both directions, y.
template <typename T, int N, int PM>
__global__ void __launch_bounds__(kMaxP) k_seq_seg_out(const SeqArgs a) {
    __shared__ SeqSmem<N, PM> sm;
    constexpr int LPP = SeqLPP<PM>::value;
    const int seg = blockIdx.x, h = blockIdx.y, row = blockIdx.z;
    const int g = h / (a.H / a.G);
    const int t0 = seg * a.seg_len, t1 = min(t0 + a.seg_len, a.L);
    const size_t row_tok = (size_t)row * a.L;
    for (int d = 0; d < a.ndir; ++d) {
        const size_t slot = seg_slot(a, row, d, seg, h);
        float st[N / LPP];
        state_load<N, LPP>(st, a.Hin + slot * a.P * N, a.P);
        if (d == 0 || a.y2) walk<T, N, PM, 1>(a, sm, d, row_tok, h, g, t0, t1, st);
        else walk<T, N, PM, 2>(a, sm, 1, row_tok, h, g, t0, t1, st);
    }
}

bool seq_supported(int P, int N) {
    return P >= 1 && P <= kMaxP && (N == 16 || N == 32 || N == 64 || N == 128);
}

namespace {

// Segment length for rows of L tokens: enough (row, head, segment)
// workgroups to fill the GPU, segments of at least 256 tokens.
int seq_seg_len(int batch, int L, int H) {
    const long pairs = (long)batch * H;
    if (pairs <= 0 || L <= 512) return L > 0 ? L : 1;
    long want = (2048 + pairs - 1) / pairs;                // segments per row
    const long most = L / 256;
    if (want > most) want = most;
    if (want <= 1) return L;
    long len = (L + want - 1) / want;
    len = (len + kSeqTile - 1) / kSeqTile * kSeqTile;
    return (int)len;
}

size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

size_t seq_workspace(int batch, int L, int H, int P, int N, bool packed) {
    if (packed) return 0;
    const int seg_len = seq_seg_len(batch, L, H);
    const size_t nseg = (L + seg_len - 1) / seg_len;
    if (nseg <= 1) return 0;
    const size_t st = (size_t)batch * 2 * nseg * H * P * N * 4;
    return 2 * al256(st) + al256((size_t)batch * 2 * nseg * H * 4);
}

template <typename T, int N, int PM>
static hipError_t launch_pm(const SeqArgs &a, int units, hipStream_t s) {
    constexpr int LPP = SeqLPP<PM>::value;
    const int threads = ((a.P * LPP + 63) / 64) * 64;
    if (a.nseg <= 1) {
        BM_LAUNCH("scan_seq", (k_scan_seq<T, N, PM>), dim3(units, a.H), dim3(threads), 0, s, a);
    } else {
        BM_LAUNCH("seq_seg_state", (k_seq_seg_state<T, N, PM>), dim3(a.nseg, a.H, a.batch * a.ndir),
                  dim3(threads), 0, s, a);
        const int nw = (a.nseg + 3) / 4 < kScanWaves ? (a.nseg + 3) / 4 : kScanWaves;
        BM_LAUNCH("seq_seg_scan", (k_seq_seg_scan<N>), dim3((a.P * N + 63) / 64, a.H, a.batch * a.ndir),
                  dim3(64 * nw), 0, s, a);
        BM_LAUNCH("seq_seg_out", (k_seq_seg_out<T, N, PM>), dim3(a.nseg, a.H, a.batch), dim3(threads), 0,
                  s, a);
    }
    return hipGetLastError();
}

template <typename T, int N>
static hipError_t launch_typed(const SeqArgs &a, int units, hipStream_t s) {
    switch (seq_pm(a.P)) {
        case 16: return launch_pm<T, N, 16>(a, units, s);
        case 32: return launch_pm<T, N, 32>(a, units, s);
        case 64: return launch_pm<T, N, 64>(a, units, s);
    }
    return launch_pm<T, N, kMaxP>(a, units, s);
}

template <typename T>
static hipError_t launch_n(const SeqArgs &a, int N, int units, hipStream_t s) {
    switch (N) {
        case 16: return launch_typed<T, 16>(a, units, s);
        case 32: return launch_typed<T, 32>(a, units, s);
        case 64: return launch_typed<T, 64>(a, units, s);
        case 128: return launch_typed<T, 128>(a, units, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scan_seq(const Problem &p, void *ws, hipStream_t s) {
    SeqArgs a;
    a.dir[0] = p.dir[0];
    a.dir[1] = p.dir[1];
    a.ndir = p.has_bwd ? 2 : 1;
    a.batch = p.batch; a.L = p.L; a.H = p.H; a.P = p.P; a.G = p.G;
    a.cu = p.cu_dev;
    a.init_state = p.init_state;
    a.final_state = p.final_state;
    a.y = p.y;
    a.dt_softplus = p.dt_softplus;
    a.y2 = p.y2;
    a.dt_bias[0] = p.dt_bias[0];
    a.dt_bias[1] = p.dt_bias[1];
    a.seg_len = p.L > 0 ? p.L : 1;
    a.nseg = 1;
    a.S = a.Hin = a.tot = nullptr;
    if (!p.cu_dev && ws && seq_workspace(p.batch, p.L, p.H, p.P, p.N, false) > 0) {
        a.seg_len = seq_seg_len(p.batch, p.L, p.H);
        a.nseg = (p.L + a.seg_len - 1) / a.seg_len;
        const size_t st = (size_t)p.batch * 2 * a.nseg * p.H * p.P * p.N * 4;
        char *w = (char *)ws;
        a.S = (float *)w;
        w += al256(st);
        a.Hin = (float *)w;
        w += al256(st);
        a.tot = (float *)w;
    }
    const int units = p.cu_dev ? p.nseq : p.batch;
    if (units == 0) return hipSuccess;
    return p.bf16 ? launch_n<uint16_t>(a, p.N, units, s) : launch_n<float>(a, p.N, units, s);
}

}  // namespace bm
