// Token-sequential bidirectional SSD scan.
//
// One workgroup per (sequence or segment, head), one lane per headdim column
// p; lane p keeps column p of the d_state x headdim state in registers and
// applies the Mamba-2 recurrence one token at a time:
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
    float *tot;               // [batch][2][nseg][H] total of a over the segment
    int dt_softplus;          // dt holds the pre-activation: softplus(dt + bias)
    const float *dt_bias[2];  // [H] per direction, or nullptr (zero)
    float *y2;                // streams kept apart: the forward stream's output
};

template <int N>
struct SeqSmem {
    float B[kSeqTile][N];
    float C[kSeqTile][N];
    float x[kSeqTile][kMaxP];
    float y[kSeqTile][kMaxP];
    float dt[kSeqTile];
};

// Walks tokens [t0, t1) of one direction (upwards for d == 0, downwards for
// d == 1) from the state in st and returns the sum of dt*A over them.
// MODE 0: state only; MODE 1: writes y; MODE 2: adds into y. y goes through
// LDS a tile at a time (the old values of a MODE 2 tile are read with the
// inputs), so no token waits on a global load.
template <typename T, int N, int MODE>
__device__ float walk(const SeqArgs &a, SeqSmem<N> &sm, int d, size_t row_tok, int h, int g,
                      int t0, int t1, float (&st)[N]) {
    // the output this direction writes (or adds into)
    float *Y = (a.y2 && d == 0) ? a.y2 : a.y;
    const int p = threadIdx.x;
    const int H = a.H, P = a.P, G = a.G;
    const DirPtrs &dp = a.dir[d];
    const T *X = (const T *)dp.x;
    const T *DT = (const T *)dp.dt;
    const T *Bm = (const T *)dp.B;
    const T *Cm = (const T *)dp.C;
    const float Ah = dp.A[h];
    const float Dh = dp.D ? dp.D[h] : 0.f;
    const int len = t1 - t0;
    float asum = 0.f;
    for (int base = 0; base < len; base += kSeqTile) {
        const int nsteps = len - base < kSeqTile ? len - base : kSeqTile;
        __syncthreads();
        for (int i = threadIdx.x; i < nsteps * N; i += blockDim.x) {
            const int s = i / N, n = i - s * N;
            const int t = d == 0 ? t0 + base + s : t1 - 1 - base - s;
            const size_t o = ((row_tok + t) * G + g) * N + n;
            sm.B[s][n] = Elem<T>::load(Bm, o);
            if (MODE != 0) sm.C[s][n] = Elem<T>::load(Cm, o);
        }
        for (int i = threadIdx.x; i < nsteps * P; i += blockDim.x) {
            const int s = i / P, pp = i - s * P;
            const int t = d == 0 ? t0 + base + s : t1 - 1 - base - s;
            const size_t o = ((row_tok + t) * H + h) * P + pp;
            sm.x[s][pp] = Elem<T>::load(X, o);
            if (MODE == 2) sm.y[s][pp] = Y[o];
        }
        for (int i = threadIdx.x; i < nsteps; i += blockDim.x) {
            const int t = d == 0 ? t0 + base + i : t1 - 1 - base - i;
            float dtv = Elem<T>::load(DT, (row_tok + t) * H + h);
            if (a.dt_softplus) dtv = softplus_dt(dtv + (a.dt_bias[d] ? a.dt_bias[d][h] : 0.f));
            sm.dt[i] = dtv;
        }
        __syncthreads();
        if (p < P) {
            for (int s = 0; s < nsteps; ++s) {
                const float dtt = sm.dt[s];
                const float at = dtt * Ah;
                asum += at;
                const float decay = expf(at);
                const float xv = sm.x[s][p];
                const float dx = dtt * xv;
                float acc = 0.f;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    st[n] = fmaf(decay, st[n], dx * sm.B[s][n]);
                    if (MODE != 0) acc = fmaf(sm.C[s][n], st[n], acc);
                }
                if (MODE == 1) sm.y[s][p] = fmaf(Dh, xv, acc);
                if (MODE == 2) sm.y[s][p] += fmaf(Dh, xv, acc);
            }
        }
        if (MODE != 0) {
            __syncthreads();
            for (int i = threadIdx.x; i < nsteps * P; i += blockDim.x) {
                const int s = i / P, pp = i - s * P;
                const int t = d == 0 ? t0 + base + s : t1 - 1 - base - s;
                Y[((row_tok + t) * H + h) * P + pp] = sm.y[s][pp];
            }
        }
    }
    return asum;
}

// Whole rows or packed sequences: one workgroup per (unit, head).
template <typename T, int N>
__global__ void __launch_bounds__(kMaxP) k_scan_seq(const SeqArgs a) {
    __shared__ SeqSmem<N> sm;
    const int unit = blockIdx.x;
    const int h = blockIdx.y;
    const int p = threadIdx.x;
    const int g = h / (a.H / a.G);
    int row, t0, t1;
    if (a.cu) { row = 0; t0 = a.cu[unit]; t1 = a.cu[unit + 1]; }
    else      { row = unit; t0 = 0; t1 = a.L; }
    const size_t row_tok = (size_t)row * a.L;
    const size_t state_off = (((size_t)unit * a.H + h) * a.P + p) * N;
    float st[N];
    if (a.init_state && p < a.P) {
#pragma unroll
        for (int n = 0; n < N; ++n) st[n] = a.init_state[state_off + n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) st[n] = 0.f;
    }
    walk<T, N, 1>(a, sm, 0, row_tok, h, g, t0, t1, st);
    if (a.final_state && p < a.P) {
#pragma unroll
        for (int n = 0; n < N; ++n) a.final_state[state_off + n] = st[n];
    }
    if (a.ndir == 2) {
#pragma unroll
        for (int n = 0; n < N; ++n) st[n] = 0.f;
        if (a.y2) walk<T, N, 1>(a, sm, 1, row_tok, h, g, t0, t1, st);
        else walk<T, N, 2>(a, sm, 1, row_tok, h, g, t0, t1, st);
    }
}

__device__ __forceinline__ size_t seg_slot(const SeqArgs &a, int row, int d, int seg, int h) {
    return (((size_t)row * 2 + d) * a.nseg + seg) * a.H + h;
}

// Pass 1: every segment from a zero state; its outgoing state and sum of a.
template <typename T, int N>
__global__ void __launch_bounds__(kMaxP) k_seq_seg_state(const SeqArgs a) {
    __shared__ SeqSmem<N> sm;
    const int seg = blockIdx.x, h = blockIdx.y;
    const int row = blockIdx.z / a.ndir, d = blockIdx.z % a.ndir;
    const int p = threadIdx.x;
    const int g = h / (a.H / a.G);
    const int t0 = seg * a.seg_len, t1 = min(t0 + a.seg_len, a.L);
    float st[N];
#pragma unroll
    for (int n = 0; n < N; ++n) st[n] = 0.f;
    const float asum = walk<T, N, 0>(a, sm, d, (size_t)row * a.L, h, g, t0, t1, st);
    const size_t slot = seg_slot(a, row, d, seg, h);
    if (p < a.P) {
#pragma unroll
        for (int n = 0; n < N; ++n) a.S[(slot * a.P + p) * N + n] = st[n];
    }
    if (p == 0) a.tot[slot] = asum;
}

// Pass 2: incoming state of every segment, one thread per state element,
// sequential over the segments in the walking direction.
template <int N>
__global__ void __launch_bounds__(256) k_seq_seg_scan(const SeqArgs a) {
    const int e = blockIdx.x * 256 + threadIdx.x;   // p * N + n
    const int h = blockIdx.y;
    const int row = blockIdx.z / a.ndir, d = blockIdx.z % a.ndir;
    const int PN = a.P * N;
    if (e >= PN) return;
    float hv = 0.f;
    if (d == 0 && a.init_state) hv = a.init_state[((size_t)row * a.H + h) * PN + e];
    for (int s = 0; s < a.nseg; ++s) {
        const int k = d == 0 ? s : a.nseg - 1 - s;
        const size_t slot = seg_slot(a, row, d, k, h);
        a.Hin[slot * PN + e] = hv;
        hv = fmaf(expf(a.tot[slot]), hv, a.S[slot * PN + e]);
    }
    if (d == 0 && a.final_state) a.final_state[((size_t)row * a.H + h) * PN + e] = hv;
}

// Pass 3: every segment from its incoming state, both directions, y.
template <typename T, int N>
__global__ void __launch_bounds__(kMaxP) k_seq_seg_out(const SeqArgs a) {
    __shared__ SeqSmem<N> sm;
    const int seg = blockIdx.x, h = blockIdx.y, row = blockIdx.z;
    const int p = threadIdx.x;
    const int g = h / (a.H / a.G);
    const int t0 = seg * a.seg_len, t1 = min(t0 + a.seg_len, a.L);
    const size_t row_tok = (size_t)row * a.L;
    for (int d = 0; d < a.ndir; ++d) {
        const size_t slot = seg_slot(a, row, d, seg, h);
        float st[N];
        if (p < a.P) {
#pragma unroll
            for (int n = 0; n < N; ++n) st[n] = a.Hin[(slot * a.P + p) * N + n];
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) st[n] = 0.f;
        }
        if (d == 0 || a.y2) walk<T, N, 1>(a, sm, d, row_tok, h, g, t0, t1, st);
        else walk<T, N, 2>(a, sm, 1, row_tok, h, g, t0, t1, st);
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

template <typename T, int N>
static hipError_t launch_typed(const SeqArgs &a, int units, hipStream_t s) {
    const int threads = ((a.P + 63) / 64) * 64;
    if (a.nseg <= 1) {
        BM_LAUNCH("scan_seq", (k_scan_seq<T, N>), dim3(units, a.H), dim3(threads), 0, s, a);
    } else {
        BM_LAUNCH("seq_seg_state", (k_seq_seg_state<T, N>), dim3(a.nseg, a.H, a.batch * a.ndir),
                  dim3(threads), 0, s, a);
        BM_LAUNCH("seq_seg_scan", (k_seq_seg_scan<N>), dim3((a.P * N + 255) / 256, a.H, a.batch * a.ndir),
                  dim3(256), 0, s, a);
        BM_LAUNCH("seq_seg_out", (k_seq_seg_out<T, N>), dim3(a.nseg, a.H, a.batch), dim3(threads), 0,
                  s, a);
    }
    return hipGetLastError();
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
