// Token-sequential bidirectional SSD scan.
//
// One workgroup per (sequence, head), one lane per headdim column p; lane p
// keeps column p of the d_state x headdim state in registers and applies the
// Mamba-2 recurrence one token at a time:
//   h <- exp(dt_t*A_h) h + dt_t B_t x_t[p],   y_t[p] = C_t . h + D_h x_t[p]
// first forward over the sequence (writing y), then backward over it with the
// reverse stream's parameters (adding into y): the flip of the DiffuMamba
// blog's bidirectional block ("network architecture") done by walking the
// indices downwards. Inputs are staged through LDS a tile of tokens at a time.
//
// This is the fp32 path (exact fp32 arithmetic, no chunking, so no cumsum
// cancellation) and the path for shapes the MFMA kernels do not cover.
#include "common.hpp"
#include "internal.hpp"

namespace bm {

constexpr int kSeqTile = 32;   // tokens staged per LDS tile
constexpr int kMaxP = 128;

struct SeqArgs {
    DirPtrs dir[2];
    int ndir;
    int L, H, P, G;
    const int32_t *cu;       // packed offsets (device) or nullptr
    const float *init_state;
    float *final_state;
    float *y;
};

template <typename T, int N>
__global__ void __launch_bounds__(kMaxP) k_scan_seq(const SeqArgs a) {
    const int unit = blockIdx.x;
    const int h = blockIdx.y;
    const int p = threadIdx.x;
    const int H = a.H, P = a.P, G = a.G, L = a.L;
    const int g = h / (H / G);
    int row, t0, t1;
    if (a.cu) { row = 0; t0 = a.cu[unit]; t1 = a.cu[unit + 1]; }
    else      { row = unit; t0 = 0; t1 = L; }
    const int len = t1 - t0;
    const size_t row_tok = (size_t)row * L;

    __shared__ float sB[kSeqTile][N];
    __shared__ float sC[kSeqTile][N];
    __shared__ float sx[kSeqTile][kMaxP];
    __shared__ float sdt[kSeqTile];

    float st[N];
    const size_t state_off = (((size_t)unit * H + h) * P + p) * N;

    for (int d = 0; d < a.ndir; ++d) {
        const DirPtrs &dp = a.dir[d];
        const T *X = (const T *)dp.x;
        const T *DT = (const T *)dp.dt;
        const T *Bm = (const T *)dp.B;
        const T *Cm = (const T *)dp.C;
        const float Ah = dp.A[h];
        const float Dh = dp.D ? dp.D[h] : 0.f;
        if (d == 0 && a.init_state && p < P) {
#pragma unroll
            for (int n = 0; n < N; ++n) st[n] = a.init_state[state_off + n];
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) st[n] = 0.f;
        }
        for (int base = 0; base < len; base += kSeqTile) {
            const int nsteps = len - base < kSeqTile ? len - base : kSeqTile;
            __syncthreads();
            for (int i = threadIdx.x; i < nsteps * N; i += blockDim.x) {
                const int s = i / N, n = i - s * N;
                const int t = d == 0 ? t0 + base + s : t1 - 1 - base - s;
                const size_t o = ((row_tok + t) * G + g) * N + n;
                sB[s][n] = Elem<T>::load(Bm, o);
                sC[s][n] = Elem<T>::load(Cm, o);
            }
            for (int i = threadIdx.x; i < nsteps * P; i += blockDim.x) {
                const int s = i / P, pp = i - s * P;
                const int t = d == 0 ? t0 + base + s : t1 - 1 - base - s;
                sx[s][pp] = Elem<T>::load(X, ((row_tok + t) * H + h) * P + pp);
            }
            for (int i = threadIdx.x; i < nsteps; i += blockDim.x) {
                const int t = d == 0 ? t0 + base + i : t1 - 1 - base - i;
                sdt[i] = Elem<T>::load(DT, (row_tok + t) * H + h);
            }
            __syncthreads();
            if (p < P) {
                for (int s = 0; s < nsteps; ++s) {
                    const int t = d == 0 ? t0 + base + s : t1 - 1 - base - s;
                    const float dtt = sdt[s];
                    const float decay = expf(dtt * Ah);
                    const float xv = sx[s][p];
                    const float dx = dtt * xv;
                    float acc = 0.f;
#pragma unroll
                    for (int n = 0; n < N; ++n) {
                        st[n] = fmaf(decay, st[n], dx * sB[s][n]);
                        acc = fmaf(sC[s][n], st[n], acc);
                    }
                    const float yv = fmaf(Dh, xv, acc);
                    float *yp = a.y + ((row_tok + t) * H + h) * P + p;
                    if (d == 0) *yp = yv; else *yp += yv;
                }
            }
        }
        if (d == 0 && a.final_state && p < P) {
#pragma unroll
            for (int n = 0; n < N; ++n) a.final_state[state_off + n] = st[n];
        }
    }
}

bool seq_supported(int P, int N) {
    return P >= 1 && P <= kMaxP && (N == 16 || N == 32 || N == 64 || N == 128);
}

template <typename T, int N>
static hipError_t launch_typed(const SeqArgs &a, int units, hipStream_t s) {
    int threads = ((a.P + 63) / 64) * 64;
    BM_LAUNCH("scan_seq", (k_scan_seq<T, N>), dim3(units, a.H), dim3(threads), 0, s, a);
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

hipError_t launch_scan_seq(const Problem &p, hipStream_t s) {
    SeqArgs a;
    a.dir[0] = p.dir[0];
    a.dir[1] = p.dir[1];
    a.ndir = p.has_bwd ? 2 : 1;
    a.L = p.L; a.H = p.H; a.P = p.P; a.G = p.G;
    a.cu = p.cu_dev;
    a.init_state = p.init_state;
    a.final_state = p.final_state;
    a.y = p.y;
    const int units = p.cu_dev ? p.nseq : p.batch;
    if (units == 0) return hipSuccess;
    return p.bf16 ? launch_n<uint16_t>(a, p.N, units, s) : launch_n<float>(a, p.N, units, s);
}

}  // namespace bm
