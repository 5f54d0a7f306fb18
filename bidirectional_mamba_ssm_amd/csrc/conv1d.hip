// Short depthwise convolution of the scan's input channels (x, then B, then
// C of one direction), one width-W filter with a bias per channel, optional
// SiLU, both directions in one launch: causal for the forward stream,
// anti-causal for the reverse stream (the reverse block runs on the flipped
// sequence and its result is flipped back, DiffuMamba blog, "network
// architecture"; width d_conv = 4 in the configuration given there). The
// forward stream can start from, and hand back, the W-1 inputs that precede
// a row: the convolution part of the block cache ("Fixed state, long reach",
// Sec. 1: the finalized prefix is summarized, the reverse pass sees only the
// active block).
//
// The operation is a stream: every input element is read once (plus a
// W-1-row halo per run of tokens that the caches catch), every output
// element written once, so the kernel is bounded by HBM. Layout: a lane owns
// four adjacent channels (8 bytes of bf16, 16 of fp32), a wave 64 such
// vectors of one token row, for a run of 16 tokens (8 for small problems);
// it loads the run and its halo into registers up front (19 independent
// loads per lane in flight), then slides the filter down the run in fp32.
// No LDS, no barriers (except one when the context is updated in place).
// Channel vectors never straddle the x | B | C boundaries, so each lane
// writes one output array with vector stores.
#include "common.hpp"
#include "internal.hpp"

namespace bm {
namespace {

constexpr int kWaves = 4;    // waves per workgroup (token runs stacked)

template <typename T, int VEC>
struct alignas(sizeof(T) * VEC) Pack {
    T v[VEC];
};

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 results -> the output vector; bf16 pairs go through the hardware
// round-to-nearest-even conversion (v_cvt_pk_bf16_f32)
template <typename T, int VEC> struct Out;
template <int VEC> struct Out<float, VEC> {
    __device__ __forceinline__ static void put(Pack<float, VEC> &o, const float *v) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) o.v[j] = v[j];
    }
};
template <int VEC> struct Out<uint16_t, VEC> {
    __device__ __forceinline__ static void put(Pack<uint16_t, VEC> &o, const float *v) {
        if constexpr (VEC == 1) {
            o.v[0] = __builtin_bit_cast(uint16_t, (__bf16)v[0]);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; j += 2) {
                const f32x2_t p = {v[j], v[j + 1]};
                const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
                o.v[j] = (uint16_t)w;
                o.v[j + 1] = (uint16_t)(w >> 16);
            }
        }
    }
};

// v * sigmoid(v) with the hardware reciprocal (about 1 ulp); exp(-v) = inf
// gives -0 for very negative v
__device__ __forceinline__ float silu(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// One direction (REV: the reverse stream) of batch row b.
template <typename T, int VEC, int W, bool PACKED, int kTok, bool REV>
__device__ __forceinline__ void conv_dir(const ConvArgs &a, int b) {
    using P = Pack<T, VEC>;
    constexpr int R = kTok + W - 1;          // rows held per lane
    constexpr bool rev = REV;
    const ConvDirPtrs d = REV ? a.bwd : a.fwd;
    const int lane = threadIdx.x;
    const int wy = threadIdx.y;
    const int cv = blockIdx.y * 64 + lane;   // channel vector of this lane
    const bool chan_ok = cv < a.nvec;
    // lanes past the last channel vector read the last one (so that every
    // load is unconditional) and store nothing
    const int c0 = (chan_ok ? cv : a.nvec - 1) * VEC;

    // filter taps and bias of the lane's channels (fp32)
    float w[VEC][W], bias[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
#pragma unroll
        for (int k = 0; k < W; ++k) w[j][k] = d.weight[(size_t)(c0 + j) * W + k];
        bias[j] = d.bias ? d.bias[c0 + j] : 0.0f;
    }
    // output array of the lane: x, B or C
    T *obase;
    int ostride, oc;
    if (c0 < a.hp) {
        obase = (T *)d.x; ostride = a.hp; oc = c0;
    } else if (c0 < a.hp + a.gn) {
        obase = (T *)d.B; ostride = a.gn; oc = c0 - a.hp;
    } else {
        obase = (T *)d.C; ostride = a.gn; oc = c0 - a.hp - a.gn;
    }
    const T *in = (const T *)d.xbc;
    const size_t row0 = (size_t)b * a.L;     // first token row of this batch row
    const int tile_tok = kTok * kWaves;

    for (int tile = blockIdx.x; tile * tile_tok < a.L; tile += gridDim.x) {
        const int t0 = tile * tile_tok + wy * kTok;
        // rows base .. base+R-1: forward [t0-(W-1), t0+kTok), reverse [t0, t0+kTok+W-1)
        const int base = rev ? t0 : t0 - (W - 1);
        P raw[R];
        const T *prow = in + ((long long)row0 + base) * a.ch + c0;   // row `base`
        if (base >= 0 && base + R <= a.L) {
            // interior run: every row exists, all loads issued back to back
#pragma unroll
            for (int i = 0; i < R; ++i) raw[i] = *(const P *)(prow + (long long)i * a.ch);
        } else {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int r = base + i;
                if (r >= 0 && r < a.L) {
                    raw[i] = *(const P *)(prow + (long long)i * a.ch);
                } else if (r < 0 && a.init) {
                    raw[i] = *(const P *)((const T *)a.init +
                                          ((size_t)b * (W - 1) + (W - 1) + r) * a.ch + c0);
                } else {
#pragma unroll
                    for (int j = 0; j < VEC; ++j) raw[i].v[j] = (T)0;
                }
            }
        }
        // packed rows: a tap reads a row only if it belongs to the token's
        // own sequence (sequences are contiguous, so equal indices suffice);
        // rows outside [0, L) carry index -1 and are zero anyway
        int sid[PACKED ? R : 1];
        if (PACKED) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int r = base + i;
                sid[i] = (r >= 0 && r < a.L) ? a.seq[r] : -1;
            }
        }
#pragma unroll
        for (int i = 0; i < kTok; ++i) {
            const int t = t0 + i;
            if (t >= a.L) break;
            float acc[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] = bias[j];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                // forward: tap k sees row t-(W-1)+k; reverse: row t+(W-1)-k
                const int ri = rev ? i + (W - 1) - k : i + k;
                bool ok = true;
                if (PACKED) ok = sid[ri] == sid[rev ? i : i + (W - 1)];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const float v = ok ? to_f(raw[ri].v[j]) : 0.0f;
                    acc[j] = __builtin_fmaf(w[j][k], v, acc[j]);
                }
            }
            if (a.act) {
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[j] = silu(acc[j]);
            }
            P o;
            Out<T, VEC>::put(o, acc);
            if (chan_ok) *(P *)(obase + (row0 + t) * ostride + oc) = o;
        }
        // forward context out: the row's last W-1 inputs, from the wave that
        // holds token L-1 (its halo reaches back W-1 rows, into the initial
        // context when the row is shorter than W-1)
        if (a.inplace) __syncthreads();          // every read of init is done
        if (!rev && a.final && chan_ok && t0 <= a.L - 1 && a.L - 1 < t0 + kTok) {
#pragma unroll
            for (int q = 0; q < W - 1; ++q) {
                // held row L-(W-1)+q; selected with constant indices so that
                // raw stays in registers
                const int want = a.L - (W - 1) + q - base;
                P v = raw[0];
#pragma unroll
                for (int i = 1; i < R; ++i)
                    if (i == want) v = raw[i];
                *(P *)((T *)a.final + ((size_t)b * (W - 1) + q) * a.ch + c0) = v;
            }
        }
    }
}

// kTok: tokens per wave (16 for long rows; 8 for small problems, where the
// grid would not fill the chip and the per-wave chain is the latency)
template <typename T, int VEC, int W, bool PACKED, int kTok>
__global__ __launch_bounds__(64 * kWaves) void k_conv(ConvArgs a) {
    const int dir = (int)(blockIdx.z % (unsigned)a.ndir);
    const int b = (int)(blockIdx.z / (unsigned)a.ndir);
    if (dir == 1)
        conv_dir<T, VEC, W, PACKED, kTok, true>(a, b);
    else
        conv_dir<T, VEC, W, PACKED, kTok, false>(a, b);
}

template <typename T, int VEC, int W, int TOK>
hipError_t launch_t(const ConvArgs &a, hipStream_t s) {
    const int tiles = (a.L + TOK * kWaves - 1) / (TOK * kWaves);
    // in place: one workgroup per (row, channel slab) walks the row in order,
    // so the initial context is read before the final one is written
    const dim3 grid(a.inplace ? 1 : tiles, (a.nvec + 63) / 64, a.batch * a.ndir);
    if (a.seq)
        BM_LAUNCH("conv1d_packed", (k_conv<T, VEC, W, true, TOK>), grid, dim3(64, kWaves), 0, s, a);
    else
        BM_LAUNCH("conv1d", (k_conv<T, VEC, W, false, TOK>), grid, dim3(64, kWaves), 0, s, a);
    return hipGetLastError();
}

template <typename T, int VEC, int W>
hipError_t launch_w(const ConvArgs &a, hipStream_t s) {
    return (long long)a.batch * a.L <= 4096 ? launch_t<T, VEC, W, 8>(a, s)
                                             : launch_t<T, VEC, W, 16>(a, s);
}

template <typename T, int VEC>
hipError_t launch_v(const ConvArgs &a, hipStream_t s) {
    switch (a.W) {
        case 2: return launch_w<T, VEC, 2>(a, s);
        case 3: return launch_w<T, VEC, 3>(a, s);
        case 4: return launch_w<T, VEC, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

__global__ void k_ctx_copy(const uint16_t *src, uint16_t *dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : (uint16_t)0;
}

hipError_t launch_ctx_copy(const void *src, void *dst, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    BM_LAUNCH("conv_ctx_copy", k_ctx_copy, dim3((unsigned)blocks), dim3(256), 0, s,
              (const uint16_t *)src, (uint16_t *)dst, n);
    return hipGetLastError();
}

// four channels per lane: 8-byte accesses for bf16, 16-byte for fp32 (for
// bf16, 8 channels per lane would double the registers a run holds and halve
// the waves a SIMD keeps in flight, which measured slower)
bool conv_vectorized(bool bf16, int hp, int gn) {
    (void)bf16;
    return hp % 4 == 0 && gn % 4 == 0;
}

hipError_t launch_conv(ConvArgs a, bool bf16, hipStream_t s) {
    if (a.L == 0 || a.batch == 0) return hipSuccess;
    const bool vec = conv_vectorized(bf16, a.hp, a.gn);
    a.nvec = a.ch / (vec ? 4 : 1);
    if (bf16)
        return vec ? launch_v<uint16_t, 4>(a, s) : launch_v<uint16_t, 1>(a, s);
    return vec ? launch_v<float, 4>(a, s) : launch_v<float, 1>(a, s);
}

}  // namespace bm
