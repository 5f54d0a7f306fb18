// Host-side interfaces between the C ABI (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bimamba.h"

namespace bm {

struct DirPtrs {
    const void *x, *dt, *B, *C;
    const float *A, *D;
};

// Problem as the launchers see it (already validated).
struct Problem {
    int batch, L, H, P, N, G, Q;
    bool bf16;
    bool has_bwd;
    DirPtrs dir[2];            // [0] forward, [1] reverse
    const int32_t *cu_dev;     // packed offsets on device, or nullptr
    const int32_t *seq_idx;    // per-token packed sequence index, or nullptr
    int nseq;                  // packed sequences (0 when not packed)
    const float *init_state;   // [units][H][P][N] or nullptr
    float *final_state;        // [units][H][P][N] or nullptr
    float *y;
    bool dt_softplus;          // dt holds the pre-activation: softplus(dt + bias)
    const float *dt_bias[2];   // with dt_softplus: [H] per direction, or nullptr (zero)
    float *y2;                 // streams kept apart: y gets the reverse stream, y2 the
                               // forward stream; nullptr: y gets their sum
};

// Profiling hooks (api.cpp): no-ops unless bimamba_profile_begin() is active
// on the calling thread. Every launcher brackets each launch with them.
void prof_before(const char *name, hipStream_t s);
void prof_after(hipStream_t s);

#define BM_LAUNCH(name, kernel, grid, block, shmem, stream, ...)            \
    do {                                                                   \
        ::bm::prof_before(name, stream);                                   \
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__); \
        ::bm::prof_after(stream);                                          \
    } while (0)

// plan.hip
hipError_t launch_store_offsets(const int32_t *cu_host, int nseq, int32_t *cu_dev,
                                hipStream_t s);
hipError_t launch_seq_index(const int32_t *cu_host, int nseq, int total,
                            int32_t *seq_idx, hipStream_t s);
hipError_t launch_zero_slots(float *data, size_t slot_elems, const int32_t *slots,
                             int n, int nslots, hipStream_t s);

// api.cpp: the forward scan behind bimamba_ssd_fwd (validation, workspace
// layout within `limit` bytes, launches); returns a bimamba_status. With
// validate_only it checks the arguments (no HIP call) and returns.
int ssd_fwd_impl(const bimamba_shape *s, const bimamba_dir *fwd, const bimamba_dir *bwd,
                 const int32_t *cu_seqlens, int nseq, const float *init_state,
                 float *final_state, float *y, float *y2, void *workspace,
                 size_t workspace_bytes, bimamba_stream stream, size_t limit,
                 bool validate_only);
// api.cpp: records a failure for bimamba_last_error and returns `code`
int api_fail(int code, const char *msg);

// ssd_chunked.hip: matrix-core chunked scan (bf16, headdim 64, d_state 128)
bool chunked_supported(const Problem &p);
// limit: the largest workspace the caller can give; segments are lengthened
// until their states fit (a whole row per segment needs none). The size
// query and the launch must be given the same limit.
size_t chunked_workspace(int batch, int L, int H, int G, int Q, size_t limit = SIZE_MAX);
hipError_t launch_chunked(const Problem &p, void *ws, size_t limit, hipStream_t s);

// ssd_seq.hip: token-sequential scan, any (P <= 128, N in {16,32,64,128}).
// Long unpacked rows with few (row, head) pairs run in segments when the
// workspace holds seq_workspace() bytes; ws may be nullptr (whole rows).
bool seq_supported(int P, int N);
size_t seq_workspace(int batch, int L, int H, int P, int N, bool packed);
hipError_t launch_scan_seq(const Problem &p, void *ws, hipStream_t s);

// ssd_bwd.hip: training backward of the bidirectional SSD
struct GradPtrs {
    float *dx, *ddt, *dA, *dB, *dC, *dD;   // dD may be nullptr
};
struct BwdProblem {
    int batch, L, H, P, N, G;
    bool bf16, has_bwd;
    DirPtrs dir[2];
    GradPtrs grad[2];
    const float *dy;
};
bool bwd_supported(int P, int N);
size_t bwd_workspace(int batch, int L, int H, int P, int N, int ndir);
hipError_t launch_bwd(const BwdProblem &p, void *ws, hipStream_t s);

// merge.hip: concatenating merge of the two streams (Linear on [y_fwd ; y_bwd])
struct MergeArgs {
    long long rows;
    int cin, cout;
    int mblk, nblk;            // token panels, output blocks (set by launch_merge)
    const float *yf, *yb;      // [rows][cin]
    const void *w;             // bf16 [cout][2 cin]
    const float *bias;         // [cout] or nullptr
    float *out;                // [rows][cout]
};
hipError_t launch_merge(MergeArgs a, hipStream_t s);

// epilogue.hip: gated RMS norm of the scan's output
struct EpiArgs {
    long long rows;
    int C, gs;                 // channels (multiple of 256, <= 8192), group size
    float eps;
    const float *y;            // [rows][C]
    const void *z;             // [rows][C] bf16 or fp32
    const float *w;            // [C]
    void *out;                 // [rows][C], z's dtype
};
hipError_t launch_gated_norm(const EpiArgs &a, bool bf16, hipStream_t s);

// conv1d.hip: short depthwise convolution of the x | B | C channels
struct ConvDirPtrs {
    const void *xbc;           // [batch][L][ch]
    const float *weight;       // [ch][W]
    const float *bias;         // [ch] or nullptr
    void *x, *B, *C;           // outputs [batch][L][hp], [batch][L][gn] x2
};
struct ConvArgs {
    ConvDirPtrs fwd;           // forward stream (causal filter)
    ConvDirPtrs bwd;           // reverse stream (anti-causal filter)
    int batch, L, hp, gn, ch, W, ndir, act;
    int nvec;                  // channel vectors per row (set by launch_conv)
    const int32_t *seq;        // packed: per-token sequence index [L], or nullptr
    const void *init;          // [batch][W-1][ch] forward context, or nullptr
    void *final;               // [batch][W-1][ch] or nullptr
    int inplace;               // final == init: one workgroup walks each row
};
bool conv_vectorized(bool bf16, int hp, int gn);
hipError_t launch_conv(ConvArgs a, bool bf16, hipStream_t s);
// dst[i] = src ? src[i] : 0 for n 16-bit words (context of an empty row)
hipError_t launch_ctx_copy(const void *src, void *dst, size_t n, hipStream_t s);

}  // namespace bm
