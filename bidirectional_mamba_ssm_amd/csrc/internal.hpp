// Host-side interfaces between the C ABI (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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

// ssd_chunked.hip: matrix-core chunked scan (bf16, headdim 64, d_state 128)
bool chunked_supported(const Problem &p);
size_t chunked_workspace(int batch, int L, int H, int G, int Q);
hipError_t launch_chunked(const Problem &p, void *ws, hipStream_t s);

// ssd_seq.hip: token-sequential scan, any (P <= 128, N in {16,32,64,128}).
// Long unpacked rows with few (row, head) pairs run in segments when the
// workspace holds seq_workspace() bytes; ws may be nullptr (whole rows).
bool seq_supported(int P, int N);
size_t seq_workspace(int batch, int L, int H, int P, int N, bool packed);
hipError_t launch_scan_seq(const Problem &p, void *ws, hipStream_t s);

}  // namespace bm
