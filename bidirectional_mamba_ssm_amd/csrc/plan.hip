// Integer planning kernels: packed-sequence offsets and per-token sequence
// indices, built on the device from host offsets passed by value (no host
// staging buffer, no synchronization), and slot clearing for state caches.
#include "common.hpp"
#include "internal.hpp"

namespace bm {

constexpr int kOffsPerLaunch = 256;

struct OffsetBatch {
    int first;                     // index of offs[0] in the full cu_seqlens
    int count;                     // number of valid entries in offs
    int32_t offs[kOffsPerLaunch + 1];
};

__global__ void k_store_offsets(OffsetBatch b, int32_t *cu_dev) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < b.count) cu_dev[b.first + i] = b.offs[i];
}

// Token t belongs to sequence j when offs[j] <= t < offs[j+1]; empty
// sequences own no token. Each launch covers tokens [offs[0], offs[count-1]).
__global__ void k_seq_index(OffsetBatch b, int32_t *seq_idx) {
    const int lo_tok = b.offs[0];
    const int hi_tok = b.offs[b.count - 1];
    int t = lo_tok + blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= hi_tok) return;
    // largest j with offs[j] <= t, then skip forward over empty sequences
    int lo = 0, hi = b.count - 1;  // invariant: offs[lo] <= t < offs[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (b.offs[mid] <= t) lo = mid; else hi = mid;
    }
    seq_idx[t] = b.first + lo;
}

static OffsetBatch make_batch(const int32_t *cu, int first, int count) {
    OffsetBatch b;
    b.first = first;
    b.count = count;
    for (int i = 0; i < count; ++i) b.offs[i] = cu[first + i];
    return b;
}

hipError_t launch_store_offsets(const int32_t *cu, int nseq, int32_t *cu_dev,
                                hipStream_t s) {
    for (int first = 0; first <= nseq; first += kOffsPerLaunch) {
        int count = nseq + 1 - first;
        if (count > kOffsPerLaunch) count = kOffsPerLaunch;
        OffsetBatch b = make_batch(cu, first, count);
        BM_LAUNCH("store_offsets", k_store_offsets, dim3(1), dim3(kOffsPerLaunch), 0, s, b, cu_dev);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_seq_index(const int32_t *cu, int nseq, int total,
                            int32_t *seq_idx, hipStream_t s) {
    (void)total;
    // consecutive launches share one boundary offset
    for (int first = 0; first < nseq; first += kOffsPerLaunch) {
        int count = nseq + 1 - first;
        if (count > kOffsPerLaunch + 1) count = kOffsPerLaunch + 1;
        OffsetBatch b = make_batch(cu, first, count);
        int ntok = cu[first + count - 1] - cu[first];
        if (ntok <= 0) continue;
        int blocks = (ntok + 255) / 256;
        BM_LAUNCH("seq_index", k_seq_index, dim3(blocks), dim3(256), 0, s, b, seq_idx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

struct SlotBatch {
    int count;        // 0 means: every slot
    int32_t slot[64];
};

__global__ void k_zero_slots(float *data, size_t slot_elems, SlotBatch b, int nslots) {
    const int which = blockIdx.y;
    const int slot = b.count ? b.slot[which] : which;
    if (slot < 0 || slot >= nslots) return;
    float4 *base = reinterpret_cast<float4 *>(data + (size_t)slot * slot_elems);
    const size_t n4 = slot_elems / 4;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (size_t)gridDim.x * blockDim.x)
        base[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (blockIdx.x == 0 && threadIdx.x < (slot_elems & 3))
        data[(size_t)slot * slot_elems + n4 * 4 + threadIdx.x] = 0.f;
}

hipError_t launch_zero_slots(float *data, size_t slot_elems, const int32_t *slots,
                             int n, int nslots, hipStream_t s) {
    int xblocks = (int)((slot_elems / 4 + 255) / 256);
    if (xblocks > 256) xblocks = 256;
    if (xblocks < 1) xblocks = 1;
    if (!slots) {
        SlotBatch b;
        b.count = 0;
        BM_LAUNCH("zero_slots", k_zero_slots, dim3(xblocks, nslots), dim3(256), 0, s, data,
                  slot_elems, b, nslots);
        return hipGetLastError();
    }
    for (int first = 0; first < n; first += 64) {
        SlotBatch b;
        b.count = n - first < 64 ? n - first : 64;
        for (int i = 0; i < b.count; ++i) b.slot[i] = slots[first + i];
        BM_LAUNCH("zero_slots", k_zero_slots, dim3(xblocks, b.count), dim3(256), 0, s, data,
                  slot_elems, b, nslots);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bm
