// C ABI of libbimamba: argument validation (host only, before any HIP call),
// workspace layout, dispatch to the kernel launchers, state-cache objects.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/bimamba.h"
#include "internal.hpp"

using namespace bm;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(BIMAMBA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int check_shape(const bimamba_shape *s, bool block_step) {
    if (!s) return fail(BIMAMBA_EINVAL, "shape is NULL");
    if (s->dtype != BIMAMBA_F32 && s->dtype != BIMAMBA_BF16)
        return fail(BIMAMBA_EINVAL, "dtype %d is not BIMAMBA_F32 or BIMAMBA_BF16", s->dtype);
    if (s->batch < 1) return fail(BIMAMBA_EINVAL, "batch %d < 1", s->batch);
    if (s->seqlen < 0) return fail(BIMAMBA_EINVAL, "seqlen %d < 0", s->seqlen);
    if (s->nheads < 1 || s->headdim < 1 || s->d_state < 1 || s->ngroups < 1)
        return fail(BIMAMBA_EINVAL, "nheads/headdim/d_state/ngroups must be >= 1");
    if (s->flags & ~BIMAMBA_DT_SOFTPLUS)
        return fail(BIMAMBA_EINVAL, "flags 0x%x: only BIMAMBA_DT_SOFTPLUS is defined", s->flags);
    if (s->nheads % s->ngroups)
        return fail(BIMAMBA_EINVAL, "ngroups %d does not divide nheads %d", s->ngroups, s->nheads);
    if (s->chunk != 64 && s->chunk != 128 && s->chunk != 256)
        return fail(BIMAMBA_EUNSUPPORTED, "chunk %d not in {64, 128, 256}", s->chunk);
    if (!seq_supported(s->headdim, s->d_state))
        return fail(BIMAMBA_EUNSUPPORTED,
                    "headdim %d / d_state %d unsupported (headdim <= 128, d_state in {16,32,64,128})",
                    s->headdim, s->d_state);
    if (block_step && (s->seqlen < 1 || s->seqlen > 256))
        return fail(BIMAMBA_EINVAL, "block length %d not in [1, 256]", s->seqlen);
    // every element index must fit comfortably in 63 bits and the token count in int32
    const long long tok = (long long)s->batch * s->seqlen;
    if (tok > (1LL << 31) - 1)
        return fail(BIMAMBA_EUNSUPPORTED, "batch*seqlen %lld exceeds 2^31-1", tok);
    return BIMAMBA_OK;
}

int check_dir(const bimamba_dir *d, const char *name, bool empty) {
    if (!d) return fail(BIMAMBA_EINVAL, "%s direction is NULL", name);
    if (!d->A) return fail(BIMAMBA_EINVAL, "%s: A is required", name);
    if (empty) return BIMAMBA_OK;   // no token: x, dt, B, C are never read
    if (!d->x || !d->dt || !d->B || !d->C)
        return fail(BIMAMBA_EINVAL, "%s: x, dt, A, B and C are required", name);
    if (!aligned16(d->x) || !aligned16(d->B) || !aligned16(d->C))
        return fail(BIMAMBA_EINVAL, "%s: x, B and C must be 16-byte aligned", name);
    return BIMAMBA_OK;
}

int check_offsets(const int32_t *cu, int nseq, int total) {
    if (nseq < 1) return fail(BIMAMBA_EINVAL, "nseq %d < 1 with cu_seqlens", nseq);
    if (cu[0] != 0) return fail(BIMAMBA_EINVAL, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int i = 0; i < nseq; ++i)
        if (cu[i + 1] < cu[i])
            return fail(BIMAMBA_EINVAL, "cu_seqlens decreases at %d (%d > %d)", i, cu[i], cu[i + 1]);
    if (cu[nseq] != total)
        return fail(BIMAMBA_EINVAL, "cu_seqlens[nseq] = %d but seqlen = %d", cu[nseq], total);
    return BIMAMBA_OK;
}

// Which kernel family serves a shape: the matrix-core chunked scan where it
// is built (bf16, headdim 64, d_state 128), the token-sequential scan
// otherwise (every fp32 problem and the remaining shapes).
bool use_chunked(const bimamba_shape *s) {
    Problem p;
    p.bf16 = s->dtype == BIMAMBA_BF16;
    p.P = s->headdim; p.N = s->d_state; p.L = s->seqlen; p.Q = s->chunk;
    return chunked_supported(p);
}

struct Layout {
    size_t cu_off = 0, seq_off = 0, scan_off = 0, scan_bytes = 0, total = 0;
};

// limit: the largest workspace available (SIZE_MAX: as much as the fastest
// form needs). Under a limit the chunked scan lengthens its segments and the
// token-sequential scan runs whole rows; the packed-sequence tables must fit.
Layout workspace_layout(const bimamba_shape *s, int nseq, size_t limit = SIZE_MAX) {
    Layout w;
    size_t off = 0;
    if (nseq > 0) {
        w.cu_off = off;
        off += align256((size_t)(nseq + 1) * 4);
        w.seq_off = off;
        off += align256((size_t)s->seqlen * 4);
    }
    w.scan_off = off;
    const size_t rest = limit > off ? limit - off : 0;
    if (use_chunked(s)) {
        w.scan_bytes = chunked_workspace(s->batch, s->seqlen, s->nheads, s->ngroups, s->chunk, rest);
    } else {
        w.scan_bytes = seq_workspace(s->batch, s->seqlen, s->nheads, s->headdim, s->d_state, nseq > 0);
        if (w.scan_bytes > rest) w.scan_bytes = 0;   // whole rows need none
    }
    off += w.scan_bytes;
    w.total = off;
    return w;
}

DirPtrs to_ptrs(const bimamba_dir *d) {
    DirPtrs p;
    p.x = d->x; p.dt = d->dt; p.B = d->B; p.C = d->C; p.A = d->A; p.D = d->D;
    return p;
}

void set_dt(Problem &p, int flags, const bimamba_dir *fwd, const bimamba_dir *bwd) {
    p.dt_softplus = (flags & BIMAMBA_DT_SOFTPLUS) != 0;
    p.dt_bias[0] = p.dt_softplus ? fwd->dt_bias : nullptr;
    p.dt_bias[1] = p.dt_softplus && bwd ? bwd->dt_bias : nullptr;
}

struct ProfRecord {
    const char *name;
    hipEvent_t start, stop;
};
thread_local bool g_prof_on = false;
thread_local std::vector<ProfRecord> g_prof;
thread_local std::vector<hipEvent_t> g_event_pool;   // reused across sessions

bool pool_event(hipEvent_t *e) {
    if (!g_event_pool.empty()) {
        *e = g_event_pool.back();
        g_event_pool.pop_back();
        return true;
    }
    return hipEventCreate(e) == hipSuccess;
}
void release_records() {
    for (auto &r : g_prof) {
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_prof.clear();
}

int check_conv_shape(const bimamba_conv_shape *s) {
    if (!s) return fail(BIMAMBA_EINVAL, "shape is NULL");
    if (s->dtype != BIMAMBA_F32 && s->dtype != BIMAMBA_BF16)
        return fail(BIMAMBA_EINVAL, "dtype %d is not BIMAMBA_F32 or BIMAMBA_BF16", s->dtype);
    if (s->batch < 1) return fail(BIMAMBA_EINVAL, "batch %d < 1", s->batch);
    if (s->seqlen < 0) return fail(BIMAMBA_EINVAL, "seqlen %d < 0", s->seqlen);
    if (s->nheads < 1 || s->headdim < 1 || s->d_state < 1 || s->ngroups < 1)
        return fail(BIMAMBA_EINVAL, "nheads/headdim/d_state/ngroups must be >= 1");
    if (s->width < 2 || s->width > 4)
        return fail(BIMAMBA_EUNSUPPORTED, "width %d not in [2, 4]", s->width);
    if (s->activation != 0 && s->activation != 1)
        return fail(BIMAMBA_EINVAL, "activation %d is neither 0 (none) nor 1 (SiLU)", s->activation);
    if (s->flags != 0)
        return fail(BIMAMBA_EINVAL, "flags 0x%x: no flag is defined", s->flags);
    const long long ch = (long long)s->nheads * s->headdim + 2LL * s->ngroups * s->d_state;
    if (ch > (1LL << 24))
        return fail(BIMAMBA_EUNSUPPORTED, "%lld channels exceed 2^24", ch);
    const long long tok = (long long)s->batch * s->seqlen;
    if (tok > (1LL << 31) - 1)
        return fail(BIMAMBA_EUNSUPPORTED, "batch*seqlen %lld exceeds 2^31-1", tok);
    if ((long long)s->batch * 2 > 65535)
        return fail(BIMAMBA_EUNSUPPORTED, "batch %d exceeds 32767", s->batch);
    return BIMAMBA_OK;
}

int check_conv_dir(const bimamba_conv_dir *d, const char *name, bool empty) {
    if (!d) return fail(BIMAMBA_EINVAL, "%s direction is NULL", name);
    if (!d->weight) return fail(BIMAMBA_EINVAL, "%s: weight is required", name);
    if ((uintptr_t)d->weight & 3u || (uintptr_t)d->bias & 3u)
        return fail(BIMAMBA_EINVAL, "%s: weight and bias must be 4-byte aligned", name);
    if (empty) return BIMAMBA_OK;
    if (!d->xbc || !d->x || !d->B || !d->C)
        return fail(BIMAMBA_EINVAL, "%s: xbc, x, B and C are required", name);
    if (!aligned16(d->xbc) || !aligned16(d->x) || !aligned16(d->B) || !aligned16(d->C))
        return fail(BIMAMBA_EINVAL, "%s: xbc, x, B and C must be 16-byte aligned", name);
    return BIMAMBA_OK;
}

// packed rows: the per-token sequence index
int check_grad(const bimamba_grad *g, const char *name, bool empty) {
    if (!g) return fail(BIMAMBA_EINVAL, "%s gradients are NULL", name);
    if (!g->dA) return fail(BIMAMBA_EINVAL, "%s: dA is required", name);
    if (!aligned16(g->dA) || !aligned16(g->dD))
        return fail(BIMAMBA_EINVAL, "%s: dA and dD must be 16-byte aligned", name);
    if (empty) return BIMAMBA_OK;
    if (!g->dx || !g->ddt || !g->dB || !g->dC)
        return fail(BIMAMBA_EINVAL, "%s: dx, ddt, dB and dC are required", name);
    if (!aligned16(g->dx) || !aligned16(g->ddt) || !aligned16(g->dB) || !aligned16(g->dC))
        return fail(BIMAMBA_EINVAL, "%s: gradient arrays must be 16-byte aligned", name);
    return BIMAMBA_OK;
}

size_t conv_workspace(int nseq, int seqlen) {
    return nseq > 0 ? align256(sizeof(int32_t) * (seqlen > 0 ? seqlen : 1)) : 0;
}

}  // namespace

namespace bm {
void prof_before(const char *name, hipStream_t s) {
    if (!g_prof_on) return;
    ProfRecord r{name, nullptr, nullptr};
    if (!pool_event(&r.start)) {
        (void)hipGetLastError();
        return;
    }
    if (!pool_event(&r.stop)) {
        (void)hipGetLastError();
        g_event_pool.push_back(r.start);
        return;
    }
    (void)hipEventRecord(r.start, s);
    g_prof.push_back(r);
}
void prof_after(hipStream_t s) {
    if (!g_prof_on || g_prof.empty()) return;
    (void)hipEventRecord(g_prof.back().stop, s);
}
}  // namespace bm

struct bimamba_state {
    float *data;
    int nslots, nheads, headdim, d_state;
    // the short convolution's context (bimamba_state_alloc_conv), or null
    void *ctx;
    int ngroups, width, cdtype;
    size_t ctx_slot_bytes;   // (width - 1) * channels * element size
};

extern "C" {

int bimamba_version(void) { return BIMAMBA_VERSION; }

int bimamba_profile_begin(void) {
    release_records();
    g_prof_on = true;
    return BIMAMBA_OK;
}

int bimamba_profile_end(char *names, int name_len, int *counts, double *ms, int cap) {
    if (!g_prof_on) return fail(BIMAMBA_EINVAL, "profiling was not begun on this thread");
    g_prof_on = false;
    std::vector<std::string> seen;
    std::vector<int> cnt;
    std::vector<double> tot;
    int status = BIMAMBA_OK;
    for (auto &r : g_prof) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
        if (e != hipSuccess && status == BIMAMBA_OK) status = hip_fail(e, "profile events");
        size_t i = 0;
        while (i < seen.size() && seen[i] != r.name) ++i;
        if (i == seen.size()) { seen.push_back(r.name); cnt.push_back(0); tot.push_back(0.0); }
        cnt[i] += 1;
        tot[i] += t;
    }
    release_records();
    if (status != BIMAMBA_OK) return status;
    for (size_t i = 0; i < seen.size() && (int)i < cap; ++i) {
        if (names && name_len > 0) {
            strncpy(names + i * name_len, seen[i].c_str(), name_len - 1);
            names[i * name_len + name_len - 1] = 0;
        }
        if (counts) counts[i] = cnt[i];
        if (ms) ms[i] = tot[i];
    }
    return (int)seen.size();
}

const char *bimamba_last_error(void) { return g_err; }

const char *bimamba_status_str(int status) {
    switch (status) {
        case BIMAMBA_OK: return "ok";
        case BIMAMBA_EINVAL: return "invalid argument";
        case BIMAMBA_EUNSUPPORTED: return "unsupported shape";
        case BIMAMBA_ENOMEM: return "out of device memory";
        case BIMAMBA_EHIP: return "HIP error";
        case BIMAMBA_EWORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

int bimamba_ssd_workspace_size(const bimamba_shape *s, int nseq, size_t *bytes) {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (!bytes) return fail(BIMAMBA_EINVAL, "bytes is NULL");
    if (nseq < 0) return fail(BIMAMBA_EINVAL, "nseq %d < 0", nseq);
    *bytes = workspace_layout(s, nseq).total;
    return BIMAMBA_OK;
}

}  // extern "C"

namespace bm {

// The forward scan. y2 == nullptr: y = sum of the streams; else y receives
// the reverse stream and y2 the forward stream. limit: as workspace_layout.
int api_fail(int code, const char *msg) { return fail(code, "%s", msg); }

int ssd_fwd_impl(const bimamba_shape *s, const bimamba_dir *fwd,
                 const bimamba_dir *bwd, const int32_t *cu_seqlens, int nseq,
                 const float *init_state, float *final_state, float *y, float *y2,
                 void *workspace, size_t workspace_bytes, bimamba_stream stream,
                 size_t limit, bool validate_only) {
    int rc = check_shape(s, false);
    if (rc) return rc;
    const bool empty = s->seqlen == 0;
    if ((rc = check_dir(fwd, "forward", empty))) return rc;
    if (bwd && (rc = check_dir(bwd, "reverse", empty))) return rc;
    if (!y && !empty) return fail(BIMAMBA_EINVAL, "y is NULL");
    if (!aligned16(y)) return fail(BIMAMBA_EINVAL, "y must be 16-byte aligned");
    if (!aligned16(init_state) || !aligned16(final_state))
        return fail(BIMAMBA_EINVAL, "init_state and final_state must be 16-byte aligned");
    if (cu_seqlens) {
        if (s->batch != 1) return fail(BIMAMBA_EINVAL, "cu_seqlens requires batch == 1");
        if ((rc = check_offsets(cu_seqlens, nseq, s->seqlen))) return rc;
        if (init_state || final_state)
            return fail(BIMAMBA_EUNSUPPORTED, "init_state/final_state are not available with cu_seqlens");
    } else if (nseq != 0) {
        return fail(BIMAMBA_EINVAL, "nseq %d given without cu_seqlens", nseq);
    }
    const Layout w = workspace_layout(s, cu_seqlens ? nseq : 0, limit);
    if (w.total > limit)
        return fail(BIMAMBA_EWORKSPACE, "the packed-sequence tables need %zu bytes, more than %zu",
                    w.total, limit);
    if (validate_only) return BIMAMBA_OK;
    if (w.total > 0) {
        if (!workspace) return fail(BIMAMBA_EWORKSPACE, "workspace of %zu bytes required", w.total);
        if (workspace_bytes < w.total)
            return fail(BIMAMBA_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, w.total);
        if ((uintptr_t)workspace & 255u)
            return fail(BIMAMBA_EINVAL, "workspace must be 256-byte aligned");
    }

    hipStream_t st = (hipStream_t)stream;
    Problem p;
    p.batch = s->batch; p.L = s->seqlen; p.H = s->nheads; p.P = s->headdim;
    p.N = s->d_state; p.G = s->ngroups; p.Q = s->chunk;
    p.bf16 = s->dtype == BIMAMBA_BF16;
    p.has_bwd = bwd != nullptr;
    p.dir[0] = to_ptrs(fwd);
    p.dir[1] = bwd ? to_ptrs(bwd) : to_ptrs(fwd);
    set_dt(p, s->flags, fwd, bwd);
    p.cu_dev = nullptr;
    p.seq_idx = nullptr;
    p.nseq = cu_seqlens ? nseq : 0;
    p.init_state = init_state;
    p.final_state = final_state;
    p.y = y;
    p.y2 = y2;

    hipError_t e;
    if (cu_seqlens) {
        char *ws = (char *)workspace;
        int32_t *cu_dev = (int32_t *)(ws + w.cu_off);
        int32_t *seq = (int32_t *)(ws + w.seq_off);
        if ((e = launch_store_offsets(cu_seqlens, nseq, cu_dev, st)) != hipSuccess)
            return hip_fail(e, "storing sequence offsets");
        if ((e = launch_seq_index(cu_seqlens, nseq, s->seqlen, seq, st)) != hipSuccess)
            return hip_fail(e, "building sequence index");
        p.cu_dev = cu_dev;
        p.seq_idx = seq;
    }
    void *scan_ws = w.scan_bytes ? (char *)workspace + w.scan_off : nullptr;
    if (use_chunked(s)) {
        if ((e = launch_chunked(p, scan_ws, limit - w.scan_off, st)) != hipSuccess)
            return hip_fail(e, "chunked scan launch");
    } else if ((e = launch_scan_seq(p, scan_ws, st)) != hipSuccess) {
        return hip_fail(e, "scan launch");
    }
    return BIMAMBA_OK;
}

}  // namespace bm

extern "C" {

int bimamba_ssd_fwd(const bimamba_shape *s, const bimamba_dir *fwd,
                    const bimamba_dir *bwd, const int32_t *cu_seqlens, int nseq,
                    const float *init_state, float *final_state, float *y,
                    void *workspace, size_t workspace_bytes,
                    bimamba_stream stream) {
    return ssd_fwd_impl(s, fwd, bwd, cu_seqlens, nseq, init_state, final_state, y, nullptr,
                        workspace, workspace_bytes, stream, SIZE_MAX, false);
}

int bimamba_ssd_fwd_streams(const bimamba_shape *s, const bimamba_dir *fwd,
                            const bimamba_dir *bwd, const int32_t *cu_seqlens, int nseq,
                            const float *init_state, float *final_state, float *y_fwd,
                            float *y_bwd, void *workspace, size_t workspace_bytes,
                            bimamba_stream stream) {
    if (!bwd) return fail(BIMAMBA_EINVAL, "both streams are required");
    if (!s) return fail(BIMAMBA_EINVAL, "shape is NULL");
    if (s->flags) return fail(BIMAMBA_EUNSUPPORTED, "streams kept apart: no shape flag is supported");
    const bool empty = s->seqlen == 0;
    if (!empty && (!y_fwd || !y_bwd)) return fail(BIMAMBA_EINVAL, "y_fwd and y_bwd are required");
    if (!aligned16(y_fwd)) return fail(BIMAMBA_EINVAL, "y_fwd must be 16-byte aligned");
    if (y_fwd == y_bwd && !empty) return fail(BIMAMBA_EINVAL, "y_fwd and y_bwd must differ");
    return ssd_fwd_impl(s, fwd, bwd, cu_seqlens, nseq, init_state, final_state, y_bwd, y_fwd,
                        workspace, workspace_bytes, stream, SIZE_MAX, false);
}

int bimamba_state_alloc(bimamba_state **out, int nslots, int nheads, int headdim,
                        int d_state) {
    if (!out) return fail(BIMAMBA_EINVAL, "out is NULL");
    *out = nullptr;
    if (nslots < 1 || nheads < 1 || headdim < 1 || d_state < 1)
        return fail(BIMAMBA_EINVAL, "state dimensions must be >= 1");
    const size_t bytes = (size_t)nslots * nheads * headdim * d_state * sizeof(float);
    float *data = nullptr;
    hipError_t e = hipMalloc((void **)&data, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(BIMAMBA_ENOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
    }
    e = hipMemset(data, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(data);
        return hip_fail(e, "zeroing state");
    }
    bimamba_state *st = new bimamba_state;
    st->data = data;
    st->nslots = nslots; st->nheads = nheads; st->headdim = headdim; st->d_state = d_state;
    st->ctx = nullptr;
    st->ngroups = st->width = st->cdtype = 0;
    st->ctx_slot_bytes = 0;
    *out = st;
    return BIMAMBA_OK;
}

int bimamba_state_alloc_conv(bimamba_state **out, int nslots, int nheads, int headdim,
                             int d_state, int ngroups, int width, int dtype) {
    if (!out) return fail(BIMAMBA_EINVAL, "out is NULL");
    *out = nullptr;
    if (ngroups < 1 || nheads % ngroups != 0)
        return fail(BIMAMBA_EINVAL, "ngroups %d must be >= 1 and divide nheads %d", ngroups, nheads);
    if (width < 2 || width > 4) return fail(BIMAMBA_EINVAL, "width %d not in 2..4", width);
    if (dtype != BIMAMBA_BF16 && dtype != BIMAMBA_F32) return fail(BIMAMBA_EINVAL, "unknown dtype %d", dtype);
    const size_t esz = dtype == BIMAMBA_BF16 ? 2 : 4;
    const size_t ch = (size_t)nheads * headdim + 2 * (size_t)ngroups * d_state;
    const size_t slot_bytes = (size_t)(width - 1) * ch * esz;
    if (slot_bytes % 16)
        return fail(BIMAMBA_EUNSUPPORTED, "a slot's context (%zu bytes) must be a multiple of 16 bytes", slot_bytes);
    bimamba_state *st = nullptr;
    int rc = bimamba_state_alloc(&st, nslots, nheads, headdim, d_state);
    if (rc) return rc;
    void *ctx = nullptr;
    hipError_t e = hipMalloc(&ctx, slot_bytes * nslots);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        bimamba_state_free(st);
        return fail(BIMAMBA_ENOMEM, "hipMalloc(%zu): %s", slot_bytes * nslots, hipGetErrorString(e));
    }
    e = hipMemset(ctx, 0, slot_bytes * nslots);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(ctx);
        bimamba_state_free(st);
        return hip_fail(e, "zeroing the convolution context");
    }
    st->ctx = ctx;
    st->ngroups = ngroups; st->width = width; st->cdtype = dtype;
    st->ctx_slot_bytes = slot_bytes;
    *out = st;
    return BIMAMBA_OK;
}

void *bimamba_state_conv_ctx(bimamba_state *st) { return st ? st->ctx : nullptr; }

int bimamba_state_reset(bimamba_state *st, const int32_t *slots, int n,
                        bimamba_stream stream) {
    if (!st) return fail(BIMAMBA_EINVAL, "state is NULL");
    if (slots) {
        if (n < 0) return fail(BIMAMBA_EINVAL, "n %d < 0", n);
        for (int i = 0; i < n; ++i)
            if (slots[i] < 0 || slots[i] >= st->nslots)
                return fail(BIMAMBA_EINVAL, "slot %d out of range [0, %d)", slots[i], st->nslots);
        if (n == 0) return BIMAMBA_OK;
    }
    const size_t slot_elems = (size_t)st->nheads * st->headdim * st->d_state;
    hipError_t e = launch_zero_slots(st->data, slot_elems, slots, n, st->nslots,
                                     (hipStream_t)stream);
    if (e == hipSuccess && st->ctx)   // the context: zeroed as floats (slots of 16-byte multiples)
        e = launch_zero_slots((float *)st->ctx, st->ctx_slot_bytes / 4, slots, n, st->nslots,
                              (hipStream_t)stream);
    return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "state reset");
}

float *bimamba_state_data(bimamba_state *st) { return st ? st->data : nullptr; }

int bimamba_state_free(bimamba_state *st) {
    if (!st) return BIMAMBA_OK;
    hipError_t e = hipFree(st->data);
    if (st->ctx) {
        const hipError_t e2 = hipFree(st->ctx);
        if (e == hipSuccess) e = e2;
    }
    delete st;
    return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "hipFree");
}

int bimamba_block_step(bimamba_state *st, const bimamba_shape *s,
                       const bimamba_dir *fwd, const bimamba_dir *bwd, int commit,
                       float *y, bimamba_stream stream) {
    if (!st) return fail(BIMAMBA_EINVAL, "state is NULL");
    int rc = check_shape(s, true);
    if (rc) return rc;
    if ((rc = check_dir(fwd, "forward", false))) return rc;
    if ((rc = check_dir(bwd, "reverse", false))) return rc;
    if (!y) return fail(BIMAMBA_EINVAL, "y is NULL");
    if (!aligned16(y)) return fail(BIMAMBA_EINVAL, "y must be 16-byte aligned");
    if (s->batch > st->nslots)
        return fail(BIMAMBA_EINVAL, "batch %d exceeds the state's %d slots", s->batch, st->nslots);
    if (s->nheads != st->nheads || s->headdim != st->headdim || s->d_state != st->d_state)
        return fail(BIMAMBA_EINVAL, "shape (H=%d, P=%d, N=%d) does not match the state (%d, %d, %d)",
                    s->nheads, s->headdim, s->d_state, st->nheads, st->headdim, st->d_state);
    Problem p;
    p.batch = s->batch; p.L = s->seqlen; p.H = s->nheads; p.P = s->headdim;
    p.N = s->d_state; p.G = s->ngroups; p.Q = s->chunk;
    p.bf16 = s->dtype == BIMAMBA_BF16;
    p.has_bwd = true;
    p.dir[0] = to_ptrs(fwd);
    p.dir[1] = to_ptrs(bwd);
    set_dt(p, s->flags, fwd, bwd);
    p.cu_dev = nullptr; p.seq_idx = nullptr; p.nseq = 0;
    p.init_state = st->data;
    p.final_state = commit ? st->data : nullptr;
    p.y = y;
    p.y2 = nullptr;
    // the block is one segment of its row: the chunked kernels need no
    // workspace then (each workgroup reads its slice of the cache before it
    // writes it back, so the in-place update is safe)
    hipError_t e = chunked_supported(p) && chunked_workspace(p.batch, p.L, p.H, p.G, p.Q) == 0
                       ? launch_chunked(p, nullptr, 0, (hipStream_t)stream)
                       : launch_scan_seq(p, nullptr, (hipStream_t)stream);
    return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "block step launch");
}

int bimamba_seq_index(const int32_t *cu_seqlens, int nseq, int total, int32_t *seq_idx,
                      bimamba_stream stream) {
    if (!cu_seqlens || !seq_idx) return fail(BIMAMBA_EINVAL, "cu_seqlens and seq_idx are required");
    if (total < 0) return fail(BIMAMBA_EINVAL, "total %d < 0", total);
    int rc = check_offsets(cu_seqlens, nseq, total);
    if (rc) return rc;
    hipError_t e = launch_seq_index(cu_seqlens, nseq, total, seq_idx, (hipStream_t)stream);
    return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "sequence index launch");
}


int bimamba_ssd_bwd_workspace_size(const bimamba_shape *s, int has_bwd, size_t *bytes) {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (!bytes) return fail(BIMAMBA_EINVAL, "bytes is NULL");
    if (!bwd_supported(s->headdim, s->d_state))
        return fail(BIMAMBA_EUNSUPPORTED, "backward: headdim %d / d_state %d not in {16, 64} x {16, 128}",
                    s->headdim, s->d_state);
    if (s->flags)
        return fail(BIMAMBA_EUNSUPPORTED, "backward: dt is taken as the forward used it (no BIMAMBA_DT_SOFTPLUS)");
    *bytes = bwd_workspace(s->batch, s->seqlen, s->nheads, s->headdim, s->d_state, has_bwd ? 2 : 1);
    return BIMAMBA_OK;
}

int bimamba_ssd_bwd(const bimamba_shape *s, const bimamba_dir *fwd, const bimamba_dir *bwd,
                    const float *dy, const bimamba_grad *gfwd, const bimamba_grad *gbwd,
                    void *workspace, size_t workspace_bytes, bimamba_stream stream) {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (!bwd_supported(s->headdim, s->d_state))
        return fail(BIMAMBA_EUNSUPPORTED, "backward: headdim %d / d_state %d not in {16, 64} x {16, 128}",
                    s->headdim, s->d_state);
    if (s->flags)
        return fail(BIMAMBA_EUNSUPPORTED, "backward: dt is taken as the forward used it (no BIMAMBA_DT_SOFTPLUS)");
    const bool empty = s->seqlen == 0;
    if ((rc = check_dir(fwd, "forward", empty))) return rc;
    if (bwd && (rc = check_dir(bwd, "reverse", empty))) return rc;
    if (!dy && !empty) return fail(BIMAMBA_EINVAL, "dy is NULL");
    if (!aligned16(dy)) return fail(BIMAMBA_EINVAL, "dy must be 16-byte aligned");
    if ((rc = check_grad(gfwd, "forward", empty))) return rc;
    if (bwd && (rc = check_grad(gbwd, "reverse", empty))) return rc;
    const size_t need = bwd_workspace(s->batch, s->seqlen, s->nheads, s->headdim, s->d_state, bwd ? 2 : 1);
    if (need) {
        if (!workspace) return fail(BIMAMBA_EWORKSPACE, "workspace of %zu bytes required", need);
        if (workspace_bytes < need)
            return fail(BIMAMBA_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
        if ((uintptr_t)workspace & 255u)
            return fail(BIMAMBA_EINVAL, "workspace must be 256-byte aligned");
    }
    BwdProblem p;
    memset(&p, 0, sizeof p);
    p.batch = s->batch;
    p.L = s->seqlen;
    p.H = s->nheads;
    p.P = s->headdim;
    p.N = s->d_state;
    p.G = s->ngroups;
    p.bf16 = s->dtype == BIMAMBA_BF16;
    p.has_bwd = bwd != nullptr;
    const bimamba_dir *dirs[2] = {fwd, bwd};
    const bimamba_grad *grads[2] = {gfwd, gbwd};
    for (int i = 0; i < (bwd ? 2 : 1); ++i) {
        p.dir[i].x = dirs[i]->x;
        p.dir[i].dt = dirs[i]->dt;
        p.dir[i].A = dirs[i]->A;
        p.dir[i].B = dirs[i]->B;
        p.dir[i].C = dirs[i]->C;
        p.dir[i].D = dirs[i]->D;
        p.grad[i].dx = grads[i]->dx;
        p.grad[i].ddt = grads[i]->ddt;
        p.grad[i].dA = grads[i]->dA;
        p.grad[i].dB = grads[i]->dB;
        p.grad[i].dC = grads[i]->dC;
        p.grad[i].dD = grads[i]->dD;
    }
    p.dy = dy;
    hipError_t e = launch_bwd(p, workspace, (hipStream_t)stream);
    return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "launching the backward");
}

int bimamba_conv1d_workspace_size(const bimamba_conv_shape *s, int nseq, size_t *bytes) {
    int rc = check_conv_shape(s);
    if (rc) return rc;
    if (!bytes) return fail(BIMAMBA_EINVAL, "bytes is NULL");
    if (nseq < 0) return fail(BIMAMBA_EINVAL, "nseq %d < 0", nseq);
    *bytes = conv_workspace(nseq, s->seqlen);
    return BIMAMBA_OK;
}

int bimamba_conv1d(const bimamba_conv_shape *s, const bimamba_conv_dir *fwd,
                   const bimamba_conv_dir *bwd, const int32_t *cu_seqlens, int nseq,
                   const void *init_ctx, void *final_ctx,
                   void *workspace, size_t workspace_bytes, bimamba_stream stream) {
    int rc = check_conv_shape(s);
    if (rc) return rc;
    const bool empty = s->seqlen == 0;
    if ((rc = check_conv_dir(fwd, "forward", empty))) return rc;
    if (bwd && (rc = check_conv_dir(bwd, "reverse", empty))) return rc;
    if (!aligned16(init_ctx) || !aligned16(final_ctx))
        return fail(BIMAMBA_EINVAL, "init_ctx and final_ctx must be 16-byte aligned");
    const int esz = s->dtype == BIMAMBA_BF16 ? 2 : 4;
    const long long ch = (long long)s->nheads * s->headdim + 2LL * s->ngroups * s->d_state;
    const size_t ctx_bytes = (size_t)s->batch * (s->width - 1) * ch * esz;
    if (init_ctx && final_ctx && init_ctx != final_ctx) {
        const char *a = (const char *)init_ctx, *b = (const char *)final_ctx;
        if (a < b + ctx_bytes && b < a + ctx_bytes)
            return fail(BIMAMBA_EINVAL, "init_ctx and final_ctx overlap without being equal");
    }
    if (cu_seqlens) {
        if (s->batch != 1) return fail(BIMAMBA_EINVAL, "cu_seqlens requires batch == 1");
        if ((rc = check_offsets(cu_seqlens, nseq, s->seqlen))) return rc;
        if (init_ctx || final_ctx)
            return fail(BIMAMBA_EUNSUPPORTED, "init_ctx/final_ctx are not available with cu_seqlens");
    } else if (nseq != 0) {
        return fail(BIMAMBA_EINVAL, "nseq %d given without cu_seqlens", nseq);
    }
    const size_t need = conv_workspace(cu_seqlens ? nseq : 0, s->seqlen);
    if (need) {
        if (!workspace) return fail(BIMAMBA_EWORKSPACE, "workspace of %zu bytes required", need);
        if (workspace_bytes < need)
            return fail(BIMAMBA_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
        if ((uintptr_t)workspace & 255u)
            return fail(BIMAMBA_EINVAL, "workspace must be 256-byte aligned");
    }
    if (empty) {
        // no token: the final context is the initial one (or zeros)
        if (!final_ctx || final_ctx == init_ctx) return BIMAMBA_OK;
        hipError_t e = launch_ctx_copy(init_ctx, final_ctx, ctx_bytes / 2, (hipStream_t)stream);
        return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "copying the context of an empty row");
    }
    ConvArgs a;
    memset(&a, 0, sizeof a);
    const bimamba_conv_dir *dirs[2] = {fwd, bwd};
    ConvDirPtrs *ptrs[2] = {&a.fwd, &a.bwd};
    for (int i = 0; i < (bwd ? 2 : 1); ++i) {
        ptrs[i]->xbc = dirs[i]->xbc;
        ptrs[i]->weight = dirs[i]->weight;
        ptrs[i]->bias = dirs[i]->bias;
        ptrs[i]->x = dirs[i]->x;
        ptrs[i]->B = dirs[i]->B;
        ptrs[i]->C = dirs[i]->C;
    }
    a.batch = s->batch;
    a.L = s->seqlen;
    a.hp = s->nheads * s->headdim;
    a.gn = s->ngroups * s->d_state;
    a.ch = (int)ch;
    a.W = s->width;
    a.ndir = bwd ? 2 : 1;
    a.act = s->activation;
    a.init = init_ctx;
    a.final = final_ctx;
    a.inplace = init_ctx && init_ctx == final_ctx;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (cu_seqlens) {
        int32_t *seq = (int32_t *)workspace;
        if ((e = launch_seq_index(cu_seqlens, nseq, s->seqlen, seq, st)) != hipSuccess)
            return hip_fail(e, "building sequence index");
        a.seq = seq;
    }
    if ((e = launch_conv(a, s->dtype == BIMAMBA_BF16, st)) != hipSuccess)
        return hip_fail(e, "launching conv1d");
    return BIMAMBA_OK;
}

int bimamba_block_step_conv(bimamba_state *st, const bimamba_conv_shape *cs,
                            const bimamba_conv_dir *cfwd, const bimamba_conv_dir *cbwd,
                            const bimamba_shape *s, const bimamba_dir *fwd,
                            const bimamba_dir *bwd, int commit, float *y,
                            bimamba_stream stream) {
    if (!st) return fail(BIMAMBA_EINVAL, "state is NULL");
    if (!st->ctx) return fail(BIMAMBA_EINVAL, "the state carries no convolution context (bimamba_state_alloc_conv)");
    if (!cs || !s) return fail(BIMAMBA_EINVAL, "shapes are NULL");
    if (!cfwd || !cbwd || !fwd || !bwd) return fail(BIMAMBA_EINVAL, "both directions are required");
    if (!y) return fail(BIMAMBA_EINVAL, "y is NULL");
    if (!aligned16(y)) return fail(BIMAMBA_EINVAL, "y must be 16-byte aligned");
    if (cs->batch != s->batch || cs->seqlen != s->seqlen || cs->nheads != s->nheads ||
        cs->headdim != s->headdim || cs->d_state != s->d_state || cs->ngroups != s->ngroups ||
        cs->dtype != s->dtype)
        return fail(BIMAMBA_EINVAL, "the convolution's shape does not match the block's");
    if (cs->width != st->width || cs->dtype != st->cdtype || cs->ngroups != st->ngroups)
        return fail(BIMAMBA_EINVAL, "the convolution (width %d, dtype %d, ngroups %d) does not match the "
                    "state's context (%d, %d, %d)", cs->width, cs->dtype, cs->ngroups, st->width,
                    st->cdtype, st->ngroups);
    if (cs->batch > st->nslots)
        return fail(BIMAMBA_EINVAL, "batch %d exceeds the state's %d slots", cs->batch, st->nslots);
    if (fwd->x != cfwd->x || fwd->B != cfwd->B || fwd->C != cfwd->C || bwd->x != cbwd->x ||
        bwd->B != cbwd->B || bwd->C != cbwd->C)
        return fail(BIMAMBA_EINVAL, "the block's x, B, C must be the convolution's outputs");
    // validate the scan's arguments before anything is launched
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (s->nheads != st->nheads || s->headdim != st->headdim || s->d_state != st->d_state)
        return fail(BIMAMBA_EINVAL, "shape (H=%d, P=%d, N=%d) does not match the state (%d, %d, %d)",
                    s->nheads, s->headdim, s->d_state, st->nheads, st->headdim, st->d_state);
    if ((rc = check_dir(fwd, "forward", false))) return rc;
    if ((rc = check_dir(bwd, "reverse", false))) return rc;
    // the context advances only with a committed block (in place: one
    // workgroup walks each row's block in order)
    rc = bimamba_conv1d(cs, cfwd, cbwd, nullptr, 0, st->ctx, commit ? st->ctx : nullptr, nullptr, 0, stream);
    if (rc) return rc;
    return bimamba_block_step(st, s, fwd, bwd, commit, y, stream);
}

int bimamba_gated_norm(long long rows, int channels, int group_size, int dtype,
                       const float *y, const void *z, const float *weight, float eps,
                       void *out, bimamba_stream stream) {
    if (dtype != BIMAMBA_F32 && dtype != BIMAMBA_BF16)
        return fail(BIMAMBA_EINVAL, "dtype %d is not BIMAMBA_F32 or BIMAMBA_BF16", dtype);
    if (rows < 0) return fail(BIMAMBA_EINVAL, "rows %lld < 0", rows);
    if (rows > (1LL << 31) - 1) return fail(BIMAMBA_EUNSUPPORTED, "rows %lld exceed 2^31-1", rows);
    if (channels <= 0 || channels % 256 || channels > 8192)
        return fail(BIMAMBA_EUNSUPPORTED, "channels %d: need a multiple of 256 up to 8192", channels);
    if (group_size <= 0 || group_size % 256 || channels % group_size)
        return fail(BIMAMBA_EINVAL, "group_size %d: need a multiple of 256 dividing %d", group_size, channels);
    if (!(eps >= 0.f) || eps > 3.0e38f) return fail(BIMAMBA_EINVAL, "eps must be finite and >= 0");
    if (rows == 0) return BIMAMBA_OK;
    if (!y || !z || !weight || !out) return fail(BIMAMBA_EINVAL, "y, z, weight and out are required");
    if (!aligned16(y) || !aligned16(z) || !aligned16(weight) || !aligned16(out))
        return fail(BIMAMBA_EINVAL, "y, z, weight and out must be 16-byte aligned");
    EpiArgs a;
    a.rows = rows;
    a.C = channels;
    a.gs = group_size;
    a.eps = eps;
    a.y = y;
    a.z = z;
    a.w = weight;
    a.out = out;
    hipError_t e = launch_gated_norm(a, dtype == BIMAMBA_BF16, (hipStream_t)stream);
    return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "launching the gated norm");
}

int bimamba_merge_linear(long long rows, int cin, int cout, const float *y_fwd,
                         const float *y_bwd, const void *weight, const float *bias,
                         float *out, bimamba_stream stream) {
    if (rows < 0) return fail(BIMAMBA_EINVAL, "rows %lld < 0", rows);
    if (rows > (1LL << 31) - 1) return fail(BIMAMBA_EUNSUPPORTED, "rows %lld exceed 2^31-1", rows);
    if (cin <= 0 || cin % 32) return fail(BIMAMBA_EUNSUPPORTED, "cin %d: need a positive multiple of 32", cin);
    if (cout <= 0 || cout % 16) return fail(BIMAMBA_EUNSUPPORTED, "cout %d: need a positive multiple of 16", cout);
    if (cin > (1 << 24) || cout > (1 << 24)) return fail(BIMAMBA_EUNSUPPORTED, "cin/cout too large");
    if (rows == 0) return BIMAMBA_OK;
    if (!y_fwd || !y_bwd || !weight || !out)
        return fail(BIMAMBA_EINVAL, "y_fwd, y_bwd, weight and out are required");
    if (!aligned16(y_fwd) || !aligned16(y_bwd) || !aligned16(weight) || !aligned16(out))
        return fail(BIMAMBA_EINVAL, "y_fwd, y_bwd, weight and out must be 16-byte aligned");
    if (!aligned16(bias)) return fail(BIMAMBA_EINVAL, "bias must be 16-byte aligned");
    MergeArgs a;
    memset(&a, 0, sizeof a);
    a.rows = rows;
    a.cin = cin;
    a.cout = cout;
    a.yf = y_fwd;
    a.yb = y_bwd;
    a.w = weight;
    a.bias = bias;
    a.out = out;
    hipError_t e = launch_merge(a, (hipStream_t)stream);
    return e == hipSuccess ? BIMAMBA_OK : hip_fail(e, "launching the merge");
}

}  // extern "C"
