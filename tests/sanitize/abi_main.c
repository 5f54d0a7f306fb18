/* Drives libbimamba's host-side argument validation (every entry point of
 * include/bimamba.h, with malformed arguments) for a build of the library's
 * host code with AddressSanitizer and UndefinedBehaviorSanitizer. Every call
 * here fails validation before any HIP call, so no GPU is needed; device
 * pointers are placeholders that are never dereferenced. Exits 0 when every
 * call returns the expected status. Test infrastructure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bimamba.h"

static int fails = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        printf("FAIL %s: %d (expected %d): %s\n", what, got, want, bimamba_last_error());
        ++fails;
    } else if (want != BIMAMBA_OK && !bimamba_last_error()[0]) {
        printf("FAIL %s: no message\n", what);
        ++fails;
    }
}

int main(void) {
    void *dev = (void *)(uintptr_t)0x100000;   /* aligned placeholder, never read */
    bimamba_shape s = {1, 128, 4, 64, 128, 1, 64, BIMAMBA_BF16, 0};
    bimamba_dir d = {dev, dev, (const float *)dev, dev, dev, NULL, NULL};
    float *y = (float *)dev;
    size_t n = 0;

    expect(bimamba_ssd_fwd(NULL, &d, NULL, NULL, 0, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "no shape");
    bimamba_shape t = s; t.dtype = 7;
    expect(bimamba_ssd_fwd(&t, &d, NULL, NULL, 0, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "dtype");
    t = s; t.chunk = 48;
    expect(bimamba_ssd_fwd(&t, &d, NULL, NULL, 0, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EUNSUPPORTED, "chunk");
    t = s; t.nheads = 3; t.ngroups = 2;
    expect(bimamba_ssd_fwd(&t, &d, NULL, NULL, 0, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "groups");
    t = s; t.flags = 8;
    expect(bimamba_ssd_fwd(&t, &d, NULL, NULL, 0, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "flags");
    expect(bimamba_ssd_fwd(&s, NULL, NULL, NULL, 0, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "no fwd");
    bimamba_dir m = d; m.x = (const void *)((uintptr_t)dev + 2);
    expect(bimamba_ssd_fwd(&s, &m, NULL, NULL, 0, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "misaligned x");
    const int32_t bad_cu[] = {0, 100, 90, 128};
    expect(bimamba_ssd_fwd(&s, &d, NULL, bad_cu, 3, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "cu decreasing");
    const int32_t short_cu[] = {0, 60, 100};
    expect(bimamba_ssd_fwd(&s, &d, NULL, short_cu, 2, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EINVAL, "cu end");
    const int32_t cu[] = {0, 60, 128};
    expect(bimamba_ssd_fwd(&s, &d, NULL, cu, 2, (const float *)dev, NULL, y, NULL, 0, NULL),
           BIMAMBA_EUNSUPPORTED, "state with cu");
    expect(bimamba_ssd_fwd(&s, &d, NULL, cu, 2, NULL, NULL, y, NULL, 0, NULL), BIMAMBA_EWORKSPACE, "no workspace");
    expect(bimamba_ssd_workspace_size(&s, 2, &n), BIMAMBA_OK, "workspace size");
    expect(bimamba_ssd_fwd(&s, &d, NULL, cu, 2, NULL, NULL, y, dev, n - 1, NULL), BIMAMBA_EWORKSPACE, "small workspace");
    expect(bimamba_ssd_workspace_size(&s, -1, &n), BIMAMBA_EINVAL, "nseq < 0");
    expect(bimamba_ssd_fwd_streams(&s, &d, NULL, NULL, 0, NULL, NULL, y, y, NULL, 0, NULL), BIMAMBA_EINVAL, "streams bwd");
    expect(bimamba_ssd_fwd_streams(&s, &d, &d, NULL, 0, NULL, NULL, y, y, NULL, 0, NULL), BIMAMBA_EINVAL, "streams alias");

    /* the no-allocation variant: tables beyond its buffer, and the checks of bimamba_ssd_fwd */
    bimamba_shape big = s; big.seqlen = (int)(BIMAMBA_NOALLOC_SCRATCH_BYTES / 4) + 64;
    const int32_t big_cu[] = {0, big.seqlen};
    expect(bimamba_ssd_fwd_noalloc(&big, &d, NULL, big_cu, 1, NULL, NULL, y, NULL), BIMAMBA_EWORKSPACE, "noalloc tables");
    expect(bimamba_ssd_fwd_noalloc(&t, &d, NULL, NULL, 0, NULL, NULL, y, NULL), BIMAMBA_EINVAL, "noalloc flags");

    /* block step and the state object */
    expect(bimamba_block_step(NULL, &s, &d, &d, 0, y, NULL), BIMAMBA_EINVAL, "no state");
    expect(bimamba_state_alloc(NULL, 1, 1, 1, 1), BIMAMBA_EINVAL, "alloc out");
    bimamba_state *st = NULL;
    expect(bimamba_state_alloc(&st, 0, 4, 64, 128), BIMAMBA_EINVAL, "alloc slots");
    expect(bimamba_state_reset(NULL, NULL, 0, NULL), BIMAMBA_EINVAL, "reset null");
    expect(bimamba_state_free(NULL), BIMAMBA_OK, "free null");
    expect(bimamba_state_data(NULL) == NULL ? 0 : 1, 0, "data null");

    /* backward, convolution, epilogue, merge */
    bimamba_grad g = {(float *)dev, (float *)dev, (float *)dev, (float *)dev, (float *)dev, NULL};
    t = s; t.headdim = 32;
    expect(bimamba_ssd_bwd(&t, &d, NULL, y, &g, NULL, NULL, 0, NULL), BIMAMBA_EUNSUPPORTED, "bwd shape");
    expect(bimamba_ssd_bwd(&s, &d, &d, y, &g, NULL, NULL, 0, NULL), BIMAMBA_EINVAL, "bwd grads");
    bimamba_conv_shape cs = {1, 128, 4, 64, 128, 1, 4, BIMAMBA_BF16, 1, 0};
    bimamba_conv_dir cd = {dev, (const float *)dev, NULL, dev, dev, dev};
    bimamba_conv_shape ct = cs; ct.width = 5;
    expect(bimamba_conv1d(&ct, &cd, NULL, NULL, 0, NULL, NULL, NULL, 0, NULL), BIMAMBA_EUNSUPPORTED, "conv width");
    expect(bimamba_conv1d(&cs, &cd, NULL, NULL, 0, dev, (void *)((uintptr_t)dev + 16), NULL, 0, NULL),
           BIMAMBA_EINVAL, "conv contexts overlap");
    expect(bimamba_conv1d_workspace_size(&cs, -2, &n), BIMAMBA_EINVAL, "conv nseq");
    expect(bimamba_state_alloc_conv(&st, 1, 4, 64, 128, 1, 5, BIMAMBA_BF16), BIMAMBA_EINVAL, "conv state width");
    expect(bimamba_state_alloc_conv(&st, 1, 1, 3, 2, 1, 4, BIMAMBA_BF16), BIMAMBA_EUNSUPPORTED, "conv state slot bytes");
    expect(bimamba_state_conv_ctx(NULL) == NULL ? 0 : 1, 0, "conv ctx null");
    expect(bimamba_block_step_conv(NULL, &cs, &cd, &cd, &s, &d, &d, 1, y, NULL), BIMAMBA_EINVAL, "conv step no state");
    expect(bimamba_gated_norm(8, 300, 300, BIMAMBA_BF16, y, dev, y, 1e-5f, dev, NULL), BIMAMBA_EUNSUPPORTED, "norm channels");
    expect(bimamba_gated_norm(8, 512, 256, 9, y, dev, y, 1e-5f, dev, NULL), BIMAMBA_EINVAL, "norm dtype");
    expect(bimamba_merge_linear(8, 33, 16, y, y, dev, NULL, y, NULL), BIMAMBA_EUNSUPPORTED, "merge cin");
    expect(bimamba_merge_linear(-1, 32, 16, y, y, dev, NULL, y, NULL), BIMAMBA_EINVAL, "merge rows");

    /* profiling and messages */
    char names[64];
    int counts[1];
    double ms[1];
    expect(bimamba_profile_end(names, 64, counts, ms, 1), BIMAMBA_EINVAL, "profile end first");
    expect(strlen(bimamba_status_str(BIMAMBA_EWORKSPACE)) > 0 ? 0 : 1, 0, "status string");
    expect(bimamba_version(), BIMAMBA_VERSION, "version");
    printf(fails ? "abi sanitized checks: %d FAILED\n" : "abi sanitized checks: ok%d\n", fails);
    return fails ? 1 : 0;
}
