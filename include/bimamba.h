/*
 * bimamba: bidirectional Mamba-2 selective state-space (SSD) mixer for
 * AMD Instinct MI355X (gfx950), plain C ABI.
 *
 * The operator (per head h, group g = h / (nheads / ngroups)):
 *
 *   forward  h_t = exp(dt_t*A_h) h_{t-1} + dt_t B_t x_t^T,  y_t = C_t^T h_t + D_h x_t
 *   reverse  the same recurrence over the time-reversed sequence with its own
 *            parameters (flip / scan / flip-back, DiffuMamba blog, "network
 *            architecture"), evaluated here by index arithmetic, never a copy
 *   output   y = y_forward + y_reverse (streams merged by addition,
 *            gist.science/ja DiffuMamba summary, Sec. 2 "proposed method")
 *
 * The recurrence is Mamba-2's selective SSM, which the DiffuMamba pages name
 * as the mixer ("Fixed state, long reach: constant-size caches in large-scale
 * block diffusion", Sec. 1: a linear-time recurrence whose hidden state is a
 * fixed-size summary of the history).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers, caller-owned; the library never
 *    keeps them past the call. Layouts are dense row-major as stated below.
 *  - Every argument is validated on the host BEFORE any HIP call. On error the
 *    function returns a negative bimamba_status, records a message readable
 *    through bimamba_last_error() (per thread) and launches nothing.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream). Nothing synchronizes. A failed launch returns BIMAMBA_EHIP.
 *  - Results are deterministic: the same inputs give the same bits.
 *  - x, B, C, y and the state arrays must be 16-byte aligned.
 */
#ifndef BIMAMBA_H
#define BIMAMBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BIMAMBA_VERSION 2

typedef enum {
    BIMAMBA_F32 = 0,   /* x, dt, B, C are float                        */
    BIMAMBA_BF16 = 1   /* x, dt, B, C are bfloat16 (raw 16-bit words)  */
} bimamba_dtype;

typedef enum {
    BIMAMBA_OK = 0,
    BIMAMBA_EINVAL = -1,        /* malformed argument                        */
    BIMAMBA_EUNSUPPORTED = -2,  /* well-formed but not built for this shape  */
    BIMAMBA_ENOMEM = -3,        /* device allocation failed (state objects)  */
    BIMAMBA_EHIP = -4,          /* a HIP call or kernel launch failed         */
    BIMAMBA_EWORKSPACE = -5     /* workspace missing or too small             */
} bimamba_status;

/* Problem shape. `chunk` is the block length Q of the SSD block
 * decomposition: tokens inside one chunk interact through the masked
 * quadratic form, chunks interact only through the carried state. It changes
 * rounding, not the mathematical result. */
typedef struct {
    int batch;      /* rows; 1 when sequences are packed                    */
    int seqlen;     /* tokens per row (packed: total tokens)                */
    int nheads;     /* H                                                    */
    int headdim;    /* P                                                    */
    int d_state;    /* N                                                    */
    int ngroups;    /* G, divides H; head h reads B/C group h/(H/G)          */
    int chunk;      /* Q: 64, 128 or 256                                    */
    int dtype;      /* bimamba_dtype of x, dt, B, C                          */
    int flags;      /* 0, or BIMAMBA_DT_SOFTPLUS                              */
} bimamba_shape;
/* Shape flag: each direction's dt holds the pre-activation of the step size
 * and the scan uses softplus(dt + dt_bias[h]) (computed in fp32 as each dt
 * is read; no stored copy). Mamba-2's step-size parameterization, the mixer
 * the DiffuMamba pages name; the pages do not give it, so this is its
 * plainest form (no clamping). bimamba_ssd_fwd and bimamba_block_step only. */
#define BIMAMBA_DT_SOFTPLUS 1

/* One direction's inputs, all read-only device pointers. The reverse
 * direction is given in the SAME (forward) time order; the library walks it
 * backwards. Directions may alias any pointer. */
typedef struct {
    const void  *x;   /* [batch][seqlen][nheads][headdim]   dtype               */
    const void  *dt;  /* [batch][seqlen][nheads]            dtype, > 0, used as
                         given (already softplus'd), or the pre-activation
                         with BIMAMBA_DT_SOFTPLUS                              */
    const float *A;   /* [nheads] float, the per-head decay rate (<= 0)         */
    const void  *B;   /* [batch][seqlen][ngroups][d_state]  dtype               */
    const void  *C;   /* [batch][seqlen][ngroups][d_state]  dtype               */
    const float *D;   /* [nheads] float skip weights; NULL means D = 0          */
    const float *dt_bias; /* [nheads] float, added to dt before softplus when
                         the shape has BIMAMBA_DT_SOFTPLUS; NULL means 0;
                         ignored otherwise                                     */
} bimamba_dir;

/* Opaque per-sequence forward-state cache (the block cache of cached block
 * diffusion, "Fixed state, long reach", Sec. 1). Device memory owned by the
 * library: float [nslots][nheads][headdim][d_state], zero after alloc. */
typedef struct bimamba_state bimamba_state;

typedef void *bimamba_stream;   /* hipStream_t */

/* Bytes of device workspace bimamba_ssd_fwd needs for this shape and number
 * of packed sequences (nseq = 0 when not packed). Writes *bytes and returns
 * BIMAMBA_OK, or an error for a shape bimamba_ssd_fwd would reject. */
int bimamba_ssd_workspace_size(const bimamba_shape *s, int nseq, size_t *bytes);

/* Bidirectional SSD over whole sequences (prefill / full-sequence denoising).
 *
 *  fwd            forward-direction inputs (required).
 *  bwd            reverse-direction inputs; NULL computes the forward stream
 *                 only.
 *  cu_seqlens     HOST int32[nseq+1] offsets of sequences packed in one row
 *                 (batch must be 1), or NULL. Non-decreasing, cu[0] = 0,
 *                 cu[nseq] = seqlen; empty sequences are allowed. Each
 *                 sequence starts from a zero state in both directions.
 *  init_state     float [batch][nheads][headdim][d_state], the forward state
 *                 before token 0 of each row, or NULL (zeros). Not with
 *                 cu_seqlens.
 *  final_state    float [batch][nheads][headdim][d_state] receiving the
 *                 forward state after each row's last token, or NULL. Not with
 *                 cu_seqlens. May equal init_state (updated in place).
 *  y              float [batch][seqlen][nheads][headdim], fully overwritten.
 *  workspace      device scratch of at least bimamba_ssd_workspace_size()
 *                 bytes, 256-byte aligned; may be NULL when that size is 0.
 *                 Its contents are dead after the stream reaches the end of
 *                 this call's work.
 */
int bimamba_ssd_fwd(const bimamba_shape *s, const bimamba_dir *fwd,
                    const bimamba_dir *bwd, const int32_t *cu_seqlens, int nseq,
                    const float *init_state, float *final_state, float *y,
                    void *workspace, size_t workspace_bytes,
                    bimamba_stream stream);

/* bimamba_ssd_fwd with no device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Arguments and results as bimamba_ssd_fwd, without the
 * workspace: the library's own static device buffer of
 * BIMAMBA_NOALLOC_SCRATCH_BYTES serves instead, held by every device the
 * library runs on until the process ends (its address is looked up once per
 * device). Within that buffer the scan lengthens its segments until their
 * states fit (a row that is one segment needs none), so every shape
 * bimamba_ssd_fwd accepts runs, except packed batches whose sequence tables
 * ((nseq + 1) * 4 + seqlen * 4 bytes, each rounded up to 256) exceed the
 * buffer: those return BIMAMBA_EWORKSPACE before any HIP call. Calls that
 * overlap on one device share the buffer and race: order them on one stream
 * (or synchronize). Nothing in the buffer needs clearing. */
#define BIMAMBA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int bimamba_ssd_fwd_noalloc(const bimamba_shape *s, const bimamba_dir *fwd,
                            const bimamba_dir *bwd, const int32_t *cu_seqlens, int nseq,
                            const float *init_state, float *final_state, float *y,
                            bimamba_stream stream);

/* The same scan with the two streams kept apart, for the concatenating merge
 * (DiffuMamba blog, "network architecture": the block concatenates the
 * forward and the flipped-back reverse output and applies a Linear layer;
 * see bimamba_merge_linear). y_fwd receives the forward stream, y_bwd the
 * reverse stream, each float [batch][seqlen][nheads][headdim], fully
 * overwritten; bwd is required; no shape flag. Other arguments as
 * bimamba_ssd_fwd. */
int bimamba_ssd_fwd_streams(const bimamba_shape *s, const bimamba_dir *fwd,
                            const bimamba_dir *bwd, const int32_t *cu_seqlens, int nseq,
                            const float *init_state, float *final_state, float *y_fwd,
                            float *y_bwd, void *workspace, size_t workspace_bytes,
                            bimamba_stream stream);
/* The concatenating merge (DiffuMamba blog, "network architecture": a Linear
 * layer from the concatenated streams back to one width):
 *
 *   out[t] = W [y_fwd[t] ; y_bwd[t]] + bias,  W: cout x (2 cin)
 *
 *  rows      tokens (>= 0)
 *  cin       channels of each stream, a multiple of 32
 *  cout      output channels, a multiple of 16
 *  y_fwd     float [rows][cin], y_bwd float [rows][cin]
 *  weight    bf16 [cout][2 cin] (row o: cin weights of the forward stream,
 *            then cin of the reverse stream: a Linear layer's layout)
 *  bias      float [cout], or NULL
 *  out       float [rows][cout]; must not overlap the inputs
 * On the bf16 matrix cores: the streams are rounded to bf16 (nearest even)
 * as they are read; products accumulate in fp32. Pointers 16-byte aligned. */
int bimamba_merge_linear(long long rows, int cin, int cout, const float *y_fwd,
                         const float *y_bwd, const void *weight, const float *bias,
                         float *out, bimamba_stream stream);
/* State cache objects. alloc allocates and zeroes (synchronously) nslots
 * forward states; reset zeroes the listed slots (HOST int32 slot indices,
 * NULL = all) asynchronously on `stream`; data returns the device pointer
 * (layout above) for saving and loading; free releases it (NULL is a no-op). */
int bimamba_state_alloc(bimamba_state **out, int nslots, int nheads,
                        int headdim, int d_state);
int bimamba_state_reset(bimamba_state *st, const int32_t *slots, int n,
                        bimamba_stream stream);
float *bimamba_state_data(bimamba_state *st);
int bimamba_state_free(bimamba_state *st);

/* A state cache object that also carries the short convolution's context
 * (the depthwise filter in front of the scan, DiffuMamba blog, "network
 * architecture", d_conv = 4): besides the nslots forward SSM states, each
 * slot's last width-1 raw forward inputs (the convolution's input channels,
 * dtype [nslots][width-1][channels], channels = nheads*headdim +
 * 2*ngroups*d_state, oldest first), so that the cache of a finalized prefix
 * is exact for the whole mixer ("Fixed state, long reach", Sec. 1). Both
 * start at zero; bimamba_state_reset zeroes both for the listed slots;
 * bimamba_state_free releases both. width 2..4, dtype BIMAMBA_BF16 or
 * BIMAMBA_F32. */
int bimamba_state_alloc_conv(bimamba_state **out, int nslots, int nheads, int headdim,
                             int d_state, int ngroups, int width, int dtype);
/* Device pointer of the convolution context (layout above) for saving and
 * loading, or NULL when the object carries none. */
void *bimamba_state_conv_ctx(bimamba_state *st);

/* One cached block-diffusion denoising step ("Fixed state, long reach",
 * Sec. 1: the forward SSM state of the finalized prefix is the cache, and the
 * reverse scan is restricted to the active block). For every slot b in
 * [0, s->batch):
 *   y[b] = forward scan of the active block resumed from state[b]
 *        + reverse scan of the block alone (zero state at the block end).
 * s->seqlen is the block length (1..256), s->batch the number of slots used
 * (<= the object's nslots), inputs are [batch][seqlen]... as in
 * bimamba_ssd_fwd. With commit != 0 the block is finalized: state[b] becomes
 * the forward state after the block's last token; otherwise the cache is
 * only read. y is float [batch][seqlen][nheads][headdim]. */
int bimamba_block_step(bimamba_state *st, const bimamba_shape *s,
                       const bimamba_dir *fwd, const bimamba_dir *bwd,
                       int commit, float *y, bimamba_stream stream);

/* Writes int32 seq_idx[total] (DEVICE), the packed-sequence index of every
 * token derived from HOST cu_seqlens[nseq+1], with the same device code the
 * scan kernels use. Exposed so the index arithmetic can be checked bit for
 * bit. */
int bimamba_seq_index(const int32_t *cu_seqlens, int nseq, int total,
                      int32_t *seq_idx, bimamba_stream stream);

/* ---- Training backward ------------------------------------------------------
 *
 * Gradients of bimamba_ssd_fwd's y (whole sequences, zero initial state, no
 * packing) with respect to every input of both streams, given dy. The
 * output being the sum of the two streams (gist.science/ja DiffuMamba
 * summary, Sec. 2), both receive the same dy; each stream has its own
 * parameters (DiffuMamba blog, "network architecture"), so each gets its
 * own gradients. The models train at 1024 tokens ("Fixed state, long
 * reach", Sec. 1, contributions) with a masked-diffusion objective
 * (DiffuMamba blog, "DiffuMamba architecture", design principles).
 * Computed in fp32 from the exact inputs (bf16 or fp32), by the chain rule
 * through the block form of the recurrence in blocks of 64 positions (the
 * shape's chunk is not used here); deterministic. */
typedef struct {
    float *dx;    /* [batch][seqlen][nheads][headdim]                          */
    float *ddt;   /* [batch][seqlen][nheads]                                   */
    float *dA;    /* [nheads]                                                  */
    float *dB;    /* [batch][seqlen][ngroups][d_state] (summed over the heads
                     of each group)                                            */
    float *dC;    /* [batch][seqlen][ngroups][d_state]                         */
    float *dD;    /* [nheads], or NULL if not wanted                           */
} bimamba_grad;
/* Bytes of device workspace bimamba_ssd_bwd needs (has_bwd: both streams). */
int bimamba_ssd_bwd_workspace_size(const bimamba_shape *s, int has_bwd, size_t *bytes);
/* dy: float [batch][seqlen][nheads][headdim]. gfwd (required) and gbwd
 * (required when bwd is given) receive the gradients; every array is fully
 * overwritten and must not overlap an input. Supported: headdim in {16, 64},
 * d_state in {16, 128}. Pointers 16-byte aligned, workspace 256-byte
 * aligned. */
int bimamba_ssd_bwd(const bimamba_shape *s, const bimamba_dir *fwd,
                    const bimamba_dir *bwd, const float *dy,
                    const bimamba_grad *gfwd, const bimamba_grad *gbwd,
                    void *workspace, size_t workspace_bytes, bimamba_stream stream);
/* ---- Gated-norm epilogue ----------------------------------------------------
 *
 * The output stage after the scan: each direction is a whole Mamba block
 * (DiffuMamba blog, "network architecture") and the mixer is Mamba-2
 * (DiffuMamba summaries, methodology); the pages do not spell the stage out,
 * and Mamba-2's default is taken: the scan output y is gated by SiLU of the
 * gate branch z, then RMS-normalized over groups of consecutive channels and
 * scaled per channel:
 *
 *   v = y * silu(z),  out = v / sqrt(mean over the group of v^2 + eps) * weight
 *
 *  rows        tokens (batch * seqlen), >= 0
 *  channels    per token (nheads * headdim): a multiple of 256, at most 8192
 *  group_size  a multiple of 256 dividing channels (channels: one group)
 *  dtype       of z and of out (bimamba_dtype)
 *  y           float [rows][channels] (bimamba_ssd_fwd's output)
 *  z           dtype [rows][channels]
 *  weight      float [channels]
 *  eps         >= 0
 *  out         dtype [rows][channels]; may not overlap the inputs
 * Pointers 16-byte aligned. Computed in fp32; bf16 output rounded to nearest
 * even. */
int bimamba_gated_norm(long long rows, int channels, int group_size, int dtype,
                       const float *y, const void *z, const float *weight, float eps,
                       void *out, bimamba_stream stream);
/* ---- Short convolution in front of the scan -------------------------------
 *
 * Each direction of the bidirectional block is a whole Mamba block with its
 * own parameters, run on the flipped sequence for the reverse direction
 * (DiffuMamba blog, "network architecture"); its configuration gives a
 * convolution of width d_conv = 4 (same section). The pages do not spell the
 * convolution out; it is taken as Mamba-2's: the channels that feed the scan,
 * x (nheads*headdim) then B then C (ngroups*d_state each), each filtered by
 * its own width-W causal filter with a bias, then SiLU v/(1+exp(-v)):
 *
 *   forward  u_t = bias + sum_{k<W} weight[k] * in_{t-(W-1)+k}
 *   reverse  u_t = bias + sum_{k<W} weight[k] * in_{t+(W-1)-k}
 *            (the same filter on the flipped sequence)
 *
 * Inputs outside a token's own row or packed sequence are zero, except that
 * the forward filter of a row may start from init_ctx. For cached block
 * diffusion ("Fixed state, long reach", Sec. 1) the forward context of the
 * finalized prefix is carried next to the SSM state, and the reverse filter
 * sees zeros after the active block. The output is rounded to the input
 * dtype (round to nearest even for bf16) and split into the x, B and C arrays
 * that bimamba_ssd_fwd / bimamba_block_step read. */
typedef struct {
    int batch;      /* rows; 1 when sequences are packed                    */
    int seqlen;     /* tokens per row (packed: total tokens)                */
    int nheads;     /* x channels: nheads * headdim                         */
    int headdim;
    int d_state;    /* B and C channels: ngroups * d_state each             */
    int ngroups;
    int width;      /* W, filter length, 2..4                               */
    int dtype;      /* bimamba_dtype of the input and of the outputs         */
    int activation; /* 0: none, 1: SiLU                                     */
    int flags;      /* reserved, must be 0                                  */
} bimamba_conv_shape;
/* One direction. The reverse direction is given in forward time order. */
typedef struct {
    const void  *xbc;     /* [batch][seqlen][channels] dtype, read-only;
                             channels = nheads*headdim + 2*ngroups*d_state,
                             ordered x | B | C                                */
    const float *weight;  /* [channels][width] float; tap width-1 multiplies
                             the token itself                                  */
    const float *bias;    /* [channels] float, or NULL for no bias            */
    void *x;              /* out [batch][seqlen][nheads][headdim]   dtype     */
    void *B;              /* out [batch][seqlen][ngroups][d_state]  dtype     */
    void *C;              /* out [batch][seqlen][ngroups][d_state]  dtype     */
} bimamba_conv_dir;
/* Bytes of device workspace bimamba_conv1d needs (nonzero only when packed). */
int bimamba_conv1d_workspace_size(const bimamba_conv_shape *s, int nseq, size_t *bytes);
/* The convolution of both directions in one launch.
 *
 *  fwd, bwd     directions; bwd NULL filters the forward direction only.
 *               Outputs must not overlap any input.
 *  cu_seqlens   HOST int32[nseq+1] packed-sequence offsets (batch 1) or NULL,
 *               as for bimamba_ssd_fwd; no filter crosses a sequence start.
 *  init_ctx     dtype [batch][width-1][channels]: the forward inputs that
 *               precede token 0 of each row, oldest first; NULL = zeros. Not
 *               with cu_seqlens.
 *  final_ctx    dtype [batch][width-1][channels] receiving each row's last
 *               width-1 forward inputs (reaching into init_ctx when the row is
 *               shorter), or NULL. Not with cu_seqlens. May equal init_ctx
 *               (updated in place: then one workgroup walks each row in
 *               order, which is meant for blocks, not long rows); any other
 *               overlap is rejected.
 *  workspace    bimamba_conv1d_workspace_size() bytes, 256-byte aligned.
 *
 * xbc, x, B, C and the contexts must be 16-byte aligned; weight and bias
 * 4-byte aligned. */
int bimamba_conv1d(const bimamba_conv_shape *s, const bimamba_conv_dir *fwd,
                   const bimamba_conv_dir *bwd, const int32_t *cu_seqlens, int nseq,
                   const void *init_ctx, void *final_ctx,
                   void *workspace, size_t workspace_bytes, bimamba_stream stream);

/* The block step from the block's raw convolution inputs, for a state made
 * by bimamba_state_alloc_conv: the short convolution of both directions over
 * the block (bimamba_conv1d; the forward filter starts from the state's
 * context, the reverse filter sees zeros after the block's end), then
 * bimamba_block_step on the filtered values, in stream order.
 *  cs        the convolution's shape: batch, seqlen, nheads, headdim,
 *            d_state, ngroups, dtype as in s; width and dtype as the
 *            state's context
 *  cfwd/cbwd raw inputs (xbc), filters, and the x, B, C the filtered values
 *            are written to (bimamba_conv_dir)
 *  s, fwd, bwd, y, commit
 *            as for bimamba_block_step; fwd/bwd's x, B and C must be
 *            cfwd/cbwd's outputs (checked)
 * With commit != 0 the SSM state and the context both move past the block
 * (the context then holds the block's last width-1 raw forward inputs);
 * otherwise neither changes. */
int bimamba_block_step_conv(bimamba_state *st, const bimamba_conv_shape *cs,
                            const bimamba_conv_dir *cfwd, const bimamba_conv_dir *cbwd,
                            const bimamba_shape *s, const bimamba_dir *fwd,
                            const bimamba_dir *bwd, int commit, float *y,
                            bimamba_stream stream);
/* Per-kernel timing for benchmarks and profilers, per calling thread.
 * Between bimamba_profile_begin() and bimamba_profile_end(), every kernel the
 * library launches from this thread is bracketed by two hipEvents recorded on
 * the kernel's own stream. bimamba_profile_end() waits for those events and,
 * for up to `cap` distinct kernels in first-launch order, writes the kernel's
 * name (NUL-terminated, at most name_len bytes each, into names + i*name_len),
 * its launch count and its summed duration in milliseconds. It returns the
 * number of distinct kernels seen, or a negative status. The work itself is
 * unchanged; only event records are added between launches. */
int bimamba_profile_begin(void);
int bimamba_profile_end(char *names, int name_len, int *counts, double *ms, int cap);

const char *bimamba_status_str(int status);
const char *bimamba_last_error(void);
int bimamba_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BIMAMBA_H */
