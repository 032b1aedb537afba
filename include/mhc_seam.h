/*
 * mhc_seam.h -- C ABI of the MI355X (gfx950) fused, delayed mHC seam.
 *
 * Sources (web pages, cited by title and section):
 *   [MEGA]  "[FlyDSL] Single-launch Mega-mHC on gfx950" (ROCm/aiter PR 6179)
 *   [FUSED] "[Triton/Gluon] [gfx950] [dsv4.1-flash] mHC fused kernel"
 *           (ROCm/aiter PR 5824)
 *
 * One seam is the mHC work between two transformer sub-layers [FUSED,
 * description].  Per token t, with n = 4 residual streams of width H, in the
 * order of [MEGA, Kernel Architecture]:
 *   1. post-mix   x'[j] = sum_i res[t][j][i] * x[t][i] + post[t][j] * y[t],
 *                 stored as the bf16 residual_out;
 *   2. collapse   u = sum_i pre[t][i] * x'[i] with the pre CARRIED from the
 *                 previous seam (the "delayed" seam [MEGA, Motivation]);
 *   3. RMSNorm    norm = u * rsqrt(mean(u^2) + eps) * gamma (bf16 [T][H]),
 *                 optionally quantised per 32 elements to ue8m0 + e4m3
 *                 [MEGA, Kernel Architecture: out_dtype];
 *   4. gates      l = rsqrt(mean(x'^2 over 4H) + eps) * (x' . fn) + bias,
 *                 next pre = sigmoid(l[0:4]), post = 2 sigmoid(l[4:8]),
 *                 res = Sinkhorn of exp(l[8:24]) as a row-major 4x4
 *                 (j = output stream, i = input stream).
 * Element rounding: fp32 arithmetic, x' and u rounded to bf16 before they
 * are used; the norm is bf16(f32(f32(u * rstd) * gamma)).
 *
 * Layouts: every tensor is dense, row-major and on the handle's device.
 *   x, residual_out  bf16 [T][4][H]   (the flattened 4H row is stream-major:
 *                                      index i*H + h, matching fn's rows)
 *   y, norm, grid    bf16 [T][H]
 *   pre, post        f32  [T][4]       pre_out, post_out  f32 [T][4]
 *   res              f32  [T][4][4]    res_out            f32 [T][4][4]
 *   codes            u8   [T][H]       OCP e4m3fn
 *   scales           u8   [T][H/32]    ue8m0: 2^(s-127) multiplies the codes
 *   fn               f32  [4H][24]     gamma bf16 [H]     bias f32 [24]
 *
 * Ownership: the caller owns every tensor and stream and keeps buffers alive
 * until the stream has finished the seam.  The handle owns its packed copy
 * of fn, its copies of gamma and bias and its per-stream scratch.
 *
 * Errors: every function returns an mhc_seam_status; nothing throws or
 * aborts across the ABI.  mhc_seam_last_error() gives a message for the
 * calling thread's most recent failure.
 */
#ifndef MHC_SEAM_H
#define MHC_SEAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mhc_seam_status {
    MHC_SEAM_OK = 0,
    MHC_SEAM_INVALID_ARG = 1,        /* bad size, pointer set, alignment, overlap */
    MHC_SEAM_UNSUPPORTED_DEVICE = 2, /* not a gfx950 device [MEGA, Limitations] */
    MHC_SEAM_OUT_OF_MEMORY = 3,
    MHC_SEAM_HIP_ERROR = 4,          /* a HIP runtime call failed */
    MHC_SEAM_CAPTURE_ALLOC = 5       /* this stream has no scratch yet and is being
                                        captured: run it once eagerly first
                                        [MEGA, Kernel Architecture: CUDA graphs] */
} mhc_seam_status;

typedef enum mhc_seam_form {
    MHC_SEAM_POST = 0,     /* post-mix with the layer output y */
    MHC_SEAM_NO_POST = 1   /* no layer output: x' = x, no residual_out */
} mhc_seam_form;

typedef enum mhc_seam_out_dtype {
    MHC_SEAM_OUT_BF16 = 0,     /* norm */
    MHC_SEAM_OUT_FP8_GRID = 1, /* norm + grid (bf16 copy of the dequantised codes) */
    MHC_SEAM_OUT_MXFP8 = 2,    /* norm + codes + scales (ue8m0 per 32) */
    MHC_SEAM_OUT_MXFP8_G128 = 3 /* norm + codes + scales (ue8m0 per 128 elements,
                                   [T][H/128]; H a multiple of 128): the
                                   128-wide grouping [MEGA, Limitations], by a
                                   quantiser pass over the norm */
} mhc_seam_out_dtype;

typedef struct mhc_seam *mhc_seam_t;

/* Create-time description.  Zero-initialise, then set the fields. */
typedef struct mhc_seam_desc {
    int32_t H;              /* stream width; multiple of 64 */
    int32_t n;              /* residual streams; must be 4 */
    float eps;              /* RMSNorm epsilon of both norms; 0 selects 1e-6 */
    int32_t sinkhorn_iters; /* 0 selects 20 */
    const float *fn;        /* device, f32 [4H][24] */
    const uint16_t *gamma;  /* device, bf16 [H] */
    const float *bias;      /* device, f32 [24] */
    int64_t max_tokens;     /* largest T a run may pass */
    int32_t device;         /* HIP device ordinal */
    /* launch-policy overrides; 0 = automatic */
    int32_t ksplit;         /* column splits per 16-token block, in 64-column
                               segments (1 = whole rows) */
    int32_t spin_polls;     /* split mode: polls a split makes for every split
                               of its block to arrive before handing its
                               segments to the finisher; 0 = default, -1 =
                               never wait */
    int32_t reserved[6];
} mhc_seam_desc;

/* Per-run arguments.  A pointer must be set exactly when the form and the
 * out_dtype use it and be NULL otherwise; anything else is INVALID_ARG
 * (incomplete post-mix inputs are an error, never silently ignored). */
typedef struct mhc_seam_args {
    int64_t T;              /* tokens; 0 is a no-op that returns OK (required
                               pointers may then be NULL) */
    int32_t form;           /* mhc_seam_form */
    int32_t identity_pre;   /* 1: first block, no carried pre (pre = 1/4) */
    int32_t out_dtype;      /* mhc_seam_out_dtype */
    int32_t unshifted;      /* 0: the delayed seam, collapse with the carried
                               pre.  1: the unshifted ordering: gates from x'
                               first, then the collapse with the fresh pre
                               (pre_out, as written); pre must be NULL and
                               identity_pre 0 [MEGA, Test Result: notes on
                               what each compared kernel computes].  Runs as
                               two launches; the second re-reads x' */
    const uint16_t *x;      /* bf16 [T][4][H]                       always */
    const uint16_t *y;      /* bf16 [T][H]                          POST */
    const float *pre;       /* f32 [T][4]                  !identity_pre && !unshifted */
    const float *post;      /* f32 [T][4]                           POST */
    const float *res;       /* f32 [T][4][4]                        POST */
    uint16_t *residual_out; /* bf16 [T][4][H]                       POST */
    uint16_t *norm;         /* bf16 [T][H]                          always */
    uint16_t *grid;         /* bf16 [T][H]                          FP8_GRID */
    uint8_t *codes;         /* e4m3fn [T][H]                        MXFP8, MXFP8_G128 */
    uint8_t *scales;        /* ue8m0 [T][H/32] (MXFP8), [T][H/128] (MXFP8_G128) */
    float *pre_out;         /* f32 [T][4]                           always */
    float *post_out;        /* f32 [T][4]                           always */
    float *res_out;         /* f32 [T][4][4]                        always */
} mhc_seam_args;

/*
 * Create a handle: checks the device is gfx950, packs fn on the device
 * (bf16 hi/lo pairs in the matrix-core operand order, [MEGA, Kernel
 * Architecture: fn pre-packed]), copies gamma and bias, allocates scratch for
 * the null stream and synchronises once.  The caller may free or reuse its
 * weight buffers after this returns.  Weights are fixed for the handle's
 * life.  Returns OK, INVALID_ARG, UNSUPPORTED_DEVICE, OUT_OF_MEMORY or
 * HIP_ERROR; *out is NULL on failure.
 */
int mhc_seam_create(const mhc_seam_desc *desc, mhc_seam_t *out);

/*
 * Enqueue one seam on `stream` (a hipStream_t; NULL is the null stream).
 * Asynchronous; no host synchronisation and no allocation, except that the
 * first run on a new stream whose launch plan splits blocks over workgroups
 * (small T, or a tail after full rounds of the CUs) allocates and zeroes
 * that stream's scratch, sized once for every T <= max_tokens
 * (CAPTURE_ALLOC if the stream is being captured at that moment).  That
 * scratch never moves, so a graph captured on the stream stays valid after
 * eager runs of any other T on it.  Runs on one stream serialise; runs of
 * one handle on different streams may overlap.
 * Rules (INVALID_ARG otherwise): T <= max_tokens and T*4*H*2 < 2^31 [MEGA,
 * Limitations]; pointers 16-byte aligned; no output range overlaps an input
 * or another output.  Groups of 32 norm elements holding inf or NaN give
 * unspecified codes and scales [MEGA, Limitations].
 */
int mhc_seam_run(mhc_seam_t h, const mhc_seam_args *args, void *stream);

/*
 * mhc_seam_run for callers that cannot allocate device memory: code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, rules and results as mhc_seam_run, with the same kernels; the
 * difference is where split-mode scratch (the per-block arrival counters and
 * hand-off masks, the partial sums and the hand-off copy of u of launches
 * that split blocks over workgroups) lives: in one fixed array of
 * MHC_SEAM_NOALLOC_SCRATCH_BYTES per GPU inside the library, set up by
 * mhc_seam_create on the handle's device and kept until the process ends.
 * This call never allocates (no hipMalloc, no host allocation) and may be
 * captured into a graph on any stream.
 * Limit: a launch plan with more than 2048 split blocks, or whose partials
 * and u exceed the array, is refused with INVALID_ARG and a message giving
 * the size (at H = 5120 every T fits; at H = 7168, whose launches are all
 * split, T up to about 2300).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other handles) race on it and must be
 * serialised by the caller.  Runs of mhc_seam_run use their own per-stream
 * scratch and do not share it.
 */
#define MHC_SEAM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int mhc_seam_run_noalloc(mhc_seam_t h, const mhc_seam_args *args, void *stream);

/*
 * Wait for every stream the handle has enqueued a seam on (and no other),
 * then free what the handle owns: the packed fn, gamma, bias and the
 * per-stream scratch ([MEGA, Technical Details]: the wrapper's per-stream
 * scratch and fn pre-pack cache).  Each of those streams must still exist
 * when this is called.  NULL is OK.  HIP_ERROR if a synchronisation fails
 * (the handle is freed all the same).
 */
int mhc_seam_destroy(mhc_seam_t h);

/*
 * Check desc and args without a device, by the same rules create and run
 * apply: the review findings on [FUSED] (optional pre_mix, dense fp32 gate
 * operands, contiguous residual_out, incomplete post-mix inputs rejected)
 * and [MEGA, Limitations] (T*4*H*2 < 2^31).  desc->fn/gamma/bias must be
 * set; device pointers are not dereferenced.  Returns OK or INVALID_ARG.
 */
int mhc_seam_validate(const mhc_seam_desc *desc, const mhc_seam_args *args);

/*
 * Launch plan the library would use for H, T and a CU count (host only, for
 * tests and tuning): the policy of [MEGA, Kernel Architecture], which picks
 * the token block, the column splits and the split count from T and the CU
 * count.  ksplit_override as in mhc_seam_desc.  OK or INVALID_ARG.
 */
typedef struct mhc_seam_plan {
    int32_t blocks;          /* 16-token blocks */
    int32_t ksplit;          /* column splits per block */
    int32_t segs_per_split;  /* 64-column segments each split covers */
    int32_t grid;            /* workgroups launched */
    int32_t row_segs;        /* whole-row mode: segments per wave (0 = split mode) */
    int32_t rows_blocks;     /* whole-row mode: blocks run whole; the remaining
                                blocks (a tail after full rounds of the CUs)
                                run as ksplit splits each, in the same launch
                                when a split has at most 8 segments, else in a
                                split launch after it (grid counts both) */
    int32_t reserved[2];
} mhc_seam_plan;

int mhc_seam_plan_for(int32_t H, int64_t T, int32_t cu_count,
                      int32_t ksplit_override, mhc_seam_plan *out);

/*
 * Status codes as text.  The errors the pages' wrapper raises (a capture
 * that would need scratch [MEGA, Kernel Architecture: CUDA graphs]; bad
 * operands, the review findings on [FUSED]) are status codes here, since
 * nothing throws across the ABI.  The string is static; unknown codes give
 * "unknown status".
 */
const char *mhc_seam_status_string(int status);

/* Message of the calling thread's most recent failed call (thread-local,
 * valid until that thread's next failing call); "" if none failed. */
const char *mhc_seam_last_error(void);

/*
 * MXFP8 quantisation of any bf16 [rows][H] device tensor in groups of
 * `group` contiguous elements (32: the seam's fused quantiser [MEGA, Kernel
 * Architecture: out_dtype]; 128: the 128-wide grouping [MEGA, Limitations]),
 * with the same device code: codes [rows][H] e4m3fn and scales
 * [rows][H/group] ue8m0 (both or neither), and/or grid [rows][H] bf16 =
 * decode(code) * 2^(scale-127).  H a multiple of 64 (of 128 for group 128),
 * rows*H*2 < 2^31, src/codes/grid 16-byte aligned.  Enqueued on `stream`;
 * INVALID_ARG or HIP_ERROR on failure.
 */
int mhc_seam_quantize(const uint16_t *src, int64_t rows, int32_t H, int32_t group,
                      uint8_t *codes, uint8_t *scales, uint16_t *grid, void *stream);

/*
 * Device-copy kernel used to measure the copy ceiling the seam is compared
 * against [MEGA, Realistic Bandwidth Ceiling]: copies `bytes` (a multiple of
 * 16; both pointers 16-byte aligned) from src to dst on `stream` with
 * 16-byte non-temporal loads and stores, one 256-thread workgroup per CU of
 * the current device.  Not part of the seam.
 */
int mhc_seam_copy(void *dst, const void *src, size_t bytes, void *stream);

/*
 * The copy ceiling at another read/write mix ([MEGA, Realistic Bandwidth
 * Ceiling] compares the seam with a copy of its bytes; the no_post seam reads
 * four bytes for each one it writes): reads src_bytes from src and writes
 * dst_bytes to dst, each byte once, with 16-byte non-temporal accesses, one
 * 256-thread workgroup per CU of the current device (fewer for small
 * sizes): S = 256 * workgroups threads, thread g XORs input chunks g, g + S,
 * ... into (g, ~g, 0, 0) and writes that XOR (j, 0, 0, 0) to output chunks
 * j = g, g + S, ....  Both sizes multiples of 16 and below 2^31, 0 < dst_bytes,
 * pointers 16-byte aligned, no overlap; INVALID_ARG
 * or HIP_ERROR otherwise.  Not part of the seam.
 */
int mhc_stream_mix(void *dst, size_t dst_bytes, const void *src, size_t src_bytes, void *stream);

/*
 * n -> 1 reduction of the residual streams, stored ("HC head reduce/store",
 * named among the unfused per-seam kernels in [FUSED, description] and not
 * described there; this is the seam's collapse step on its own):
 *   out[t][h] = bf16( sum_i w[t][i] * x[t][i][h] )
 * in binary32 as the collapse chain (a rounded product, then fused
 * multiply-adds in stream order, bf16 round-to-nearest-even at the end).
 *   x    bf16 [T][4][H]  device, read only
 *   w    f32  [T][4]     device per-token weights (the pre gate), or NULL for
 *                        weights of 1/4
 *   out  bf16 [T][H]     device, written; must not overlap x or w
 * H a positive multiple of 8; x, w and out 16-byte aligned.  Needs no
 * handle; enqueued on `stream` (a hipStream_t, NULL for the default
 * stream).  INVALID_ARG or HIP_ERROR on failure; T == 0 does nothing.
 */
int mhc_head_reduce(const uint16_t *x, const float *w, int64_t T, int32_t H, uint16_t *out,
                    void *stream);

/*
 * Consumer GEMM of the MXFP8 norm ([MEGA, Kernel Architecture]: the seam's
 * ue8m0/e4m3 output feeds the next layer's GEMM; [MEGA, Test Result] prices
 * the format with that GEMM).  Both operands are MXFP8 along K, in the layout
 * the seam writes (MHC_SEAM_OUT_MXFP8), so its codes and scales are `a` and
 * `a_scales` unchanged:
 *   out[t][n] = bf16( sum_k a(t,k) b(n,k) ),
 *   a(t,k) = e4m3(a[t][k]) * 2^(a_scales[t][k/32] - 127),
 *   b(n,k) = e4m3(b[n][k]) * 2^(b_scales[n][k/32] - 127),
 * accumulated in binary32 by gfx950's block-scaled MFMA, rounded once to bf16.
 *   a        u8  [T][K]     device e4m3fn codes (activations)
 *   a_scales u8  [T][K/32]  device ue8m0
 *   b        u8  [N][K]     device e4m3fn codes (weights, K contiguous)
 *   b_scales u8  [N][K/32]  device ue8m0
 *   out      bf16 [T][N]    device, written; must not overlap the inputs
 * K a positive multiple of 128 and at most 8192, N > 0, a and b 16-byte
 * aligned, the scales 4-byte aligned.  Needs no handle; enqueued on
 * `stream`.  INVALID_ARG or HIP_ERROR on failure; T == 0 does nothing.
 * Special values: codes 0x7f / 0xff and the scale byte 0xff are NaN (the OCP
 * MX encodings), so every output whose row of a or column of b holds one is
 * NaN.  The accumulator is binary32: results keep its subnormals, and an
 * output whose partial sums leave its range is +-inf (or NaN) even where the
 * exact sum would fit bf16.  The seam itself writes scale bytes 0..254 only.
 */
int mhc_mxfp8_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                   const uint8_t *b_scales, int64_t T, int32_t N, int32_t K, uint16_t *out,
                   void *stream);

/*
 * The output blocks mhc_mxfp8_gemm launches for T x N on a device with
 * cu_count compute units (the GEMM of [MEGA, Kernel Architecture]'s
 * consumer, above): *tm x *tn outputs per workgroup, staged *stages deep in
 * LDS.  Host only, no device call; the same choice the launch makes.
 * INVALID_ARG unless T is in 1 .. 2^31 - 1, N > 0, cu_count > 0 and the
 * three outputs are non-null.
 */
int mhc_mxfp8_gemm_blocks(int64_t T, int32_t N, int32_t cu_count, int32_t *tm, int32_t *tn,
                          int32_t *stages);

#ifdef __cplusplus
}
#endif

#endif /* MHC_SEAM_H */
