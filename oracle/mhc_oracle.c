/*
 * mhc_oracle.c -- plain, slow CPU oracle for the fused, delayed mHC seam.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links, calls or includes it, and it shares no code with the GPU path.
 *
 * Sources (web pages, cited by title and section):
 *   [MEGA]   "[FlyDSL] Single-launch Mega-mHC on gfx950" (ROCm/aiter PR 6179)
 *   [FUSED]  "[Triton/Gluon] [gfx950] [dsv4.1-flash] mHC fused kernel"
 *            (ROCm/aiter PR 5824)
 *
 * What is computed.  [MEGA, Motivation] lists the seam's work in one launch:
 * post-mix, input mix with the carried pre, RMSNorm, gate projection,
 * Sinkhorn and next pre, writing the bf16 norm and optionally its per-32
 * ue8m0 FP8 quantisation.  [MEGA, Kernel Architecture] fixes the order:
 * post-mix -> collapse -> sum of squares + gate projection -> reduce -> rstd
 * -> Sinkhorn -> layer input.  The pages print no formulas; the per-token
 * definitions below are the plain reading of that step list with n = 4
 * residual streams of width H:
 *
 *   x'[j]  = sum_i res[j][i] * x[i] + post[j] * y        (post-mix)
 *   u      = sum_i pre[i] * x'[i]                         (collapse)
 *   norm   = u * rsqrt(mean(u^2) + eps) * gamma           (RMSNorm)
 *   l[k]   = rsqrt(mean(x'^2 over 4H) + eps) * (x' . fn[:,k]) + bias[k]
 *   pre'   = sigmoid(l[0:4]); post' = 2*sigmoid(l[4:8])
 *   res'   = Sinkhorn(exp(l[8:24] as a 4x4 matrix))
 *
 * Rounding points (a reading; the pages only say bf16 activations and
 * fp32 gates).  f32() is IEEE binary32 round-to-nearest-even, bf16() is
 * binary32 -> bfloat16 round-to-nearest-even.
 *   - the post-mix and collapse chains are binary32, left to right, the
 *     first term a rounded product and every later term one fused
 *     multiply-add (fmaf);
 *   - x' is rounded to bf16 (it is the stored residual) and that rounded
 *     value feeds the collapse, the sum of squares and the gate projection;
 *   - u is rounded to bf16 before the norm;
 *   - sums of squares, dot products, rstd, the gates and Sinkhorn are
 *     evaluated in binary64 and rounded to binary32 where stored;
 *   - norm = bf16( f32( f32(u * rstd_u) * gamma ) ), rstd_u rounded to f32.
 *
 * Forms [MEGA, Test Plan] "post, no_post, identity_pre":
 *   - no_post: there is no layer output; x' = x and no residual is written;
 *   - identity_pre (first block, no carried pre): pre = (1/4, 1/4, 1/4, 1/4).
 *
 * Quantiser [MEGA, Motivation / Kernel Architecture / Limitations]: per 32
 * contiguous norm elements one ue8m0 scale byte and 32 OCP e4m3fn codes;
 * fp8_grid is the bf16 copy of the dequantised codes.  Reading of the scale
 * rule: the smallest integer k with 448 * 2^k >= amax, clamped to
 * [-127, 127] (all-zero groups take -127); scale byte = k + 127.  The crafted
 * groups "amax = 448 * 2^k" of [MEGA, Test Plan] sit exactly on this rule's
 * boundary.  Groups holding inf or NaN are unspecified [MEGA, Limitations].
 *
 * Parity pins for every function here live in the test suite: closed forms,
 * invariants, library special cases and brute force (see the tests named
 * test_oracle_*).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- scalar conversions -------------------------------------------------- */

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* ---- gates: sigmoid and Sinkhorn ------------------------------------------ */

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/*
 * Sinkhorn, the step after rstd in [MEGA, Kernel Architecture]:
 * M[j][i] = exp(logit[4j+i]); each iteration divides every row by its sum
 * over i, then every column by its sum over j.  j is the output stream.
 */
static void sinkhorn4(const double *logit16, int iters, double *out16)
{
    double m[4][4];
    for (int j = 0; j < 4; ++j)
        for (int i = 0; i < 4; ++i)
            m[j][i] = exp(logit16[4 * j + i]);
    for (int it = 0; it < iters; ++it) {
        for (int j = 0; j < 4; ++j) {
            double s = 0.0;
            for (int i = 0; i < 4; ++i)
                s += m[j][i];
            for (int i = 0; i < 4; ++i)
                m[j][i] /= s;
        }
        for (int i = 0; i < 4; ++i) {
            double s = 0.0;
            for (int j = 0; j < 4; ++j)
                s += m[j][i];
            for (int j = 0; j < 4; ++j)
                m[j][i] /= s;
        }
    }
    for (int j = 0; j < 4; ++j)
        for (int i = 0; i < 4; ++i)
            out16[4 * j + i] = m[j][i];
}

/* ---- the seam -------------------------------------------------------------- */

/*
 * One seam over tokens [t0, t1).  Layouts are dense row-major:
 *   x [T][4][H] bf16, y [T][H] bf16, pre/post [T][4] f32, res [T][4][4] f32,
 *   fn [4H][24] f32 (row r = i*H + h of the flattened stream-major row),
 *   gamma [H] bf16, bias [24] f32;
 *   residual_out [T][4][H] bf16, norm [T][H] bf16,
 *   pre_out/post_out [T][4] f32, res_out [T][4][4] f32.
 * post_form = 0 selects no_post: y, post, res and residual_out are unused.
 * identity_pre = 1: pre is unused.
 * xb and u are caller-provided work rows of 4H and H floats.
 */
/* step 2: u = bf16(sum_i p[i] * xb[i]) elementwise over the row (the
 * binary32 chain: a rounded product, then fmaf) */
static void collapse_row(int32_t H, const float p[4], const float *xb, float *u)
{
    for (int h = 0; h < H; ++h) {
        float c = p[0] * xb[0 * (size_t)H + h];
        c = fmaf(p[1], xb[1 * (size_t)H + h], c);
        c = fmaf(p[2], xb[2 * (size_t)H + h], c);
        c = fmaf(p[3], xb[3 * (size_t)H + h], c);
        u[h] = bf16_to_f32(f32_to_bf16(c));
    }
}

/* steps 2-3: collapse x'b with p (rounded to bf16) and RMSNorm it with gamma */
static void collapse_norm(int64_t t, int32_t H, float eps, const float p[4],
                          const float *xb, const uint16_t *gamma, uint16_t *norm,
                          float *u)
{
    collapse_row(H, p, xb, u);
    double su = 0.0;
    for (int h = 0; h < H; ++h)
        su += (double)u[h] * (double)u[h];
    float rstd_u = (float)(1.0 / sqrt(su / (double)H + (double)eps));
    for (int h = 0; h < H; ++h) {
        float a = u[h] * rstd_u;
        float b = a * bf16_to_f32(gamma[h]);
        norm[(size_t)t * H + h] = f32_to_bf16(b);
    }
}

/* steps 4-5: gate projection over the flattened 4H row, then the next gates */
static void next_gates(int64_t t, int32_t H, float eps, int iters, const float *xb,
                       const float *fn, const float *bias, float *pre_out,
                       float *post_out, float *res_out)
{
    const int64_t K = 4 * (int64_t)H;
    double ss = 0.0;
    for (int64_t r = 0; r < K; ++r)
        ss += (double)xb[r] * (double)xb[r];
    double rstd_g = 1.0 / sqrt(ss / (double)K + (double)eps);
    double l[24];
    for (int k = 0; k < 24; ++k) {
        double d = 0.0;
        for (int64_t r = 0; r < K; ++r)
            d += (double)xb[r] * (double)fn[r * 24 + k];
        l[k] = rstd_g * d + (double)bias[k];
    }
    for (int i = 0; i < 4; ++i)
        pre_out[(size_t)t * 4 + i] = (float)sigmoid(l[i]);
    for (int j = 0; j < 4; ++j)
        post_out[(size_t)t * 4 + j] = (float)(2.0 * sigmoid(l[4 + j]));
    double m[16];
    sinkhorn4(l + 8, iters, m);
    for (int e = 0; e < 16; ++e)
        res_out[(size_t)t * 16 + e] = (float)m[e];
}

/*
 * unshifted = 1 selects the other ordering of the method ([MEGA], Test
 * Result, the notes on what each compared kernel computes: an unshifted
 * variant): the gates are computed from x' first and the collapse uses the
 * fresh pre (pre_out as stored, binary32) instead of the carried one; the
 * RMSNorm and everything else are as in the delayed seam.  pre is unused.
 */
static void seam_token(int64_t t, int32_t H, int post_form, int identity_pre,
                       int unshifted, float eps, int iters, const uint16_t *x,
                       const uint16_t *y, const float *pre, const float *post,
                       const float *res, const float *fn,
                       const uint16_t *gamma, const float *bias,
                       uint16_t *residual_out, uint16_t *norm, float *pre_out,
                       float *post_out, float *res_out, float *xb, float *u)
{
    const uint16_t *xt = x + (size_t)t * 4 * H;

    /* step 1: post-mix; x' rounded to bf16 is the stored residual */
    for (int j = 0; j < 4; ++j) {
        for (int h = 0; h < H; ++h) {
            float v;
            if (post_form) {
                const float *r = res + (size_t)t * 16 + 4 * j;
                float a = r[0] * bf16_to_f32(xt[0 * (size_t)H + h]);
                a = fmaf(r[1], bf16_to_f32(xt[1 * (size_t)H + h]), a);
                a = fmaf(r[2], bf16_to_f32(xt[2 * (size_t)H + h]), a);
                a = fmaf(r[3], bf16_to_f32(xt[3 * (size_t)H + h]), a);
                a = fmaf(post[(size_t)t * 4 + j],
                         bf16_to_f32(y[(size_t)t * H + h]), a);
                uint16_t b = f32_to_bf16(a);
                residual_out[((size_t)t * 4 + j) * H + h] = b;
                v = bf16_to_f32(b);
            } else {
                v = bf16_to_f32(xt[(size_t)j * H + h]);
            }
            xb[(size_t)j * H + h] = v;
        }
    }

    if (unshifted) {
        next_gates(t, H, eps, iters, xb, fn, bias, pre_out, post_out, res_out);
        collapse_norm(t, H, eps, pre_out + (size_t)t * 4, xb, gamma, norm, u);
        return;
    }
    /* step 2-3: collapse with the carried pre (the delayed step), RMSNorm */
    float p[4];
    for (int i = 0; i < 4; ++i)
        p[i] = identity_pre ? 0.25f : pre[(size_t)t * 4 + i];
    collapse_norm(t, H, eps, p, xb, gamma, norm, u);
    /* step 4-5: gate projection and next gates */
    next_gates(t, H, eps, iters, xb, fn, bias, pre_out, post_out, res_out);
}

/* oracle_seam: tokens [t0, t1) of a seam over T tokens; work holds
 * oracle_max_threads() * 5 * H floats.  Returns 0, or -1 on bad sizes. */
int oracle_seam(int64_t T, int32_t H, int64_t t0, int64_t t1, int32_t post_form,
                int32_t identity_pre, int32_t unshifted, float eps, int32_t iters,
                const uint16_t *x, const uint16_t *y, const float *pre,
                const float *post, const float *res, const float *fn,
                const uint16_t *gamma, const float *bias,
                uint16_t *residual_out, uint16_t *norm, float *pre_out,
                float *post_out, float *res_out, float *work)
{
    if (T < 0 || H <= 0 || t0 < 0 || t1 > T || t0 > t1 || iters < 0 ||
        (unshifted && identity_pre))
        return -1;
    /* work: per thread 5H floats (x' rows and u) */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = t0; t < t1; ++t) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        float *xb = work + (size_t)tid * 5 * H;
        float *u = xb + 4 * (size_t)H;
        seam_token(t, H, post_form, identity_pre, unshifted, eps, iters, x, y, pre, post,
                   res, fn, gamma, bias, residual_out, norm, pre_out, post_out,
                   res_out, xb, u);
    }
    return 0;
}

/*
 * oracle_head_reduce: the n -> 1 reduction of the streams, stored.
 * [FUSED, description] names an HC head reduce/store kernel among the
 * unfused per-seam kernels and says nothing more about it.  The reading
 * taken here: the collapse step on its own over the stored streams,
 *   out[t][h] = bf16( sum_i w[t][i] * x[t][i][h] )
 * with the collapse's binary32 chain (collapse_row), w f32 [T][4] per-token
 * weights (the pre gate), or w == NULL for the identity weights 1/4.
 * x bf16 [T][4][H], out bf16 [T][H].  Returns 0, or -1 on bad sizes.
 */
int oracle_head_reduce(int64_t T, int32_t H, const uint16_t *x, const float *w,
                       uint16_t *out)
{
    if (T < 0 || H <= 0)
        return -1;
    const float quarter[4] = {0.25f, 0.25f, 0.25f, 0.25f};
#pragma omp parallel
    {
        float *xb = malloc(sizeof(float) * 5 * (size_t)H);
        float *u = xb + 4 * (size_t)H;
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (size_t r = 0; r < 4 * (size_t)H; ++r)
                xb[r] = bf16_to_f32(x[(size_t)t * 4 * H + r]);
            collapse_row(H, w ? w + (size_t)t * 4 : quarter, xb, u);
            for (int h = 0; h < H; ++h)
                out[(size_t)t * H + h] = f32_to_bf16(u[h]);
        }
        free(xb);
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing of the CPU baseline only). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- quantiser ------------------------------------------------------------- */

/* value of a positive OCP e4m3fn code c in [0, 126] (0x7f is NaN) */
static double e4m3_value(int c)
{
    int e = (c >> 3) & 15, m = c & 7;
    return e ? ldexp(8 + m, e - 10) : ldexp(m, -9);
}

/*
 * Nearest e4m3fn code to v (|v| <= 448 here by construction of the scale),
 * ties to the even code, i.e. the even mantissa.  Zero keeps its sign.
 */
static uint8_t e4m3_encode(double v)
{
    int sign = signbit(v) ? 1 : 0;
    double a = fabs(v);
    int c = 0;
    while (c < 126 && e4m3_value(c + 1) <= a)
        ++c;
    /* now value(c) <= a < value(c+1), or c == 126 */
    if (c < 126) {
        double lo = a - e4m3_value(c), hi = e4m3_value(c + 1) - a;
        if (hi < lo || (hi == lo && (c & 1)))
            ++c;
    }
    return (uint8_t)((sign << 7) | c);
}

/* smallest integer k with 448 * 2^k >= amax, clamped to [-127, 127] */
static int scale_exp(double amax)
{
    if (amax == 0.0)
        return -127;
    int k = -127;
    while (k < 127 && ldexp(448.0, k) < amax)
        ++k;
    return k;
}

/*
 * Quantise a bf16 norm [T][H] (any norm, the GPU's own included) in groups
 * of G contiguous elements along H: G = 32 is the seam's MXFP8 output
 * [MEGA, Kernel Architecture: out_dtype]; G = 128 is the 128-wide grouping
 * for 128 x 128-block checkpoints that [MEGA, Limitations] lists as missing,
 * read here as the same ue8m0 scale rule over 128 elements.
 * codes [T][H] u8, scales [T][H/G] u8, grid [T][H] bf16; any may be NULL.
 * H must be a multiple of G.  Returns 0, or -1 on bad sizes.
 */
int oracle_quantize_groups(int64_t T, int32_t H, int32_t G, const uint16_t *norm,
                           uint8_t *codes, uint8_t *scales, uint16_t *grid)
{
    if (T < 0 || H <= 0 || (G != 32 && G != 128) || H % G)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int g = 0; g < H / G; ++g) {
            const uint16_t *v = norm + (size_t)t * H + (size_t)G * g;
            double amax = 0.0;
            for (int e = 0; e < G; ++e) {
                double a = fabs((double)bf16_to_f32(v[e]));
                if (a > amax)
                    amax = a;
            }
            int k = scale_exp(amax);
            if (scales)
                scales[(size_t)t * (H / G) + g] = (uint8_t)(k + 127);
            for (int e = 0; e < G; ++e) {
                uint8_t c = e4m3_encode(ldexp((double)bf16_to_f32(v[e]), -k));
                size_t idx = (size_t)t * H + (size_t)G * g + e;
                if (codes)
                    codes[idx] = c;
                if (grid) {
                    double q = e4m3_value(c & 0x7f);
                    if (c & 0x80)
                        q = -q;
                    grid[idx] = f32_to_bf16((float)ldexp(q, k));
                }
            }
        }
    }
    return 0;
}

/* the seam's per-32 quantiser */
int oracle_quantize(int64_t T, int32_t H, const uint16_t *norm, uint8_t *codes,
                    uint8_t *scales, uint16_t *grid)
{
    return oracle_quantize_groups(T, H, 32, norm, codes, scales, grid);
}

/* ---- bulk entry points used by the pins ------------------------------------ */

void oracle_f32_to_bf16(int64_t n, const float *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16(in[i]);
}

/* codes of bf16 values v scaled by 2^-k */
void oracle_e4m3_encode_scaled(int64_t n, const uint16_t *v, int32_t k,
                               uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_encode(ldexp((double)bf16_to_f32(v[i]), -k));
}

/* value of an e4m3fn code with its sign (0x7f / 0xff: NaN) */
static double e4m3_signed(int c)
{
    double q = (c & 0x7f) == 0x7f ? NAN : e4m3_value(c & 0x7f);
    return (c & 0x80) ? -q : q;
}

/* value of a ue8m0 scale byte: 2^(s-127) for s = 0..254; 0xff is NaN in the
 * OCP Microscaling (MX) format, the format of the seam's codes and scales */
static double e8m0_value(int s)
{
    return s == 0xff ? NAN : ldexp(1.0, s - 127);
}

void oracle_e4m3_decode(int64_t n, const uint8_t *codes, double *out)
{
    for (int64_t i = 0; i < n; ++i) {
        out[i] = e4m3_signed(codes[i]);
    }
}

/*
 * oracle_mxfp8_gemm: the consumer GEMM of the MXFP8 norm.  [MEGA, Kernel
 * Architecture] feeds the ue8m0/e4m3 output to the next layer's GEMM and
 * [MEGA, Test Result] prices the scale format with that GEMM included; the
 * pages give no GEMM of their own.  Reading: both operands in the seam's
 * MXFP8 format along K (e4m3fn codes, one ue8m0 scale per 32 consecutive K
 * elements), the activations a [T][K] and the weights b [N][K]:
 *   out[t][n] = sum_k dec(a[t][k]) 2^(sa[t][k/32]-127) dec(b[n][k]) 2^(sb[n][k/32]-127)
 * evaluated in binary64 (every product is exact there; the sums cannot
 * overflow binary64); absum gets sum_k |a b| for the accumulation bound of a
 * binary32 evaluation.  A scale byte of 0xff is NaN (OCP MX), so every output
 * whose row or column holds one is NaN.
 * Returns 0, or -1 on bad sizes (K a multiple of 32).
 */
int oracle_mxfp8_gemm(int64_t T, int32_t N, int32_t K, const uint8_t *a, const uint8_t *sa,
                      const uint8_t *b, const uint8_t *sb, double *out, double *absum)
{
    if (T < 0 || N <= 0 || K <= 0 || K % 32)
        return -1;
    const int KB = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int kb = 0; kb < KB; ++kb) {
                const double ea = e8m0_value(sa[(size_t)t * KB + kb]);
                const double eb = e8m0_value(sb[(size_t)n * KB + kb]);
                for (int e = 0; e < 32; ++e) {
                    const int k = kb * 32 + e;
                    const double p = e4m3_signed(a[(size_t)t * K + k]) * ea *
                                     (e4m3_signed(b[(size_t)n * K + k]) * eb);
                    acc += p;
                    mag += fabs(p);
                }
            }
            out[(size_t)t * N + n] = acc;
            if (absum)
                absum[(size_t)t * N + n] = mag;
        }
    }
    return 0;
}

void oracle_scale_exp(int64_t n, const double *amax, int32_t *k_out)
{
    for (int64_t i = 0; i < n; ++i)
        k_out[i] = scale_exp(amax[i]);
}

/* res inputs and Sinkhorn pins: n matrices of 16 logits each */
void oracle_sinkhorn(int64_t n, const double *logits, int32_t iters,
                     double *out)
{
    for (int64_t i = 0; i < n; ++i)
        sinkhorn4(logits + 16 * i, iters, out + 16 * i);
}

void oracle_sigmoid(int64_t n, const double *in, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = sigmoid(in[i]);
}
