// seam_kernels.hip -- gfx950 kernels of the fused, delayed mHC seam.
//
// Sources (web pages, cited by title and section):
//   [MEGA]  "[FlyDSL] Single-launch Mega-mHC on gfx950" (ROCm/aiter PR 6179)
//   [FUSED] "[Triton/Gluon] [gfx950] [dsv4.1-flash] mHC fused kernel"
//
// One launch does the whole seam [MEGA, Motivation]: post-mix -> collapse
// with the carried pre -> sum of squares + gate projection -> reduce -> rstd
// -> Sinkhorn -> layer input [MEGA, Kernel Architecture].
//
// Work decomposition (our design for CDNA4, not the pages'):
//  * A workgroup is 8 wave64s and owns a block of 16 tokens.  Each wave walks
//    32-column chunks of the H columns; in a chunk, lane l holds token l%16
//    and the 8 columns 8*(l/16)..+8 of all four streams, which is exactly the
//    A operand of v_mfma_f32_16x16x32_bf16 for one stream.  The gate
//    projection x'[4H] . fn[4H,24] is therefore 4 MFMA K-steps per chunk
//    against fn pre-packed as bf16 hi/lo pairs in B-operand order [MEGA,
//    Kernel Architecture: "fn pre-packed as bf16 hi/lo in MFMA B order"]:
//    x' is exactly bf16, so x'*hi and x'*lo are exact products and the
//    result carries ~16 bits of fn.  Three 16-column tiles hold
//    hi[0:16], (hi[16:24] | lo[16:24]) and lo[0:16].
//  * Whole-row mode (ksplit = 1, large T): each wave keeps its chunks of the
//    bf16 collapse u in VGPRs until rstd is known, so x is read from HBM once
//    and u never leaves the chip; the workgroup reduces its 8 waves' partials
//    through LDS and finishes the norm, the quantiser and the gates itself.
//  * Split mode (ksplit > 1, small T): the 16-token block's chunks are split
//    over ksplit workgroups [MEGA, Kernel Architecture: split-K].  Each
//    writes its partials and its u chunks to scratch, then bumps the block's
//    agent-scope counter; the last-arriving workgroup sums the partials in
//    split order (deterministic), computes rstd and the gates and writes the
//    whole block's norm.  No workgroup ever waits on another, so nothing can
//    hang; the counter is reset by the finisher for the next launch.
//
// Elementwise chains use explicit fmaf in the order fixed by the seam's
// definition (the first term a rounded product, then fused multiply-adds,
// left to right); the library is compiled with -ffp-contract=off.  Sums of
// squares are accumulated in fp64 so that rstd rounds like the definition.

#include "seam_internal.h"

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ u32 pack_bf16(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(u32, v);
}

__device__ __forceinline__ void unpack8(const u32x4 &v, float (&f)[8])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf_lo(v[q]);
        f[2 * q + 1] = bf_hi(v[q]);
    }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8])
{
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        v[q] = pack_bf16(f[2 * q], f[2 * q + 1]);
    return v;
}

__device__ __forceinline__ u32x4 ld_nt(const uint16_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void st_nt(uint16_t *p, const u32x4 &v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- fn pack --
//
// pack[((c*4 + j)*3 + tile)*64 + lane] holds, as 8 bf16, the B operand lane
// `lane` feeds for chunk c, stream j and tile `tile`: rows
// r = j*H + 32c + 8*(lane/16) + e (e = 0..7) of column col(tile, lane%16),
// hi = bf16(fn), lo = bf16(fn - hi).
__global__ void fn_pack_kernel(const float *__restrict__ fn, int H, u32x4 *__restrict__ pack,
                               int total)
{
    int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    int lane = idx & 63;
    int tile = (idx >> 6) % 3;
    int j = (idx / 192) & 3;
    int c = idx / 768;
    int n = lane & 15, g = lane >> 4;
    int col;
    bool lo;
    if (tile == 0) {
        col = n;
        lo = false;
    } else if (tile == 2) {
        col = n;
        lo = true;
    } else {
        col = 16 + (n & 7);
        lo = n >= 8;
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        size_t r = (size_t)j * H + (size_t)c * kChunk + 8 * g + e;
        float f = fn[r * 24 + col];
        float hi = (float)(__bf16)f;
        v[e] = lo ? (float)(__bf16)(f - hi) : hi;
    }
    pack[idx] = pack8(v);
}

// ------------------------------------------------------------- quantiser --
//
// Per 32 contiguous norm elements (the four lanes l, l^16, l^32, l^48 of one
// chunk): amax, the ue8m0 exponent k = smallest integer with 448*2^k >= amax
// clamped to [-127, 127] (zero groups: -127), e4m3fn codes of v*2^-k with
// round to nearest even, and optionally the bf16 grid decode(code)*2^k
// [MEGA, Kernel Architecture: out_dtype; Limitations: per-32 ue8m0].
__device__ __forceinline__ int group_scale_exp(const u32x4 &nv)
{
    u32 m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        m = max(m, nv[q] & 0x7fffu);
        m = max(m, (nv[q] >> 16) & 0x7fffu);
    }
    m = max(m, (u32)__shfl_xor((int)m, 16));
    m = max(m, (u32)__shfl_xor((int)m, 32));
    int e = (int)(m >> 7), mant = (int)(m & 0x7f);
    // amax = (1 + mant/128) 2^(e-127); 448 = 1.75 * 2^8
    int k = (e == 0) ? -127 : e - 135 + (mant > 0x60 ? 1 : 0);
    return max(k, -127);
}

__device__ __forceinline__ u32 e4m3_code(float v, int k)
{
    float s = ldexpf(v, -k);
    u32 b = __float_as_uint(s);
    u32 sign = (b >> 24) & 0x80u;
    u32 a = b & 0x7fffffffu;
    u32 code;
    if (a >= 0x3c800000u) {                      // |s| >= 2^-6: normal e4m3
        u32 r = a + 0x7ffffu + ((a >> 20) & 1u); // round 23 -> 3 mantissa bits
        code = (r >> 20) - (120u << 3);
    } else {                                      // subnormal range: q * 2^-9
        code = (u32)rintf(__uint_as_float(a) * 512.0f);
    }
    return code | sign;
}

__device__ __forceinline__ float e4m3_dequant(u32 code, int k)
{
    u32 mag = code & 0x7fu;
    float f = (mag >= 8u) ? __uint_as_float((mag << 20) + 0x3c000000u) : (float)mag * 0x1p-9f;
    f = ldexpf(f, k);
    return (code & 0x80u) ? -f : f;
}

// ---------------------------------------------------------------- seam ----

struct Coef {
    float r[16];  // res[t][j][i] at 4j+i
    float p[4];   // post[t][j]
    float c[4];   // carried pre[t][i]
};

__device__ __forceinline__ void load_coef(const SeamParams &P, int form, int tc, Coef &k)
{
    if (form == kPost) {
        const f32x4 *r4 = reinterpret_cast<const f32x4 *>(P.res + (size_t)tc * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 v = r4[q];
            k.r[4 * q] = v[0];
            k.r[4 * q + 1] = v[1];
            k.r[4 * q + 2] = v[2];
            k.r[4 * q + 3] = v[3];
        }
        f32x4 v = *reinterpret_cast<const f32x4 *>(P.post + (size_t)tc * 4);
        k.p[0] = v[0], k.p[1] = v[1], k.p[2] = v[2], k.p[3] = v[3];
    }
    if (P.identity_pre) {
        k.c[0] = k.c[1] = k.c[2] = k.c[3] = 0.25f;
    } else {
        f32x4 v = *reinterpret_cast<const f32x4 *>(P.pre + (size_t)tc * 4);
        k.c[0] = v[0], k.c[1] = v[1], k.c[2] = v[2], k.c[3] = v[3];
    }
}

struct Acc {
    f32x4 t0, t1, t2;  // MFMA tiles
    double ssg, ssu;   // sums of squares of x' (4H) and u (H)
};

// Stream one 32-column chunk c of this lane's token: post-mix (stores the
// residual), collapse, sums of squares and the 12 MFMAs.  Returns u (bf16).
template <int FORM>
__device__ __forceinline__ u32x4 stream_chunk(const SeamParams &P, int tc, bool tvalid, int c,
                                              int grp, int lane, const Coef &k, Acc &acc)
{
    const int H = P.H;
    const int h0 = c * kChunk + grp * 8;
    const uint16_t *xr = P.x + (size_t)tc * 4 * H + h0;
    u32x4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        xv[j] = ld_nt(xr + (size_t)j * H);
    const u32x4 *fb = reinterpret_cast<const u32x4 *>(P.fnp) + (size_t)c * (4 * 3 * 64) + lane;

    u32x4 xb[4];
    if (FORM == kPost) {
        u32x4 yv = ld_nt(P.y + (size_t)tc * H + h0);
        float xf[4][8], yf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            unpack8(xv[i], xf[i]);
        unpack8(yv, yf);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = k.r[4 * j] * xf[0][e];
                a = __builtin_fmaf(k.r[4 * j + 1], xf[1][e], a);
                a = __builtin_fmaf(k.r[4 * j + 2], xf[2][e], a);
                a = __builtin_fmaf(k.r[4 * j + 3], xf[3][e], a);
                a = __builtin_fmaf(k.p[j], yf[e], a);
                o[e] = a;
            }
            xb[j] = pack8(o);
        }
        if (tvalid) {
            uint16_t *rr = P.resid + (size_t)tc * 4 * H + h0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st_nt(rr + (size_t)j * H, xb[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xb[j] = xv[j];
    }

    float xbf[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        unpack8(xb[j], xbf[j]);
    float uf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float cc = k.c[0] * xbf[0][e];
        cc = __builtin_fmaf(k.c[1], xbf[1][e], cc);
        cc = __builtin_fmaf(k.c[2], xbf[2][e], cc);
        cc = __builtin_fmaf(k.c[3], xbf[3][e], cc);
        uf[e] = cc;
    }
    u32x4 u = pack8(uf);
    float ub[8];
    unpack8(u, ub);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc.ssg += (double)xbf[j][e] * (double)xbf[j][e];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc.ssu += (double)ub[e] * (double)ub[e];

#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 b0 = fb[(j * 3 + 0) * 64];
        u32x4 b1 = fb[(j * 3 + 1) * 64];
        u32x4 b2 = fb[(j * 3 + 2) * 64];
        acc.t0 = mfma16(xb[j], b0, acc.t0);
        acc.t1 = mfma16(xb[j], b1, acc.t1);
        acc.t2 = mfma16(xb[j], b2, acc.t2);
    }
    return u;
}

struct Smem {
    float dot[kWaves][kBlockTokens][24];
    double ss[kWaves][kBlockTokens][2];
    float tot[kBlockTokens][24];
    double rstd_g[kBlockTokens];
    float rstd_u[kBlockTokens];
    int last;
};

// Each wave's MFMA tiles and sums of squares -> LDS (per wave).
__device__ __forceinline__ void wave_partials_to_lds(Smem &sm, const Acc &acc, int wave, int lane)
{
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int m = 4 * grp + i;
        sm.dot[wave][m][n] = acc.t0[i] + acc.t2[i];
        float v = acc.t1[i];
        float w = __shfl_xor(v, 8);
        if (n < 8)
            sm.dot[wave][m][16 + n] = v + w;
    }
    double g = acc.ssg, u = acc.ssu;
    g += __shfl_xor(g, 16);
    u += __shfl_xor(u, 16);
    g += __shfl_xor(g, 32);
    u += __shfl_xor(u, 32);
    if (grp == 0) {
        sm.ss[wave][n][0] = g;
        sm.ss[wave][n][1] = u;
    }
}

// Next gates of the block's 16 tokens from sm.tot and sm.rstd_g: waves 0-3,
// 16 lanes per token, lane e holds logit 8+e of the 4x4 res matrix (row
// j = e/4 is the output stream) and, for e < 8, the pre/post logit e.
__device__ void gates(const SeamParams &P, Smem &sm, int b, int wave, int lane)
{
    if (wave >= 4)
        return;
    const int m = 4 * wave + (lane >> 4), e = lane & 15;
    const int t = b * kBlockTokens + m;
    const double rg = sm.rstd_g[m];
    float lr = (float)(rg * (double)sm.tot[m][8 + e] + (double)P.bias[8 + e]);
    float lg = (float)(rg * (double)sm.tot[m][e & 7] + (double)P.bias[e & 7]);
    // Sinkhorn of exp(l) [MEGA, Kernel Architecture]; the row max is taken
    // out first, which the first row normalisation cancels exactly.
    float rmax = fmaxf(lr, __shfl_xor(lr, 1));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 2));
    float M = expf(lr - rmax);
    for (int it = 0; it < P.iters; ++it) {
        float s = M + __shfl_xor(M, 1);
        s = s + __shfl_xor(s, 2);
        M = M / s;
        s = M + __shfl_xor(M, 4);
        s = s + __shfl_xor(s, 8);
        M = M / s;
    }
    if (t < P.T) {
        P.res_out[(size_t)t * 16 + e] = M;
        float sg = 1.0f / (1.0f + expf(-lg));
        if (e < 4)
            P.pre_out[(size_t)t * 4 + e] = sg;
        else if (e < 8)
            P.post_out[(size_t)t * 4 + (e - 4)] = 2.0f * sg;
    }
}

// Norm (and quantised outputs) of one chunk from its bf16 u.
template <int OUT>
__device__ __forceinline__ void finish_chunk(const SeamParams &P, const u32x4 &u, float rs, int t,
                                             bool tvalid, int c, int grp)
{
    const int H = P.H;
    const int h0 = c * kChunk + grp * 8;
    u32x4 gv = *reinterpret_cast<const u32x4 *>(P.gamma + h0);
    float uf[8], gf[8], nf[8];
    unpack8(u, uf);
    unpack8(gv, gf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float a = uf[e] * rs;
        nf[e] = a * gf[e];
    }
    u32x4 nv = pack8(nf);
    if (tvalid)
        st_nt(P.norm + (size_t)t * H + h0, nv);
    if (OUT != kBf16) {
        int k = group_scale_exp(nv);
        float v[8];
        unpack8(nv, v);
        u32 code[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            code[e] = e4m3_code(v[e], k);
        if (OUT == kMxfp8) {
            if (tvalid) {
                u32x2 cw;
                cw[0] = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
                cw[1] = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
                *reinterpret_cast<u32x2 *>(P.codes + (size_t)t * H + h0) = cw;
                if (grp == 0)
                    P.scales[(size_t)t * (H / kChunk) + c] = (uint8_t)(k + 127);
            }
        } else {
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                q[e] = e4m3_dequant(code[e], k);
            if (tvalid)
                st_nt(P.grid + (size_t)t * H + h0, pack8(q));
        }
    }
}

// Block totals (sum of the 8 waves in LDS, fixed order) into sm.tot and
// the per-token rstds.  Threads 0..383: dots; 384..399: sums of squares.
__device__ __forceinline__ void block_totals_from_waves(const SeamParams &P, Smem &sm, int tid)
{
    if (tid < kBlockTokens * 24) {
        int m = tid / 24, q = tid % 24;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            s += sm.dot[w][m][q];
        sm.tot[m][q] = s;
    } else if (tid < kBlockTokens * 25) {
        int m = tid - kBlockTokens * 24;
        double g = 0.0, u = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            g += sm.ss[w][m][0];
            u += sm.ss[w][m][1];
        }
        sm.rstd_g[m] = 1.0 / sqrt(g / (4.0 * P.H) + (double)P.eps);
        sm.rstd_u[m] = (float)(1.0 / sqrt(u / (double)P.H + (double)P.eps));
    }
}

// Whole-row mode: one workgroup per 16-token block, RC chunks of u per wave
// held in VGPRs.
template <int FORM, int OUT, int RC>
__global__ __launch_bounds__(kThreads, 1) void seam_rows_kernel(SeamParams P)
{
    __shared__ Smem sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tok = lane & 15, grp = lane >> 4;
    const int b = blockIdx.x;
    const int t = b * kBlockTokens + tok;
    const bool tvalid = t < P.T;
    const int tc = tvalid ? t : P.T - 1;

    Coef k;
    load_coef(P, FORM, tc, k);
    Acc acc;
    acc.t0 = acc.t1 = acc.t2 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.ssg = acc.ssu = 0.0;
    u32x4 ureg[RC];
#pragma unroll
    for (int i = 0; i < RC; ++i) {
        int c = wave + kWaves * i;
        if (c < P.nchunks)
            ureg[i] = stream_chunk<FORM>(P, tc, tvalid, c, grp, lane, k, acc);
    }
    wave_partials_to_lds(sm, acc, wave, lane);
    __syncthreads();
    block_totals_from_waves(P, sm, tid);
    __syncthreads();
    const float rs = sm.rstd_u[tok];
#pragma unroll
    for (int i = 0; i < RC; ++i) {
        int c = wave + kWaves * i;
        if (c < P.nchunks)
            finish_chunk<OUT>(P, ureg[i], rs, t, tvalid, c, grp);
    }
    gates(P, sm, b, wave, lane);
}

// Split mode: workgroup (block b, split s) streams its chunk range, writes
// partials and u to scratch; the last arriver of block b finishes it.
template <int FORM, int OUT>
__global__ __launch_bounds__(kThreads, 1) void seam_split_kernel(SeamParams P)
{
    __shared__ Smem sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tok = lane & 15, grp = lane >> 4;
    // WG id -> (block, split): every split of a block gets an id of the same
    // residue mod 8, i.e. the same XCD under round-robin dispatch, so the
    // block's partials stay in one L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int b = (slot / P.ksplit) * 8 + xcd;
    const int s = slot % P.ksplit;
    if (b >= P.nblocks)
        return;
    const int t = b * kBlockTokens + tok;
    const bool tvalid = t < P.T;
    const int tc = tvalid ? t : P.T - 1;

    Coef k;
    load_coef(P, FORM, tc, k);
    Acc acc;
    acc.t0 = acc.t1 = acc.t2 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.ssg = acc.ssu = 0.0;
    const int c0 = s * P.chunks_per_split;
    const int c1 = min(c0 + P.chunks_per_split, P.nchunks);
    for (int c = c0 + wave; c < c1; c += kWaves) {
        u32x4 u = stream_chunk<FORM>(P, tc, tvalid, c, grp, lane, k, acc);
        if (tvalid)
            *reinterpret_cast<u32x4 *>(P.uscr + (size_t)t * P.H + c * kChunk + grp * 8) = u;
    }
    wave_partials_to_lds(sm, acc, wave, lane);
    __syncthreads();
    float *part = P.part + ((size_t)b * P.ksplit + s) * kBlockTokens * kPartFloats;
    if (tid < kBlockTokens * 24) {
        int m = tid / 24, q = tid % 24;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            sum += sm.dot[w][m][q];
        part[m * kPartFloats + q] = sum;
    } else if (tid < kBlockTokens * 25) {
        int m = tid - kBlockTokens * 24;
        double g = 0.0, u = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            g += sm.ss[w][m][0];
            u += sm.ss[w][m][1];
        }
        double *pd = reinterpret_cast<double *>(part + m * kPartFloats + 24);
        pd[0] = g;
        pd[1] = u;
    }
    // release this workgroup's scratch writes, then arrive
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        int old = __hip_atomic_fetch_add(P.counters + b, 1, __ATOMIC_ACQ_REL,
                                         __HIP_MEMORY_SCOPE_AGENT);
        sm.last = (old == P.ksplit - 1);
    }
    __syncthreads();
    if (!sm.last)
        return;
    __threadfence();  // acquire the other splits' writes
    if (tid == 0)
        __hip_atomic_store(P.counters + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // totals over splits in split order
    const float *pb = P.part + (size_t)b * P.ksplit * kBlockTokens * kPartFloats;
    if (tid < kBlockTokens * 24) {
        int m = tid / 24, q = tid % 24;
        float sum = 0.f;
        for (int ss = 0; ss < P.ksplit; ++ss)
            sum += pb[((size_t)ss * kBlockTokens + m) * kPartFloats + q];
        sm.tot[m][q] = sum;
    } else if (tid < kBlockTokens * 25) {
        int m = tid - kBlockTokens * 24;
        double g = 0.0, u = 0.0;
        for (int ss = 0; ss < P.ksplit; ++ss) {
            const double *pd = reinterpret_cast<const double *>(
                pb + ((size_t)ss * kBlockTokens + m) * kPartFloats + 24);
            g += pd[0];
            u += pd[1];
        }
        sm.rstd_g[m] = 1.0 / sqrt(g / (4.0 * P.H) + (double)P.eps);
        sm.rstd_u[m] = (float)(1.0 / sqrt(u / (double)P.H + (double)P.eps));
    }
    __syncthreads();
    const float rs = sm.rstd_u[tok];
    for (int c = wave; c < P.nchunks; c += kWaves) {
        u32x4 u = *reinterpret_cast<const u32x4 *>(P.uscr + (size_t)tc * P.H + c * kChunk + grp * 8);
        finish_chunk<OUT>(P, u, rs, t, tvalid, c, grp);
    }
    gates(P, sm, b, wave, lane);
}

// Copy kernel for the bandwidth ceiling: 16-byte non-temporal loads/stores.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src,
                                                   u32x4 *__restrict__ dst, size_t n)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

template <int FORM, int OUT>
hipError_t launch_form_out(const SeamParams &p, int rc, int grid, hipStream_t s)
{
    dim3 g(grid), b(kThreads);
    if (p.ksplit > 1) {
        hipLaunchKernelGGL((seam_split_kernel<FORM, OUT>), g, b, 0, s, p);
        return hipGetLastError();
    }
    switch (rc) {
    case 1: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 1>), g, b, 0, s, p); break;
    case 2: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 2>), g, b, 0, s, p); break;
    case 4: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 4>), g, b, 0, s, p); break;
    case 8: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 8>), g, b, 0, s, p); break;
    case 12: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 12>), g, b, 0, s, p); break;
    case 16: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 16>), g, b, 0, s, p); break;
    case 20: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 20>), g, b, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int reg_chunks_instance(int needed)
{
    static const int inst[] = {1, 2, 4, 8, 12, 16, 20};
    for (int v : inst)
        if (v >= needed)
            return v;
    return 0;
}

hipError_t launch_fn_pack(const float *fn, int H, void *pack, hipStream_t s)
{
    int total = (H / kChunk) * 4 * 3 * 64;
    int threads = 256;
    hipLaunchKernelGGL(fn_pack_kernel, dim3((total + threads - 1) / threads), dim3(threads), 0, s,
                       fn, H, reinterpret_cast<u32x4 *>(pack), total);
    return hipGetLastError();
}

hipError_t launch_seam(const SeamParams &p, int form, int out, int reg_chunks, int grid,
                       hipStream_t s)
{
    if (form == kPost) {
        if (out == kBf16) return launch_form_out<kPost, kBf16>(p, reg_chunks, grid, s);
        if (out == kFp8Grid) return launch_form_out<kPost, kFp8Grid>(p, reg_chunks, grid, s);
        return launch_form_out<kPost, kMxfp8>(p, reg_chunks, grid, s);
    }
    if (out == kBf16) return launch_form_out<kNoPost, kBf16>(p, reg_chunks, grid, s);
    if (out == kFp8Grid) return launch_form_out<kNoPost, kFp8Grid>(p, reg_chunks, grid, s);
    return launch_form_out<kNoPost, kMxfp8>(p, reg_chunks, grid, s);
}

hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s)
{
    size_t n = bytes / 16;
    if (n == 0)
        return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 256 * 16)
        blocks = 256 * 16;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(src), reinterpret_cast<u32x4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace mhc
