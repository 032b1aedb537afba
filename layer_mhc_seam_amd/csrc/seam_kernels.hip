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
//  * A workgroup is 8 wave64s and owns a block of 16 tokens.  Columns are
//    walked in 64-column segments (128 bytes of one row of one stream).  In
//    the "row layout" every memory instruction of a wave covers 8 tokens x
//    one full 128-byte line each: lane l handles token 8h + l/8 (h = 0, 1 is
//    the half of the block) and the 8 columns 8*(l%8)..+8 of the segment.
//    Every HBM access is a full-line access; an MFMA-shaped access (16 rows x
//    64 bytes per instruction) was measured to cap the same traffic at about
//    3.5 TB/s, two thirds of the copy rate.
//  * Post-mix, residual store, collapse, sums of squares, the norm and the
//    quantiser are elementwise or per token and run in the row layout.  Only
//    the gate projection x'[4H] . fn[4H,24] needs the matrix cores: each
//    stream's bf16 x' goes through a 2 KB per-wave LDS buffer and is read
//    back as the A operand of v_mfma_f32_16x16x32_bf16 (lane l: token l%16,
//    k-group l/16), against fn pre-packed as bf16 hi/lo pairs in B-operand
//    order (the pages pack fn the same way [MEGA, Kernel Architecture]).  x'
//    is exactly bf16, so x'*hi and x'*lo are exact products and the dots
//    carry ~16 bits of fn.  Tiles: hi[0:16], (hi[16:24] | lo[16:24]),
//    lo[0:16].
//  * Whole-row mode (large T): the bf16 collapse u of the block stays on chip
//    (LDS, the rest in VGPRs) until rstd is known, so x is read from HBM once
//    and u never leaves the chip; the workgroup reduces its waves' partials
//    through LDS and finishes the norm, the quantiser and the gates itself.
//    A short tail of blocks after full rounds of the CUs runs in split mode
//    in the same launch.
//  * Split mode (small T): a block's segments are split over up to 20
//    workgroups [MEGA, Kernel Architecture: split-K].  Each writes its
//    partials, arrives on the block's agent-scope counter, waits (bounded)
//    for the others, sums the partials itself and normalises its own u; the
//    last arriver also computes the gates.  A split that cannot wait hands
//    its u to the last arriver through scratch (protocol with split_body).
//  * The unshifted ordering runs as a post-mix + gates launch (runtime flag
//    skip_norm), then a collapse + norm launch over x' (skip_gates; the
//    collapse-only form kCollapse, without the gate projection, for
//    whole-row plans).
//
// Elementwise chains use explicit fmaf in the order the seam's definition
// fixes (the first term a rounded product, then fused multiply-adds, left to
// right); the library is compiled with -ffp-contract=off.  Sums of squares
// are accumulated in fp64 so that rstd rounds like the definition.

#include "seam_internal.h"

#ifndef SEAM_PREFETCH
#define SEAM_PREFETCH 1
#endif
#ifndef SEAM_PREFETCH_NOPOST
#define SEAM_PREFETCH_NOPOST 1
#endif
#ifndef SEAM_FN_RING
#define SEAM_FN_RING 1
#endif

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 pair -> packed bf16 pair, round to nearest even: one
// v_cvt_pk_bf16_f32 (built from two scalar casts, the compiler converted
// many pairs one value at a time and merged the halves)
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32 pack_bf16(float lo, float hi)
{
    const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
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

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Loads use buffer resources: base in SGPRs + a 32-bit per-lane offset (one
// VGPR) + a wave-uniform offset (SGPR), so the unrolled loop needs no 64-bit
// VGPR addresses.  All offsets stay below 2^31 (T*4*H*2 < 2^31 is one of the
// library's argument rules).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kAuxNT = 2;     // non-temporal (streaming) cache policy
constexpr int kAuxPlain = 0;
constexpr int kAuxSc1 = 16;   // device-coherent (agent scope) access

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

template <int AUX>
__device__ __forceinline__ u32x4 bload(rsrc_t r, int voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
}

// Stores use global_store with a uniform base and a 32-bit byte offset
// (saddr form).  Buffer stores on this target have shown their data VGPRs
// overwritten by the next VALU instruction before the wave's last lanes were
// read (no wait state is inserted), so the kernels do not use them.
template <typename V>
__device__ __forceinline__ void gstore_nt(void *base, uint32_t off, const V &v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<V *>(static_cast<char *>(base) + off));
}

template <typename V>
__device__ __forceinline__ void gstore(void *base, uint32_t off, const V &v)
{
    *reinterpret_cast<V *>(static_cast<char *>(base) + off) = v;
}

// ---------------------------------------------------------------- fn pack --
//
// pack[((c*4 + j)*3 + tile)*64 + lane] holds, as 8 bf16, the B operand lane
// `lane` feeds for 32-column chunk c, stream j and tile `tile`: rows
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

// ------------------------------------------------------ lane exchanges ----
// XOR exchanges inside a 16-lane row with DPP (no LDS round trip):
// xor 1 and 2 are quad permutes, xor 4 is a half-row mirror followed by a
// quad reversal, xor 8 a row mirror followed by a half-row mirror.  Sums
// built as XOR butterflies give the same bits in every lane of the group.
enum { kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppQuadRev = 0x1B, kDppRowRor = 0x120,
       kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141 };

template <int CTRL>
__device__ __forceinline__ u32 dpp_u32(u32 v)
{
    return (u32)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

template <int X>
__device__ __forceinline__ u32 xor_lane(u32 v)
{
    static_assert(X == 1 || X == 2 || X == 4 || X == 8, "xor within a 16-lane row");
    if (X == 1)
        return dpp_u32<kDppQuadXor1>(v);
    if (X == 2)
        return dpp_u32<kDppQuadXor2>(v);
    if (X == 4)
        return dpp_u32<kDppQuadRev>(dpp_u32<kDppRowHalfMirror>(v));
    return dpp_u32<kDppRowHalfMirror>(dpp_u32<kDppRowMirror>(v));
}

// the value of the lane R places away within the lane's 16-lane row, by a
// row rotation: one DPP move.  Its uses here do not depend on the direction.
template <int R>
__device__ __forceinline__ float ror_lane(float v)
{
    static_assert(R > 0 && R < 16, "rotation within a 16-lane row");
    return __uint_as_float(dpp_u32<kDppRowRor + R>(__float_as_uint(v)));
}

template <int X>
__device__ __forceinline__ float xor_lane(float v)
{
    return __uint_as_float(xor_lane<X>(__float_as_uint(v)));
}

template <int X>
__device__ __forceinline__ double xor_lane(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = xor_lane<X>((u32)b), hi = xor_lane<X>((u32)(b >> 32));
    return __longlong_as_double((long long)(lo | (hi << 32)));
}

// ------------------------------------------------------------- quantiser --
//
// Per 32 contiguous norm elements (the four lanes 4k..4k+3 of a row-layout
// segment): amax, the ue8m0 exponent k = smallest integer with 448*2^k >=
// amax clamped to [-127, 127] (zero groups: -127), e4m3fn codes of v*2^-k
// with round to nearest even, and optionally the bf16 grid decode(code)*2^k
// [MEGA, Kernel Architecture: out_dtype; Limitations: per-32 ue8m0].
// Largest |bf16| of the 8 values of a piece, as a bit pattern (sign cleared;
// ordered like the magnitudes).
__device__ __forceinline__ u32 amax_bits8(const u32x4 &nv)
{
    u32 m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        m = max(m, nv[q] & 0x7fffu);
        m = max(m, (nv[q] >> 16) & 0x7fffu);
    }
    return m;
}

// The ue8m0 exponent of a group whose amax has bf16 bit pattern m.
__device__ __forceinline__ int scale_exp_of_bits(u32 m)
{
    int e = (int)(m >> 7), mant = (int)(m & 0x7f);
    // amax = (1 + mant/128) 2^(e-127); 448 = 1.75 * 2^8
    int k = (e == 0) ? -127 : e - 135 + (mant > 0x60 ? 1 : 0);
    return max(k, -127);
}

// k of the 32-element group held by this lane's quad (lanes 4k..4k+3)
__device__ __forceinline__ int group_scale_exp(const u32x4 &nv)
{
    u32 m = amax_bits8(nv);
    m = max(m, xor_lane<1>(m));
    m = max(m, xor_lane<2>(m));
    return scale_exp_of_bits(m);
}

// Scale operand of gfx950's scaled fp8 conversions: the binary32 whose
// exponent field is the ue8m0 byte k + 127, i.e. 2^k (a field of 0 stands
// for 2^-127).  The encode divides by it and the decode multiplies by it,
// both exactly (powers of two).
__device__ __forceinline__ float e8m0_scale(int k) { return __uint_as_float((u32)(k + 127) << 23); }

// e4m3fn codes of v*2^-k for the 8 bf16 values of a piece, packed 4 per
// word (round to nearest even; |v*2^-k| <= 448 by the choice of k, so
// nothing saturates).  Checked bit for bit against the oracle's quantiser
// over every finite bf16 value and every k.
__device__ __forceinline__ bf16x2 bf16_pair(u32 w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ u32x2 e4m3_codes8(const u32x4 &nv, int k)
{
    // each word is copied to a scalar before the bit cast: this clang folds a
    // bit cast of a vector element to the vector's first element
    const u32 w0 = nv[0], w1 = nv[1], w2 = nv[2], w3 = nv[3];
    const float sc = e8m0_scale(k);
    s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, bf16_pair(w0), sc, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, bf16_pair(w1), sc, true);
    s16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, bf16_pair(w2), sc, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, bf16_pair(w3), sc, true);
    u32x2 w;
    w[0] = __builtin_bit_cast(u32, lo);
    w[1] = __builtin_bit_cast(u32, hi);
    return w;
}

// bf16 grid decode(code) * 2^k of the 8 codes of a piece (exact; values of
// 2^128 and above, reachable only at k >= 120, are inf like any binary32
// overflow).
__device__ __forceinline__ u32x4 e4m3_grid8(const u32x2 &w, int k)
{
    const u32 c0 = w[0], c1 = w[1];
    const float sc = e8m0_scale(k);
    const bf16x2 g0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, sc, false);
    const bf16x2 g1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, sc, true);
    const bf16x2 g2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, sc, false);
    const bf16x2 g3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, sc, true);
    u32x4 g;
    g[0] = __builtin_bit_cast(u32, g0);
    g[1] = __builtin_bit_cast(u32, g1);
    g[2] = __builtin_bit_cast(u32, g2);
    g[3] = __builtin_bit_cast(u32, g3);
    return g;
}

// Quantised outputs of one 8-value piece of a row-layout segment: scale byte
// (shared by the 4 lanes of the group), e4m3 codes and/or the bf16 grid.
__device__ __forceinline__ void quant_piece(const u32x4 &nv, uint8_t *codes,
                                            uint32_t code_off, uint8_t *scales,
                                            uint32_t scale_off, uint16_t *grid,
                                            uint32_t grid_off)
{
    const int k = group_scale_exp(nv);
    const u32x2 w = e4m3_codes8(nv, k);
    if (codes) {
        gstore_nt(codes, code_off, w);
        // the four lanes of the group hold the same k: all store it
        gstore(scales, scale_off, (uint8_t)(k + 127));
    }
    if (grid)
        gstore_nt(grid, grid_off, e4m3_grid8(w, k));
}

// ---------------------------------------------------------------- seam ----

// Per wave: the transpose rows while streaming, then (after the wave's last
// segment) its partial dot products.
union WaveLds {
    u32x4 tb[kBlockTokens][9];  // transpose rows, padded to 144 B
    float dot[kBlockTokens][24];
};

struct Smem {
    float coef[kBlockTokens][24];   // res (row-major 4x4), post, carried pre
    WaveLds w[kWaves];
    double ss[kWaves][kBlockTokens][2];
    float tot[kBlockTokens][24];
    double rstd_g[kBlockTokens];
    alignas(16) float rstd_u[kBlockTokens];
    float bias[24];
    u32 epoch;  // split mode: this launch's base of the block's arrival counter
};

struct Bufs {
    rsrc_t x, y, fn, gamma;
};

__device__ __forceinline__ Bufs make_bufs(const SeamParams &P)
{
    const uint32_t th = (uint32_t)P.T * (uint32_t)P.H;
    Bufs b;
    b.x = make_rsrc(P.x, th * 8u);
    b.y = make_rsrc(P.y, P.y ? th * 2u : 0u);
    b.fn = make_rsrc(P.fnp, (uint32_t)P.nchunks * (4u * 3u * 64u * 16u));
    b.gamma = make_rsrc(P.gamma, (uint32_t)P.H * 2u);
    return b;
}

// Row-layout geometry of one lane: piece q (8 columns) of the segment and
// the two tokens 8h + sub of the block.
struct Lane {
    int q, sub;
    int x[2];   // byte offset of token row h in [T][4][H] bf16, at piece q
    int h[2];   // ... in [T][H] bf16
    int c[2];   // ... in [T][H] u8
    int s[2];   // row offset in [T][H/32] u8
};

__device__ __forceinline__ Lane lane_geometry(const SeamParams &P, int b, int lane)
{
    Lane L;
    L.q = lane & 7;
    L.sub = lane >> 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // rows past T read and rewrite row T-1: identical bytes, no branches
        const int tc = min(b * kBlockTokens + 8 * h + L.sub, P.T - 1);
        L.x[h] = tc * (8 * P.H) + L.q * 16;
        L.h[h] = tc * (2 * P.H) + L.q * 16;
        L.c[h] = tc * P.H + L.q * 8;
        L.s[h] = tc * P.nchunks;
    }
    return L;
}

// Carried gates of the block's 16 tokens -> LDS (threads 0..383).
template <int FORM>
__device__ __forceinline__ void load_coef(const SeamParams &P, Smem &sm, int b, int tid)
{
    if (tid < kBlockTokens * 24) {
        const int m = tid / 24, e = tid % 24;
        const int tc = min(b * kBlockTokens + m, P.T - 1);
        float v;
        if (e < 16)
            v = FORM == kPost ? P.res[(size_t)tc * 16 + e] : 0.f;
        else if (e < 20)
            v = FORM == kPost ? P.post[(size_t)tc * 4 + (e - 16)] : 0.f;
        else
            v = P.identity_pre ? 0.25f : P.pre[(size_t)tc * 4 + (e - 20)];
        sm.coef[m][e] = v;
    } else if (tid < kBlockTokens * 24 + 24) {
        sm.bias[tid - kBlockTokens * 24] = P.bias[tid - kBlockTokens * 24];
    }
}

// x (4 streams) and y of one segment for both token halves.
struct SegXY {
    u32x4 x[2][4];
    u32x4 y[2];
};

// HALF0: only token half 0 (rows 0-7) is loaded and processed.  For T <= 8
// the rows of half 1 all stand for token T-1, which half 0 already holds, so
// the split kernel's decode instance leaves them out.
template <int FORM, bool HALF0 = false>
__device__ __forceinline__ void load_seg(const SeamParams &P, const Bufs &B, const Lane &L,
                                         int seg, SegXY &v)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (HALF0 && h == 1)
            break;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v.x[h][j] = bload<kAuxNT>(B.x, L.x[h], seg * 128 + j * 2 * P.H);
        if (FORM == kPost)
            v.y[h] = bload<kAuxNT>(B.y, L.h[h], seg * 128);
    }
}

struct Acc {
    f32x4 t0, t1, t2;  // MFMA tiles of the gate projection
    f32x4 tq;          // MFMA tile x' x'^T: its diagonal is each token's sum of x'^2
    double ssu[2];     // sum of squares of u (per token half)
};

// One segment: post-mix (residual store), collapse, sums of squares and the
// 24 MFMAs of the gate projection.  Returns the segment's u for both halves.
// B operands of stream j for segment seg: chunks 2*seg + s2, tiles 0..2.
__device__ __forceinline__ void load_fn(const Bufs &B, int lane, int seg, int j,
                                        u32x4 (&fb)[2][3])
{
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int tile = 0; tile < 3; ++tile)
            fb[s2][tile] = bload<kAuxPlain>(B.fn, lane * 16,
                                            ((((2 * seg + s2) * 4 + j) * 3 + tile) * 64) * 16);
}

// PRE: the fn operands were loaded ahead into fpre.  RING: they are in the
// ring fring, and once stream j's MFMAs have read them, stream j of segment
// `next` (if >= 0) is loaded into the same slot.
template <int FORM, bool PRE = false, bool HALF0 = false, bool RING = false>
__device__ __forceinline__ void process_seg(const SeamParams &P, const Bufs &B, const Lane &L,
                                            Smem &sm, int wave, int lane, int seg,
                                            const SegXY &v, Acc &acc, u32x4 (&u)[2],
                                            const u32x4 (*fpre)[2][3] = nullptr,
                                            u32x4 (*fring)[2][3] = nullptr, int next = -1)
{
    constexpr bool kGates = FORM != kCollapse;   // the gate projection's operands and MFMAs
    float uacc[2][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 fb[2][3];
        if constexpr (!kGates) {
        } else if (PRE || RING) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int tile = 0; tile < 3; ++tile)
                    fb[s2][tile] = PRE ? fpre[j][s2][tile] : fring[j][s2][tile];
        } else {
            load_fn(B, lane, seg, j, fb);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (HALF0 && h == 1)
                break;
            const int m = 8 * h + L.sub;
            u32x4 xb;
            if (FORM == kPost) {
                const f32x4 r = *reinterpret_cast<const f32x4 *>(&sm.coef[m][4 * j]);
                const float pj = sm.coef[m][16 + j];
                float xf[4][8], yf[8], o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    unpack8(v.x[h][i], xf[i]);
                unpack8(v.y[h], yf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float a = r[0] * xf[0][e];
                    a = __builtin_fmaf(r[1], xf[1][e], a);
                    a = __builtin_fmaf(r[2], xf[2][e], a);
                    a = __builtin_fmaf(r[3], xf[3][e], a);
                    a = __builtin_fmaf(pj, yf[e], a);
                    o[e] = a;
                }
                xb = pack8(o);
                gstore_nt(P.resid, (uint32_t)(L.x[h] + seg * 128 + j * 2 * P.H), xb);
            } else {
                xb = v.x[h][j];
            }
            if constexpr (kGates)
                sm.w[wave].tb[m][L.q] = xb;
            float xbf[8];
            unpack8(xb, xbf);
            const float pc = sm.coef[m][20 + j];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                uacc[h][e] = j == 0 ? pc * xbf[e] : __builtin_fmaf(pc, xbf[e], uacc[h][e]);
        }
        // A operands of stream j from the transpose rows: token lane%16,
        // columns 32*s2 + 8*(lane/16)..+8 of the segment.  The same register
        // is also the B operand of x' x'^T (B column n = token n), whose
        // diagonal accumulates the sums of squares on the matrix cores: the
        // bf16 products are exact and add in fp32.
        if constexpr (kGates) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const u32x4 a = sm.w[wave].tb[lane & 15][4 * s2 + (lane >> 4)];
                acc.t0 = mfma16(a, fb[s2][0], acc.t0);
                acc.t1 = mfma16(a, fb[s2][1], acc.t1);
                acc.t2 = mfma16(a, fb[s2][2], acc.t2);
                acc.tq = mfma16(a, a, acc.tq);
            }
            if (RING && next >= 0)
                load_fn(B, lane, next, j, fring[j]);
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (HALF0 && h == 1)
            break;
        u[h] = pack8(uacc[h]);
        float ub[8];
        unpack8(u[h], ub);
        // the bf16 squares are exact in fp32; 8 of them add in fp32, then
        // the segment's sum joins the fp64 total
        float su = ub[0] * ub[0];
#pragma unroll
        for (int e = 1; e < 8; ++e)
            su = __builtin_fmaf(ub[e], ub[e], su);
        acc.ssu[h] += (double)su;
    }
    // Materialise the running sums here: otherwise the compiler sinks the
    // fp64 chains to their use after the loop and keeps every segment's
    // inputs alive until then.
    asm volatile("" : "+v"(acc.ssu[0]), "+v"(acc.ssu[1]));
}

// Each wave's MFMA tiles and per-token sums of squares -> LDS.
__device__ __forceinline__ void wave_partials_to_lds(Smem &sm, const Acc &acc, const Lane &L,
                                                     int wave, int lane)
{
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int m = 4 * grp + i;
        sm.w[wave].dot[m][n] = acc.t0[i] + acc.t2[i];
        float v = acc.t1[i];
        float w = xor_lane<8>(v);
        if (n < 8)
            sm.w[wave].dot[m][16 + n] = v + w;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        double u = acc.ssu[h];
        u += xor_lane<1>(u);
        u += xor_lane<2>(u);
        u += xor_lane<4>(u);
        if (L.q == 0)
            sm.ss[wave][8 * h + L.sub][1] = u;
    }
    // the diagonal of x' x'^T: element (m, m) sits in lane m + 16 (m / 4),
    // register m % 4
    if (n >> 2 == grp) {
        const int i = n & 3;
        const float d = i == 0 ? acc.tq[0] : i == 1 ? acc.tq[1] : i == 2 ? acc.tq[2] : acc.tq[3];
        sm.ss[wave][n][0] = (double)d;
    }
}

// Sums over the 8 waves in LDS (fixed order): thread tid < 384 gets the dot
// (token tid/24, column tid%24); threads 384..399 the two sums of squares of
// token tid-384.
__device__ __forceinline__ void wave_sums(Smem &sm, int tid, float *dot_out, double *ss_out)
{
    if (tid < kBlockTokens * 24) {
        int m = tid / 24, q = tid % 24;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            s += sm.w[w].dot[m][q];
        *dot_out = s;
    } else if (tid < kBlockTokens * 25) {
        int m = tid - kBlockTokens * 24;
        double g = 0.0, u = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            g += sm.ss[w][m][0];
            u += sm.ss[w][m][1];
        }
        ss_out[0] = g;
        ss_out[1] = u;
    }
}

__device__ __forceinline__ void set_rstd(const SeamParams &P, Smem &sm, int m, double g, double u)
{
    sm.rstd_g[m] = 1.0 / sqrt(g / (4.0 * P.H) + (double)P.eps);
    sm.rstd_u[m] = (float)(1.0 / sqrt(u / (double)P.H + (double)P.eps));
}

// Next gates of the block's 16 tokens from sm.tot and sm.rstd_g: waves 0-3,
// 16 lanes per token, lane e holds logit 8+e of the 4x4 res matrix (row
// j = e/4 is the output stream) and, for e < 8, the pre/post logit e.
// Row sums (over lanes e^1, e^2) and column sums (over e^4, e^8) are DPP
// butterflies, so every entry of a row or column is divided by the same
// sum; the division is a hardware reciprocal and a multiply.
__device__ __forceinline__ float recip_sum(float s)
{
    // a column of entries that all underflowed keeps a finite scale
    return __builtin_amdgcn_rcpf(fmaxf(s, 1.17549435e-38f));
}

__device__ void gates(const SeamParams &P, Smem &sm, int b, int wave, int lane)
{
    if (wave >= 4)
        return;
    const int m = 4 * wave + (lane >> 4), e = lane & 15;
    const int t = b * kBlockTokens + m;
    const double rg = sm.rstd_g[m];
    float lr = (float)(rg * (double)sm.tot[m][8 + e] + (double)sm.bias[8 + e]);
    float lg = (float)(rg * (double)sm.tot[m][e & 7] + (double)sm.bias[e & 7]);
    // Sinkhorn of exp(l) [MEGA, Kernel Architecture]; the row max is taken
    // out first, which the first row normalisation cancels exactly.
    float rmax = fmaxf(lr, xor_lane<1>(lr));
    rmax = fmaxf(rmax, xor_lane<2>(rmax));
    float M = expf(lr - rmax);
    // Row sums over the quad (pairs {i, i^1}, then the two pairs); column
    // sums over lanes i, i+4, i+8, i+12 (pairs {i, i+8} by a rotation of 8,
    // then the other pair by a rotation of 4).  Every lane of a row or
    // column adds the same two pair sums, so all its entries are divided by
    // the same value; each step is a single DPP add.
    for (int it = 0; it < P.iters; ++it) {
        float s = M + xor_lane<1>(M);
        s = s + xor_lane<2>(s);
        M = M * recip_sum(s);
        s = M + ror_lane<8>(M);
        s = s + ror_lane<4>(s);
        M = M * recip_sum(s);
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

// bf16 norm of one 8-value piece: bf16(f32(f32(u * rstd) * gamma))
__device__ __forceinline__ u32x4 norm8(const u32x4 &u, const u32x4 &gv, float rs)
{
    float uf[8], gf[8], nf[8];
    unpack8(u, uf);
    unpack8(gv, gf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float a = uf[e] * rs;
        nf[e] = a * gf[e];
    }
    return pack8(nf);
}

// Norm (and quantised outputs) of one segment half from its bf16 u.  The
// 128-wide groups are quantised by the whole-row finish (finish_pair_g128),
// so here they get the norm only.
template <int OUT>
__device__ __forceinline__ void finish_half(const SeamParams &P, const Lane &L, int h, int seg,
                                            const u32x4 &u, const u32x4 &gv, float rs)
{
    const u32x4 nv = norm8(u, gv, rs);
    gstore_nt(P.norm, (uint32_t)(L.h[h] + seg * 128), nv);
    if (OUT == kMxfp8)
        quant_piece(nv, P.codes, (uint32_t)(L.c[h] + seg * 64), P.scales,
                    (uint32_t)(L.s[h] + 2 * seg + (L.q >> 2)), nullptr, 0);
    else if (OUT == kFp8Grid)
        quant_piece(nv, nullptr, 0, nullptr, 0, P.grid, (uint32_t)(L.h[h] + seg * 128));
}

// Largest |bf16| bit pattern over the 8 lanes of a token row (lanes 8s..8s+7)
__device__ __forceinline__ u32 row_amax_bits(u32 m)
{
    m = max(m, xor_lane<1>(m));
    m = max(m, xor_lane<2>(m));
    m = max(m, xor_lane<4>(m));
    return m;
}

// 128-wide groups: codes of one segment half with the group's exponent k,
// and the scale byte (written by piece 0 of the row when `scale` is set).
__device__ __forceinline__ void store_g128(const SeamParams &P, const Lane &L, int h, int seg,
                                           const u32x4 &nv, int k, bool scale)
{
    gstore_nt(P.codes, (uint32_t)(L.c[h] + seg * 64), e4m3_codes8(nv, k));
    if (scale && L.q == 0)
        gstore(P.scales, (uint32_t)((L.s[h] >> 2) + (seg >> 1)), (uint8_t)(k + 127));
}

// Norm and 128-wide-group MXFP8 of segments seg0 and seg0 + 1 (one group
// per token row: the same 8 lanes hold the row's pieces of both segments).
__device__ __forceinline__ void finish_pair_g128(const SeamParams &P, const Bufs &B, const Lane &L,
                                                 int seg0, const u32x4 (&u)[2][2], float rs0,
                                                 float rs1)
{
    const u32x4 g0 = bload<kAuxPlain>(B.gamma, L.q * 16, seg0 * 128);
    const u32x4 g1 = bload<kAuxPlain>(B.gamma, L.q * 16, (seg0 + 1) * 128);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float rs = h ? rs1 : rs0;
        const u32x4 n0 = norm8(u[0][h], g0, rs), n1 = norm8(u[1][h], g1, rs);
        gstore_nt(P.norm, (uint32_t)(L.h[h] + seg0 * 128), n0);
        gstore_nt(P.norm, (uint32_t)(L.h[h] + (seg0 + 1) * 128), n1);
        const int k = scale_exp_of_bits(row_amax_bits(max(amax_bits8(n0), amax_bits8(n1))));
        store_g128(P, L, h, seg0, n0, k, true);
        store_g128(P, L, h, seg0 + 1, n1, k, false);
    }
}

// Whole-row mode: one workgroup per 16-token block; wave w walks segments
// w + 8i, i < RS (H = 512 * RS).  u: the first UL segments of each wave in
// LDS (2 KB each), the rest in VGPRs.
constexpr int kMaxLdsSegs = 8;  // 8 waves x 8 x 2 KB = 128 KB of LDS

// Split mode's per-block words (the protocol is described with split_body):
// the arrival counter, then two hand-off mask sets (63 splits per 64-bit
// word, bit 63 = CLOSED) that alternate launch by launch.  The counter never
// goes back: a launch's arrivals are its value modulo kEpoch, and the last
// arriver moves it on to the next multiple of kEpoch.
enum { kSyncArrive = 0, kSyncMask = 4 };
constexpr int kMaskSplits = 63;
constexpr int kMaskWords = (kMaxSplits + kMaskSplits - 1) / kMaskSplits;
constexpr uint64_t kClosed = 1ull << 63;
constexpr u32 kEpoch = 4096;  // > kMaxSplits, and a divisor of 2^32 (the counter wraps)
static_assert(kSyncMask + 2 * 2 * kMaskWords <= 32, "sync words exceed one line");

// What a split workgroup does after arriving (kept in LDS, shared by its waves)
enum SplitRole {
    kRoleFinish = 0,    // normalise its own segments
    kRoleFinisher = 1,  // the last arriver: its own segments, the gates, hand-offs
    kRoleHandOff = 2,   // its wait ran out: hand its segments over
    kRoleDone = 3,      // nothing left: handed off, or no norm in this launch
};

template <int FORM, int OUT, int MAXU, bool HALF0 = false>
__device__ __forceinline__ void split_body(const SeamParams &P, Smem &sm, uint64_t *handed,
                                           int &role, u32x4 *ulds, int b, int s);

// Workgroups past the first P.rows_blocks run the last blocks in split mode
// (ksplit splits of at most 8 segments each, one per wave): a small tail of
// blocks left over after full rounds of the CUs is spread over many short
// workgroups instead of leaving a near-empty last round of whole blocks.
template <int FORM, int OUT, int RS>
__global__ __launch_bounds__(kThreads, 1) void seam_rows_kernel(SeamParams P)
{
    constexpr int UL = RS < kMaxLdsSegs ? RS : kMaxLdsSegs;
    constexpr int UR = RS - UL > 0 ? RS - UL : 1;
    constexpr int D = FORM == kNoPost ? SEAM_PREFETCH_NOPOST : SEAM_PREFETCH;
    __shared__ Smem sm;
    __shared__ u32x4 ul[kWaves][UL][2][64];
    // 128-wide groups: row amax of the VGPR-resident segments, per wave
    __shared__ u32 gx[OUT == kMxfp8G128 ? kWaves : 1][UR][2][8];
    __shared__ uint64_t handed[kMaskWords];
    __shared__ int role;
    if ((int)blockIdx.x >= P.rows_blocks) {
        const int w = blockIdx.x - P.rows_blocks;
        split_body<FORM, OUT, 1>(P, sm, handed, role, nullptr, P.rows_blocks + w / P.ksplit,
                                 w % P.ksplit);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const Bufs B = make_bufs(P);
    const Lane L = lane_geometry(P, b, lane);
    load_coef<FORM>(P, sm, b, tid);

    Acc acc;
    acc.t0 = acc.t1 = acc.t2 = acc.tq = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.ssu[0] = acc.ssu[1] = 0.0;
    u32x4 ureg[UR][2];
    SegXY ring[D + 1];
    auto seg_of = [&](int i) { return wave + kWaves * i; };
    // Software pipeline: x/y of segment i+D are in flight while segment i is
    // computed.  nseg == 8 * RS here, so every branch below is resolved at
    // compile time and the waitcnt pass sees straight-line code.
    //
    // Vector memory loads complete in issue order, so a wait for one load
    // also waits for every load issued before it.  In the plain schedule the
    // fn operands of segment i are loaded after the HBM prefetch of segment
    // i+1, and the first MFMA of segment i waits for that prefetch too.  With
    // the fn ring (no_post form, whose registers hold the 96 it needs), a
    // segment's fn operands are loaded one segment ahead, stream by stream as
    // the previous segment's MFMAs free their slots, and the x of segment i+2
    // is issued after all of them: no wait covers a recent HBM load.
    constexpr bool kRing = FORM == kNoPost && SEAM_FN_RING && D == 1;
    u32x4 fring[kRing ? 4 : 1][2][3];
    if (kRing) {
        load_seg<FORM>(P, B, L, seg_of(0), ring[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            load_fn(B, lane, seg_of(0), j, fring[j]);
        if (RS > 1)
            load_seg<FORM>(P, B, L, seg_of(1), ring[1]);
    } else {
#pragma unroll
        for (int i = 0; i < D && i < RS; ++i)
            load_seg<FORM>(P, B, L, seg_of(i), ring[i]);
    }
    __syncthreads();  // coefficients in LDS
#pragma unroll
    for (int i = 0; i < RS; ++i) {
        const int seg = seg_of(i);
        if (!kRing && i + D < RS)
            load_seg<FORM>(P, B, L, seg_of(i + D), ring[(i + D) % (D + 1)]);
        u32x4 u[2];
        if (kRing) {
            process_seg<FORM, false, false, true>(P, B, L, sm, wave, lane, seg, ring[i % 2], acc,
                                                  u, nullptr, fring,
                                                  i + 1 < RS ? seg_of(i + 1) : -1);
            if (i + 2 < RS)
                load_seg<FORM>(P, B, L, seg_of(i + 2), ring[i % 2]);
        } else {
            process_seg<FORM>(P, B, L, sm, wave, lane, seg, ring[i % (D + 1)], acc, u);
        }
        if (i < UL) {
            ul[wave][i][0][lane] = u[0];
            ul[wave][i][1][lane] = u[1];
        } else {
            ureg[i - UL][0] = u[0];
            ureg[i - UL][1] = u[1];
        }
        // keep the scheduler from merging iterations: the pipeline depth is
        // the one written here, and register pressure stays bounded
        __builtin_amdgcn_sched_barrier(0);
    }
    // gamma of the wave's segments: the first GD in flight during the
    // reductions, then GD ahead of the finish loop
    constexpr int GD = 4;
    u32x4 gv[RS];
    if (OUT != kMxfp8G128)
#pragma unroll
        for (int i = 0; i < GD && i < RS; ++i)
            gv[i] = bload<kAuxPlain>(B.gamma, L.q * 16, seg_of(i) * 128);
    wave_partials_to_lds(sm, acc, L, wave, lane);
    __syncthreads();
    {
        float d;
        double ss[2];
        wave_sums(sm, tid, &d, ss);
        if (tid < kBlockTokens * 24)
            sm.tot[tid / 24][tid % 24] = d;
        else if (tid < kBlockTokens * 25)
            set_rstd(P, sm, tid - kBlockTokens * 24, ss[0], ss[1]);
    }
    __syncthreads();
    const float rs0 = sm.rstd_u[L.sub], rs1 = sm.rstd_u[8 + L.sub];
    if (OUT == kMxfp8G128) {
        // 128-wide groups pair segments 2g, 2g + 1.  Segments in LDS (the
        // first 8 UL) go pair by pair to any wave; those in VGPRs (i >= UL,
        // owned by waves w and w ^ 1) swap their row amax through LDS.
        if (!P.skip_norm) {
            if (RS > UL) {
                u32x4 nv[UR][2];
#pragma unroll
                for (int i = UL; i < RS; ++i) {
                    const int seg = wave + kWaves * i;
                    const u32x4 gs = bload<kAuxPlain>(B.gamma, L.q * 16, seg * 128);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        nv[i - UL][h] = norm8(ureg[i - UL][h], gs, h ? rs1 : rs0);
                        gstore_nt(P.norm, (uint32_t)(L.h[h] + seg * 128), nv[i - UL][h]);
                        const u32 m = row_amax_bits(amax_bits8(nv[i - UL][h]));
                        if (L.q == 0)
                            gx[wave][i - UL][h][L.sub] = m;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int i = UL; i < RS; ++i) {
                    const int seg = wave + kWaves * i;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32 m = max(gx[wave][i - UL][h][L.sub], gx[wave ^ 1][i - UL][h][L.sub]);
                        store_g128(P, L, h, seg, nv[i - UL][h], scale_exp_of_bits(m),
                                   (wave & 1) == 0);
                    }
                }
            }
            for (int g = wave; g < 4 * UL; g += kWaves) {
                u32x4 u[2][2];
#pragma unroll
                for (int k = 0; k < 2; ++k)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        u[k][h] = ul[(2 * g + k) % kWaves][(2 * g + k) / kWaves][h][lane];
                finish_pair_g128(P, B, L, 2 * g, u, rs0, rs1);
            }
        }
    } else if (!P.skip_norm)
#pragma unroll
    for (int i = 0; i < RS; ++i) {
        const int seg = seg_of(i);
        if (i + GD < RS)
            gv[i + GD] = bload<kAuxPlain>(B.gamma, L.q * 16, seg_of(i + GD) * 128);
        const u32x4 u0 = i < UL ? ul[wave][i][0][lane] : ureg[i - UL][0];
        const u32x4 u1 = i < UL ? ul[wave][i][1][lane] : ureg[i - UL][1];
        finish_half<OUT>(P, L, 0, seg, u0, gv[i], rs0);
        finish_half<OUT>(P, L, 1, seg, u1, gv[i], rs1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (FORM != kCollapse && !P.skip_gates)
        gates(P, sm, b, wave, lane);
}

// ------------------------------------------------------------ split mode --
//
// Workgroup (block b, split s) streams segments [s0, s1) of block b.  Every
// split writes its partials, then arrives on the block's counter.  The last
// arriver (the finisher) sets the CLOSED bit of the block's hand-off mask
// with one atomic OR, sums the partials and computes the gates.  The other
// splits poll the counter, with a bound, until every split has arrived, then
// sum the partials' squares themselves (same data, same order: the same
// rstd bits) and normalise their own segments from the u they kept on chip,
// as the pages' distributed finish does [MEGA, Kernel Architecture].  A
// split whose bound runs out (its block's other splits are not all
// resident, e.g. the GPU is shared) writes its u to scratch and sets its bit
// in the hand-off mask; the finisher finishes the segments of every split
// whose bit its OR got back, and a split that finds CLOSED already set in
// the value its own OR returns finishes itself (every split has arrived by
// then).  So every segment is normalised exactly once and no workgroup waits
// without a bound.  Nothing is reset on the way out: the finisher moves the
// arrival counter on to the next epoch and clears the mask set of the
// previous launch, which the next launch uses; launches on a stream do not
// overlap, so no split of either touches it meanwhile.
//
// Cross-workgroup data (partials, counters, handed-off u) moves with
// relaxed agent-scope atomic accesses, which are coherent across XCDs (sc1)
// without writing back or invalidating the L2; an explicit s_waitcnt before
// each signalling atomic orders the data before the signal.  Agent-scope
// fences were measured to cost ~1 us per workgroup here (each one writes
// back the XCD's dirty L2).
//
// MAXU > 0: each wave keeps up to MAXU segments of u on chip (segs per
// split <= 8 * MAXU; VGPRs for MAXU = 1, LDS above).  MAXU == 0: u goes to
// scratch as it is made and every split hands off (the finisher normalises
// the whole block).

// The sync words, like the partials and the handed-off u, are indexed from
// the first split block (rows_blocks).  A word set serves whichever block
// uses it next: every launch leaves its counter at a multiple of kEpoch
// and the mask set of the next launch clear, whatever the block or plan.
__device__ __forceinline__ int *block_sync(const SeamParams &P, int b)
{
    return P.sync + (size_t)(b - P.rows_blocks) * P.sync_stride;
}

__device__ __forceinline__ void st_rel(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rel(double *p, double v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_rel(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_rel(const double *p)
{
    return __hip_atomic_load(const_cast<double *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_rel(const int *p)
{
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rel(int *p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-mode scratch covers the split blocks only: blocks [rows_blocks,
// nblocks), i.e. tokens from 16 * rows_blocks on (0 in a launch that is all
// splits).  Byte offset of a token row's u (a [T][H] bf16 offset, L.h) in
// the handed-off u, and the first partial record of block b.
__device__ __forceinline__ int uscr_off(const SeamParams &P, int row_off)
{
    return row_off - P.rows_blocks * kBlockTokens * 2 * P.H;
}

__device__ __forceinline__ float *block_part(const SeamParams &P, int b)
{
    return P.part + (size_t)(b - P.rows_blocks) * P.ksplit * kBlockTokens * kPartFloats;
}

// u of one segment half to / from scratch (two coherent 8-byte accesses)
__device__ __forceinline__ void st_u(const SeamParams &P, const Lane &L, int h, int seg,
                                     const u32x4 &u)
{
    uint64_t *p = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(P.uscr) +
                                               uscr_off(P, L.h[h]) + seg * 128);
    __hip_atomic_store(p, ((uint64_t)u[1] << 32) | u[0], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, ((uint64_t)u[3] << 32) | u[2], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u32x4 ld_u(const SeamParams &P, const Lane &L, int h, int seg)
{
    uint64_t *p = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(P.uscr) +
                                               uscr_off(P, L.h[h]) + seg * 128);
    uint64_t a = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t c = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return u32x4{(u32)a, (u32)(a >> 32), (u32)c, (u32)(c >> 32)};
}

// Norm of segments [s0, s1) of this block with u from scratch (all waves).
template <int OUT, bool HALF0>
__device__ void finish_from_scratch(const SeamParams &P, const Bufs &B, const Lane &L, int wave,
                                    int s0, int s1, float rs0, float rs1)
{
    for (int seg0 = s0 + wave; seg0 < s1; seg0 += 4 * kWaves) {
        u32x4 u[4][2], gv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int seg = min(seg0 + k * kWaves, s1 - 1);
            gv[k] = bload<kAuxPlain>(B.gamma, L.q * 16, seg * 128);
            u[k][0] = ld_u(P, L, 0, seg);
            u[k][1] = HALF0 ? u[k][0] : ld_u(P, L, 1, seg);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int seg = seg0 + k * kWaves;
            if (seg < s1) {
                finish_half<OUT>(P, L, 0, seg, u[k][0], gv[k], rs0);
                if (!HALF0)
                    finish_half<OUT>(P, L, 1, seg, u[k][1], gv[k], rs1);
            }
        }
    }
}

__device__ __forceinline__ uint64_t *block_mask(int *sync, u32 epoch)
{
    return reinterpret_cast<uint64_t *>(sync + kSyncMask) + ((epoch / kEpoch) & 1) * kMaskWords;
}

// Poll the block's arrival counter until every split has arrived (wave 0),
// at most spin_limit + 1 times.
#ifndef SEAM_POLL_SLEEP
#define SEAM_POLL_SLEEP 2
#endif
__device__ __forceinline__ bool wait_arrivals(const SeamParams &P, int *sync, u32 epoch, int lane)
{
    for (int it = 0; it <= P.spin_limit; ++it) {
        int n = 0;
        if (lane == 0)
            n = ld_rel(sync + kSyncArrive);
        // the finisher may already have moved the counter on by kEpoch
        if ((u32)__shfl(n, 0) - epoch >= (u32)P.ksplit)
            return true;
        __builtin_amdgcn_s_sleep(SEAM_POLL_SLEEP);
    }
    return false;
}

// Adds quad q of records k0, k0 + 4, ..., k0 + 4 (NB - 1) of one token
// (byte offset `off` within a split's records) to d (dots) or g, u (the
// sums of squares).  All NB loads are issued before the first add, so the
// batch costs one round trip to the coherent level.  Records past the
// block's last split lie outside the resource: those loads return +0.0
// without a memory access.  They are added all the same (conditional adds
// would let the compiler sink each load to its add): every sum starts at
// +0.0, so adding +0.0 leaves its bits unchanged.
template <int NB>
__device__ __forceinline__ void add_records(rsrc_t rp, int k0, int off, bool sums, f32x4 &d,
                                            double &g, double &u)
{
    constexpr int kRecBytes = kBlockTokens * kPartFloats * 4;  // one split's records
    u32x4 v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
        v[i] = bload<kAuxSc1>(rp, (k0 + 4 * i) * kRecBytes + off, 0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (sums) {
            g += __longlong_as_double((long long)(((uint64_t)v[i][1] << 32) | v[i][0]));
            u += __longlong_as_double((long long)(((uint64_t)v[i][3] << 32) | v[i][2]));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                d[c] += __uint_as_float(v[i][c]);
        }
    }
}

// Sums over the splits of the block's partial records (128 B per split and
// token: 24 dots, then the fp64 sums of squares of x' and u), then rstd of
// the block's tokens.  Thread (m, q, j), j = tid % 4, of the 16 x 7 x 4
// grid loads quad q (16 bytes) of token m's records from splits j, j + 4,
// ... (device-coherent loads) and adds them in that order; the 4 threads
// then combine with two DPP steps, so every split that runs this gets the
// same bits.  Quads 0-5 are the dots (DOTS: the finisher, for the gates),
// quad 6 the two sums, whose thread also computes the token's rstd.  Rows
// past the last token (T not a multiple of 16) load nothing: their lanes
// rewrite the last token's row and read its rstd instead.
template <bool DOTS>
__device__ void reduce_partials(const SeamParams &P, Smem &sm, int b, int tid)
{
    const int valid = min(kBlockTokens, P.T - b * kBlockTokens);
    const int j = tid & 3, mq = tid >> 2;
    if (mq >= kBlockTokens * 7)
        return;
    const int m = mq / 7, q = mq % 7;
    // uniform per group of 4 lanes, so the DPP steps below see whole groups
    if (!(q == 6 || DOTS) || m >= valid)
        return;
    const rsrc_t rp = make_rsrc(block_part(P, b),
                                (uint32_t)(P.ksplit * kBlockTokens * kPartFloats * 4));
    const int off = (m * kPartFloats + 4 * q) * 4;
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    double g = 0.0, u = 0.0;
    const bool sums = q == 6;
    // records per thread, sized so that no batch is mostly empty
    const int per = (P.ksplit + 3) / 4;
    if (per <= 1)
        add_records<1>(rp, j, off, sums, d, g, u);
    else if (per <= 2)
        add_records<2>(rp, j, off, sums, d, g, u);
    else if (per <= 3)
        add_records<3>(rp, j, off, sums, d, g, u);
    else if (per <= 5)
        add_records<5>(rp, j, off, sums, d, g, u);
    else if (per <= 10)
        add_records<10>(rp, j, off, sums, d, g, u);
    else
        for (int k0 = j; k0 < P.ksplit; k0 += 4 * 16)
            add_records<16>(rp, k0, off, sums, d, g, u);
    if (sums) {
        g += xor_lane<1>(g);
        u += xor_lane<1>(u);
        g += xor_lane<2>(g);
        u += xor_lane<2>(u);
        if (j == 0)
            set_rstd(P, sm, m, g, u);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float v = d[c];
            v += xor_lane<1>(v);
            v += xor_lane<2>(v);
            if (j == 0)
                sm.tot[m][4 * q + c] = v;
        }
    }
}

// u of the split's segments: MAXU = 1 in VGPRs; MAXU > 1 in the LDS array
// `ulds` ([kWaves][MAXU][2][64]); MAXU = 0 straight to scratch.  HALF0: the
// launch has T <= 8 tokens, all in half 0 of block 0 (see load_seg).
template <int FORM, int OUT, int MAXU, bool HALF0>
__device__ __forceinline__ void split_body(const SeamParams &P, Smem &sm, uint64_t *handed,
                                           int &role, u32x4 *ulds, int b, int s)
{
    constexpr bool kVgprU = MAXU == 1;
    constexpr bool kLdsU = MAXU > 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Bufs B = make_bufs(P);
    const Lane L = lane_geometry(P, b, lane);
    int *sync = block_sync(P, b);
    load_coef<FORM>(P, sm, b, tid);

    Acc acc;
    acc.t0 = acc.t1 = acc.t2 = acc.tq = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.ssu[0] = acc.ssu[1] = 0.0;
    const int s0 = s * P.segs_per_split;
    const int s1 = min(s0 + P.segs_per_split, P.nseg);
    const bool busy = s0 + wave < s1;  // this wave has at least one segment
    u32x4 ureg[kVgprU ? MAXU : 1][2];
    auto uslot = [&](int i, int h) -> u32x4 & {
        return ulds[((wave * (kLdsU ? MAXU : 1) + i) * 2 + h) * 64 + lane];
    };
    if (kVgprU) {
        // every load of the wave's segments (and, with one segment per
        // wave, its fn operands) is in flight before the coefficient barrier
        constexpr bool kPreFn = MAXU == 1;
        SegXY v[kVgprU ? MAXU : 1];
        u32x4 f0[kPreFn ? 4 : 1][2][3];
        if (busy) {
#pragma unroll
            for (int i = 0; i < (kVgprU ? MAXU : 1); ++i)
                load_seg<FORM, HALF0>(P, B, L, min(s0 + wave + kWaves * i, s1 - 1), v[i]);
            if (kPreFn && FORM != kCollapse)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    load_fn(B, lane, s0 + wave, j, f0[kPreFn ? j : 0]);
        }
        __syncthreads();  // coefficients in LDS
        if (busy) {
            process_seg<FORM, kPreFn, HALF0>(P, B, L, sm, wave, lane, s0 + wave, v[0], acc,
                                             ureg[0], f0);
#pragma unroll
            for (int i = 1; i < (kVgprU ? MAXU : 1); ++i) {
                const int seg = s0 + wave + kWaves * i;
                if (seg < s1)
                    process_seg<FORM, false, HALF0>(P, B, L, sm, wave, lane, seg, v[i], acc,
                                                    ureg[i]);
            }
        }
    } else {
        // the prefetch is issued unconditionally (clamped to a segment
        // already read) so that the waitcnt pass keeps it in flight
        SegXY cur, nxt;
        if (busy)
            load_seg<FORM, HALF0>(P, B, L, s0 + wave, cur);
        __syncthreads();  // coefficients in LDS
        for (int seg = s0 + wave, i = 0; seg < s1; seg += kWaves, ++i) {
            load_seg<FORM, HALF0>(P, B, L, min(seg + kWaves, s1 - 1), nxt);
            u32x4 u[2];
            process_seg<FORM, false, HALF0>(P, B, L, sm, wave, lane, seg, cur, acc, u);
            if (kLdsU) {
                uslot(i, 0) = u[0];
                uslot(i, 1) = u[1];
            } else {
                st_u(P, L, 0, seg, u[0]);
                if (!HALF0)
                    st_u(P, L, 1, seg, u[1]);
            }
            cur = nxt;
        }
    }
    wave_partials_to_lds(sm, acc, L, wave, lane);
    __syncthreads();
    {
        float *part = block_part(P, b) + (size_t)s * kBlockTokens * kPartFloats;
        float d;
        double ss[2];
        wave_sums(sm, tid, &d, ss);
        if (tid < kBlockTokens * 24) {
            st_rel(part + (tid / 24) * kPartFloats + tid % 24, d);
        } else if (tid < kBlockTokens * 25) {
            double *pd =
                reinterpret_cast<double *>(part + (tid - kBlockTokens * 24) * kPartFloats + 24);
            st_rel(pd, ss[0]);
            st_rel(pd + 1, ss[1]);
        }
    }
    // gamma of the split's own segments, in flight while the block gathers
    u32x4 gv[MAXU > 0 ? MAXU : 1];
    if (MAXU > 0 && busy)
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
            gv[MAXU > 0 ? i : 0] =
                bload<kAuxPlain>(B.gamma, L.q * 16, min(s0 + wave + kWaves * i, s1 - 1) * 128);
    __builtin_amdgcn_s_waitcnt(0);  // partials (and handed-off u) before the arrival
    __syncthreads();
    if (tid == 0) {
        const u32 old = __hip_atomic_fetch_add(reinterpret_cast<u32 *>(sync + kSyncArrive), 1u,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.epoch = old & ~(kEpoch - 1);
        role = (int)(old & (kEpoch - 1)) == P.ksplit - 1 ? kRoleFinisher : kRoleFinish;
    }
    __syncthreads();
    const bool finisher = role == kRoleFinisher;
    const u32 epoch = sm.epoch;
    uint64_t *mask = block_mask(sync, epoch);
    const int nwords = (P.ksplit + kMaskSplits - 1) / kMaskSplits;
    if (finisher) {
        // every split has arrived: move the counter on to the next epoch, and
        // clear the other mask set (the previous launch's) for the next one
        if (tid == 0)
            __hip_atomic_fetch_add(reinterpret_cast<u32 *>(sync + kSyncArrive),
                                   kEpoch - (u32)P.ksplit, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        if (tid >= 64 && tid < 64 + kMaskWords)
            __hip_atomic_store(block_mask(sync, epoch + kEpoch) + (tid - 64), (uint64_t)0,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    bool reduce = finisher;
    if (finisher) {
        // splits that handed off before this point are finished here.  The
        // OR is made, and waited for, by the last lanes of the last wave,
        // which has no share of the reduction: its round trip overlaps the
        // reduction's loads instead of preceding them
        static_assert(kBlockTokens * 7 * 4 <= kThreads - 64,
                      "the last wave takes no part in the reduction");
        const int w = tid - (kThreads - kMaskWords);
        if (w >= 0 && w < nwords)
            handed[w] = __hip_atomic_fetch_or(mask + w, kClosed, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) & ~kClosed;
    } else if (P.skip_norm) {
        role = kRoleDone;
    } else {
        // MAXU > 0: wait, with a bound, until every split has arrived; on a
        // time out (and always when MAXU == 0) hand the segments off
        if (wave == 0)
            role = (MAXU > 0 && wait_arrivals(P, sync, epoch, lane)) ? kRoleFinish : kRoleHandOff;
        __syncthreads();
        if (role == kRoleHandOff) {
            if (MAXU > 0) {
#pragma unroll
                for (int i = 0; i < MAXU; ++i) {
                    const int seg = s0 + wave + kWaves * i;
                    if (seg < s1) {
                        st_u(P, L, 0, seg, kVgprU ? ureg[kVgprU ? i : 0][0] : uslot(i, 0));
                        if (!HALF0)
                            st_u(P, L, 1, seg, kVgprU ? ureg[kVgprU ? i : 0][1] : uslot(i, 1));
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) {
                const uint64_t old = __hip_atomic_fetch_or(
                    mask + s / kMaskSplits, 1ull << (s % kMaskSplits), __ATOMIC_RELAXED,
                    __HIP_MEMORY_SCOPE_AGENT);
                // closed: every split has arrived; finish here after all
                role = (old & kClosed) ? kRoleFinish : kRoleDone;
            }
            __syncthreads();
        }
        reduce = role == kRoleFinish;
    }
    if (finisher && !P.skip_gates)
        reduce_partials<true>(P, sm, b, tid);
    else if (reduce)
        reduce_partials<false>(P, sm, b, tid);
    __syncthreads();

    // rows past the block's last token rewrite that token's row, with its rstd
    const int last = min(kBlockTokens, P.T - b * kBlockTokens) - 1;
    const float rs0 = sm.rstd_u[min(L.sub, last)], rs1 = sm.rstd_u[min(8 + L.sub, last)];
    // with at most 4 segments per split, waves 4-7 have none: they compute
    // the gates while waves 0-3 normalise
    const bool gates_early = P.segs_per_split <= 4;
    if (finisher && !P.skip_gates && gates_early && wave >= 4)
        gates(P, sm, b, wave - 4, lane);
    if (!P.skip_norm && (finisher || role == kRoleFinish)) {
        // this split's own segments
        if (MAXU > 0) {
#pragma unroll
            for (int i = 0; i < MAXU; ++i) {
                const int seg = s0 + wave + kWaves * i;
                if (seg < s1) {
                    finish_half<OUT>(P, L, 0, seg, kVgprU ? ureg[kVgprU ? i : 0][0] : uslot(i, 0),
                                     gv[MAXU > 0 ? i : 0], rs0);
                    if (!HALF0)
                        finish_half<OUT>(P, L, 1, seg,
                                         kVgprU ? ureg[kVgprU ? i : 0][1] : uslot(i, 1),
                                         gv[MAXU > 0 ? i : 0], rs1);
                }
            }
        } else {
            finish_from_scratch<OUT, HALF0>(P, B, L, wave, s0, s1, rs0, rs1);
        }
    }
    if (finisher) {
        if (!P.skip_gates && !gates_early)
            gates(P, sm, b, wave, lane);
        // segments of the splits that handed off
        for (int w = 0; w < nwords; ++w) {
            uint64_t bits = handed[w];
            while (bits) {
                const int k = w * kMaskSplits + __builtin_ctzll(bits);
                bits &= bits - 1;
                finish_from_scratch<OUT, HALF0>(P, B, L, wave, k * P.segs_per_split,
                                                min((k + 1) * P.segs_per_split, P.nseg), rs0,
                                                rs1);
            }
        }
    }
}

template <int FORM, int OUT, int MAXU, bool HALF0 = false>
__global__ __launch_bounds__(kThreads, 1) void seam_split_kernel(SeamParams P)
{
    __shared__ Smem sm;
    __shared__ uint64_t handed[kMaskWords];
    __shared__ int role;
    __shared__ u32x4 ulds[MAXU > 1 ? kWaves * MAXU * 2 * 64 : 1];  // the waves' u (MAXU > 1)
    split_body<FORM, OUT, MAXU, HALF0>(P, sm, handed, role, ulds,
                                       P.rows_blocks + blockIdx.x / P.ksplit,
                                       blockIdx.x % P.ksplit);
}

// Standalone per-32 MXFP8 quantiser of a bf16 [rows][H] tensor with the
// seam's device code: each wave takes 8 rows x 64 columns per step in the
// row layout (lane: row l/8, columns 8*(l%8)..+8), grid-stride over tiles.
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *__restrict__ src,
                                                       int rows, int H, uint8_t *codes,
                                                       uint8_t *scales, uint16_t *grid)
{
    const int lane = threadIdx.x & 63;
    const int q = lane & 7, sub = lane >> 3;
    const int nseg = H / kSeg, nchunks = H / kChunk;
    const int ntiles = ((rows + 7) / 8) * nseg;
    const rsrc_t r = make_rsrc(src, (uint32_t)rows * (uint32_t)H * 2u);
    for (int tile = blockIdx.x * 4 + (threadIdx.x >> 6); tile < ntiles; tile += gridDim.x * 4) {
        const int rt = tile / nseg, seg = tile % nseg;
        // rows past the end re-read and rewrite the last row: identical bytes
        const int row = min(rt * 8 + sub, rows - 1);
        const u32x4 nv = bload<kAuxNT>(r, row * (2 * H) + q * 16, seg * 128);
        quant_piece(nv, codes, (uint32_t)(row * H + seg * 64 + q * 8), scales,
                    (uint32_t)(row * nchunks + 2 * seg + (q >> 2)), grid,
                    (uint32_t)(row * (2 * H) + seg * 128 + q * 16));
    }
}

// The same quantiser in 128-wide groups: a wave takes 8 rows x 128 columns
// (two segments) per step; the 8 lanes of a row hold the group (16 values
// each), reduce its amax with DPP and share one scale byte.
__global__ __launch_bounds__(256) void quantize128_kernel(const uint16_t *__restrict__ src,
                                                          int rows, int H, uint8_t *codes,
                                                          uint8_t *scales, uint16_t *grid)
{
    const int lane = threadIdx.x & 63;
    const int q = lane & 7, sub = lane >> 3;
    const int ngroups = H / 128;
    const int ntiles = ((rows + 7) / 8) * ngroups;
    const rsrc_t r = make_rsrc(src, (uint32_t)rows * (uint32_t)H * 2u);
    for (int tile = blockIdx.x * 4 + (threadIdx.x >> 6); tile < ntiles; tile += gridDim.x * 4) {
        const int rt = tile / ngroups, g = tile % ngroups;
        // rows past the end re-read and rewrite the last row: identical bytes
        const int row = min(rt * 8 + sub, rows - 1);
        const u32x4 nv0 = bload<kAuxNT>(r, row * (2 * H) + q * 16, (2 * g) * 128);
        const u32x4 nv1 = bload<kAuxNT>(r, row * (2 * H) + q * 16, (2 * g + 1) * 128);
        u32 m = max(amax_bits8(nv0), amax_bits8(nv1));
        m = max(m, xor_lane<1>(m));
        m = max(m, xor_lane<2>(m));
        m = max(m, xor_lane<4>(m));
        const int k = scale_exp_of_bits(m);
        const u32x2 w0 = e4m3_codes8(nv0, k), w1 = e4m3_codes8(nv1, k);
        if (codes) {
            gstore_nt(codes, (uint32_t)(row * H + 2 * g * 64 + q * 8), w0);
            gstore_nt(codes, (uint32_t)(row * H + (2 * g + 1) * 64 + q * 8), w1);
            if (q == 0)
                gstore(scales, (uint32_t)(row * ngroups + g), (uint8_t)(k + 127));
        }
        if (grid) {
            gstore_nt(grid, (uint32_t)(row * (2 * H) + 2 * g * 128 + q * 16), e4m3_grid8(w0, k));
            gstore_nt(grid, (uint32_t)(row * (2 * H) + (2 * g + 1) * 128 + q * 16),
                      e4m3_grid8(w1, k));
        }
    }
}

template <int FORM, int OUT>
hipError_t launch_rows(const SeamParams &p, int rs, int grid, hipStream_t s);

// Split workgroups of blocks [rows_blocks, nblocks): the whole launch in
// split mode (rows_blocks = 0), or the tail after a whole-row launch.
template <int FORM, int OUT>
hipError_t launch_split(const SeamParams &p, int grid, hipStream_t s)
{
    dim3 g(grid), b(kThreads);
    {
        const int per_wave = (p.segs_per_split + kWaves - 1) / kWaves;
        if (per_wave <= 1 && p.T <= 8)   // decode: token half 0 only
            hipLaunchKernelGGL((seam_split_kernel<FORM, OUT, 1, true>), g, b, 0, s, p);
        else if (per_wave <= 1)
            hipLaunchKernelGGL((seam_split_kernel<FORM, OUT, 1>), g, b, 0, s, p);
        else if (per_wave <= 2)
            hipLaunchKernelGGL((seam_split_kernel<FORM, OUT, 2>), g, b, 0, s, p);
        else if (per_wave <= 3)
            hipLaunchKernelGGL((seam_split_kernel<FORM, OUT, 3>), g, b, 0, s, p);
        else if (per_wave <= 4)
            hipLaunchKernelGGL((seam_split_kernel<FORM, OUT, 4>), g, b, 0, s, p);
        else if (per_wave <= 5)
            hipLaunchKernelGGL((seam_split_kernel<FORM, OUT, 5>), g, b, 0, s, p);
        else
            hipLaunchKernelGGL((seam_split_kernel<FORM, OUT, 0>), g, b, 0, s, p);
        return hipGetLastError();
    }
}

template <int FORM, int OUT>
hipError_t launch_form_out(const SeamParams &p, int rs, int grid, hipStream_t s)
{
    if (rs == 0)
        return launch_split<FORM, OUT>(p, grid, s);
    if (p.rows_blocks < p.nblocks && p.segs_per_split > kWaves) {
        // a tail whose splits take more than one segment per wave: the
        // whole-row kernel keeps only one-segment splits in line (their u in
        // VGPRs; larger ones raised its register pressure and spills, which
        // slowed every whole-row block), so the tail's splits follow in a
        // launch of their own
        const hipError_t e = launch_rows<FORM, OUT>(p, rs, p.rows_blocks, s);
        if (e != hipSuccess)
            return e;
        return launch_split<FORM, OUT>(p, (p.nblocks - p.rows_blocks) * p.ksplit, s);
    }
    return launch_rows<FORM, OUT>(p, rs, grid, s);
}

template <int FORM, int OUT>
hipError_t launch_rows(const SeamParams &p, int rs, int grid, hipStream_t s)
{
    dim3 g(grid), b(kThreads);
    switch (rs) {
    case 1: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 1>), g, b, 0, s, p); break;
    case 2: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 2>), g, b, 0, s, p); break;
    case 4: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 4>), g, b, 0, s, p); break;
    case 8: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 8>), g, b, 0, s, p); break;
    case 10: hipLaunchKernelGGL((seam_rows_kernel<FORM, OUT, 10>), g, b, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool row_segs_instance(int rs) { return rs == 1 || rs == 2 || rs == 4 || rs == 8 || rs == 10; }

hipError_t launch_fn_pack(const float *fn, int H, void *pack, hipStream_t s)
{
    int total = (H / kChunk) * 4 * 3 * 64;
    int threads = 256;
    hipLaunchKernelGGL(fn_pack_kernel, dim3((total + threads - 1) / threads), dim3(threads), 0, s,
                       fn, H, reinterpret_cast<u32x4 *>(pack), total);
    return hipGetLastError();
}

hipError_t launch_seam(const SeamParams &p, int form, int out, int row_segs, int grid,
                       hipStream_t s)
{
    if (form == kCollapse) {
        // whole-row launches only, a tail of one-segment splits in line
        if (row_segs == 0 || (p.rows_blocks < p.nblocks && p.segs_per_split > kWaves) ||
            !p.skip_gates)
            return hipErrorInvalidValue;
        if (out == kMxfp8G128) return launch_rows<kCollapse, kMxfp8G128>(p, row_segs, grid, s);
        if (out == kBf16) return launch_rows<kCollapse, kBf16>(p, row_segs, grid, s);
        if (out == kFp8Grid) return launch_rows<kCollapse, kFp8Grid>(p, row_segs, grid, s);
        return launch_rows<kCollapse, kMxfp8>(p, row_segs, grid, s);
    }
    if (out == kMxfp8G128) {
        // fused 128-wide groups: whole-row launches without a split tail only
        if (row_segs == 0 || p.rows_blocks != grid)
            return hipErrorInvalidValue;
        return form == kPost ? launch_rows<kPost, kMxfp8G128>(p, row_segs, grid, s)
                             : launch_rows<kNoPost, kMxfp8G128>(p, row_segs, grid, s);
    }
    if (form == kPost) {
        if (out == kBf16) return launch_form_out<kPost, kBf16>(p, row_segs, grid, s);
        if (out == kFp8Grid) return launch_form_out<kPost, kFp8Grid>(p, row_segs, grid, s);
        return launch_form_out<kPost, kMxfp8>(p, row_segs, grid, s);
    }
    if (out == kBf16) return launch_form_out<kNoPost, kBf16>(p, row_segs, grid, s);
    if (out == kFp8Grid) return launch_form_out<kNoPost, kFp8Grid>(p, row_segs, grid, s);
    return launch_form_out<kNoPost, kMxfp8>(p, row_segs, grid, s);
}

hipError_t launch_quantize(const uint16_t *src, int rows, int H, int group, uint8_t *codes,
                           uint8_t *scales, uint16_t *grid, hipStream_t s)
{
    const int ntiles = ((rows + 7) / 8) * (H / (group == 128 ? 128 : kSeg));
    int blocks = (ntiles + 3) / 4;
    if (blocks > 256 * 8)
        blocks = 256 * 8;
    if (group == 128)
        hipLaunchKernelGGL(quantize128_kernel, dim3(blocks), dim3(256), 0, s, src, rows, H,
                           codes, scales, grid);
    else
        hipLaunchKernelGGL(quantize_kernel, dim3(blocks), dim3(256), 0, s, src, rows, H, codes,
                           scales, grid);
    return hipGetLastError();
}

}  // namespace mhc
