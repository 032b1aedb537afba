// gemm_kernels.hip -- the consumer GEMM of the MXFP8 norm.
//
// "[FlyDSL] Single-launch Mega-mHC on gfx950", Kernel Architecture and Test
// Result: the seam's ue8m0/e4m3 output is the next layer's GEMM input, and
// the scale format is priced with that GEMM included.  Here both operands
// are MXFP8 along K (e4m3fn codes, one ue8m0 scale per 32 consecutive K
// elements), as the seam writes them, so the seam's codes and scales are
// the A operand as they are:
//   out[t][n] = bf16( sum_k a[t][k] 2^(sa[t][k/32]-127) b[n][k] 2^(sb[n][k/32]-127) )
// a [T][K], sa [T][K/32], b [N][K] (weights), sb [N][K/32]; fp32 accumulate.
//
// gfx950's block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, fp8 e4m3
// operands) applies the scales itself.  Its operand layout, fixed with an
// in-bounds probe on the device: lane l, byte j of an operand holds row
// (A) or column (B) l % 16 at k = 16 (l / 16) + j for j < 16 and at
// k = 64 + 16 (l / 16) + j - 16 for j >= 16; byte 0 of lane l's scale
// register is the scale of row/column l % 16, K block l / 16 (the
// instruction's byte selects pick another byte of the register).  So each
// lane reads two 16-byte pieces of its row and one scale byte per 128-wide
// K step.
//
// Tiled kernels (T > 32): a workgroup computes a TM x TN block of out, each
// wave WM x WN of it.  Each 128-wide K step of the block's A and B rows and
// their scales is staged in LDS, double-buffered: the next step's global
// loads are in flight while the current one is multiplied, and each row
// leaves global memory once per workgroup.  Two shapes: 256 x 256 blocks on
// 8 waves of 128 x 64 for large T, 128 x 128 blocks on 4 waves of 64 x 64
// where the large blocks would leave CUs idle.  A few-row kernel without
// staging serves T <= 32.
#include <hip/hip_runtime.h>

#include "seam_internal.h"

#ifndef GEMM_BIG_COST
#define GEMM_BIG_COST 28
#endif

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStep = 128;   // K per MFMA
constexpr int kRow = 144;    // LDS bytes per staged row: 128 + 16 of padding, so that
                             // the 16 lanes of a 16-byte read phase hit all 64 banks

__device__ __forceinline__ i32x8 join(const u32x4 &lo, const u32x4 &hi)
{
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// The block-scaled MFMA with scale bytes oa of sa and ob of sb (both
// constants once the caller's loops are unrolled: every case is one
// instruction with its byte selects).
__device__ __forceinline__ f32x4 mfma_sel(const i32x8 &a, const i32x8 &b, const f32x4 &c, int sa,
                                          int oa, int sb, int ob)
{
#define MFMA_SEL(A, B)                                                                     \
    case A * 4 + B:                                                                        \
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, A, sa, B, sb);
    switch (oa * 4 + ob) {
        MFMA_SEL(0, 0) MFMA_SEL(0, 1) MFMA_SEL(0, 2) MFMA_SEL(0, 3)
        MFMA_SEL(1, 0) MFMA_SEL(1, 1) MFMA_SEL(1, 2) MFMA_SEL(1, 3)
        MFMA_SEL(2, 0) MFMA_SEL(2, 1) MFMA_SEL(2, 2) MFMA_SEL(2, 3)
        MFMA_SEL(3, 0) MFMA_SEL(3, 1) MFMA_SEL(3, 2) MFMA_SEL(3, 3)
    }
#undef MFMA_SEL
    return c;
}

// ------------------------------------------------------------ tiled kernels --
//
// A workgroup of NW = (TM / WM) (TN / WN) waves, one thread per staged row's
// scale dword (TM + TN threads).  Per 128-wide K step a wave reads its A and
// B rows from LDS once, (WM + WN) x 128 bytes, for WM x WN x 128
// multiply-adds: the 128 x 64 wave tile reads 0.75 KB per MFMA, the 64 x 64
// one 1 KB.
//
// Large blocks (TM = TN = 256, WM = 128, WN = 64; 148 KB of LDS, 228
// VGPRs): at T = 16384, N = K = 5120 about 460-520 us from box to box (a
// 256 x 128 block took 650 us, 4 waves of 128 x 128 about 570 us).
template <int TM_, int TN_, int WM_, int WN_>
struct Tile {
    static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
    static constexpr int NW = (TM / WM) * (TN / WN);
    static constexpr int kThreads = 64 * NW;
    static constexpr int kChunksA = TM * 8 / kThreads;   // 16-byte chunks per thread and step
    static constexpr int kChunksB = TN * 8 / kThreads;
    // Scales are staged transposed: byte g * kScaleA + (TM / 16) r + I holds
    // the scale of A row 16 I + r, K block g (B alike).  A lane (row r of
    // its tiles, K block g) reads the scales of its WM / 16 A tiles as one
    // word of WM / 16 bytes and those of its WN / 16 B tiles likewise, and
    // the MFMA's byte select picks each tile's byte.  The 16 bytes between
    // K blocks put the four blocks' reads on other banks.
    static constexpr int kScaleA = TM + 16, kScaleB = TN + 16;
    static_assert(kThreads == TM + TN, "one thread per staged row's scales");
    static_assert(kChunksA * kThreads == TM * 8 && kChunksB * kThreads == TN * 8, "chunks");
    static_assert(WM % 64 == 0 && WN % 64 == 0, "scale words of whole dwords");
};

template <class C>
struct StageT {
    uint8_t a[C::TM * kRow];
    uint8_t b[C::TN * kRow];
    uint8_t sa[4 * C::kScaleA];
    uint8_t sb[4 * C::kScaleB];
};

template <class C>
struct RegsT {
    u32x4 a[C::kChunksA], b[C::kChunksB];
    u32 s;   // the scale dword (4 K blocks) of one A row (threads < TM) or B row
};

// A block's operand sources: buffer resources based at the block's first
// row, so that every offset fits 32 bits whatever T * K, and this thread's
// row offsets, which do not change from step to step (the step is the
// uniform offset).  Thread t stages 16-byte chunks t + kThreads i of the A
// and B rows (8 threads per 128-byte row) and the scale dword of A row t
// (t < TM) or B row t - TM; rows past the end re-read the last.
template <class C>
struct SrcT {
    rsrc_t a, b, s;
    int oa[C::kChunksA], ob[C::kChunksB], os;
};

template <class C>
__device__ __forceinline__ SrcT<C> src_tile(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                                            const uint8_t *sb, int K, int m_blk, int n_blk, int T,
                                            int N, int tid)
{
    const int ra = min(C::TM, T - m_blk), rb = min(C::TN, N - n_blk), kb = K / 32;
    SrcT<C> s;
    s.a = make_rsrc(a + (size_t)m_blk * K, (uint32_t)(ra * K));
    s.b = make_rsrc(b + (size_t)n_blk * K, (uint32_t)(rb * K));
#pragma unroll
    for (int i = 0; i < C::kChunksA; ++i) {
        const int c = tid + C::kThreads * i, row = c >> 3, col = (c & 7) * 16;
        s.oa[i] = min(row, ra - 1) * K + col;
    }
#pragma unroll
    for (int i = 0; i < C::kChunksB; ++i) {
        const int c = tid + C::kThreads * i, row = c >> 3, col = (c & 7) * 16;
        s.ob[i] = min(row, rb - 1) * K + col;
    }
    // waves 0 .. TM/64 - 1 take A rows, the others B rows: the resource is
    // uniform across each wave
    if (tid < C::TM) {
        s.s = make_rsrc(sa + (size_t)m_blk * kb, (uint32_t)(ra * kb));
        s.os = min(tid, ra - 1) * kb;
    } else {
        s.s = make_rsrc(sb + (size_t)n_blk * kb, (uint32_t)(rb * kb));
        s.os = min(tid - C::TM, rb - 1) * kb;
    }
    return s;
}

template <class C>
__device__ __forceinline__ void fetch_tile(const SrcT<C> &s, int ks, RegsT<C> &r)
{
#pragma unroll
    for (int i = 0; i < C::kChunksA; ++i)
        r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(s.a, s.oa[i], ks * kStep, 0);
#pragma unroll
    for (int i = 0; i < C::kChunksB; ++i)
        r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(s.b, s.ob[i], ks * kStep, 0);
    r.s = __builtin_amdgcn_raw_buffer_load_b32(s.s, s.os, 4 * ks, 0);
}

template <class C>
__device__ __forceinline__ void stash_tile(StageT<C> &st, int tid, const RegsT<C> &r)
{
#pragma unroll
    for (int i = 0; i < C::kChunksA; ++i) {
        const int c = tid + C::kThreads * i, row = c >> 3, col = (c & 7) * 16;
        *reinterpret_cast<u32x4 *>(st.a + row * kRow + col) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < C::kChunksB; ++i) {
        const int c = tid + C::kThreads * i, row = c >> 3, col = (c & 7) * 16;
        *reinterpret_cast<u32x4 *>(st.b + row * kRow + col) = r.b[i];
    }
    // scale bytes of row R (A for tid < TM, then B), transposed
    const bool is_a = tid < C::TM;
    uint8_t *t = is_a ? st.sa : st.sb;
    const int R = is_a ? tid : tid - C::TM, tile = R >> 4, rr = R & 15;
    const int gs = is_a ? C::kScaleA : C::kScaleB, rs = is_a ? C::TM / 16 : C::TN / 16;
#pragma unroll
    for (int g = 0; g < 4; ++g)
        t[g * gs + rr * rs + tile] = (uint8_t)(r.s >> (8 * g));
}

// Block order.  Workgroup w runs on XCD w % 8 (the dispatcher deals
// consecutive workgroups out to the 8 XCDs in turn; nothing here depends on
// it for correctness).  XCD x takes the x-th eighth of the blocks in a
// grouped order: groups of 8 row blocks, all column blocks of a group before
// the next, so that the workgroups resident on an XCD share A rows and B
// rows at about the same K step in that XCD's L2.
constexpr int kGroupRows = 8;

__device__ __forceinline__ bool block_of(int w, int mb, int nb, int &m, int &n)
{
    const int total = mb * nb, per_xcd = (total + 7) / 8;
    const int L = (w % 8) * per_xcd + w / 8;
    if (L >= total)
        return false;
    const int group = L / (kGroupRows * nb), first = group * kGroupRows;
    const int gm = min(mb - first, kGroupRows), in = L % (kGroupRows * nb);
    m = first + in % gm;
    n = in / gm;
    return true;
}

// Scale words of a wave's NB tiles (NB / 4 dwords, one byte per tile)
template <int NB>
__device__ __forceinline__ void scale_words(const uint8_t *p, u32 (&w)[NB / 4])
{
    if (NB / 4 == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
        w[0] = v[0];
        w[NB / 4 == 2 ? 1 : 0] = v[1];
    } else {
#pragma unroll
        for (int q = 0; q < NB / 4; ++q)
            w[q] = *reinterpret_cast<const u32 *>(p + 4 * q);
    }
}

template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void mxfp8_gemm_tile_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa,
    const uint8_t *__restrict__ b, const uint8_t *__restrict__ sb, int T, int N, int K,
    uint16_t *__restrict__ out)
{
    constexpr int MI = C::WM / 16, NJ = C::WN / 16;   // MFMA tiles of a wave block
    __shared__ StageT<C> st[2];
    static_assert(2 * sizeof(StageT<C>) >= C::TM * C::TN * 2, "the output tile fits the stages");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int mi, ni;
    if (!block_of(blockIdx.x, (T + C::TM - 1) / C::TM, (N + C::TN - 1) / C::TN, mi, ni))
        return;
    const int m_blk = mi * C::TM, n_blk = ni * C::TN;
    const int wm = (wave / (C::TN / C::WN)) * C::WM, wn = (wave % (C::TN / C::WN)) * C::WN;
    const int g = lane >> 4, r = lane & 15;
    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int steps = K / kStep;
    const SrcT<C> src = src_tile<C>(a, sa, b, sb, K, m_blk, n_blk, T, N, tid);
    RegsT<C> rg;
    fetch_tile<C>(src, 0, rg);
    stash_tile<C>(st[0], tid, rg);
    __syncthreads();   // step 0 in LDS
    // The step loop has no branch (the last step re-reads itself into the
    // idle buffer): a conditional stash made the compiler sink the MFMAs
    // into the join block behind the stash.  The scheduling barriers keep
    // the next step's global loads at the top of the step, ahead of the
    // MFMAs (left to itself the compiler issued them after the last MFMA,
    // into registers the fragments had just freed, and the stash then waited
    // out their whole latency every step), and the MFMAs ahead of the stash.
    for (int ks = 0; ks < steps; ++ks) {
        const StageT<C> &cur = st[ks & 1];
        fetch_tile<C>(src, min(ks + 1, steps - 1), rg);
        __builtin_amdgcn_sched_barrier(0);
        u32 sca[MI / 4], scb[NJ / 4];
        scale_words<MI>(cur.sa + g * C::kScaleA + r * (C::TM / 16) + wm / 16, sca);
        scale_words<NJ>(cur.sb + g * C::kScaleB + r * (C::TN / 16) + wn / 16, scb);
        i32x8 fb[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint8_t *p = cur.b + (wn + 16 * j + r) * kRow + 16 * g;
            fb[j] = join(*reinterpret_cast<const u32x4 *>(p),
                         *reinterpret_cast<const u32x4 *>(p + 64));
        }
        // a wave issuing its MFMAs goes ahead of the other wave of its SIMD,
        // whose LDS reads then overlap them (2% faster at 16384 x 5120 x 5120)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint8_t *p = cur.a + (wm + 16 * i + r) * kRow + 16 * g;
            const i32x8 fa = join(*reinterpret_cast<const u32x4 *>(p),
                                  *reinterpret_cast<const u32x4 *>(p + 64));
            const int sai = (int)sca[i >> 2];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = mfma_sel(fa, fb[j], acc[i][j], sai, i & 3, (int)scb[j >> 2], j & 3);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);   // the step's MFMAs issue before the stash
        stash_tile<C>(st[(ks + 1) & 1], tid, rg);
        __syncthreads();
    }
    // out tile in LDS as bf16 [TM][TN] (lane l holds rows 4 (l / 16) + e,
    // column l % 16 of each 16 x 16 tile), then 16-byte row pieces to memory
    uint16_t *ot = reinterpret_cast<uint16_t *>(&st[0]);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const __bf16 v = (__bf16)acc[i][j][e];
                ot[(wm + 16 * i + 4 * g + e) * C::TN + wn + 16 * j + r] =
                    __builtin_bit_cast(uint16_t, v);
            }
    __syncthreads();
    const bool whole = N % 8 == 0;
    for (int c = tid; c < C::TM * C::TN / 8; c += C::kThreads) {
        const int row = c / (C::TN / 8), col = (c % (C::TN / 8)) * 8;
        const int gr = m_blk + row, gc = n_blk + col;
        if (gr >= T || gc >= N)
            continue;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ot + row * C::TN + col);
        uint16_t *dst = out + (size_t)gr * N + gc;
        if (whole) {
            *reinterpret_cast<u32x4 *>(dst) = v;
        } else {
            const uint16_t *e8 = ot + row * C::TN + col;
            for (int e = 0; e < 8 && gc + e < N; ++e)
                dst[e] = e8[e];
        }
    }
}

using BigTile = Tile<256, 256, 128, 64>;
using MidTile = Tile<128, 128, 64, 64>;

// ----------------------------------------------------------- few rows --

// Few rows (T <= 32, decode): TILES 16-row tiles of out
// against 16 columns of the weights per workgroup, the K steps dealt to the
// 8 waves in turn, every operand straight from memory into MFMA layout
// (within a workgroup nothing is read twice, so there is nothing to stage).
// N / 16 workgroups then stream the weights once, where the 256-row blocks
// leave all but N / 128 CUs idle (T = 4, N = K = 5120: 52 us).  Each wave's
// partial tile goes through LDS and wave 0 adds the 8 in wave order.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyChunk = 4;   // K steps per wave whose loads are in flight together

template <int TILES>
__global__ __launch_bounds__(64 * kSkinnyWaves) void mxfp8_gemm_skinny_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa,
    const uint8_t *__restrict__ b, const uint8_t *__restrict__ sb, int T, int N, int K,
    uint16_t *__restrict__ out)
{
    __shared__ f32x4 red[kSkinnyWaves][TILES][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16;
    const int r = lane & 15, g = lane >> 4;
    const int steps = K / kStep, kb = K / 32;
    const int rb = min(16, N - n0);
    const rsrc_t ra_ = make_rsrc(a, (uint32_t)(T * K));
    const rsrc_t rsa = make_rsrc(sa, (uint32_t)(T * kb));
    const rsrc_t rb_ = make_rsrc(b + (size_t)n0 * K, (uint32_t)(rb * K));
    const rsrc_t rsb = make_rsrc(sb + (size_t)n0 * kb, (uint32_t)(rb * kb));
    int oa[TILES], osa[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int row = min(16 * t + r, T - 1);   // rows past T re-read the last
        oa[t] = row * K + 16 * g;
        osa[t] = row * kb;
    }
    const int ob = min(r, rb - 1) * K + 16 * g, osb = min(r, rb - 1) * kb;
    f32x4 acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = wave; c0 < steps; c0 += kSkinnyWaves * kSkinnyChunk) {
        i32x8 fa[kSkinnyChunk][TILES], fb[kSkinnyChunk];
        int sca[kSkinnyChunk][TILES], scb[kSkinnyChunk];
#pragma unroll
        for (int c = 0; c < kSkinnyChunk; ++c) {
            const int ks = min(c0 + kSkinnyWaves * c, steps - 1);   // past the end: re-read, unused
            fb[c] = join(__builtin_amdgcn_raw_buffer_load_b128(rb_, ob, ks * kStep, 0),
                         __builtin_amdgcn_raw_buffer_load_b128(rb_, ob + 64, ks * kStep, 0));
            scb[c] = (int)(__builtin_amdgcn_raw_buffer_load_b32(rsb, osb, 4 * ks, 0) >> (8 * g));
#pragma unroll
            for (int t = 0; t < TILES; ++t) {
                fa[c][t] = join(__builtin_amdgcn_raw_buffer_load_b128(ra_, oa[t], ks * kStep, 0),
                                __builtin_amdgcn_raw_buffer_load_b128(ra_, oa[t] + 64, ks * kStep,
                                                                      0));
                sca[c][t] =
                    (int)(__builtin_amdgcn_raw_buffer_load_b32(rsa, osa[t], 4 * ks, 0) >> (8 * g));
            }
        }
#pragma unroll
        for (int c = 0; c < kSkinnyChunk; ++c) {
            if (c0 + kSkinnyWaves * c < steps) {
#pragma unroll
                for (int t = 0; t < TILES; ++t)
                    acc[t] = mfma_sel(fa[c][t], fb[c], acc[t], sca[c][t], 0, scb[c], 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t)
        red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        f32x4 sum = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < kSkinnyWaves; ++w)
            sum += red[w][t][lane];
        // lane l holds rows 4 (l / 16) + e, column l % 16 of the tile
        const int col = n0 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * t + 4 * g + e;
            if (row < T && col < N)
                out[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, (__bf16)sum[e]);
        }
    }
}

}  // namespace

template <class C>
static hipError_t launch_tile(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                              const uint8_t *sb, int T, int N, int K, uint16_t *out, hipStream_t s)
{
    const int64_t total = (int64_t)((T + C::TM - 1) / C::TM) * ((N + C::TN - 1) / C::TN);
    if (total > INT32_MAX / 2)
        return hipErrorInvalidValue;
    const int grid = (int)((total + 7) / 8 * 8);   // whole rounds of the 8 XCDs
    hipLaunchKernelGGL(mxfp8_gemm_tile_kernel<C>, dim3(grid), dim3(C::kThreads), 0, s, a, sa, b,
                       sb, T, N, K, out);
    return hipGetLastError();
}

hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                             const uint8_t *sb, int T, int N, int K, uint16_t *out, int cus,
                             hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    if (T <= 32) {
        const int grid = (N + 15) / 16;
        if (T <= 16)
            hipLaunchKernelGGL(mxfp8_gemm_skinny_kernel<1>, dim3(grid), dim3(64 * kSkinnyWaves), 0,
                               s, a, sa, b, sb, T, N, K, out);
        else
            hipLaunchKernelGGL(mxfp8_gemm_skinny_kernel<2>, dim3(grid), dim3(64 * kSkinnyWaves), 0,
                               s, a, sa, b, sb, T, N, K, out);
        return hipGetLastError();
    }
    // the large blocks where their rounds of the CUs cost less than the mid
    // blocks': one large block does 4 mid blocks' work in about 2.8 times
    // their time (N = K = 5120: mid blocks up to T = 1536 and at 4096, large
    // ones at 2048, 3072 and from 8192 on)
    const int64_t rounds_big = ((int64_t)((T + 255) / 256) * ((N + 255) / 256) + cus - 1) / cus;
    const int64_t rounds_mid = ((int64_t)((T + 127) / 128) * ((N + 127) / 128) + cus - 1) / cus;
    if (GEMM_BIG_COST * rounds_big < 10 * rounds_mid)
        return launch_tile<BigTile>(a, sa, b, sb, T, N, K, out, s);
    return launch_tile<MidTile>(a, sa, b, sb, T, N, K, out, s);
}

}  // namespace mhc
