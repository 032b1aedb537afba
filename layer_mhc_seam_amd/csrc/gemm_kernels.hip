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
// register is the scale of row/column l % 16, K block l / 16.  So each lane
// loads two 16-byte pieces of its row and one scale byte per 128-wide K step.
//
// Tiling: a workgroup of 8 waves computes a 256 x 128 block of out, each
// wave 64 x 64 (4 x 4 MFMA tiles, 16 fp32 accumulators), two waves per SIMD.
// Each 128-wide K step of the block's A and B rows and their scale dwords
// (one coalesced dword per row: per-lane byte loads touch 16 rows each and
// doubled the L1 requests) is staged in LDS, double-buffered: the next
// step's global loads are in flight while the current one is multiplied,
// and each row leaves global memory once per workgroup.  A 128 x 128 block
// on 4 waves needed about 64 bytes of operands per clock per CU at full
// MFMA rate, about all that a CU's L1 delivers; 256 x 128 needs about 48.
#include <hip/hip_runtime.h>

#include "seam_internal.h"

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileM = 256;  // workgroup block: rows of out (tokens)
constexpr int kTileN = 128;  // ... columns of out
constexpr int kWave = 64;    // wave block (both ways)
constexpr int kStep = 128;   // K per MFMA

constexpr int kRow = 144;    // LDS bytes per staged row: 128 + 16 of padding, so that
                             // the 8 lanes of a 16-byte read phase hit all 32 banks
constexpr int kThreadsG = 512;
constexpr int kChunksA = kTileM * 8 / kThreadsG;   // 16-byte chunks per thread and step
constexpr int kChunksB = kTileN * 8 / kThreadsG;

// one K step of the workgroup's operands: A and B rows (128 bytes each) and
// their scale dwords (4 ue8m0 bytes: the step's four 32-wide K blocks)
struct Stage {
    uint8_t a[kTileM * kRow];
    uint8_t b[kTileN * kRow];
    u32 sa[kTileM];
    u32 sb[kTileN];
};

struct Regs {
    u32x4 a[kChunksA], b[kChunksB];
    u32 s;
};

__device__ __forceinline__ i32x8 join(const u32x4 &lo, const u32x4 &hi)
{
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// step ks into registers: thread t takes 16-byte chunks t + 512 i of the A
// and B rows (8 threads per 128-byte row, coalesced) and, for t < 384, one
// scale dword (A rows, then B rows); rows past the end re-read the last
__device__ __forceinline__ void fetch_step(const uint8_t *__restrict__ a,
                                          const uint8_t *__restrict__ sa,
                                          const uint8_t *__restrict__ b,
                                          const uint8_t *__restrict__ sb, int K, int ks,
                                          int m_blk, int n_blk, int T, int N, int tid, Regs &r)
{
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int c = tid + kThreadsG * i, row = c >> 3, col = (c & 7) * 16;
        const int ta = min(m_blk + row, T - 1);
        r.a[i] = *reinterpret_cast<const u32x4 *>(a + (size_t)ta * K + ks * kStep + col);
    }
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) {
        const int c = tid + kThreadsG * i, row = c >> 3, col = (c & 7) * 16;
        const int nb = min(n_blk + row, N - 1);
        r.b[i] = *reinterpret_cast<const u32x4 *>(b + (size_t)nb * K + ks * kStep + col);
    }
    const int kb = K / 32;
    if (tid < kTileM) {
        const int ta = min(m_blk + tid, T - 1);
        r.s = *reinterpret_cast<const u32 *>(sa + (size_t)ta * kb + 4 * ks);
    } else if (tid < kTileM + kTileN) {
        const int nb = min(n_blk + tid - kTileM, N - 1);
        r.s = *reinterpret_cast<const u32 *>(sb + (size_t)nb * kb + 4 * ks);
    }
}

__device__ __forceinline__ void stash_step(Stage &st, int tid, const Regs &r)
{
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int c = tid + kThreadsG * i, row = c >> 3, col = (c & 7) * 16;
        *reinterpret_cast<u32x4 *>(st.a + row * kRow + col) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) {
        const int c = tid + kThreadsG * i, row = c >> 3, col = (c & 7) * 16;
        *reinterpret_cast<u32x4 *>(st.b + row * kRow + col) = r.b[i];
    }
    if (tid < kTileM)
        st.sa[tid] = r.s;
    else if (tid < kTileM + kTileN)
        st.sb[tid - kTileM] = r.s;
}

// Block order.  Workgroup w runs on XCD w % 8 (the dispatcher deals
// consecutive workgroups out to the 8 XCDs in turn; nothing here depends on
// it for correctness).  XCD x takes the x-th eighth of the blocks in a
// grouped order: groups of kGroupM row blocks, all column blocks of a group
// before the next, so the workgroups resident on an XCD share A rows and B
// rows at about the same K step in that XCD's L2.
constexpr int kGroupM = 2;

__device__ __forceinline__ bool block_of(int w, int mb, int nb, int &m, int &n)
{
    const int total = mb * nb, per_xcd = (total + 7) / 8;
    const int L = (w % 8) * per_xcd + w / 8;
    if (L >= total)
        return false;
    const int group = L / (kGroupM * nb), first = group * kGroupM;
    const int gm = min(mb - first, kGroupM), in = L % (kGroupM * nb);
    m = first + in % gm;
    n = in / gm;
    return true;
}

__global__ __launch_bounds__(kThreadsG) void mxfp8_gemm_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa,
    const uint8_t *__restrict__ b, const uint8_t *__restrict__ sb, int T, int N, int K,
    uint16_t *__restrict__ out)
{
    __shared__ Stage st[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int mi, ni;
    if (!block_of(blockIdx.x, (T + kTileM - 1) / kTileM, (N + kTileN - 1) / kTileN, mi, ni))
        return;
    const int m_blk = mi * kTileM, n_blk = ni * kTileN;
    const int wm = (wave >> 1) * kWave, wn = (wave & 1) * kWave;   // wave block in the tile
    const int g = lane >> 4, r = lane & 15;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int steps = K / kStep;
    Regs rg;
    fetch_step(a, sa, b, sb, K, 0, m_blk, n_blk, T, N, tid, rg);
    stash_step(st[0], tid, rg);
    __syncthreads();   // step 0 in LDS
    for (int ks = 0; ks < steps; ++ks) {
        const Stage &cur = st[ks & 1];
        if (ks + 1 < steps)
            fetch_step(a, sa, b, sb, K, ks + 1, m_blk, n_blk, T, N, tid, rg);
        // this lane's scale bytes of the step: rows of its tiles, K block g
        const uint8_t *csa = reinterpret_cast<const uint8_t *>(cur.sa);
        const uint8_t *csb = reinterpret_cast<const uint8_t *>(cur.sb);
        int sca[4], scb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sca[i] = csa[(wm + 16 * i + r) * 4 + g];
            scb[i] = csb[(wn + 16 * i + r) * 4 + g];
        }
        i32x8 fb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint8_t *p = cur.b + (wn + 16 * j + r) * kRow + 16 * g;
            fb[j] = join(*reinterpret_cast<const u32x4 *>(p),
                         *reinterpret_cast<const u32x4 *>(p + 64));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint8_t *p = cur.a + (wm + 16 * i + r) * kRow + 16 * g;
            const i32x8 fa = join(*reinterpret_cast<const u32x4 *>(p),
                                  *reinterpret_cast<const u32x4 *>(p + 64));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                // formats 0, 0: fp8 e4m3 for A and B; scale byte 0 of each
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fa, fb[j], acc[i][j], 0, 0, 0, sca[i], 0, scb[j]);
        }
        if (ks + 1 < steps)
            stash_step(st[(ks + 1) & 1], tid, rg);
        __syncthreads();
    }
    // lane l holds rows 4 (l / 16) + e, column l % 16 of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n_blk + wn + 16 * j + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m_blk + wm + 16 * i + 4 * g + e;
                if (row < T && col < N) {
                    const __bf16 v = (__bf16)acc[i][j][e];
                    out[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, v);
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Large shapes: a 256 x 256 block of out per workgroup of 8 waves (two per
// SIMD), each wave 128 x 64 = 8 x 4 MFMA tiles of 16 x 16 (128 fp32
// accumulators per lane).  Per 128-wide K step a wave reads its A and B rows
// from LDS once, (128 + 64) x 128 bytes, for 128 x 64 x 128 multiply-adds:
// fewer LDS bytes per flop than the 64 x 64 wave tile above, whose 128 KB of
// reads and 48 KB of writes per step per CU outlasted the step's MFMAs.
// Staging as in the kernel above (padded 144-byte rows, double-buffered, the
// next step's global loads in flight during the current step's MFMAs), with
// buffer loads from per-block resources and the scales staged transposed
// (below); the output is rounded to bf16 into LDS and stored in 16-byte row
// pieces.  At T = 16384, N = K = 5120: about 510 us (4 waves of 128 x 128
// each: 616 us; the 256 x 128 kernel: 660 us).
constexpr int kBig = 256;          // block rows and columns
constexpr int kBigWaveM = 128;     // wave block rows
constexpr int kBigWaveN = 64;      // wave block columns
constexpr int kBigThreads = 512;   // 8 waves
constexpr int kBigChunks = kBig * 8 / kBigThreads;   // 16-byte chunks per thread, per operand

// Scales are staged transposed: byte g * kScaleG + 16 r + I holds the scale
// of row 16 I + r, K block g.  A lane (row r of its tiles, K block g) then
// reads the scales of its 8 A tiles as one 8-byte word and those of its 4 B
// tiles as one dword, and the MFMA's byte select picks each tile's byte.
// The 16 bytes between K blocks put the four blocks' reads on other banks.
constexpr int kScaleG = 16 * 16 + 16;
struct StageBig {
    uint8_t a[kBig * kRow];
    uint8_t b[kBig * kRow];
    uint8_t sa[4 * kScaleG];
    uint8_t sb[4 * kScaleG];
};
static_assert(2 * sizeof(StageBig) >= kBig * kBig * 2, "the output tile fits the stages");

struct RegsBig {
    u32x4 a[kBigChunks], b[kBigChunks];
    u32 s;   // the scale dword (4 K blocks) of one A row (threads < 256) or B row
};

// Block order for the large tiles: as block_of, in groups of 8 row blocks,
// so that an XCD's share (one eighth of the blocks) is a few groups and its
// resident workgroups cover 8 row blocks x 4 column blocks at a time.
constexpr int kGroupBig = 8;
// the large tiles are considered from this many rows of out
#ifndef GEMM_BIG_MIN_ROWS
#define GEMM_BIG_MIN_ROWS 2048
#endif
constexpr int kBigMinRows = GEMM_BIG_MIN_ROWS;

__device__ __forceinline__ bool block_of_big(int w, int mb, int nb, int &m, int &n)
{
    const int total = mb * nb, per_xcd = (total + 7) / 8;
    const int L = (w % 8) * per_xcd + w / 8;
    if (L >= total)
        return false;
    const int group = L / (kGroupBig * nb), first = group * kGroupBig;
    const int gm = min(mb - first, kGroupBig), in = L % (kGroupBig * nb);
    m = first + in % gm;
    n = in / gm;
    return true;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// A block's operand sources: buffer resources based at the block's first
// row, so that every offset fits 32 bits whatever T * K, and this thread's
// row offsets, which do not change from step to step (the step is the
// uniform offset).  Thread t stages 16-byte chunks t + 512 i of the A and B
// rows (8 threads per 128-byte row) and the scale dword of A row t (waves
// 0-3) or B row t - 256 (waves 4-7); rows past the end re-read the last.
struct SrcBig {
    rsrc_t a, b, s;
    int oa[kBigChunks], ob[kBigChunks], os;
};

__device__ __forceinline__ SrcBig src_big(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                                          const uint8_t *sb, int K, int m_blk, int n_blk, int T,
                                          int N, int tid, int wave)
{
    const int ra = min(kBig, T - m_blk), rb = min(kBig, N - n_blk), kb = K / 32;
    SrcBig s;
    s.a = make_rsrc(a + (size_t)m_blk * K, (uint32_t)(ra * K));
    s.b = make_rsrc(b + (size_t)n_blk * K, (uint32_t)(rb * K));
#pragma unroll
    for (int i = 0; i < kBigChunks; ++i) {
        const int c = tid + kBigThreads * i, row = c >> 3, col = (c & 7) * 16;
        s.oa[i] = min(row, ra - 1) * K + col;
        s.ob[i] = min(row, rb - 1) * K + col;
    }
    if (wave < 4) {
        s.s = make_rsrc(sa + (size_t)m_blk * kb, (uint32_t)(ra * kb));
        s.os = min(tid, ra - 1) * kb;
    } else {
        s.s = make_rsrc(sb + (size_t)n_blk * kb, (uint32_t)(rb * kb));
        s.os = min(tid - kBig, rb - 1) * kb;
    }
    return s;
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

__device__ __forceinline__ void fetch_big(const SrcBig &s, int ks, RegsBig &r)
{
#pragma unroll
    for (int i = 0; i < kBigChunks; ++i) {
        r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(s.a, s.oa[i], ks * kStep, 0);
        r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(s.b, s.ob[i], ks * kStep, 0);
    }
    r.s = __builtin_amdgcn_raw_buffer_load_b32(s.s, s.os, 4 * ks, 0);
}

__device__ __forceinline__ void stash_big(StageBig &st, int tid, const RegsBig &r)
{
#pragma unroll
    for (int i = 0; i < kBigChunks; ++i) {
        const int c = tid + kBigThreads * i, row = c >> 3, col = (c & 7) * 16;
        *reinterpret_cast<u32x4 *>(st.a + row * kRow + col) = r.a[i];
        *reinterpret_cast<u32x4 *>(st.b + row * kRow + col) = r.b[i];
    }
    // scale bytes of row R = tid mod 256 (A for tid < 256, then B), transposed
    uint8_t *t = tid < kBig ? st.sa : st.sb;
    const int R = tid & (kBig - 1), tile = R >> 4, rr = R & 15;
#pragma unroll
    for (int g = 0; g < 4; ++g)
        t[g * kScaleG + rr * 16 + tile] = (uint8_t)(r.s >> (8 * g));
}

__global__ __launch_bounds__(kBigThreads, 1) void mxfp8_gemm_big_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa,
    const uint8_t *__restrict__ b, const uint8_t *__restrict__ sb, int T, int N, int K,
    uint16_t *__restrict__ out)
{
    constexpr int WN = kBigWaveN;
    constexpr int NJ = WN / 16;                 // MFMA tiles across a wave block
    constexpr int kThreads = kBigThreads;
    __shared__ StageBig st[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int mi, ni;
    if (!block_of_big(blockIdx.x, (T + kBig - 1) / kBig, (N + kBig - 1) / kBig, mi, ni))
        return;
    const int m_blk = mi * kBig, n_blk = ni * kBig;
    const int wm = (wave / (kBig / WN)) * kBigWaveM, wn = (wave % (kBig / WN)) * WN;
    const int g = lane >> 4, r = lane & 15;
    f32x4 acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int steps = K / kStep;
    const SrcBig src = src_big(a, sa, b, sb, K, m_blk, n_blk, T, N, tid, wave);
    RegsBig rg;
    fetch_big(src, 0, rg);
    stash_big(st[0], tid, rg);
    __syncthreads();   // step 0 in LDS
    // The step loop has no branch (the last step re-reads itself into the
    // idle buffer): a conditional stash made the compiler sink the MFMAs
    // into the join block behind the stash.  The scheduling barriers keep
    // the next step's global loads at the top of the step, ahead of the
    // MFMAs (left to itself the compiler issued them after the last MFMA,
    // into registers the fragments had just freed, and the stash then waited
    // out their whole latency every step), and the MFMAs ahead of the stash.
    for (int ks = 0; ks < steps; ++ks) {
        const StageBig &cur = st[ks & 1];
        fetch_big(src, min(ks + 1, steps - 1), rg);
        __builtin_amdgcn_sched_barrier(0);
        const u32 scb = *reinterpret_cast<const u32 *>(cur.sb + g * kScaleG + r * 16 + wn / 16);
        const u32x2 sca = *reinterpret_cast<const u32x2 *>(cur.sa + g * kScaleG + r * 16 + wm / 16);
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
        for (int i = 0; i < 8; ++i) {
            const uint8_t *p = cur.a + (wm + 16 * i + r) * kRow + 16 * g;
            const i32x8 fa = join(*reinterpret_cast<const u32x4 *>(p),
                                  *reinterpret_cast<const u32x4 *>(p + 64));
            const int sai = (int)sca[i >> 2];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = mfma_sel(fa, fb[j], acc[i][j], sai, i & 3, (int)scb, j);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);   // the step's MFMAs issue before the stash
        stash_big(st[(ks + 1) & 1], tid, rg);
        __syncthreads();
    }
    // out tile in LDS as bf16 [256][256] (lane l holds rows 4 (l / 16) + e,
    // column l % 16 of each 16 x 16 tile), then 16-byte row pieces to memory
    uint16_t *ot = reinterpret_cast<uint16_t *>(&st[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const __bf16 v = (__bf16)acc[i][j][e];
                ot[(wm + 16 * i + 4 * g + e) * kBig + wn + 16 * j + r] =
                    __builtin_bit_cast(uint16_t, v);
            }
    __syncthreads();
    const bool whole = N % 8 == 0;
    for (int c = tid; c < kBig * kBig / 8; c += kThreads) {
        const int row = c / (kBig / 8), col = (c % (kBig / 8)) * 8;
        const int gr = m_blk + row, gc = n_blk + col;
        if (gr >= T || gc >= N)
            continue;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ot + row * kBig + col);
        uint16_t *dst = out + (size_t)gr * N + gc;
        if (whole) {
            *reinterpret_cast<u32x4 *>(dst) = v;
        } else {
            const uint16_t *e8 = ot + row * kBig + col;
            for (int e = 0; e < 8 && gc + e < N; ++e)
                dst[e] = e8[e];
        }
    }
}

// Few rows (T <= 64, decode and short prefill): TILES 16-row tiles of out
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

hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                             const uint8_t *sb, int T, int N, int K, uint16_t *out, int cus,
                             hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    if (T <= 64) {
        const int grid = (N + 15) / 16;
        if (T <= 16)
            hipLaunchKernelGGL(mxfp8_gemm_skinny_kernel<1>, dim3(grid), dim3(64 * kSkinnyWaves), 0,
                               s, a, sa, b, sb, T, N, K, out);
        else if (T <= 32)
            hipLaunchKernelGGL(mxfp8_gemm_skinny_kernel<2>, dim3(grid), dim3(64 * kSkinnyWaves), 0,
                               s, a, sa, b, sb, T, N, K, out);
        else
            hipLaunchKernelGGL(mxfp8_gemm_skinny_kernel<4>, dim3(grid), dim3(64 * kSkinnyWaves), 0,
                               s, a, sa, b, sb, T, N, K, out);
        return hipGetLastError();
    }
    // the 256 x 256 blocks where their rounds of the CUs cost less: one such
    // block takes about 1.7x a 256 x 128 block (twice the work, measured
    // 1.18x more efficient)
    const int64_t rounds_big =
        ((int64_t)((T + kBig - 1) / kBig) * ((N + kBig - 1) / kBig) + cus - 1) / cus;
    const int64_t rounds_small =
        ((int64_t)((T + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN) + cus - 1) / cus;
    if (T >= kBigMinRows && N >= kBig && 17 * rounds_big < 10 * rounds_small) {
        const int64_t total = (int64_t)((N + kBig - 1) / kBig) * ((T + kBig - 1) / kBig);
        if (total > INT32_MAX / 2)
            return hipErrorInvalidValue;
        const int grid = (int)((total + 7) / 8 * 8);   // whole rounds of the 8 XCDs
        hipLaunchKernelGGL(mxfp8_gemm_big_kernel, dim3(grid), dim3(kBigThreads), 0, s, a, sa, b,
                           sb, T, N, K, out);
        return hipGetLastError();
    }
    const int64_t total = (int64_t)((N + kTileN - 1) / kTileN) * ((T + kTileM - 1) / kTileM);
    if (total > INT32_MAX / 2)
        return hipErrorInvalidValue;
    const int grid = (int)((total + 7) / 8 * 8);   // whole rounds of the 8 XCDs
    hipLaunchKernelGGL(mxfp8_gemm_kernel, dim3(grid), dim3(kThreadsG), 0, s, a, sa, b, sb, T, N,
                       K, out);
    return hipGetLastError();
}

}  // namespace mhc
