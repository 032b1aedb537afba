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
// Tiled kernel: a workgroup computes a TM x TN block of out, each wave
// WM x WN of it.  Each 128-wide K step of the block's A and B rows and their
// scales is loaded straight into one of S stages of LDS: the next S - 1
// steps' loads are in flight while the current one is multiplied, and each
// row leaves global memory once per workgroup.  256 x 256 and 128 x 256
// blocks on 8 waves for large T; 128 x 128 down to 16 x 32 blocks on 4 or 2
// waves where fewer blocks fit the CUs, the shape chosen by the bytes each
// CU streams.
#include <hip/hip_runtime.h>

#include "seam_internal.h"

#ifndef GEMM_BIG_COST   // relative cost of a round of 256 x 256 blocks
#define GEMM_BIG_COST 20
#endif
#ifndef GEMM_MID_COST   // and of a round of 128 x 128 blocks, two per CU
#define GEMM_MID_COST 13
#endif

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStep = 128;   // K per MFMA

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
// A workgroup of NW = (TM / WM) (TN / WN) waves computes a TM x TN block of
// out, each wave WM x WN of it, over 128-wide K steps.  Each step's A and B
// rows and their scales go from memory straight into LDS
// (buffer_load_dwordx4 ... lds: the 64 lanes of a wave fill one 1 KB run,
// lane l at byte 16 l), so no register holds them on the way and no LDS
// write instruction is issued.  S stages of LDS keep the next S - 1 steps'
// loads in flight while one step is multiplied.  Per step a wave reads its
// A and B rows from LDS once, (WM + WN) x 128 bytes, for WM x WN x 128
// multiply-adds: the 64 x 128 wave tile reads 0.75 KB per MFMA, the 64 x 64
// one 1 KB.
//
// A run is 8 rows of 128 bytes with no padding.  The 16-byte piece c of
// row R sits in slot c ^ ((R >> 1) & 7) of the row, which puts the 16 lanes
// of a fragment read phase (rows 16 I .. 16 I + 15, one piece each) on 16
// different 16-byte groups of the 64 banks.  The scales are staged as they
// lie in memory, one dword (4 K blocks) per row, A rows then B rows, and a
// lane reads its K block's byte.
template <int TM_, int TN_, int WM_, int WN_, int S_>
struct Tile {
    static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_, S = S_;
    static constexpr int NW = (TM / WM) * (TN / WN);
    static constexpr int kThreads = 64 * NW;
    static constexpr int kRunsA = TM / 8 / NW, kRunsB = TN / 8 / NW;   // 1 KB runs per wave and step
    static constexpr int kLoads = kRunsA + kRunsB + 1;                 // and its scale dwords
    static_assert(kRunsA * 8 * NW == TM && kRunsB * 8 * NW == TN, "whole runs per wave");
    // wave w loads the scale dwords of 64 rows: the A rows, padded to kAS,
    // then the B rows (A rows past TM and waves past the last B row re-read
    // the last row into the padding, so that every wave has the same loads
    // in flight)
    static constexpr int kAS = (TM + 63) / 64 * 64;
    static_assert(kAS + TN <= 64 * NW, "one wave per 64 rows' scale dwords");
    static_assert(S >= 2 && (S - 1) * kLoads < 64, "the loads in flight fit the vmcnt counter");
};

template <class C>
struct StageT {
    uint8_t a[C::TM * kStep];
    uint8_t b[C::TN * kStep];
    uint8_t s[C::NW * 64 * 4];
};

typedef __attribute__((address_space(3))) void *lds_ptr;

// s_waitcnt on the vector memory counter alone: this wave's loads but the
// last N have completed
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The workgroup barrier without __syncthreads()'s release fence, which
// would wait for every load in flight (the stages' loads included).  Every
// LDS read of a wave has completed before the wave gets here (its MFMAs have
// consumed them), and the memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void block_barrier()
{
    asm volatile("s_barrier" ::: "memory");
}

// A block's operand sources: buffer resources based at the block's first
// row, so that every offset fits 32 bits whatever T * K, and this lane's
// offsets, which do not change from step to step (the step is the uniform
// offset).  Wave w fills A runs w kRunsA + i and B runs w kRunsB + i (rows
// 8 run + l / 8, slot l % 8 of lane l) and the scale dwords of rows
// 64 w + l of A then B; rows past the end re-read the last.
template <class C>
struct SrcT {
    rsrc_t a, b, s;
    int oa[C::kRunsA], ob[C::kRunsB], os;
};

template <class C>
__device__ __forceinline__ SrcT<C> src_tile(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                                            const uint8_t *sb, int K, int m_blk, int n_blk, int T,
                                            int N, int wave, int lane)
{
    const int ra = min(C::TM, T - m_blk), rb = min(C::TN, N - n_blk), kb = K / 32;
    SrcT<C> s;
    s.a = make_rsrc(a + (size_t)m_blk * K, (uint32_t)(ra * K));
    s.b = make_rsrc(b + (size_t)n_blk * K, (uint32_t)(rb * K));
    const int slot = lane & 7;
#pragma unroll
    for (int i = 0; i < C::kRunsA; ++i) {
        const int row = 8 * (wave * C::kRunsA + i) + (lane >> 3);
        s.oa[i] = min(row, ra - 1) * K + 16 * (slot ^ ((row >> 1) & 7));
    }
#pragma unroll
    for (int i = 0; i < C::kRunsB; ++i) {
        const int row = 8 * (wave * C::kRunsB + i) + (lane >> 3);
        s.ob[i] = min(row, rb - 1) * K + 16 * (slot ^ ((row >> 1) & 7));
    }
    const int R = 64 * wave + lane;
    if (64 * wave < C::kAS) {   // uniform across the wave
        s.s = make_rsrc(sa + (size_t)m_blk * kb, (uint32_t)(ra * kb));
        s.os = min(R, ra - 1) * kb;
    } else {
        s.s = make_rsrc(sb + (size_t)n_blk * kb, (uint32_t)(rb * kb));
        s.os = min(R - C::kAS, rb - 1) * kb;
    }
    return s;
}

// this wave's C::kLoads loads of step ks into stage st
template <class C>
__device__ __forceinline__ void fetch_step(const SrcT<C> &s, int ks, StageT<C> &st, int wave)
{
#pragma unroll
    for (int i = 0; i < C::kRunsA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            s.a, (lds_ptr)(st.a + 1024 * (wave * C::kRunsA + i)), 16, s.oa[i], ks * kStep, 0, 0);
#pragma unroll
    for (int i = 0; i < C::kRunsB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            s.b, (lds_ptr)(st.b + 1024 * (wave * C::kRunsB + i)), 16, s.ob[i], ks * kStep, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.s, (lds_ptr)(st.s + 256 * wave), 4, s.os, 4 * ks,
                                             0, 0);
}

// Block order.  Workgroup w runs on XCD w % 8 (the dispatcher deals
// consecutive workgroups out to the 8 XCDs in turn; nothing here depends on
// it for correctness).  XCD x takes the x-th eighth of the blocks in a
// grouped order: groups of 4 row blocks, all column blocks of a group before
// the next, so that the workgroups resident on an XCD share A rows and B
// rows at about the same K step in that XCD's L2 (groups of 8 and 16 were
// 2.5% and 5% slower at T = 16384, N = K = 5120).
constexpr int kGroupRows = 4;

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

template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void mxfp8_gemm_tile_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa,
    const uint8_t *__restrict__ b, const uint8_t *__restrict__ sb, int T, int N, int K,
    uint16_t *__restrict__ out)
{
    constexpr int MI = C::WM / 16, NJ = C::WN / 16, S = C::S;
    __shared__ StageT<C> st[S];
    static_assert(S * sizeof(StageT<C>) >= C::TM * C::TN * 2, "the output tile fits the stages");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int mi, ni;
    if (!block_of(blockIdx.x, (T + C::TM - 1) / C::TM, (N + C::TN - 1) / C::TN, mi, ni))
        return;
    const int m_blk = mi * C::TM, n_blk = ni * C::TN;
    const int wm = (wave / (C::TN / C::WN)) * C::WM, wn = (wave % (C::TN / C::WN)) * C::WN;
    const int g = lane >> 4, r = lane & 15;
    const int p0 = 16 * (g ^ (r >> 1)), p1 = p0 ^ 64;   // slots of pieces g and g + 4 of row r
    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int steps = K / kStep;
    const SrcT<C> src = src_tile<C>(a, sa, b, sb, K, m_blk, n_blk, T, N, wave, lane);
    // Steps past the end re-read the last into a free stage: every step has
    // the same loads in flight, so the waits are constants and the loop has
    // no branch.
#pragma unroll
    for (int p = 0; p < S - 1; ++p)
        fetch_step<C>(src, min(p, steps - 1), st[p], wave);
    int cur_s = 0, next_s = S - 1;
    for (int ks = 0; ks < steps; ++ks) {
        wait_vm<(S - 2) * C::kLoads>();   // this wave's loads of step ks are in LDS
        block_barrier();                   // every wave's are, and step ks - 1's stage is free
        fetch_step<C>(src, min(ks + S - 1, steps - 1), st[next_s], wave);
        // the loads go out ahead of the step's LDS reads and MFMAs
        __builtin_amdgcn_sched_barrier(0);
        const StageT<C> &cur = st[cur_s];
        i32x8 fb[NJ];
        int scb[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint8_t *p = cur.b + (wn + 16 * j + r) * kStep;
            fb[j] = join(*reinterpret_cast<const u32x4 *>(p + p0),
                         *reinterpret_cast<const u32x4 *>(p + p1));
            scb[j] = cur.s[(C::kAS + wn + 16 * j + r) * 4 + g];
        }
        // a wave issuing its MFMAs goes ahead of the other wave of its SIMD,
        // whose LDS reads then overlap them
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint8_t *p = cur.a + (wm + 16 * i + r) * kStep;
            const i32x8 fa = join(*reinterpret_cast<const u32x4 *>(p + p0),
                                  *reinterpret_cast<const u32x4 *>(p + p1));
            const int sai = cur.s[(wm + 16 * i + r) * 4 + g];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = mfma_sel(fa, fb[j], acc[i][j], sai, 0, scb[j], 0);
        }
        __builtin_amdgcn_s_setprio(0);
        cur_s = cur_s == S - 1 ? 0 : cur_s + 1;
        next_s = next_s == S - 1 ? 0 : next_s + 1;
    }
    wait_vm<0>();      // the re-reads past the end have landed
    __syncthreads();   // and every wave is done with the stages
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

// 256 x 256 blocks fill 132 KB of LDS with two stages, one workgroup per
// CU, on 8 waves of 64 x 128 (each holding its 8 B fragments of a step and
// streaming 4 A fragments: 2.8% faster at T = 16384, N = K = 5120, than
// 128 x 64, 255 VGPRs); 128 x 256 blocks (8 waves of 64 x 64) 150 KB with three.  128 x 128
// blocks: three stages (99 KB) where one round of workgroups covers the
// blocks, else two (66 KB), so that two workgroups share a CU.
// The narrower blocks, for one round of the CUs, take three stages, those
// of 16 or 32 rows six (with 6 KB or 8 KB per step, three stages left the
// loads short of the CU's rate: 10.6 against 8.9 us at T <= 16, N = K =
// 5120; more stages gained nothing, for these or the larger shapes).
using BigTile = Tile<256, 256, 64, 128, 2>;
using MidTile3 = Tile<128, 128, 64, 64, 3>;
using MidTile2 = Tile<128, 128, 64, 64, 2>;
using WideTile = Tile<128, 256, 64, 64, 3>;
using NarrowTile = Tile<128, 64, 64, 32, 3>;
using SmallTile = Tile<64, 64, 32, 32, 3>;
using TinyTile = Tile<64, 32, 32, 16, 3>;
using Tile32 = Tile<32, 32, 16, 16, 6>;
using MicroTile = Tile<16, 32, 16, 16, 6>;

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

GemmBlocks gemm_blocks(int64_t T, int N, int cus)
{
    // Where one round of workgroups covers the 128 x 128 blocks, the step
    // loop's loads bound the time: each CU streams (TM + TN) x K bytes per
    // block at a rate of its own, whatever the stages or waves (the loads
    // alone take 24-30 us of the 31-34 us of 128 x 128 blocks at T = 64-384,
    // N = K = 5120).  So the launch takes the shape whose CU with the most
    // blocks streams the fewest bytes, the larger on a tie; for T <= 32 also
    // past one round (many weight columns).  Blocks of 16 or 32 rows take six
    // stages, the others three.
    const int64_t mid = ((T + 127) / 128) * (int64_t)((N + 127) / 128);
    if (mid <= cus || T <= 32) {
        static const int shapes[6][2] = {{16, 32}, {32, 32}, {64, 32}, {64, 64},
                                         {128, 64}, {128, 128}};
        int best = 0;
        int64_t best_cost = INT64_MAX;
        for (int i = 0; i < 6; ++i) {
            const int tm = shapes[i][0], tn = shapes[i][1];
            const int64_t blocks = ((T + tm - 1) / tm) * (int64_t)((N + tn - 1) / tn);
            const int64_t cost = (blocks + cus - 1) / cus * (tm + tn);
            if (cost <= best_cost) {
                best = i;
                best_cost = cost;
            }
        }
        return {shapes[best][0], shapes[best][1], shapes[best][0] <= 32 ? 6 : 3};
    }
    // Past one round of 128 x 128 blocks: 128 x 256 blocks where they fit
    // one round (N = K = 5120, T = 1024-1536: 53-55 us against 56-58 for
    // 128 x 128 blocks two per CU); past that the large blocks where their
    // rounds cost less than the mid blocks' at two per CU (one round of
    // large blocks takes about 1.5 times as long; N = K = 5120: mid blocks
    // at 4096, large ones at 2048, 3072 and from 6144 on)
    const int64_t wide = ((T + 127) / 128) * (int64_t)((N + 255) / 256);
    if (wide <= cus)
        return {128, 256, 3};
    const int64_t rounds_big = (((T + 255) / 256) * (int64_t)((N + 255) / 256) + cus - 1) / cus;
    const int64_t rounds_mid = (mid + 2 * cus - 1) / (2 * cus);
    if (GEMM_MID_COST * rounds_mid < GEMM_BIG_COST * rounds_big)
        return {128, 128, 2};
    return {256, 256, 2};
}

hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                             const uint8_t *sb, int T, int N, int K, uint16_t *out, int cus,
                             hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    const GemmBlocks g = gemm_blocks(T, N, cus);
#define SHAPE(C)                                                                            \
    if (g.tm == C::TM && g.tn == C::TN && g.stages == C::S)                                 \
        return launch_tile<C>(a, sa, b, sb, T, N, K, out, s);
    SHAPE(MicroTile)
    SHAPE(Tile32)
    SHAPE(TinyTile)
    SHAPE(SmallTile)
    SHAPE(NarrowTile)
    SHAPE(MidTile3)
    SHAPE(MidTile2)
    SHAPE(WideTile)
    SHAPE(BigTile)
#undef SHAPE
    return hipErrorInvalidValue;
}

}  // namespace mhc
