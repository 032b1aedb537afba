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
// Tiling: a workgroup of 4 waves computes a 128 x 128 block of out, each
// wave 64 x 64 (4 x 4 MFMA tiles, 16 fp32 accumulators), with the next K
// step's operands in flight while the current one is multiplied.
#include <hip/hip_runtime.h>

#include "seam_internal.h"

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;   // workgroup block (rows and columns)
constexpr int kWave = 64;    // wave block
constexpr int kStep = 128;   // K per MFMA

struct Frags {
    i32x8 a[4], b[4];
    int sa[4], sb[4];
};

__device__ __forceinline__ i32x8 join(const u32x4 &lo, const u32x4 &hi)
{
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// operand pieces of K step ks: rows ra[i] of a, rows rb[i] of b
__device__ __forceinline__ void load_frags(const uint8_t *__restrict__ a,
                                           const uint8_t *__restrict__ sa,
                                           const uint8_t *__restrict__ b,
                                           const uint8_t *__restrict__ sb, int K, int ks,
                                           const int (&ra)[4], const int (&rb)[4], int g,
                                           Frags &f)
{
    const int k0 = ks * kStep + 16 * g, kb = ks * (kStep / 32) + g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint8_t *pa = a + (size_t)ra[i] * K + k0;
        f.a[i] = join(*reinterpret_cast<const u32x4 *>(pa),
                      *reinterpret_cast<const u32x4 *>(pa + 64));
        const uint8_t *pb = b + (size_t)rb[i] * K + k0;
        f.b[i] = join(*reinterpret_cast<const u32x4 *>(pb),
                      *reinterpret_cast<const u32x4 *>(pb + 64));
        f.sa[i] = sa[(size_t)ra[i] * (K / 32) + kb];
        f.sb[i] = sb[(size_t)rb[i] * (K / 32) + kb];
    }
}

__device__ __forceinline__ void mma(const Frags &f, f32x4 (&acc)[4][4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            // formats 0, 0: fp8 e4m3 for A and B; scale byte 0 of each
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                f.a[i], f.b[j], acc[i][j], 0, 0, 0, f.sa[i], 0, f.sb[j]);
}

__global__ __launch_bounds__(256) void mxfp8_gemm_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa,
    const uint8_t *__restrict__ b, const uint8_t *__restrict__ sb, int T, int N, int K,
    uint16_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m0 = blockIdx.y * kTile + (wave >> 1) * kWave;
    const int n0 = blockIdx.x * kTile + (wave & 1) * kWave;
    const int g = lane >> 4, r = lane & 15;
    // rows past T / columns past N re-read the last one; their results are
    // not stored
    int ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = min(m0 + 16 * i + r, T - 1);
        rb[i] = min(n0 + 16 * i + r, N - 1);
    }
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int steps = K / kStep;
    Frags cur, nxt;
    load_frags(a, sa, b, sb, K, 0, ra, rb, g, cur);
    for (int ks = 0; ks < steps; ++ks) {
        if (ks + 1 < steps)
            load_frags(a, sa, b, sb, K, ks + 1, ra, rb, g, nxt);
        mma(cur, acc);
        cur = nxt;
    }
    // lane l holds rows 4 (l / 16) + e, column l % 16 of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + 16 * j + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + 16 * i + 4 * g + e;
                if (row < T && col < N) {
                    const __bf16 v = (__bf16)acc[i][j][e];
                    out[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, v);
                }
            }
        }
}

}  // namespace

hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                             const uint8_t *sb, int T, int N, int K, uint16_t *out, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    dim3 grid((N + kTile - 1) / kTile, (T + kTile - 1) / kTile);
    hipLaunchKernelGGL(mxfp8_gemm_kernel, grid, dim3(256), 0, s, a, sa, b, sb, T, N, K, out);
    return hipGetLastError();
}

}  // namespace mhc
