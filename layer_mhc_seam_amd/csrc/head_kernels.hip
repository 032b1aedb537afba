// head_kernels.hip -- n -> 1 reduction of the residual streams, stored.
//
// "[Triton/Gluon] [gfx950] [dsv4.1-flash] mHC fused kernel", description,
// names an HC head reduce/store kernel among the unfused per-seam kernels
// and says nothing more about it.  The reading taken here: the seam's
// collapse step on its own over the stored streams,
//   out[t][h] = bf16( w0 x0 + w1 x1 + w2 x2 + w3 x3 )      (x_i = x[t][i][h])
// evaluated as the collapse chain: a rounded product, then three fused
// multiply-adds in stream order, one bf16 round-to-nearest-even at the end.
// w is f32 [T][4] per token (the pre gate); without it every weight is 1/4.
//
// It is a pure stream: 8H bytes of x and 16 bytes of w read, 2H bytes
// written per token, no reuse.  Each wave owns one token row at a time and
// each of its load instructions covers 1 KB of one stream row (64 lanes x
// 16 B), the access shape that reaches the device's best copy rate; loads
// and stores are non-temporal.  Workgroups walk the tokens grid-stride.
#include <hip/hip_runtime.h>

#include "seam_internal.h"

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadWaves = 4;

__device__ __forceinline__ u32 pack_pair(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
    return __builtin_bit_cast(u32, v);
}

// one 16-byte chunk (8 columns) of the four streams -> 8 outputs
__device__ __forceinline__ u32x4 reduce8(const u32x4 (&s)[4], const float (&w)[4])
{
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float lo = w[0] * __uint_as_float(s[0][q] << 16);
        float hi = w[0] * __uint_as_float(s[0][q] & 0xffff0000u);
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            lo = fmaf(w[i], __uint_as_float(s[i][q] << 16), lo);
            hi = fmaf(w[i], __uint_as_float(s[i][q] & 0xffff0000u), hi);
        }
        r[q] = pack_pair(lo, hi);
    }
    return r;
}

// U chunks per lane in flight (4U loads of 16 B)
template <int U>
__global__ __launch_bounds__(kHeadWaves * 64) void head_reduce_kernel(
    const u32x4 *__restrict__ x, const float *__restrict__ w, int64_t T, int H8,
    u32x4 *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t stride = (int64_t)gridDim.x * kHeadWaves;
    for (int64_t t = (int64_t)blockIdx.x * kHeadWaves + wave; t < T; t += stride) {
        float wt[4] = {0.25f, 0.25f, 0.25f, 0.25f};
        if (w) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wt[i] = w[t * 4 + i];
        }
        const u32x4 *xr = x + t * 4 * H8;
        u32x4 *orow = out + t * H8;
        for (int c0 = lane; c0 < H8; c0 += 64 * U) {
            u32x4 s[U][4];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int c = c0 + 64 * k;
                if (c < H8)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s[k][i] = __builtin_nontemporal_load(xr + (int64_t)i * H8 + c);
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int c = c0 + 64 * k;
                if (c < H8)
                    __builtin_nontemporal_store(reduce8(s[k], wt), orow + c);
            }
        }
    }
}

}  // namespace

hipError_t launch_head_reduce(const uint16_t *x, const float *w, int64_t T, int H, uint16_t *out,
                              int cus, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    // One workgroup per four tokens (grid-stride only past 64 workgroups per
    // CU) and ten chunks per lane in flight: at H = 5120 a lane then issues
    // its whole share of the four stream rows at once (40 loads, 173 VGPRs).
    // Measured at T = 16384, H = 5120: 137.8 us = 6.09 TB/s, the device's copy
    // rate; two or four chunks per lane, or fewer workgroups, ran 1-7% slower.
    constexpr int kWgsPerCu = 64, kChunks = 10;
    const int64_t want = (T + kHeadWaves - 1) / kHeadWaves;
    const int grid = (int)(want < (int64_t)cus * kWgsPerCu ? want : (int64_t)cus * kWgsPerCu);
    hipLaunchKernelGGL(head_reduce_kernel<kChunks>, dim3(grid), dim3(kHeadWaves * 64), 0, s,
                       reinterpret_cast<const u32x4 *>(x), w, T, H / 8,
                       reinterpret_cast<u32x4 *>(out));
    return hipGetLastError();
}

}  // namespace mhc
