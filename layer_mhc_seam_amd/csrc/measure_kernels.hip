// measure_kernels.hip -- streaming kernels that set the bandwidth ceilings
// the seam is measured against; not part of the seam.
//
// "[FlyDSL] Single-launch Mega-mHC on gfx950", Realistic Bandwidth Ceiling,
// compares the seam with a plain device copy of its bytes.  copy_kernel is
// that copy.  stream_mix_kernel generalises it to a kernel that reads R and
// writes W bytes, each byte once, so that a seam whose reads and writes are
// not balanced (the no_post form reads four bytes for each one it writes)
// has a ceiling with its own mix.

#include "seam_internal.h"

namespace mhc {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

// Copy: 16-byte non-temporal loads and stores, four loads in flight per
// thread, grid-stride.  Launched with one 256-thread workgroup per CU, the
// fastest of the shapes measured (grids of 256..16384 workgroups x 1..8
// loads in flight, and hipMemcpy).
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src,
                                                   u32x4 *__restrict__ dst, size_t n)
{
    constexpr int U = 4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u)
            __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Read n_in and write n_out 16-byte chunks, each once, over the whole grid
// whatever the ratio: thread g XORs input chunks g, g + S, g + 2S, ... (S
// threads in the grid; four loads in flight) into a value that starts as
// (g, ~g, 0, 0), then stores that value XOR (j, 0, 0, 0) to output chunks
// j = g, g + S, ....  Every store depends on all of the thread's loads, so
// none is dropped.
__global__ __launch_bounds__(256) void stream_mix_kernel(const u32x4 *__restrict__ src,
                                                         size_t n_in, u32x4 *__restrict__ dst,
                                                         size_t n_out)
{
    const size_t S = (size_t)gridDim.x * blockDim.x;
    const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {(u32)g, ~(u32)g, 0u, 0u};
    size_t i = g;
    for (; i + 3 * S < n_in; i += 4 * S) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * S);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    for (; i < n_in; i += S)
        acc ^= __builtin_nontemporal_load(src + i);
    for (size_t j = g; j < n_out; j += S)
        __builtin_nontemporal_store(acc ^ u32x4{(u32)j, 0u, 0u, 0u}, dst + j);
}

}  // namespace

hipError_t launch_copy(void *dst, const void *src, size_t bytes, int cus, hipStream_t s)
{
    size_t n = bytes / 16;
    if (n == 0)
        return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > (size_t)cus)
        blocks = (size_t)cus;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(src), reinterpret_cast<u32x4 *>(dst), n);
    return hipGetLastError();
}

hipError_t launch_stream_mix(void *dst, size_t dst_bytes, const void *src, size_t src_bytes,
                             int cus, hipStream_t s)
{
    const size_t n_out = dst_bytes / 16, n_in = src_bytes / 16;
    const size_t n = n_out > n_in ? n_out : n_in;
    if (n == 0)
        return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > (size_t)cus)
        blocks = (size_t)cus;
    hipLaunchKernelGGL(stream_mix_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(src), n_in, reinterpret_cast<u32x4 *>(dst),
                       n_out);
    return hipGetLastError();
}

}  // namespace mhc
