// seam_internal.h -- shared between the HIP kernels and the host runtime of
// libmhc_seam.so (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mhc {

constexpr int kBlockTokens = 16;   // tokens per block: the MFMA M dimension
constexpr int kWaves = 8;          // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;         // columns per quantiser group / MFMA K step
constexpr int kSeg = 64;           // columns per segment (one 128-byte line per row)
constexpr int kPartFloats = 32;    // per (block, split, token) partial record
constexpr int kMaxSplits = 128;    // splits per block (<= H/64 for H <= 8192)

// kCollapse: x collapsed with pre, its sums of squares and the norm only
// (no post-mix, no gate projection): the second launch of the unshifted
// ordering, whose gates the first launch computed
enum Form { kPost = 0, kNoPost = 1, kCollapse = 2 };
enum Out { kBf16 = 0, kFp8Grid = 1, kMxfp8 = 2, kMxfp8G128 = 3 };

struct SeamParams {
    int T, H, nchunks, nseg;
    int nblocks, ksplit, segs_per_split;
    int rows_blocks;          // blocks [0, rows_blocks) whole-row, the rest split
    float eps;
    int iters;
    int identity_pre;
    int skip_norm;            // post-mix and gates only (no collapse output)
    int skip_gates;           // collapse, norm and quantiser only (no gates)
    const uint16_t *x;
    const uint16_t *y;
    const float *pre;
    const float *post;
    const float *res;
    const void *fnp;          // packed fn: [nchunks][4][3][64] x 16 bytes
    const uint16_t *gamma;
    const float *bias;
    uint16_t *resid;
    uint16_t *norm;
    uint16_t *grid;
    uint8_t *codes;
    uint8_t *scales;
    float *pre_out;
    float *post_out;
    float *res_out;
    // split-mode scratch; partials and u cover the split blocks only (blocks
    // rows_blocks .. nblocks-1, tokens 16*rows_blocks .. T-1)
    float *part;              // [nblocks - rows_blocks][ksplit][16][kPartFloats]
    uint16_t *uscr;           // [T - 16*rows_blocks][H] bf16 u of handed-off splits
    int *sync;                // [nblocks - rows_blocks][sync_stride]: arrival counter, two
                              // hand-off mask sets
    int sync_stride;          // ints per block (one 128-byte line)
    int spin_limit;           // polls a waiting split makes before handing off
};

// bytes of the packed fn for width H
inline size_t fn_pack_bytes(int H) { return (size_t)(H / kChunk) * 4 * 3 * 64 * 16; }

// whole-row kernels are compiled for nseg == 8 * rs with these rs
bool row_segs_instance(int rs);

hipError_t launch_fn_pack(const float *fn, int H, void *pack, hipStream_t s);
hipError_t launch_seam(const SeamParams &p, int form, int out, int row_segs,
                       int grid, hipStream_t s);
hipError_t launch_copy(void *dst, const void *src, size_t bytes, int cus, hipStream_t s);
hipError_t launch_stream_mix(void *dst, size_t dst_bytes, const void *src, size_t src_bytes,
                             int cus, hipStream_t s);
// The MXFP8 GEMM's output blocks for T x N on cus CUs: TM x TN and the
// number of LDS stages (host only; the launch takes exactly this shape)
struct GemmBlocks {
    int tm, tn, stages;
};
GemmBlocks gemm_blocks(int64_t T, int N, int cus);
hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                             const uint8_t *sb, int T, int N, int K, uint16_t *out, int cus,
                             hipStream_t s);
hipError_t launch_head_reduce(const uint16_t *x, const float *w, int64_t T, int H, uint16_t *out,
                              int cus, hipStream_t s);
hipError_t launch_quantize(const uint16_t *src, int rows, int H, int group, uint8_t *codes,
                           uint8_t *scales, uint16_t *grid, hipStream_t s);

}  // namespace mhc
