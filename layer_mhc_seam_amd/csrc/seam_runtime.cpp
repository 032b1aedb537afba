// seam_runtime.cpp -- host runtime and C ABI of libmhc_seam.so.
//
// Sources (web pages, cited by title and section):
//   [MEGA]  "[FlyDSL] Single-launch Mega-mHC on gfx950" (ROCm/aiter PR 6179)
//   [FUSED] "[Triton/Gluon] [gfx950] [dsv4.1-flash] mHC fused kernel"
//
// Argument rules follow the review findings on [FUSED] ("Copilot review
// overview": pre_mix optional, dense fp32 gate operands, contiguous
// residual_out, incomplete post-mix inputs must not be ignored) and [MEGA,
// Limitations] (gfx950 only, T*4*H*2 < 2^31).  Per-stream scratch and the fn
// pack are filled by eager calls only; a capture that would need a new
// allocation fails [MEGA, Kernel Architecture: CUDA graphs].

#include <algorithm>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/mhc_seam.h"
#include "seam_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    if (e == hipErrorOutOfMemory)
        return fail(MHC_SEAM_OUT_OF_MEMORY, "%s: %s", what, hipGetErrorString(e));
    return fail(MHC_SEAM_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

struct Scratch {
    void *base = nullptr;
    size_t bytes = 0;
};

struct Range {
    uintptr_t lo, hi;
    const char *name;
};

// Streams a handle has enqueued seams on, kept without allocating: up to
// kCap distinct streams are remembered; past that the set only notes that
// it overflowed, and destroy waits for the whole device instead.
struct StreamSet {
    static constexpr int kCap = 64;
    hipStream_t s[kCap];
    int n = 0;
    bool overflow = false;
    void add(hipStream_t st)
    {
        for (int i = 0; i < n; ++i)
            if (s[i] == st)
                return;
        if (n < kCap)
            s[n++] = st;
        else
            overflow = true;
    }
};

}  // namespace

struct mhc_seam {
    int H = 0;
    float eps = 1e-6f;
    int iters = 20;
    int64_t max_tokens = 0;
    int device = 0;
    int cu_count = 0;
    int ksplit_override = 0;
    int spin_polls = 0;
    void *fnp = nullptr;
    uint16_t *gamma = nullptr;
    float *bias = nullptr;
    size_t scratch_max = 0;   // split-mode scratch per stream, for any T <= max_tokens
    std::mutex mu;
    std::unordered_map<hipStream_t, Scratch> scratch;
    StreamSet streams;        // every stream a seam was enqueued on
};

namespace {

constexpr int64_t kOffsetLimit = int64_t(1) << 31;

int check_desc(const mhc_seam_desc *d)
{
    if (!d)
        return fail(MHC_SEAM_INVALID_ARG, "desc is NULL");
    if (d->n != 4)
        return fail(MHC_SEAM_INVALID_ARG, "n must be 4 (got %d)", d->n);
    if (d->H <= 0 || d->H % mhc::kSeg != 0)
        return fail(MHC_SEAM_INVALID_ARG, "H must be a positive multiple of 64 (got %d)", d->H);
    if (!(d->eps >= 0.0f) || d->eps > 1.0f)
        return fail(MHC_SEAM_INVALID_ARG, "eps must be in [0, 1] (0 selects 1e-6)");
    if (d->sinkhorn_iters < 0 || d->sinkhorn_iters > 1000)
        return fail(MHC_SEAM_INVALID_ARG, "sinkhorn_iters must be in [0, 1000]");
    if (!d->fn || !d->gamma || !d->bias)
        return fail(MHC_SEAM_INVALID_ARG, "fn, gamma and bias are required");
    if (d->max_tokens < 0)
        return fail(MHC_SEAM_INVALID_ARG, "max_tokens must be >= 0");
    if (d->max_tokens * 4 * (int64_t)d->H * 2 >= kOffsetLimit)
        return fail(MHC_SEAM_INVALID_ARG, "max_tokens*4*H*2 must be < 2^31");
    if (d->ksplit < 0 || d->ksplit > d->H / mhc::kSeg || d->ksplit > mhc::kMaxSplits)
        return fail(MHC_SEAM_INVALID_ARG, "ksplit must be in [0, min(H/64, %d)]", mhc::kMaxSplits);
    if (d->spin_polls < -1)
        return fail(MHC_SEAM_INVALID_ARG, "spin_polls must be >= -1");
    for (int v : d->reserved)
        if (v)
            return fail(MHC_SEAM_INVALID_ARG, "reserved desc fields must be zero");
    return MHC_SEAM_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_args(int H, int64_t max_tokens, const mhc_seam_args *a)
{
    if (!a)
        return fail(MHC_SEAM_INVALID_ARG, "args is NULL");
    if (a->T < 0)
        return fail(MHC_SEAM_INVALID_ARG, "T must be >= 0");
    if (a->T > max_tokens)
        return fail(MHC_SEAM_INVALID_ARG, "T=%lld exceeds max_tokens=%lld", (long long)a->T,
                    (long long)max_tokens);
    if (a->T * 4 * (int64_t)H * 2 >= kOffsetLimit)
        return fail(MHC_SEAM_INVALID_ARG, "T*4*H*2 must be < 2^31");
    if (a->form != MHC_SEAM_POST && a->form != MHC_SEAM_NO_POST)
        return fail(MHC_SEAM_INVALID_ARG, "unknown form %d", a->form);
    if (a->identity_pre != 0 && a->identity_pre != 1)
        return fail(MHC_SEAM_INVALID_ARG, "identity_pre must be 0 or 1");
    if (a->out_dtype < MHC_SEAM_OUT_BF16 || a->out_dtype > MHC_SEAM_OUT_MXFP8_G128)
        return fail(MHC_SEAM_INVALID_ARG, "unknown out_dtype %d", a->out_dtype);
    if (a->out_dtype == MHC_SEAM_OUT_MXFP8_G128 && H % 128)
        return fail(MHC_SEAM_INVALID_ARG, "128-wide groups need H a multiple of 128");
    if (a->unshifted != 0 && a->unshifted != 1)
        return fail(MHC_SEAM_INVALID_ARG, "unshifted must be 0 or 1");
    if (a->unshifted && a->identity_pre)
        return fail(MHC_SEAM_INVALID_ARG, "unshifted takes the fresh pre: identity_pre must be 0");

    const bool post = a->form == MHC_SEAM_POST;
    const bool idp = a->identity_pre == 1 || a->unshifted == 1;
    const int64_t T = a->T, th = T * H;
    const bool mx = a->out_dtype == MHC_SEAM_OUT_MXFP8 || a->out_dtype == MHC_SEAM_OUT_MXFP8_G128;
    struct Slot {
        const void *p;
        bool needed;
        int64_t bytes;
        bool output;
        const char *name;
    } slots[] = {
        {a->x, true, th * 4 * 2, false, "x"},
        {a->y, post, th * 2, false, "y"},
        {a->pre, !idp, T * 16, false, "pre"},
        {a->post, post, T * 16, false, "post"},
        {a->res, post, T * 64, false, "res"},
        {a->residual_out, post, th * 4 * 2, true, "residual_out"},
        {a->norm, true, th * 2, true, "norm"},
        {a->grid, a->out_dtype == MHC_SEAM_OUT_FP8_GRID, th * 2, true, "grid"},
        {a->codes, mx, th, true, "codes"},
        {a->scales, mx, T * (H / (a->out_dtype == MHC_SEAM_OUT_MXFP8_G128 ? 128 : 32)), true,
         "scales"},
        {a->pre_out, true, T * 16, true, "pre_out"},
        {a->post_out, true, T * 16, true, "post_out"},
        {a->res_out, true, T * 64, true, "res_out"},
    };
    std::vector<Range> ranges;
    for (const Slot &s : slots) {
        if (s.needed && !s.p && T > 0)   // T == 0 touches nothing: empty tensors may be NULL
            return fail(MHC_SEAM_INVALID_ARG, "%s is required by this form/out_dtype", s.name);
        if (!s.needed && s.p)
            return fail(MHC_SEAM_INVALID_ARG,
                        "%s must be NULL for this form/out_dtype (it would be ignored)", s.name);
        if (s.p && !aligned16(s.p))
            return fail(MHC_SEAM_INVALID_ARG, "%s must be 16-byte aligned", s.name);
        if (s.p && s.bytes > 0) {
            uintptr_t lo = reinterpret_cast<uintptr_t>(s.p);
            ranges.push_back({lo, lo + (uintptr_t)s.bytes, s.name});
        }
    }
    // no output may overlap an input or another output
    for (size_t i = 0; i < ranges.size(); ++i)
        for (size_t j = i + 1; j < ranges.size(); ++j) {
            bool out_i = false, out_j = false;
            for (const Slot &s : slots) {
                if (s.name == ranges[i].name)
                    out_i = s.output;
                if (s.name == ranges[j].name)
                    out_j = s.output;
            }
            if (!out_i && !out_j)
                continue;
            if (ranges[i].lo < ranges[j].hi && ranges[j].lo < ranges[i].hi)
                return fail(MHC_SEAM_INVALID_ARG, "%s overlaps %s", ranges[i].name,
                            ranges[j].name);
        }
    return MHC_SEAM_OK;
}

// Launch policy.  Whole-row mode (one workgroup per 16-token block, u kept
// on chip) when the blocks alone fill most of the chip and H/512 is one of
// the compiled segment counts; otherwise split mode, each block's 64-column
// segments spread so that blocks * ksplit is about one workgroup per CU.
// Split mode with ksplit = 1 serves widths the whole-row kernels are not
// compiled for.
constexpr int kDefaultMaxSplits = 20;

void make_plan(int H, int64_t T, int cu, int ksplit_override, mhc_seam_plan *pl)
{
    std::memset(pl, 0, sizeof *pl);
    const int nseg = H / mhc::kSeg;
    const int nb = (int)((T + mhc::kBlockTokens - 1) / mhc::kBlockTokens);
    const bool rows_ok = nseg % mhc::kWaves == 0 && mhc::row_segs_instance(nseg / mhc::kWaves);
    pl->blocks = nb;
    if (rows_ok && (ksplit_override == 1 || (ksplit_override == 0 && nb * 2 > cu))) {
        // whole rows; a tail of r <= cu/2 blocks after full rounds of the
        // CUs is split so that it does not cost a whole extra round
        pl->row_segs = nseg / mhc::kWaves;
        const int r = nb % cu;
        // The tail's r blocks split into as many workgroups as fit on the CUs
        // together (splits that are not all resident hand off, measured far
        // slower: T = 6144 took 217 us with 1280 tail splits), at least two
        // per block.  Splits of at most 8 segments run in the whole-row
        // launch; larger ones in a split launch after it.
        int ks = r > 0 ? std::min({cu / r, nseg, mhc::kMaxSplits}) : 1;
        const int sps = (nseg + std::max(ks, 1) - 1) / std::max(ks, 1);
        ks = (nseg + sps - 1) / sps;
        if (ksplit_override == 0 && nb >= cu && r > 0 && ks >= 2 && r * ks <= cu) {
            pl->rows_blocks = nb - r;
            pl->ksplit = ks;
            pl->segs_per_split = sps;
            pl->grid = pl->rows_blocks + r * ks;
        } else {
            pl->rows_blocks = nb;
            pl->ksplit = 1;
            pl->segs_per_split = nseg;
            pl->grid = nb;
        }
        return;
    }
    int ks;
    // up to 20 splits per block while every split workgroup is resident
    // (measured fastest at H = 5120 for T = 4 ... 2048)
    if (ksplit_override > 0)
        ks = ksplit_override;
    else
        ks = std::min({std::max(1, cu / std::max(nb, 1)), kDefaultMaxSplits, std::max(1, nseg / 2)});
    ks = std::min(std::min(ks, nseg), mhc::kMaxSplits);
    const int sps = (nseg + ks - 1) / ks;
    ks = (nseg + sps - 1) / sps;  // no empty splits
    pl->ksplit = ks;
    pl->segs_per_split = sps;
    pl->grid = nb * ks;
    pl->row_segs = 0;
    pl->rows_blocks = 0;
}

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Split-mode scratch: [per-block sync words for every block max_tokens can
// have] [partials of the plan's split blocks] [u of the split blocks' tokens,
// for splits that hand off].  The sync words sit first at a fixed offset so
// that they stay valid between runs of any T: zero when allocated, and every
// launch leaves each block's arrival counter at a multiple of its epoch step
// and the hand-off mask set of the block's next launch clear.  Partials and u
// cover only the blocks that run split (all of them in split mode, the tail
// in a mixed launch).
int sync_stride(int) { return 32; }

size_t sync_bytes(int H, int64_t max_tokens)
{
    return round256((size_t)((max_tokens + mhc::kBlockTokens - 1) / mhc::kBlockTokens) *
                    sync_stride(H) * 4);
}

int64_t split_blocks(const mhc_seam_plan &pl) { return pl.blocks - pl.rows_blocks; }

size_t part_bytes(const mhc_seam_plan &pl)
{
    return round256((size_t)split_blocks(pl) * pl.ksplit * mhc::kBlockTokens * mhc::kPartFloats *
                    4);
}

size_t scratch_bytes(int H, int64_t T, int64_t max_tokens, const mhc_seam_plan &pl)
{
    if (split_blocks(pl) == 0 || T == 0)
        return 0;
    const int64_t split_tokens = T - (int64_t)pl.rows_blocks * mhc::kBlockTokens;
    return sync_bytes(H, max_tokens) + part_bytes(pl) + round256((size_t)split_tokens * H * 2);
}

// Largest scratch any T <= max_tokens needs under the handle's policy.
size_t max_scratch_bytes(const mhc_seam &h)
{
    size_t best = 0;
    int64_t nbmax = (h.max_tokens + mhc::kBlockTokens - 1) / mhc::kBlockTokens;
    for (int64_t nb = 1; nb <= nbmax; ++nb) {
        int64_t T = std::min(h.max_tokens, nb * mhc::kBlockTokens);
        mhc_seam_plan pl;
        make_plan(h.H, T, h.cu_count, h.ksplit_override, &pl);
        best = std::max(best, scratch_bytes(h.H, T, h.max_tokens, pl));
    }
    return best;
}

// The stream's scratch, allocated (h.scratch_max bytes, enough for every T
// the handle accepts) and zeroed on the stream's first use, and never moved
// afterwards: a graph captured on the stream keeps pointing at it.
int ensure_scratch(mhc_seam &h, hipStream_t stream, Scratch **out)
{
    std::lock_guard<std::mutex> lock(h.mu);
    auto it = h.scratch.find(stream);
    if (it != h.scratch.end()) {
        *out = &it->second;
        return MHC_SEAM_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess)
        return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return fail(MHC_SEAM_CAPTURE_ALLOC,
                    "stream has no scratch yet and is being captured; run the seam once "
                    "eagerly on this stream first");
    Scratch s;
    if ((e = hipMalloc(&s.base, h.scratch_max)) != hipSuccess)
        return hip_fail(e, "hipMalloc(scratch)");
    // zero the whole area once: the block counters must start at a multiple
    // of the epoch step with both mask sets clear; every launch leaves them so
    if ((e = hipMemsetAsync(s.base, 0, h.scratch_max, stream)) != hipSuccess) {
        (void)hipFree(s.base);
        return hip_fail(e, "hipMemsetAsync(scratch)");
    }
    s.bytes = h.scratch_max;
    *out = &(h.scratch[stream] = s);
    return MHC_SEAM_OK;
}

// ------------------------------------------------ no-allocation scratch ----
//
// mhc_seam_run_noalloc takes its split-mode scratch from this fixed array
// instead of allocating: one copy per GPU, alive until the process ends,
// shared by every handle and stream on that GPU (runs that overlap on one
// GPU race on it).  Layout: [sync words of up to kNoAllocSyncBlocks split
// blocks][partials][u], the sync words at a fixed offset so that they keep
// their state from run to run.  In host code `scratch` only names the
// symbol: the device address comes from hipGetSymbolAddress, once per
// device at set-up (mhc_seam_create), and only that address is used.
constexpr size_t kNoAllocBytes = size_t(32) << 20;
constexpr int kNoAllocSyncBlocks = 2048;
constexpr size_t kNoAllocSyncBytes = (size_t)kNoAllocSyncBlocks * 32 * 4;
constexpr int kNoAllocMaxDevices = 64;
static_assert(MHC_SEAM_NOALLOC_SCRATCH_BYTES == kNoAllocBytes, "header and library agree");

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

std::mutex g_noalloc_mu;
void *g_noalloc_ptr[kNoAllocMaxDevices];   // device address of `scratch`, per device

// Once per device, with that device current: find the array's device
// address and clear it (block counters at zero, both mask sets clear).
int noalloc_setup(int device)
{
    if (device < 0 || device >= kNoAllocMaxDevices)
        return MHC_SEAM_OK;   // the no-allocation entry point then refuses this device
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (g_noalloc_ptr[device])
        return MHC_SEAM_OK;
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return hip_fail(e, "hipGetSymbolAddress(no-allocation scratch)");
    if ((e = hipMemset(ptr, 0, kNoAllocBytes)) != hipSuccess)
        return hip_fail(e, "hipMemset(no-allocation scratch)");
    g_noalloc_ptr[device] = ptr;
    return MHC_SEAM_OK;
}

void *noalloc_ptr(int device)
{
    if (device < 0 || device >= kNoAllocMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    return g_noalloc_ptr[device];
}

// Residency guard: a split may only wait for its finisher when all split
// workgroups can be resident at once (one workgroup per CU); in a mixed
// launch they are the tail, dispatched after the whole blocks.
int spin_limit(const mhc_seam &h, const mhc_seam_plan &pl)
{
    if (h.spin_polls < 0 || pl.grid - pl.rows_blocks > h.cu_count)
        return -1;
    return h.spin_polls > 0 ? h.spin_polls : 4000;
}

// Points p's split-mode scratch into [base, ...) laid out as sync words
// (sync_len bytes), partials, u.
void set_scratch(mhc::SeamParams &p, char *base, size_t sync_len, const mhc_seam_plan &pl, int H)
{
    p.sync = reinterpret_cast<int *>(base);
    p.sync_stride = sync_stride(H);
    base += sync_len;
    p.part = reinterpret_cast<float *>(base);
    base += part_bytes(pl);
    p.uscr = reinterpret_cast<uint16_t *>(base);
}

int run_seam(mhc_seam *h, const mhc_seam_args *a, void *stream_ptr, bool noalloc);

}  // namespace

extern "C" {

const char *mhc_seam_status_string(int status)
{
    switch (status) {
    case MHC_SEAM_OK: return "ok";
    case MHC_SEAM_INVALID_ARG: return "invalid argument";
    case MHC_SEAM_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case MHC_SEAM_OUT_OF_MEMORY: return "out of device memory";
    case MHC_SEAM_HIP_ERROR: return "HIP runtime error";
    case MHC_SEAM_CAPTURE_ALLOC: return "scratch allocation needed during stream capture";
    default: return "unknown status";
    }
}

const char *mhc_seam_last_error(void) { return g_last_error.c_str(); }

int mhc_seam_validate(const mhc_seam_desc *desc, const mhc_seam_args *args)
{
    int st = check_desc(desc);
    if (st != MHC_SEAM_OK)
        return st;
    if (!args)
        return MHC_SEAM_OK;
    return check_args(desc->H, desc->max_tokens, args);
}

int mhc_seam_plan_for(int32_t H, int64_t T, int32_t cu_count, int32_t ksplit_override,
                      mhc_seam_plan *out)
{
    if (!out || H <= 0 || H % mhc::kSeg || T < 0 || cu_count <= 0 || ksplit_override < 0 ||
        ksplit_override > H / mhc::kSeg)
        return fail(MHC_SEAM_INVALID_ARG, "bad plan query");
    make_plan(H, T, cu_count, ksplit_override, out);
    return MHC_SEAM_OK;
}

int mhc_seam_create(const mhc_seam_desc *desc, mhc_seam_t *out)
{
    if (!out)
        return fail(MHC_SEAM_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int st = check_desc(desc);
    if (st != MHC_SEAM_OK)
        return st;
    hipError_t e;
    int ndev = 0;
    if ((e = hipGetDeviceCount(&ndev)) != hipSuccess)
        return hip_fail(e, "hipGetDeviceCount");
    if (desc->device < 0 || desc->device >= ndev)
        return fail(MHC_SEAM_INVALID_ARG, "device %d out of range (%d devices)", desc->device, ndev);
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, desc->device)) != hipSuccess)
        return hip_fail(e, "hipGetDeviceProperties");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MHC_SEAM_UNSUPPORTED_DEVICE, "device %d is %s; this library is built for gfx950",
                    desc->device, prop.gcnArchName);
    int prev = 0;
    (void)hipGetDevice(&prev);
    if ((e = hipSetDevice(desc->device)) != hipSuccess)
        return hip_fail(e, "hipSetDevice");

    mhc_seam *h = new (std::nothrow) mhc_seam;
    if (!h)
        return fail(MHC_SEAM_OUT_OF_MEMORY, "host allocation failed");
    h->H = desc->H;
    h->eps = desc->eps > 0.0f ? desc->eps : 1e-6f;
    h->iters = desc->sinkhorn_iters > 0 ? desc->sinkhorn_iters : 20;
    h->max_tokens = desc->max_tokens;
    h->device = desc->device;
    h->cu_count = prop.multiProcessorCount;
    h->ksplit_override = desc->ksplit;
    h->spin_polls = desc->spin_polls;

    auto cleanup = [&](int status) {
        mhc_seam_destroy(h);
        (void)hipSetDevice(prev);
        return status;
    };
    size_t pack_bytes = mhc::fn_pack_bytes(h->H);
    if ((e = hipMalloc(&h->fnp, pack_bytes)) != hipSuccess)
        return cleanup(hip_fail(e, "hipMalloc(fn pack)"));
    if ((e = hipMalloc(reinterpret_cast<void **>(&h->gamma), (size_t)h->H * 2)) != hipSuccess)
        return cleanup(hip_fail(e, "hipMalloc(gamma)"));
    if ((e = hipMalloc(reinterpret_cast<void **>(&h->bias), 24 * sizeof(float))) != hipSuccess)
        return cleanup(hip_fail(e, "hipMalloc(bias)"));
    if ((e = hipMemcpy(h->gamma, desc->gamma, (size_t)h->H * 2, hipMemcpyDefault)) != hipSuccess)
        return cleanup(hip_fail(e, "copy gamma"));
    if ((e = hipMemcpy(h->bias, desc->bias, 24 * sizeof(float), hipMemcpyDefault)) != hipSuccess)
        return cleanup(hip_fail(e, "copy bias"));
    if ((e = mhc::launch_fn_pack(desc->fn, h->H, h->fnp, nullptr)) != hipSuccess)
        return cleanup(hip_fail(e, "fn pack launch"));
    if ((st = noalloc_setup(h->device)) != MHC_SEAM_OK)
        return cleanup(st);
    h->scratch_max = max_scratch_bytes(*h);
    if (h->scratch_max) {
        Scratch *s = nullptr;
        int st2 = ensure_scratch(*h, nullptr, &s);
        if (st2 != MHC_SEAM_OK)
            return cleanup(st2);
    }
    if ((e = hipDeviceSynchronize()) != hipSuccess)
        return cleanup(hip_fail(e, "hipDeviceSynchronize after create"));
    (void)hipSetDevice(prev);
    *out = h;
    return MHC_SEAM_OK;
}

int mhc_seam_run(mhc_seam_t h, const mhc_seam_args *a, void *stream_ptr)
{
    return run_seam(h, a, stream_ptr, false);
}

int mhc_seam_run_noalloc(mhc_seam_t h, const mhc_seam_args *a, void *stream_ptr)
{
    return run_seam(h, a, stream_ptr, true);
}

}  // extern "C"

namespace {

int run_seam(mhc_seam *h, const mhc_seam_args *a, void *stream_ptr, bool noalloc)
{
    if (!h)
        return fail(MHC_SEAM_INVALID_ARG, "handle is NULL");
    int st = check_args(h->H, h->max_tokens, a);
    if (st != MHC_SEAM_OK)
        return st;
    if (a->T == 0)
        return MHC_SEAM_OK;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    mhc_seam_plan pl;
    make_plan(h->H, a->T, h->cu_count, h->ksplit_override, &pl);

    mhc::SeamParams p;
    std::memset(&p, 0, sizeof p);
    p.T = (int)a->T;
    p.H = h->H;
    p.nchunks = h->H / mhc::kChunk;
    p.nseg = h->H / mhc::kSeg;
    p.nblocks = pl.blocks;
    p.ksplit = pl.ksplit;
    p.segs_per_split = pl.segs_per_split;
    p.rows_blocks = pl.rows_blocks;
    p.eps = h->eps;
    p.iters = h->iters;
    p.identity_pre = a->identity_pre;
    p.x = a->x;
    p.y = a->y;
    p.pre = a->pre;
    p.post = a->post;
    p.res = a->res;
    p.fnp = h->fnp;
    p.gamma = h->gamma;
    p.bias = h->bias;
    p.resid = a->residual_out;
    p.norm = a->norm;
    p.grid = a->grid;
    p.codes = a->codes;
    p.scales = a->scales;
    p.pre_out = a->pre_out;
    p.post_out = a->post_out;
    p.res_out = a->res_out;

    int prev = 0;
    (void)hipGetDevice(&prev);
    if (prev != h->device)
        (void)hipSetDevice(h->device);
    {
        std::lock_guard<std::mutex> lock(h->mu);
        h->streams.add(stream);
    }
    if (scratch_bytes(h->H, a->T, h->max_tokens, pl)) {
        if (noalloc) {
            // the fixed per-device array: sync words of the split blocks,
            // then their partials and u
            const size_t need = kNoAllocSyncBytes + part_bytes(pl) +
                                round256((size_t)(a->T - (int64_t)pl.rows_blocks *
                                                             mhc::kBlockTokens) * h->H * 2);
            char *base = static_cast<char *>(noalloc_ptr(h->device));
            if (!base)
                st = fail(MHC_SEAM_INVALID_ARG,
                          "no-allocation scratch is not set up for device %d", h->device);
            else if (split_blocks(pl) > kNoAllocSyncBlocks || need > kNoAllocBytes)
                st = fail(MHC_SEAM_INVALID_ARG,
                          "T=%lld at H=%d needs %zu bytes of split-mode scratch (%lld split "
                          "blocks); the no-allocation entry point has %zu bytes for at most %d "
                          "split blocks",
                          (long long)a->T, h->H, need, (long long)split_blocks(pl),
                          kNoAllocBytes, kNoAllocSyncBlocks);
            else
                set_scratch(p, base, kNoAllocSyncBytes, pl, h->H);
        } else {
            Scratch *s = nullptr;
            st = ensure_scratch(*h, stream, &s);
            if (st == MHC_SEAM_OK)
                set_scratch(p, static_cast<char *>(s->base), sync_bytes(h->H, h->max_tokens), pl,
                            h->H);
        }
        if (st != MHC_SEAM_OK) {
            if (prev != h->device)
                (void)hipSetDevice(prev);
            return st;
        }
        p.spin_limit = spin_limit(*h, pl);
    }
    // 128-wide groups: fused into the finish of whole-row launches; with
    // split workgroups the seam writes the bf16 norm and a quantiser pass
    // follows
    const bool g128 = a->out_dtype == MHC_SEAM_OUT_MXFP8_G128;
    const bool g128_fused = g128 && pl.row_segs != 0 && pl.rows_blocks == pl.grid;
    const int kout = g128 ? (g128_fused ? (int)mhc::kMxfp8G128 : (int)MHC_SEAM_OUT_BF16)
                          : a->out_dtype;
    if (g128 && !g128_fused)
        p.codes = p.scales = nullptr;
    hipError_t e;
    if (!a->unshifted) {
        e = mhc::launch_seam(p, a->form, kout, pl.row_segs, pl.grid, stream);
    } else {
        // pass 1: post-mix (residual_out) and the fresh gates; no collapse
        mhc::SeamParams pa = p;
        pa.identity_pre = 1;
        pa.skip_norm = 1;
        pa.norm = pa.grid = nullptr;
        pa.codes = pa.scales = nullptr;
        e = mhc::launch_seam(pa, a->form, MHC_SEAM_OUT_BF16, pl.row_segs, pl.grid, stream);
        // pass 2: x' (residual_out, or x in the no_post form) collapsed with
        // the fresh pre, RMSNorm and quantiser; the gates are not redone
        if (e == hipSuccess) {
            mhc::SeamParams pb = p;
            pb.x = a->form == MHC_SEAM_POST ? a->residual_out : a->x;
            pb.y = nullptr;
            pb.post = pb.res = nullptr;
            pb.resid = nullptr;
            pb.identity_pre = 0;
            pb.pre = a->pre_out;
            pb.skip_gates = 1;
            pb.pre_out = pb.post_out = pb.res_out = nullptr;
            // whole-row plans take the collapse-only form (no fn operands,
            // no gate projection); split plans the no_post form
            const bool collapse = pl.row_segs != 0 &&
                                  !(pl.rows_blocks < pl.blocks &&
                                    pl.segs_per_split > mhc::kWaves);
            e = mhc::launch_seam(pb, collapse ? (int)mhc::kCollapse : (int)MHC_SEAM_NO_POST, kout,
                                 pl.row_segs, pl.grid, stream);
        }
    }
    if (e == hipSuccess && g128 && !g128_fused)
        e = mhc::launch_quantize(a->norm, (int)a->T, h->H, 128, a->codes, a->scales, nullptr,
                                 stream);
    if (prev != h->device)
        (void)hipSetDevice(prev);
    if (e != hipSuccess)
        return hip_fail(e, "seam launch");
    return MHC_SEAM_OK;
}

}  // namespace

extern "C" {

int mhc_seam_destroy(mhc_seam_t h)
{
    if (!h)
        return MHC_SEAM_OK;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(h->device);
    // the handle's memory is in use until every seam it enqueued has run:
    // wait for the streams it ran on, and only those
    hipError_t e = hipSuccess;
    if (h->streams.overflow) {
        e = hipDeviceSynchronize();
    } else {
        for (int i = 0; i < h->streams.n; ++i) {
            hipError_t e2 = hipStreamSynchronize(h->streams.s[i]);
            if (e == hipSuccess)
                e = e2;
        }
    }
    for (auto &kv : h->scratch)
        if (kv.second.base)
            (void)hipFree(kv.second.base);
    if (h->fnp)
        (void)hipFree(h->fnp);
    if (h->gamma)
        (void)hipFree(h->gamma);
    if (h->bias)
        (void)hipFree(h->bias);
    (void)hipSetDevice(prev);
    delete h;
    if (e != hipSuccess)
        return hip_fail(e, "hipStreamSynchronize in destroy");
    return MHC_SEAM_OK;
}

int mhc_seam_quantize(const uint16_t *src, int64_t rows, int32_t H, int32_t group,
                      uint8_t *codes, uint8_t *scales, uint16_t *grid, void *stream)
{
    if (group != 32 && group != 128)
        return fail(MHC_SEAM_INVALID_ARG, "quantize groups are 32 or 128 elements");
    if (rows < 0 || H <= 0 || H % mhc::kSeg || H % group)
        return fail(MHC_SEAM_INVALID_ARG,
                    "quantize needs rows >= 0 and H a multiple of 64 and of the group");
    if (rows * (int64_t)H * 2 >= kOffsetLimit)
        return fail(MHC_SEAM_INVALID_ARG, "rows*H*2 must be < 2^31");
    if (!codes != !scales)
        return fail(MHC_SEAM_INVALID_ARG, "codes and scales come together");
    if (rows == 0)
        return MHC_SEAM_OK;
    if (!src || (!codes && !grid))
        return fail(MHC_SEAM_INVALID_ARG, "quantize needs src and codes+scales and/or grid");
    const void *ptrs[] = {src, codes, grid};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return fail(MHC_SEAM_INVALID_ARG, "src, codes and grid must be 16-byte aligned");
    hipError_t e = mhc::launch_quantize(src, (int)rows, H, group, codes, scales, grid,
                                        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "quantize launch");
    return MHC_SEAM_OK;
}

int mhc_seam_copy(void *dst, const void *src, size_t bytes, void *stream)
{
    if (!dst || !src || bytes % 16 || !aligned16(dst) || !aligned16(src))
        return fail(MHC_SEAM_INVALID_ARG, "copy needs 16-byte aligned pointers and size");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return hip_fail(e, "device attributes");
    e = mhc::launch_copy(dst, src, bytes, cus, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "copy launch");
    return MHC_SEAM_OK;
}

int mhc_stream_mix(void *dst, size_t dst_bytes, const void *src, size_t src_bytes, void *stream)
{
    if (!dst || !src || dst_bytes % 16 || src_bytes % 16 || !aligned16(dst) || !aligned16(src))
        return fail(MHC_SEAM_INVALID_ARG, "stream mix needs 16-byte aligned pointers and sizes");
    if (dst_bytes == 0 || dst_bytes >= (size_t(1) << 31) || src_bytes >= (size_t(1) << 31))
        return fail(MHC_SEAM_INVALID_ARG,
                    "stream mix needs 0 < dst_bytes < 2^31 and src_bytes < 2^31");
    const uintptr_t dlo = reinterpret_cast<uintptr_t>(dst), slo = reinterpret_cast<uintptr_t>(src);
    if (dlo < slo + src_bytes && slo < dlo + dst_bytes)
        return fail(MHC_SEAM_INVALID_ARG, "stream mix: dst overlaps src");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return hip_fail(e, "device attributes");
    e = mhc::launch_stream_mix(dst, dst_bytes, src, src_bytes, cus,
                               reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "stream mix launch");
    return MHC_SEAM_OK;
}

int mhc_head_reduce(const uint16_t *x, const float *w, int64_t T, int32_t H, uint16_t *out,
                    void *stream)
{
    if (T < 0 || H <= 0 || H % 8)
        return fail(MHC_SEAM_INVALID_ARG, "head reduce needs T >= 0 and H a positive multiple of 8");
    if (T > (INT64_MAX / 8) / H)
        return fail(MHC_SEAM_INVALID_ARG, "T*4*H*2 overflows");
    if (T == 0)
        return MHC_SEAM_OK;
    if (!x || !out)
        return fail(MHC_SEAM_INVALID_ARG, "head reduce needs x and out");
    if (!aligned16(x) || !aligned16(out) || (w && !aligned16(w)))
        return fail(MHC_SEAM_INVALID_ARG, "x, w and out must be 16-byte aligned");
    const uintptr_t olo = reinterpret_cast<uintptr_t>(out), ohi = olo + (uintptr_t)(T * H * 2);
    const uintptr_t xlo = reinterpret_cast<uintptr_t>(x), xhi = xlo + (uintptr_t)(T * H * 8);
    const uintptr_t wlo = reinterpret_cast<uintptr_t>(w), whi = wlo + (uintptr_t)(T * 16);
    if ((olo < xhi && xlo < ohi) || (w && olo < whi && wlo < ohi))
        return fail(MHC_SEAM_INVALID_ARG, "out overlaps x or w");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return hip_fail(e, "device attributes");
    e = mhc::launch_head_reduce(x, w, T, H, out, cus, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "head reduce launch");
    return MHC_SEAM_OK;
}

int mhc_mxfp8_gemm_blocks(int64_t T, int32_t N, int32_t cu_count, int32_t *tm, int32_t *tn,
                          int32_t *stages)
{
    if (T <= 0 || T > INT32_MAX || N <= 0 || cu_count <= 0 || !tm || !tn || !stages)
        return fail(MHC_SEAM_INVALID_ARG,
                    "gemm blocks need T in 1..2^31-1, N > 0, cu_count > 0 and three outputs");
    const mhc::GemmBlocks g = mhc::gemm_blocks(T, N, cu_count);
    *tm = g.tm;
    *tn = g.tn;
    *stages = g.stages;
    return MHC_SEAM_OK;
}

int mhc_mxfp8_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                   const uint8_t *b_scales, int64_t T, int32_t N, int32_t K, uint16_t *out,
                   void *stream)
{
    if (T < 0 || N <= 0 || K <= 0 || K % 128 || K > 8192)
        return fail(MHC_SEAM_INVALID_ARG,
                    "gemm needs T >= 0, N > 0 and K a positive multiple of 128, at most 8192");
    if (T > INT32_MAX || T * (int64_t)K >= ((int64_t)1 << 40) || T * (int64_t)N >= ((int64_t)1 << 40) ||
        (int64_t)N * K >= ((int64_t)1 << 40))
        return fail(MHC_SEAM_INVALID_ARG, "gemm sizes too large");
    if (T == 0)
        return MHC_SEAM_OK;
    if (!a || !a_scales || !b || !b_scales || !out)
        return fail(MHC_SEAM_INVALID_ARG, "gemm needs a, a_scales, b, b_scales and out");
    if (!aligned16(a) || !aligned16(b) || (reinterpret_cast<uintptr_t>(a_scales) & 3) ||
        (reinterpret_cast<uintptr_t>(b_scales) & 3))
        return fail(MHC_SEAM_INVALID_ARG,
                    "a and b must be 16-byte aligned, a_scales and b_scales 4-byte aligned");
    struct R { const void *p; size_t n; } in[] = {{a, (size_t)T * K}, {a_scales, (size_t)T * (K / 32)},
                                                  {b, (size_t)N * K}, {b_scales, (size_t)N * (K / 32)}};
    const uintptr_t olo = reinterpret_cast<uintptr_t>(out), ohi = olo + (size_t)T * N * 2;
    for (const R &r : in) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(r.p);
        if (olo < lo + r.n && lo < ohi)
            return fail(MHC_SEAM_INVALID_ARG, "out overlaps an input");
    }
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return hip_fail(e, "device attributes");
    e = mhc::launch_mxfp8_gemm(a, a_scales, b, b_scales, (int)T, N, K, out, cus,
                               reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "gemm launch");
    return MHC_SEAM_OK;
}

}  // extern "C"
