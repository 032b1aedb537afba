// split_protocol_model.cpp -- a threaded CPU model of the seam's split-mode
// protocol (the cross-workgroup finish of layer_mhc_seam_amd/csrc/
// seam_kernels.hip, split_body), for the tests.
//
// "[FlyDSL] Single-launch Mega-mHC on gfx950", Kernel Architecture: split-K
// over workgroups, the last-arriving workgroup finishes; the distributed
// finish with a residency guard and a bounded spin with hand-off "never
// hangs".  Each split of a block is a thread here; the block's words are
// the kernel's: a 32-bit arrival counter that never goes back (a launch's
// arrivals are its value modulo kEpoch), and two hand-off mask sets of 63
// splits per 64-bit word plus a CLOSED bit, used in alternate launches.
//
// What a thread does, in the kernel's order:
//   store its partial record; arrive (fetch_add 1 on the counter);
//   the last arriver (the finisher) moves the counter on to the next
//   multiple of kEpoch, clears the other mask set, sets CLOSED with one
//   fetch_or (getting back the splits that handed off before), reduces the
//   partials, normalises its own segments, computes the gates and finishes
//   every handed-off split's segments from the u it left;
//   any other split polls the counter (at most spin + 1 times; spin < 0:
//   never) until every split has arrived, then reduces and normalises its
//   own segments; if its polls run out it stores its u, sets its bit with
//   a fetch_or and, if that returns CLOSED, finishes itself after all.
//   Splits start late at random, some much later than their block's wait
//   bound (a workgroup that is not resident), and stall at random between
//   any two of these steps.
//
// Memory ordering: on the GPU the data (partials, handed-off u) is written
// with device-coherent stores and waited for (s_waitcnt) before the
// signalling atomic, and the waiters' device-coherent loads are issued
// after the poll that saw the count; here the same order is a release on the
// signalling read-modify-writes and an acquire on the polls and the reads.
//
// Checks, per launch: exactly one finisher per block; each split's segments
// normalised exactly once; gates computed once per block; every partial
// and every handed-off u read is the one this launch wrote; afterwards each
// counter sits at a multiple of kEpoch and the mask set of the next launch
// is clear.  Launches run one after another (stream order) and change the
// split count and the block-to-word-set assignment between launches.
//
// Usage: split_protocol_model SEED LAUNCHES  (exit status 0 = all checks held)

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

namespace {

constexpr uint32_t kEpoch = 4096;       // > splits per block, divides 2^32
constexpr int kMaskSplits = 63;         // splits per mask word; bit 63 is CLOSED
constexpr int kMaxSplits = 128;
constexpr int kMaskWords = (kMaxSplits + kMaskSplits - 1) / kMaskSplits;
constexpr uint64_t kClosed = 1ull << 63;

struct BlockWords {
    std::atomic<uint32_t> arrive{0};
    std::atomic<uint64_t> mask[2][kMaskWords];
    BlockWords()
    {
        for (auto &set : mask)
            for (auto &w : set)
                w.store(0);
    }
};

std::atomic<uint64_t> *mask_set(BlockWords &bw, uint32_t epoch)
{
    return bw.mask[(epoch / kEpoch) & 1];
}

uint64_t tag(int launch, int block, int split, int what)
{
    return ((uint64_t)(launch + 1) << 40) ^ ((uint64_t)block << 20) ^ ((uint64_t)split << 2) ^
           (uint64_t)what;
}

std::atomic<int> g_fail{0};

void check(bool ok, const char *what, int launch, int block, int split)
{
    if (!ok) {
        if (g_fail.fetch_add(1) < 10)
            std::fprintf(stderr, "launch %d block %d split %d: %s\n", launch, block, split, what);
    }
}

struct Launch {
    int id, nblocks, ks, spin;
    bool skip_norm;
    std::vector<int> words_of;                  // block -> word set
    std::vector<std::atomic<uint64_t>> part;    // [block][split] partial record
    std::vector<std::atomic<uint64_t>> uscr;    // [block][split] handed-off u
    std::vector<std::atomic<int>> normed;       // [block][split] times normalised
    std::vector<std::atomic<int>> finishers;    // [block]
    std::vector<std::atomic<int>> gates;        // [block]
    std::vector<int> delay_us;                  // [block][split] start delay
    std::vector<unsigned> stall;                // [block][split] seed of stalls between steps
    Launch(int id_, int nb, int ks_, int spin_, bool skip)
        : id(id_), nblocks(nb), ks(ks_), spin(spin_), skip_norm(skip), words_of(nb),
          part(nb * ks_), uscr(nb * ks_), normed(nb * ks_), finishers(nb), gates(nb),
          delay_us(nb * ks_, 0), stall(nb * ks_, 0)
    {
        for (auto &a : part) a.store(0);
        for (auto &a : uscr) a.store(0);
        for (auto &a : normed) a.store(0);
        for (auto &a : finishers) a.store(0);
        for (auto &a : gates) a.store(0);
    }
};

void reduce_partials(Launch &L, int b, int s)
{
    for (int k = 0; k < L.ks; ++k)
        check(L.part[b * L.ks + k].load(std::memory_order_acquire) == tag(L.id, b, k, 1),
              "reduction read a partial of another launch", L.id, b, s);
}

// A workgroup can stall between any two steps (preempted, its CU shared):
// with a split's stall seed set, each step point sleeps 0-300 us at random.
struct Stall {
    std::minstd_rand r;
    bool on;
    Stall(unsigned seed) : r(seed), on(seed != 0) {}
    void operator()()
    {
        if (on && r() % 4 == 0)
            std::this_thread::sleep_for(std::chrono::microseconds(r() % 300));
    }
};

void split(Launch &L, std::vector<BlockWords> &words, int b, int s)
{
    if (L.delay_us[b * L.ks + s])
        std::this_thread::sleep_for(std::chrono::microseconds(L.delay_us[b * L.ks + s]));
    Stall stall(L.stall[b * L.ks + s]);
    BlockWords &bw = words[L.words_of[b]];
    L.part[b * L.ks + s].store(tag(L.id, b, s, 1), std::memory_order_relaxed);
    stall();
    const uint32_t old = bw.arrive.fetch_add(1, std::memory_order_acq_rel);
    stall();
    const uint32_t epoch = old & ~(kEpoch - 1);
    const bool finisher = (int)(old & (kEpoch - 1)) == L.ks - 1;
    std::atomic<uint64_t> *mask = mask_set(bw, epoch);
    const int nwords = (L.ks + kMaskSplits - 1) / kMaskSplits;
    if (finisher) {
        L.finishers[b].fetch_add(1);
        bw.arrive.fetch_add(kEpoch - (uint32_t)L.ks, std::memory_order_relaxed);
        std::atomic<uint64_t> *next = mask_set(bw, epoch + kEpoch);
        for (int w = 0; w < kMaskWords; ++w)
            next[w].store(0, std::memory_order_relaxed);
        stall();
        uint64_t handed[kMaskWords] = {};
        for (int w = 0; w < nwords; ++w)
            handed[w] = mask[w].fetch_or(kClosed, std::memory_order_acq_rel) & ~kClosed;
        reduce_partials(L, b, s);
        if (!L.skip_norm)
            L.normed[b * L.ks + s].fetch_add(1);
        L.gates[b].fetch_add(1);
        for (int w = 0; w < nwords; ++w)
            for (uint64_t bits = handed[w]; bits; bits &= bits - 1) {
                const int k = w * kMaskSplits + __builtin_ctzll(bits);
                check(k < L.ks && k != s, "hand-off bit of no other split", L.id, b, k);
                check(L.uscr[b * L.ks + k].load(std::memory_order_acquire) == tag(L.id, b, k, 2),
                      "finisher read a u of another launch", L.id, b, k);
                L.normed[b * L.ks + k].fetch_add(1);
            }
        return;
    }
    if (L.skip_norm)
        return;
    bool arrived = false;
    for (int it = 0; it <= L.spin; ++it) {
        const uint32_t n = bw.arrive.load(std::memory_order_acquire);
        if (n - epoch >= (uint32_t)L.ks) {   // the finisher may have moved it on by kEpoch
            arrived = true;
            break;
        }
        std::this_thread::yield();
    }
    if (arrived) {
        reduce_partials(L, b, s);
        L.normed[b * L.ks + s].fetch_add(1);
        return;
    }
    L.uscr[b * L.ks + s].store(tag(L.id, b, s, 2), std::memory_order_relaxed);
    stall();
    const uint64_t was = mask[s / kMaskSplits].fetch_or(1ull << (s % kMaskSplits),
                                                        std::memory_order_acq_rel);
    if (was & kClosed) {   // every split has arrived: finish here after all
        reduce_partials(L, b, s);
        L.normed[b * L.ks + s].fetch_add(1);
    }
}

}  // namespace

int main(int argc, char **argv)
{
    const unsigned seed = argc > 1 ? (unsigned)std::atoi(argv[1]) : 1;
    const int launches = argc > 2 ? std::atoi(argv[2]) : 60;
    std::mt19937 rng(seed);
    const int nwordsets = 6;
    std::vector<BlockWords> words(nwordsets);
    // start the counters just below the 32-bit wrap on some word sets
    for (int i = 0; i < nwordsets; i += 2)
        words[i].arrive.store(0u - 3 * kEpoch);
    const int splits[] = {1, 2, 3, 4, 5, 10, 20, 40, 62, 63, 64, 80, 127, 128};
    int handoffs = 0, waits = 0;
    for (int l = 0; l < launches; ++l) {
        const int ks = splits[rng() % (sizeof splits / sizeof *splits)];
        const int nb = 1 + (int)(rng() % 3);
        // spin < 0: never wait; 0: one poll; large: wait for everyone
        const int spins[] = {-1, 0, 1, 50, 1000000};
        const int spin = spins[rng() % 5];
        Launch L(l, nb, ks, spin, rng() % 8 == 0);
        std::vector<int> ws(nwordsets);
        for (int i = 0; i < nwordsets; ++i)
            ws[i] = i;
        std::shuffle(ws.begin(), ws.end(), rng);
        for (int b = 0; b < nb; ++b)
            L.words_of[b] = ws[b];
        // some splits start late (delayed), a few very late (a suspended,
        // not resident workgroup) -- never with an unbounded spin, which
        // the residency guard allows only when all splits are resident
        for (int i = 0; i < nb * ks; ++i) {
            const unsigned r = rng() % 16;
            L.delay_us[i] = r < 3 ? (int)(rng() % 200) : (r == 3 && spin < 1000 ? 3000 : 0);
            L.stall[i] = rng() % 3 == 0 ? (unsigned)rng() | 1u : 0u;
        }
        std::vector<std::thread> th;
        for (int b = 0; b < nb; ++b)
            for (int s = 0; s < ks; ++s)
                th.emplace_back(split, std::ref(L), std::ref(words), b, s);
        for (auto &t : th)
            t.join();
        for (int b = 0; b < nb; ++b) {
            check(L.finishers[b].load() == 1, "not exactly one finisher", l, b, -1);
            check(L.gates[b].load() == 1, "gates not computed once", l, b, -1);
            // a launch without the norm (the unshifted ordering's first
            // launch) normalises nothing; any other normalises every
            // split's segments exactly once
            for (int s = 0; s < ks; ++s)
                check(L.normed[b * ks + s].load() == (L.skip_norm ? 0 : 1),
                      "segments not normalised exactly once", l, b, s);
            BlockWords &bw = words[L.words_of[b]];
            const uint32_t c = bw.arrive.load();
            check(c % kEpoch == 0, "counter not at a multiple of the epoch step", l, b, -1);
            for (int w = 0; w < kMaskWords; ++w)
                check(mask_set(bw, c)[w].load() == 0, "next launch's mask set not clear", l, b,
                      -1);
            for (int s = 0; s < ks; ++s)
                handoffs += L.uscr[b * ks + s].load() != 0;
            waits += ks;
        }
    }
    std::printf("launches %d, splits %d, hand-offs %d, failures %d\n", launches, waits, handoffs,
                g_fail.load());
    return g_fail.load() ? 1 : 0;
}
