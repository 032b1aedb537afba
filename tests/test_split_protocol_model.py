"""CPU model of the split-mode protocol (tests/split_protocol_model.cpp).

The seam's split launches finish a block across workgroups: an arrival
counter that never goes back (epochs of 4096), two alternating hand-off mask
sets with a CLOSED bit, a bounded wait and a hand-off to the last arriver
("[FlyDSL] Single-launch Mega-mHC on gfx950", Kernel Architecture: split-K
with the last-arriving workgroup finishing; DIST_FINISH's residency guard,
bounded spin and hand-off, which never hangs).  The model runs each split
as a thread, with random start delays, suspended splits, every kind of
wait bound, split counts 1..128 changing from launch to launch on the same
block words, and counters that wrap past 2^32.  It checks that each block
has exactly one finisher, every split's segments are normalised exactly
once, every partial and handed-off u read belongs to the launch, and the
words are left ready for the next launch.

It also builds copies of the model with one protocol mistake planted each
(on the CPU), which the same checks must catch.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "split_protocol_model.cpp")

MUTANTS = {
    # the finisher does not move the counter on to the next epoch
    "no_epoch_step": ("        bw.arrive.fetch_add(kEpoch - (uint32_t)L.ks, std::memory_order_relaxed);\n",
                      ""),
    # the finisher does not clear the mask set of the next launch
    "stale_next_mask_set": ("            next[w].store(0, std::memory_order_relaxed);\n",
                            "            (void)next;\n"),
    # a split that finds CLOSED after handing off does not finish itself
    "closed_hand_off_dropped": ("    if (was & kClosed) {   // every split has arrived: finish here after all",
                                "    if (false) {"),
    # waiters compare the raw counter instead of its value in this epoch
    "wait_ignores_epoch": ("if (n - epoch >= (uint32_t)L.ks) {", "if (n >= (uint32_t)L.ks) {"),
    # the finisher reads the hand-off mask before closing it (a split that
    # hands off in between is finished by nobody)
    "finisher_reads_mask_without_closing": (
        "handed[w] = mask[w].fetch_or(kClosed, std::memory_order_acq_rel) & ~kClosed;",
        "handed[w] = mask[w].load(std::memory_order_acquire) & ~kClosed;"),
}


def build(tmp_path, src_text, name, sanitize=False):
    src = tmp_path / f"{name}.cpp"
    src.write_text(src_text)
    exe = tmp_path / name
    cmd = ["g++", "-std=c++17", "-pthread", "-Wall", str(src), "-o", str(exe)]
    cmd += ["-O1", "-g", "-fsanitize=thread"] if sanitize else ["-O2"]
    subprocess.run(cmd, check=True)
    return str(exe)


def run(exe, seed, launches, timeout=300):
    return subprocess.run([exe, str(seed), str(launches)], capture_output=True, text=True,
                          timeout=timeout)


def test_protocol_holds(tmp_path):
    exe = build(tmp_path, open(SRC).read(), "model")
    for seed in (1, 2, 3):
        r = run(exe, seed, 150)
        assert r.returncode == 0, r.stdout + r.stderr
        print(r.stdout.strip())


def test_protocol_model_under_thread_sanitizer(tmp_path):
    """Host build under ThreadSanitizer: the model itself has no data race
    (every shared word is an atomic), so its verdicts are about the
    protocol."""
    exe = build(tmp_path, open(SRC).read(), "model_tsan", sanitize=True)
    r = run(exe, 4, 30)
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stdout + r.stderr[-3000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_model_catches_planted_protocol_mistakes(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site of {name} not found"
    exe = build(tmp_path, text.replace(old, new), name)
    failed = False
    for seed in range(1, 9):
        r = run(exe, seed, 80, timeout=120)
        if r.returncode != 0:
            failed = True
            break
    assert failed, f"the model did not catch {name}"
