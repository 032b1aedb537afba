"""GPU parity of the HIP seam (through the C ABI) against the CPU oracle.

Workloads are the seam shapes of "[FlyDSL] Single-launch Mega-mHC on gfx950"
(performance tables, H = 5120) plus an H = 512 oracle case; forms and
outputs follow its Test Plan (post, no_post, identity_pre; bf16, fp8_grid,
mxfp8) and T covers empty, ragged and multi-block cases.
"""
import numpy as np
import pytest
import torch

from bits import exact_bf16
from seam_harness import (check_all, check_bf16, check_gates, check_quant, dev_inputs,
                          host_case, make_seam, run_gpu, run_oracle, to_dev, to_host)
from layer_mhc_seam_amd import synth

pytestmark = pytest.mark.gpu


def _gpu_ok():
    return torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not _gpu_ok():
        pytest.skip("no GPU")


def full_case(name, form=None, out=None, idp=False, seed=0, ksplit=0):
    w = synth.WORKLOADS[name]
    form = form or w.form
    out = out or w.out_dtype
    c = host_case(w.T, w.H, seed=seed, y_boost_every=w.y_boost_every)
    s = make_seam(c, w.T, ksplit=ksplit)
    got = run_gpu(s, c, form, idp, out)
    want = run_oracle(c, form, idp)
    stats = check_all(got, want, form, out)
    s.close()
    return stats


@pytest.mark.parametrize("name", ["tiny_post_bf16", "decode_post_bf16",
                                  "prefill384_post_mxfp8", "tail4160_nopost_bf16"])
def test_workload_parity_full(name):
    print(name, full_case(name), flush=True)


@pytest.mark.parametrize("form", ["post", "no_post"])
@pytest.mark.parametrize("out", ["bf16", "fp8_grid", "mxfp8", "mxfp8_g128"])
@pytest.mark.parametrize("idp", [False, True])
def test_forms_and_outputs_small(form, out, idp):
    c = host_case(40, 512, seed=3)
    s = make_seam(c, 40)
    got = run_gpu(s, c, form, idp, out)
    check_all(got, run_oracle(c, form, idp), form, out)


@pytest.mark.parametrize("T,H", [(5, 512), (8, 5120)])
@pytest.mark.parametrize("form", ["post", "no_post"])
@pytest.mark.parametrize("out", ["bf16", "fp8_grid", "mxfp8", "mxfp8_g128"])
@pytest.mark.parametrize("idp", [False, True])
def test_decode_forms_and_outputs(T, H, form, out, idp):
    """T <= 8 runs the split kernel's decode instance, which loads and
    normalises token half 0 only (the rows of half 1 all stand for token
    T - 1): every form and output there, T = 8 being the largest such T."""
    c = host_case(T, H, seed=T + H)
    s = make_seam(c, T)
    for _ in range(2):
        got = run_gpu(s, c, form, idp, out)
        check_all(got, run_oracle(c, form, idp), form, out)
    s.close()


@pytest.mark.parametrize("T", [1, 3, 15, 16, 17, 63, 64, 100])
@pytest.mark.parametrize("H", [256, 5120])
def test_ragged_token_counts(T, H):
    c = host_case(T, H, seed=T)
    s = make_seam(c, 128)
    got = run_gpu(s, c, "post", False, "mxfp8")
    check_all(got, run_oracle(c), "post", "mxfp8")


@pytest.mark.parametrize("ksplit", [1, 2, 3, 4, 5, 7, 20, 40, 80])
def test_forced_split_counts(ksplit):
    c = host_case(50, 5120, seed=11)
    s = make_seam(c, 64, ksplit=ksplit)
    got = run_gpu(s, c, "post", False, "fp8_grid")
    check_all(got, run_oracle(c), "post", "fp8_grid")


@pytest.mark.parametrize("T,ksplit", [(4, 10), (4, 80), (50, 5), (64, 40), (384, 10), (100, 1),
                                      (64, 4), (50, 2), (1024, 3)])
@pytest.mark.parametrize("spin", [-1, 1, 0])
def test_split_finish_paths(T, ksplit, spin):
    """Split mode with the distributed finish (spin 0: default wait), with
    waits that run out after one poll (spin 1: some splits may hand off) and
    with no wait at all (spin -1: every non-last split hands its segments to
    the finisher through scratch).  Splits of 1-5 segments per wave cover u
    kept in VGPRs (1) and in LDS (2-5)."""
    c = host_case(T, 5120, seed=T + ksplit)
    s = make_seam(c, T, ksplit=ksplit, spin_polls=spin)
    want = run_oracle(c)
    for _ in range(3):   # the block words carry over from launch to launch
        got = run_gpu(s, c, "post", False, "mxfp8")
        check_all(got, want, "post", "mxfp8")


@pytest.mark.parametrize("spin", [0, -1])
def test_split_state_carries_across_plans(spin):
    """One handle and stream, launches whose plans differ (split counts 20,
    10, 4 and 1, a mixed tail, whole rows) in a sequence that revisits each
    block with a different split count, then 41 launches in a row: the block
    words (arrival counter and the alternating mask sets) must stay valid
    through every change."""
    Ts = [64, 384, 4, 1024, 64, 4160, 4, 384, 16, 1024, 64]
    cases = {T: host_case(T, 5120, seed=90 + T) for T in set(Ts)}
    for c in cases.values():        # one handle: the same weights for every case
        c.update(fn=cases[4160]["fn"], gamma=cases[4160]["gamma"], bias=cases[4160]["bias"])
    wants = {T: run_oracle(c) for T, c in cases.items()}
    s = make_seam(cases[4160], 4160, spin_polls=spin)
    for T in Ts:
        got = run_gpu(s, cases[T], "post", False, "bf16")
        check_all(got, wants[T], "post", "bf16")
    first = run_gpu(s, cases[4], "post", False, "bf16")
    check_all(first, wants[4], "post", "bf16")
    for _ in range(40):
        again = run_gpu(s, cases[4], "post", False, "bf16")
        for k in first:
            assert np.array_equal(again[k], first[k]), k
    s.close()


@pytest.mark.parametrize("T,spin", [(4160, 0), (4160, -1), (4496, 0), (4512, 0), (5120, 0),
                                    (6144, 0), (6144, -1), (16400, 0)])
def test_split_tail_after_whole_rows(T, spin):
    """Whole-row blocks plus a split tail: T = 4160 leaves 4 blocks after one
    round of 256 CUs (40 splits of 2 segments each, in the whole-row launch;
    with spin -1 every tail split hands off), 4496 leaves 25 (10 splits of 8
    segments, 250 workgroups), 16400 leaves 1.  4512 (26 x 9 splits of 9
    segments), 5120 (64 x 4 of 20) and 6144 (128 x 2 of 40) run their tail
    splits in a split launch after the whole-row launch."""
    c = host_case(T, 5120, seed=T)
    s = make_seam(c, T, spin_polls=spin)
    want = run_oracle(c)
    for _ in range(2):
        got = run_gpu(s, c, "post", False, "mxfp8")
        check_all(got, want, "post", "mxfp8")
    s.close()


@pytest.mark.parametrize("H", [64, 192, 320, 1024, 2048, 4096, 7168])
def test_other_widths(H):
    c = host_case(33, H, seed=5)
    s = make_seam(c, 33)
    got = run_gpu(s, c, "post", False, "mxfp8")
    check_all(got, run_oracle(c), "post", "mxfp8")


@pytest.mark.parametrize("T,H", [(2048, 7168), (300, 7168), (1100, 3072)])
def test_widths_without_whole_row_kernels(T, H):
    """Widths whose H/512 has no whole-row instance run split mode at any T;
    with more than 5 segments per wave the splits stream u to scratch and the
    finisher normalises every segment (H = 7168: 112 segments)."""
    from layer_mhc_seam_amd.seam import plan
    p = plan(H, T, 256)
    assert p["row_segs"] == 0
    c = host_case(T, H, seed=T + H)
    s = make_seam(c, T)
    got = run_gpu(s, c, "post", False, "mxfp8")
    check_all(got, run_oracle(c), "post", "mxfp8")
    s.close()


def test_empty_input_is_noop():
    c = host_case(8, 512)
    s = make_seam(c, 8)
    z = {k: v[:0] for k, v in dev_inputs(c).items()}
    o = s.run(**z)
    torch.cuda.synchronize()
    assert o["norm"].shape == (0, 512)


@pytest.mark.parametrize("T", [4, 384, 4160])
def test_g128_output(T):
    """128-wide groups at the workload widths: split, mixed and whole-row
    plans, codes and scales bit-exact against the oracle on the GPU norm."""
    c = host_case(T, 5120, seed=60 + T, y_boost_every=64)
    s = make_seam(c, T)
    got = run_gpu(s, c, "post", False, "mxfp8_g128")
    assert got["scales"].shape == (T, 5120 // 128)
    check_all(got, run_oracle(c), "post", "mxfp8_g128")
    s.close()


@pytest.mark.parametrize("T,H,form", [(4096, 5120, "post"), (3000, 5120, "post"),
                                      (3000, 5120, "no_post"), (2080, 512, "post"),
                                      (2080, 1024, "post"), (2080, 2048, "no_post"),
                                      (2080, 4096, "post")])
def test_g128_fused_whole_row(T, H, form):
    """Whole-row launches quantise the 128-wide groups in their finish: every
    compiled row width (pairs of LDS segments; at H = 5120 also the VGPR
    segments whose row amax two waves swap), a ragged last block, both forms.
    Codes and scales bit-exact against the oracle on the GPU norm."""
    from layer_mhc_seam_amd.seam import plan
    p = plan(H, T)
    assert p["row_segs"] > 0 and p["rows_blocks"] == p["grid"]
    c = host_case(T, H, seed=70 + T + H, y_boost_every=64)
    s = make_seam(c, T)
    for _ in range(2):
        got = run_gpu(s, c, form, False, "mxfp8_g128")
        assert got["scales"].shape == (T, H // 128)
        check_all(got, run_oracle(c, form), form, "mxfp8_g128")
    s.close()


def test_g128_fused_prefill16k_sampled():
    """T = 16384, H = 5120 with fused 128-wide groups: the oracle recomputes a
    sample of tokens; the quantiser checks every group of the full output."""
    T, H = 16384, 5120
    c = host_case(T, H, seed=5)
    s = make_seam(c, T)
    got = run_gpu(s, c, "post", False, "mxfp8_g128")
    check_quant(got, "mxfp8_g128")
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([np.arange(16), np.arange(T - 16, T),
                                    rng.choice(T, 64, replace=False)]))
    want = run_oracle(c, "post", False, idx=idx)
    sub = {k: v[idx] for k, v in got.items() if k in ("residual_out", "norm", "pre_out",
                                                      "post_out", "res_out")}
    check_all(sub, want, "post", "bf16")
    s.close()


def test_prefill16k_full_parity():
    """Full-size large-prefill seam (T = 16384, H = 5120, post, fp8_grid) in
    the launch configuration the benchmark times, against the oracle on
    every token: residual bitwise, norm at the ulp bar, gates, and the grid
    bit-exact on the GPU's own norm."""
    w = synth.WORKLOADS["prefill16k_post_fp8grid"]
    c = host_case(w.T, w.H, seed=0)
    s = make_seam(c, w.T)
    got = run_gpu(s, c, w.form, False, w.out_dtype)
    s.close()
    want = run_oracle(c, w.form, False)
    stats = check_all(got, want, w.form, w.out_dtype)
    print("prefill16k", stats, flush=True)


def test_crafted_quantiser_groups_through_gamma():
    """x[:,0,:] = 1, pre = e0, res = I, post = 0 makes u = 1 and the norm equal
    gamma (rstd = 1/sqrt(1+eps) is within half a bf16 ulp of 1), so gamma
    writes crafted groups into the fused quantiser: amax = 448*2^k and its
    neighbours, zeros, subnormals, near-max (Mega-mHC page, Test Plan)."""
    H = 1024
    T = 3
    rng = np.random.default_rng(7)
    groups = []
    for k in (-126, -120, -60, -9, -1, 0, 1, 7, 60, 119):
        top = 448.0 * 2.0 ** k
        for nb in (-1, 0, 1):
            g = exact_bf16(np.round(rng.standard_normal(32) * 8) * 2.0 ** (k + 2)) \
                if k > -120 else np.zeros(32, np.uint16)
            g[rng.integers(32)] = np.uint16(int(exact_bf16([top])[0]) + nb)
            groups.append(g)
    groups.append(np.zeros(32, np.uint16))
    groups.append(np.arange(1, 33, dtype=np.uint16))
    while len(groups) < H // 32:
        groups.append(exact_bf16(rng.standard_normal(32).astype(np.float32)
                                 .astype(np.float16).astype(np.float32)))
    gamma = np.concatenate(groups[: H // 32])
    c = host_case(T, H, seed=1)
    c["gamma"] = gamma
    c["x"][:, 0, :] = exact_bf16(np.ones(H))
    c["res"] = np.broadcast_to(np.eye(4, dtype=np.float32), (T, 4, 4)).copy()
    c["post"] = np.zeros((T, 4), np.float32)
    c["pre"] = np.tile(np.array([1, 0, 0, 0], np.float32), (T, 1))
    for out in ("mxfp8", "fp8_grid", "mxfp8_g128"):
        s = make_seam(c, T)
        got = run_gpu(s, c, "post", False, out)
        assert np.array_equal(got["norm"][0], gamma)
        check_quant(got, out)
        check_all(got, run_oracle(c), "post", out)
        s.close()


def test_repeated_launches_are_bitwise_identical():
    c = host_case(384, 5120, seed=2, y_boost_every=64)
    s = make_seam(c, 384)
    d = dev_inputs(c)
    first = {k: v.clone() for k, v in s.run(out_dtype="mxfp8", **d).items()}
    for _ in range(20):
        o = s.run(out_dtype="mxfp8", **d)
    torch.cuda.synchronize()
    for k in first:
        assert torch.equal(first[k].view(torch.uint8), o[k].view(torch.uint8)), k


def test_two_streams_one_handle():
    c1 = host_case(200, 5120, seed=3)
    c2 = host_case(200, 5120, seed=4)
    c2["fn"], c2["gamma"], c2["bias"] = c1["fn"], c1["gamma"], c1["bias"]
    s = make_seam(c1, 256)
    d1, d2 = dev_inputs(c1), dev_inputs(c2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = s.run(**d1, stream=s1)
        with torch.cuda.stream(s2):
            o2 = s.run(**d2, stream=s2)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    w1, w2 = run_oracle(c1), run_oracle(c2)
    for o1, o2 in outs:
        check_all({k: to_host(v) for k, v in o1.items()}, w1, "post", "bf16")
        check_all({k: to_host(v) for k, v in o2.items()}, w2, "post", "bf16")


@pytest.mark.parametrize("T", [384, 5120])
def test_graph_capture_replays_match_eager(T):
    """Split mode (T = 384) and a whole-row launch followed by its tail's
    split launch (T = 5120) captured in one graph: every replay equals the
    eager run."""
    c = host_case(T, 5120, seed=6, y_boost_every=64)
    s = make_seam(c, T)
    d = dev_inputs(c)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = {k: v.clone() for k, v in s.run(out_dtype="mxfp8", **d, stream=stream).items()}
        out = {k: torch.empty_like(v) for k, v in eager.items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        s.run(out_dtype="mxfp8", **d, out=out, stream=stream)
    for _ in range(4):
        for v in out.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(eager[k].view(torch.uint8), out[k].view(torch.uint8)), k


def test_graph_survives_larger_eager_runs_on_its_stream():
    """A graph captured at T = 4 on a side stream keeps the stream's scratch
    pointers; eager seams of T = 384 and 4160 on the same stream afterwards
    must not move that scratch, so later replays still match eager results
    bitwise."""
    c4 = host_case(4, 5120, seed=12)
    big = {T: host_case(T, 5120, seed=13 + T) for T in (384, 4160)}
    for c in big.values():
        c.update(fn=c4["fn"], gamma=c4["gamma"], bias=c4["bias"])
    s = make_seam(c4, 4160)
    stream = torch.cuda.Stream()
    d4 = dev_inputs(c4)
    with torch.cuda.stream(stream):
        eager = {k: v.clone() for k, v in s.run(**d4, stream=stream).items()}
        out = {k: torch.empty_like(v) for k, v in eager.items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        s.run(**d4, out=out, stream=stream)
    for T, c in big.items():
        with torch.cuda.stream(stream):
            o = s.run(**dev_inputs(c), stream=stream)
        torch.cuda.synchronize()
        check_all({k: to_host(v) for k, v in o.items()}, run_oracle(c), "post", "bf16")
        for _ in range(2):
            for v in out.values():
                v.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k in eager:
                assert torch.equal(eager[k].view(torch.uint8), out[k].view(torch.uint8)), (T, k)
    del g
    s.close()


def test_capture_without_scratch_is_refused():
    from layer_mhc_seam_amd.seam import SeamError, CAPTURE_ALLOC
    c = host_case(64, 5120, seed=8)
    s = make_seam(c, 64)
    d = dev_inputs(c)
    out = s.run(**d)                     # allocates outputs eagerly
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()         # no scratch on this stream yet
    g = torch.cuda.CUDAGraph()
    with pytest.raises(SeamError) as ei:
        with torch.cuda.graph(g, stream=stream):
            s.run(**d, out=out, stream=stream)
    assert ei.value.status == CAPTURE_ALLOC


def test_copy_kernel():
    from layer_mhc_seam_amd.seam import copy
    src = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    copy(dst, src, src.numel())
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("rd,wr", [(4096, 4096), (1 << 20, 1 << 18), (40 * 4096, 4096),
                                   (4096, 1 << 16), (0, 4096), (4096 * 3 + 16, 4096),
                                   (256 * 4096 * 16 * 3 + 48, 1 << 20)])
def test_stream_mix_kernel(rd, wr):
    """The ceiling kernel for other read/write mixes, against a model of its
    definition: with S = 256 * min(CUs, ceil(max chunks / 256)) threads,
    thread g XORs input chunks g, g + S, ... into (g, ~g, 0, 0) and writes
    that XOR (j, 0, 0, 0) to output chunks j = g, g + S, ...."""
    from layer_mhc_seam_amd.seam import stream_mix
    g = torch.Generator(device="cuda").manual_seed(rd + wr)
    src = torch.randint(0, 1 << 30, (max(rd, 16) // 4,), generator=g, device="cuda",
                        dtype=torch.int32)
    dst = torch.zeros(wr // 4, dtype=torch.int32, device="cuda")
    stream_mix(dst, wr, src, rd)
    torch.cuda.synchronize()
    n_in, n_out = rd // 16, wr // 16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = 256 * min(cus, -(-max(n_in, n_out) // 256))
    acc = np.zeros((S, 4), np.uint32)
    acc[:, 0] = np.arange(S, dtype=np.uint32)
    acc[:, 1] = ~np.arange(S, dtype=np.uint32)
    s = src.cpu().numpy().view(np.uint32)[: rd // 4].reshape(-1, 4)
    for i0 in range(0, n_in, S):
        blk = s[i0:i0 + S]
        acc[:blk.shape[0]] ^= blk
    j = np.arange(n_out)
    want = acc[j % S].copy()
    want[:, 0] ^= j.astype(np.uint32)
    assert np.array_equal(dst.cpu().numpy().view(np.uint32).reshape(-1, 4), want)
