"""GPU parity of the unshifted ordering against the oracle: gates from x'
first, then the collapse with the fresh pre ("[FlyDSL] Single-launch
Mega-mHC on gfx950", Test Result, the notes on what each compared kernel
computes).  The library runs it as two launches (post-mix and gates, then
collapse, RMSNorm and quantiser over the stored x').

Two checks per case:
  * the strict one: the GPU norm is the delayed seam's norm (oracle) with
    the carried pre replaced by the GPU's own pre_out, at the seam's usual
    bar (<= 1 bf16 ulp on >= 99.99%, <= 2 ulp everywhere): the collapse must
    use exactly the gates the first launch wrote;
  * end to end against the oracle's unshifted seam: residual bitwise, gates
    within 1e-3, and every norm element within 2 ulp or, where it is not,
    within 1e-4 of its token's norm RMS.  The oracle's fresh pre is fp64;
    the GPU's comes from fp32 MFMA dots and differs by ~1e-7, far inside the
    gate tolerance.  That moves u across a bf16 rounding boundary now and
    then (up to 2 ulp of the norm), and where the four streams cancel (u
    near 0) the same absolute difference is many ulp of a tiny value.
"""
import numpy as np
import pytest
import torch

from bits import bf16_to_f32, ulp_diff
from seam_harness import (check_bf16, check_gates, check_quant, dev_inputs, host_case,
                          make_seam, run_gpu, run_oracle, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_unshifted(got, c, form, out, idx=None):
    sub = got if idx is None else {k: v[idx] for k, v in got.items()}
    want = run_oracle(c, form, idx=idx, unshifted=True)
    if form == "post":
        check_bf16("residual_out", sub["residual_out"], want["residual_out"], bitwise=True)
    check_gates(sub, want)
    d = ulp_diff(sub["norm"], want["norm"])
    g, w = bf16_to_f32(sub["norm"]).astype(np.float64), bf16_to_f32(want["norm"]).astype(np.float64)
    rms = np.sqrt((w * w).mean(axis=-1, keepdims=True))
    bad = (d > 2) & (np.abs(g - w) > 1e-4 * rms)
    assert not bad.any(), f"norm: {int(bad.sum())} elements beyond 2 ulp and 1e-4 x rms"
    if out != "bf16":
        check_quant(got, out)
    again = run_oracle(c, form, idx=idx, pre=sub["pre_out"])
    return check_bf16("norm with the GPU's fresh pre", sub["norm"], again["norm"])


@pytest.mark.parametrize("form", ["post", "no_post"])
@pytest.mark.parametrize("out", ["bf16", "fp8_grid", "mxfp8"])
@pytest.mark.parametrize("ksplit", [0, 1])
def test_unshifted_forms_and_outputs(form, out, ksplit):
    """Split plans (ksplit 0 at this size) and whole-row plans (ksplit 1),
    whose second launch is the collapse-only kernel."""
    c = host_case(40, 512, seed=31)
    s = make_seam(c, 40, ksplit=ksplit)
    got = run_gpu(s, c, form, False, out, unshifted=True)
    check_unshifted(got, c, form, out)


@pytest.mark.parametrize("T", [1, 17, 100, 384])
def test_unshifted_split_mode(T):
    c = host_case(T, 5120, seed=32 + T)
    s = make_seam(c, T)
    got = run_gpu(s, c, "post", False, "mxfp8", unshifted=True)
    check_unshifted(got, c, "post", "mxfp8")


@pytest.mark.parametrize("ksplit,spin", [(40, 0), (40, -1), (3, 0), (1, 0)])
def test_unshifted_split_paths(ksplit, spin):
    """Waiting splits, splits that all hand off, LDS-resident u, whole rows."""
    c = host_case(64, 5120, seed=40 + ksplit)
    s = make_seam(c, 64, ksplit=ksplit, spin_polls=spin)
    for _ in range(2):
        got = run_gpu(s, c, "post", False, "fp8_grid", unshifted=True)
        check_unshifted(got, c, "post", "fp8_grid")


@pytest.mark.parametrize("T,form,out", [(4160, "no_post", "bf16"), (5120, "post", "mxfp8")])
def test_unshifted_tail_wave(T, form, out):
    """Whole-row launches with a split tail: in the same launch (T = 4160)
    and in a split launch after each of the two passes (T = 5120)."""
    c = host_case(T, 5120, seed=45, y_boost_every=64 if out == "mxfp8" else 0)
    s = make_seam(c, T)
    got = run_gpu(s, c, form, False, out, unshifted=True)
    check_unshifted(got, c, form, out)


def test_unshifted_prefill16k_sampled():
    T = 16384
    c = host_case(T, 5120, seed=46)
    s = make_seam(c, T)
    got = run_gpu(s, c, "post", False, "fp8_grid", unshifted=True)
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([np.arange(16), np.arange(T - 16, T),
                                    rng.choice(T, 96, replace=False)]))
    check_unshifted(got, c, "post", "fp8_grid", idx=idx)
    s.close()


def test_unshifted_graph_replays_match_eager():
    c = host_case(384, 5120, seed=47, y_boost_every=64)
    s = make_seam(c, 384)
    d = dev_inputs(c, unshifted=True)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = {k: v.clone() for k, v in
                 s.run(out_dtype="mxfp8", unshifted=True, **d, stream=stream).items()}
        out = {k: torch.empty_like(v) for k, v in eager.items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        s.run(out_dtype="mxfp8", unshifted=True, **d, out=out, stream=stream)
    for _ in range(3):
        for v in out.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(eager[k].view(torch.uint8), out[k].view(torch.uint8)), k
    check_unshifted({k: to_host(v) for k, v in eager.items()}, c, "post", "mxfp8")


def test_unshifted_g128_fused_whole_row():
    """The second launch quantises 128-wide groups in its whole-row finish."""
    c = host_case(3000, 5120, seed=48)
    s = make_seam(c, 3000)
    got = run_gpu(s, c, "post", False, "mxfp8_g128", unshifted=True)
    check_unshifted(got, c, "post", "mxfp8_g128")
