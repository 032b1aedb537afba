"""mhc_seam_run_noalloc, the entry point that allocates nothing, against
mhc_seam_run.

It runs the same kernels; only its split-mode scratch differs (the
library's fixed per-GPU array instead of per-stream allocations).  So its
outputs must equal mhc_seam_run's bit for bit on the same inputs, which is
stricter than the parity bar both are held to against the oracle.  Two and
more calls in a row, each smaller than the one before, also check that the
array's sync words stay valid from call to call.
"""
import numpy as np
import pytest
import torch

from seam_harness import check_all, dev_inputs, host_case, make_seam, run_oracle, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs_like(o):
    return {k: torch.empty_like(v) for k, v in o.items()}


def _same(a, b):
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


def _pair(s, c, out_dtype, form="post"):
    """(mhc_seam_run outputs, mhc_seam_run_noalloc outputs) on case c."""
    d = dev_inputs(c, form)
    ref = s.run(**d, form=form, out_dtype=out_dtype)
    out = _outputs_like(ref)
    s.run(**d, form=form, out_dtype=out_dtype, out=out, noalloc=True)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_run_on_shrinking_calls():
    """Calls in a row, each smaller than the last: a whole-row launch with
    its tail's splits in a launch after it (T = 5120), a whole-row launch
    with the tail's splits in it (4160), split launches (384, 40) and the
    decode instance (4).  Every output equals mhc_seam_run's, and the
    first, second and last also meet the oracle bar."""
    H = 5120
    cases = {T: host_case(T, H, seed=100 + T, y_boost_every=64) for T in (5120, 4160, 384, 40, 4)}
    for c in cases.values():
        c.update(fn=cases[5120]["fn"], gamma=cases[5120]["gamma"], bias=cases[5120]["bias"])
    s = make_seam(cases[5120], 5120)
    for T, out_dtype in ((5120, "fp8_grid"), (4160, "mxfp8"), (384, "mxfp8"), (40, "fp8_grid"),
                         (4, "bf16")):
        ref, got = _pair(s, cases[T], out_dtype)
        _same(ref, got)
        if T in (5120, 4160, 4):
            check_all({k: to_host(v) for k, v in got.items()}, run_oracle(cases[T]), "post",
                      out_dtype)
    s.close()


def test_noalloc_other_width_and_no_post():
    """A width whose launches are all split (H = 7168: every split hands its
    u over through the array) in the no_post form, then a smaller T, then
    the limit: a T whose u does not fit the array is refused."""
    from layer_mhc_seam_amd.seam import INVALID_ARG, SeamError
    H = 7168
    c = host_case(1500, H, seed=110)
    s = make_seam(c, 4000)
    for T in (1500, 300):
        sub = {k: (v[:T] if k in ("x", "y", "pre", "post", "res") else v) for k, v in c.items()}
        ref, got = _pair(s, sub, "bf16", form="no_post")
        _same(ref, got)
    check_all({k: to_host(v) for k, v in got.items()},
              run_oracle({k: (v[:300] if k in ("x", "y", "pre", "post", "res") else v)
                          for k, v in c.items()}, "no_post"), "no_post", "bf16")
    big = host_case(4000, H, seed=111)
    big.update(fn=c["fn"], gamma=c["gamma"], bias=c["bias"])
    with pytest.raises(SeamError) as ei:
        s.run(**dev_inputs(big, "no_post"), form="no_post", noalloc=True)
    assert ei.value.status == INVALID_ARG and "no-allocation" in str(ei.value)
    s.close()


def test_noalloc_is_capturable_on_a_fresh_stream():
    """No eager call is needed before capture (nothing to allocate); graph
    replays equal the eager mhc_seam_run result."""
    c = host_case(384, 5120, seed=120, y_boost_every=64)
    s = make_seam(c, 384)
    d = dev_inputs(c)
    ref = {k: v.clone() for k, v in s.run(**d, out_dtype="mxfp8").items()}
    out = _outputs_like(ref)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        s.run(**d, out_dtype="mxfp8", out=out, stream=stream, noalloc=True)
    for _ in range(3):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(ref, out)
    del g
    s.close()
