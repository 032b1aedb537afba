"""GPU parity of the n -> 1 head reduce (mhc_head_reduce) against the oracle.

The reading ("[Triton/Gluon] [gfx950] [dsv4.1-flash] mHC fused kernel",
description, names an HC head reduce/store kernel and no more): the seam's
collapse chain on its own, bf16(sum_i w_i x_i) in binary32 with fused
multiply-adds in stream order.  Both sides evaluate the same chain, so the
bar is bitwise equality.
"""
import numpy as np
import pytest
import torch

import oracle
from bits import bf16_to_f32
from seam_harness import host_case, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_head_reduce(x, w, **kw):
    from layer_mhc_seam_amd.seam import head_reduce
    out = head_reduce(to_dev(x), None if w is None else to_dev(w), **kw)
    torch.cuda.synchronize()
    return to_host(out)


def assert_bitwise(got, want):
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} elements differ, first at {list(zip(*bad))[:6]}"


# H: one chunk per lane and less, a ragged last pass over the lanes, the
# seam's widths; T: single tokens, a ragged last workgroup, several rounds
# of the grid
@pytest.mark.parametrize("T,H", [(1, 8), (3, 136), (7, 512), (5, 1000), (64, 5120),
                                 (130, 7168), (2049, 512)])
@pytest.mark.parametrize("weights", ["pre", "identity"])
def test_head_reduce_matches_oracle(T, H, weights):
    c = host_case(T, H, seed=60 + T)
    w = c["pre"] if weights == "pre" else None
    assert_bitwise(gpu_head_reduce(c["x"], w), oracle.head_reduce(c["x"], w))


def test_head_reduce_signed_and_zero_weights():
    """Negative, zero and large weights (the chain's products and sums in
    every sign combination), and tokens whose weights are all zero."""
    T, H = 40, 512
    c = host_case(T, H, seed=70)
    rng = np.random.default_rng(71)
    w = (rng.standard_normal((T, 4)) * 3).astype(np.float32)
    w[::7] = 0.0
    w[3] = [1e30, -1e30, 1.0, 0.5]
    got = gpu_head_reduce(c["x"], w)
    assert_bitwise(got, oracle.head_reduce(c["x"], w))
    assert (bf16_to_f32(got[::7]) == 0).all()          # +0 or -0 (0 times a negative)


def test_head_reduce_prefill16k_sampled():
    """T = 16384, H = 5120 in the benchmark's launch; sampled rows against
    the oracle, including the first and last workgroups."""
    T, H = 16384, 5120
    c = host_case(T, H, seed=72)
    got = gpu_head_reduce(c["x"], c["pre"])
    rng = np.random.default_rng(2)
    idx = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T),
                                    rng.choice(T, 48, replace=False)]))
    assert_bitwise(got[idx], oracle.head_reduce(c["x"][idx], c["pre"][idx]))


def test_head_reduce_empty_and_given_output():
    from layer_mhc_seam_amd.seam import head_reduce
    x = torch.zeros((0, 4, 512), dtype=torch.bfloat16, device="cuda")
    assert head_reduce(x).shape == (0, 512)
    c = host_case(9, 256, seed=73)
    out = torch.full((9, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    r = head_reduce(to_dev(c["x"]), to_dev(c["pre"]), out=out)
    torch.cuda.synchronize()
    assert r.data_ptr() == out.data_ptr()
    assert_bitwise(to_host(out), oracle.head_reduce(c["x"], c["pre"]))


def test_head_reduce_rejects_bad_tensors():
    from layer_mhc_seam_amd.seam import head_reduce
    x = torch.zeros((4, 4, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        head_reduce(x.float())
    with pytest.raises(ValueError):
        head_reduce(x, torch.zeros((4, 3), device="cuda"))
    with pytest.raises(RuntimeError):
        head_reduce(torch.zeros((4, 4, 12), dtype=torch.bfloat16, device="cuda"))


def test_head_reduce_graph_replays_match_eager():
    from layer_mhc_seam_amd.seam import head_reduce
    c = host_case(300, 5120, seed=74)
    x, w = to_dev(c["x"]), to_dev(c["pre"])
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = head_reduce(x, w, stream=stream).clone()
        out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        head_reduce(x, w, out=out, stream=stream)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    assert_bitwise(to_host(eager), oracle.head_reduce(c["x"], c["pre"]))
