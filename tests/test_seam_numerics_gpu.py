"""GPU parity of the parts of the seam that unit-scale inputs at the default
settings cannot see: the Sinkhorn iteration count, and RMSNorm's epsilon.

* The gates' tolerance (1e-3) cannot tell 20 Sinkhorn iterations from 19 or
  21 on ordinary logits, which converge fast.  So the seam runs at 1, 2 and
  3 iterations against the oracle at the same count, in every launch mode
  (split, whole-row, whole-row plus split tail); and with fn = 0 and res
  logits crafted in bias (block-triangular, no doubly stochastic scaling,
  convergence like 1/n) its res_out is compared with the closed form at
  1, 2, 3 and the default 20 iterations at a bar (2e-5) far below the 1e-3
  step between 20 and 21.
* Tokens with a mean square near or below eps (x, y scaled by 2^-10, 2^-12)
  and zero tokens, in both forms and every launch mode.  A CPU test
  (test_eps_regime_cases) shows the same cases fail a seam whose epsilon is
  outside the root.

The iteration count and eps come from "[FlyDSL] Single-launch Mega-mHC on
gfx950", Kernel Architecture (rstd -> Sinkhorn) and the seam's definition
(20-iteration Sinkhorn, RMSNorm eps 1e-6).
"""
import numpy as np
import pytest
import torch

from seam_harness import (check_all, eps_regime_case, host_case, make_seam, run_gpu,
                          run_oracle)
from test_oracle_pins import triangular_block_closed_form, triangular_block_logits

pytestmark = pytest.mark.gpu

H = 5120
# T -> launch mode at H = 5120 on 256 CUs: split (several splits per block),
# whole-row (129 blocks > 128), whole-row plus a split tail (260 = 256 + 4)
PLANS = {40: "split", 2064: "whole_row", 4160: "whole_row_plus_split_tail"}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_plan(T, mode):
    from layer_mhc_seam_amd.seam import plan
    p = plan(H, T)
    if mode == "split":
        assert p["row_segs"] == 0 and p["ksplit"] > 1
    elif mode == "whole_row":
        assert p["row_segs"] > 0 and p["rows_blocks"] == p["grid"]
    else:
        assert p["row_segs"] > 0 and 0 < p["rows_blocks"] < p["blocks"]


@pytest.mark.parametrize("T", sorted(PLANS))
@pytest.mark.parametrize("iters", [1, 2, 3])
def test_sinkhorn_iteration_counts(T, iters):
    _check_plan(T, PLANS[T])
    c = host_case(T, H, seed=40 + T)
    s = make_seam(c, T, sinkhorn_iters=iters)
    got = run_gpu(s, c, "post", False, "bf16")
    check_all(got, run_oracle(c, iters=iters), "post", "bf16")
    s.close()


BLOCKS = [(1.0, 1.0, 3.0), (2.0, 0.25, 5.0)]


@pytest.mark.parametrize("T", [4, 40, 2064])
@pytest.mark.parametrize("iters", [1, 2, 3, 0])
def test_sinkhorn_closed_form_through_bias(T, iters):
    """fn = 0: every logit equals its bias, so res_out is the closed form of
    the block-triangular logits at the seam's iteration count (0 selects
    the default, 20), and pre_out / post_out are sigma / 2 sigma of bias."""
    n = iters or 20
    c = host_case(T, H, seed=50 + T)
    c["fn"] = np.zeros((4 * H, 24), np.float32)
    bias = np.zeros(24, np.float32)
    bias[:8] = np.linspace(-2, 2, 8)
    bias[8:] = triangular_block_logits(BLOCKS).reshape(16)
    c["bias"] = bias
    s = make_seam(c, T, sinkhorn_iters=iters)
    got = run_gpu(s, c, "post", False, "bf16")
    want = np.broadcast_to(triangular_block_closed_form(BLOCKS, n), (T, 4, 4))
    err = np.abs(got["res_out"].astype(np.float64) - want).max()
    assert err <= 2e-5, f"res_out off the {n}-iteration closed form by {err}"
    # one iteration more or fewer moves M[0][1] by more than 1e-3 at n = 20
    step = abs(triangular_block_closed_form(BLOCKS, n + 1) - triangular_block_closed_form(
        BLOCKS, n)).max()
    assert step > 50 * 2e-5
    sig = 1.0 / (1.0 + np.exp(-bias[:8].astype(np.float64)))
    np.testing.assert_allclose(got["pre_out"], np.broadcast_to(sig[:4], (T, 4)), atol=2e-7)
    np.testing.assert_allclose(got["post_out"], np.broadcast_to(2 * sig[4:], (T, 4)), atol=4e-7)
    check_all(got, run_oracle(c, iters=n), "post", "bf16")
    s.close()


@pytest.mark.parametrize("T", sorted(PLANS))
@pytest.mark.parametrize("form", ["post", "no_post"])
def test_eps_regime_tokens(T, form):
    """Tokens at mean squares ~1, ~1e-6 (= eps), ~6e-8 and 0: the norm and
    the gates depend on where eps enters both rstd's."""
    _check_plan(T, PLANS[T])
    c = eps_regime_case(T, H, seed=60 + T)
    s = make_seam(c, T)
    got = run_gpu(s, c, form, False, "mxfp8")
    check_all(got, run_oracle(c, form), form, "mxfp8")
    z = np.arange(3, T, 4)     # signed zeros in, signed zeros out
    assert not (got["norm"][z] & 0x7FFF).any(), "zero tokens must give a zero norm"
    s.close()


def test_eps_regime_decode():
    """The decode instance (T <= 8: token half 0 only) with tokens at every
    scale."""
    c = eps_regime_case(8, H, seed=68)
    s = make_seam(c, 8)
    for form in ("post", "no_post"):
        got = run_gpu(s, c, form, False, "fp8_grid")
        check_all(got, run_oracle(c, form), form, "fp8_grid")
    s.close()
