"""The device quantiser (shared by the seam and mhc_seam_quantize) against
the oracle's quantiser, bit for bit: every finite bf16 value at every scale
exponent k it can meet (|v| <= 448 * 2^k), with each group's amax pinned to
the top of k's range so that k is the one intended.  Per-32 ue8m0 + e4m3fn
as in "[FlyDSL] Single-launch Mega-mHC on gfx950", Kernel Architecture
(out_dtype) and Test Plan (crafted quantiser groups)."""
import numpy as np
import pytest
import torch

import oracle
from bits import bf16_to_f32, exact_bf16
from seam_harness import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def exhaustive_groups():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f32(b).astype(np.float64)
    finite = np.isfinite(vals)
    groups = []
    for k in range(-127, 121):
        top = 448.0 * 2.0 ** k
        amax = exact_bf16([top])[0] if k < 120 else np.uint16(0x7F7F)
        amax_v = float(bf16_to_f32(np.array([amax]))[0])
        sel = b[finite & (np.abs(vals) <= amax_v)]
        n = (len(sel) + 30) // 31
        body = np.resize(sel, n * 31).reshape(n, 31)
        groups.append(np.concatenate([np.full((n, 1), amax, np.uint16), body], axis=1))
    g = np.concatenate(groups)
    H = 5120
    per_row = H // 32
    rows = (len(g) + per_row - 1) // per_row
    g = np.resize(g, (rows * per_row, 32))
    return g.reshape(rows, H)


def test_quantiser_exhaustive_against_oracle():
    from layer_mhc_seam_amd.seam import quantize
    norm = exhaustive_groups()
    codes, scales, grid = quantize(to_dev(norm))
    torch.cuda.synchronize()
    codes, scales, grid = to_host(codes), to_host(scales), to_host(grid)
    oc, os_, og = oracle.quantize(norm)
    assert np.array_equal(scales, os_), "scales differ"
    bad = np.argwhere(codes != oc)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {[(hex(norm[r, c]), hex(codes[r, c]), hex(oc[r, c])) for r, c in bad[:5]]}"
    bad = np.argwhere(grid != og)
    assert len(bad) == 0, f"{len(bad)} grid values differ, first {[(hex(norm[r, c]), hex(grid[r, c]), hex(og[r, c])) for r, c in bad[:5]]}"


@pytest.mark.parametrize("rows,H", [(1, 64), (3, 128), (9, 5120), (17, 192)])
def test_quantize_ragged_shapes(rows, H):
    from layer_mhc_seam_amd.seam import quantize
    rng = np.random.default_rng(rows)
    norm = oracle.f32_to_bf16((rng.standard_normal((rows, H)) *
                               np.exp(rng.standard_normal((rows, 1)) * 5)).astype(np.float32))
    codes, scales, grid = quantize(to_dev(norm))
    torch.cuda.synchronize()
    oc, os_, og = oracle.quantize(norm)
    assert np.array_equal(to_host(codes), oc)
    assert np.array_equal(to_host(scales), os_)
    assert np.array_equal(to_host(grid), og)


def test_quantiser_g128_exhaustive_values_against_oracle():
    """The same exhaustive set of values laid out in 128-wide groups: each
    group is four of the 32-element groups above, so its scale is the
    largest of theirs and every value meets k's it can meet."""
    from layer_mhc_seam_amd.seam import quantize
    norm = exhaustive_groups()
    codes, scales, grid = quantize(to_dev(norm), group=128)
    torch.cuda.synchronize()
    oc, os_, og = oracle.quantize(norm, 128)
    assert np.array_equal(to_host(scales), os_), "scales differ"
    assert np.array_equal(to_host(codes), oc), "codes differ"
    assert np.array_equal(to_host(grid), og), "grid differs"


@pytest.mark.parametrize("rows,H", [(1, 128), (3, 256), (9, 5120), (17, 384)])
def test_quantize_g128_ragged_shapes(rows, H):
    from layer_mhc_seam_amd.seam import quantize
    rng = np.random.default_rng(rows + 100)
    norm = oracle.f32_to_bf16((rng.standard_normal((rows, H)) *
                               np.exp(rng.standard_normal((rows, H // 32, 1)) * 5)
                               .repeat(32, axis=-1).reshape(rows, H)).astype(np.float32))
    codes, scales, grid = quantize(to_dev(norm), group=128)
    torch.cuda.synchronize()
    oc, os_, og = oracle.quantize(norm, 128)
    assert np.array_equal(to_host(codes), oc)
    assert np.array_equal(to_host(scales), os_)
    assert np.array_equal(to_host(grid), og)


def test_quantize_rejects_bad_groups():
    from layer_mhc_seam_amd.seam import SeamError, quantize
    src = torch.zeros((2, 192), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(SeamError):
        quantize(src, group=128)                     # 192 is not a multiple of 128
    with pytest.raises(SeamError):
        quantize(src, group=64)
