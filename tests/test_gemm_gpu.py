"""GPU parity of the MXFP8 consumer GEMM (mhc_mxfp8_gemm) against the oracle.

Reading ("[FlyDSL] Single-launch Mega-mHC on gfx950", Kernel Architecture
and Test Result: the ue8m0/e4m3 norm feeds the next layer's GEMM): both
operands MXFP8 along K, out = bf16(a b^T).  The oracle evaluates the exact
sum in binary64.

The GPU's arithmetic is gfx950's block-scaled MFMA, which does not add its
128 products exactly: a one-instruction probe of a 16 x 16 x 128 tile gives
the GEMM kernel's bits exactly, and both differ from the exact sum on a few
per cent of the elements.  A model that aligns each group of 8 products to
the largest of them and keeps 14 fraction bits (truncating) reproduces
98-99% of the bits.  The bar is the worst case of that alignment over a
128-wide step, 128 * 2^-14 * max |a b|, summed over the K / 128 steps and
bounded by K * 2^-14 * max_k |a| * max_k |b|, plus half a bf16 ulp of the
result (doubled):
    |gpu - exact| <= 2^-8 |exact| + K 2^-14 max|a[t, :]| max|b[n, :]|,
and at least 90% of the elements equal to bf16(exact) (96-99% measured).

Extreme scales: the instruction adds the two scale exponents before scaling
(bytes 0 / 254 are exact), keeps binary32 subnormals, overflows to +-inf
when partial sums leave binary32's range, and reads the scale byte 0xff as
NaN, the OCP MX definition the oracle follows.
"""
import numpy as np
import pytest
import torch

import oracle
from bits import bf16_to_f32
from seam_harness import check_quant, dev_inputs, host_case, make_seam, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


FINITE = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], np.uint8)


def mx_operands(T, N, K, seed, scale_lo=122, scale_hi=133):
    rng = np.random.default_rng(seed)
    a = rng.choice(FINITE, (T, K))
    b = rng.choice(FINITE, (N, K))
    sa = rng.integers(scale_lo, scale_hi, (T, K // 32)).astype(np.uint8)
    sb = rng.integers(scale_lo, scale_hi, (N, K // 32)).astype(np.uint8)
    return a, sa, b, sb


def gpu_gemm(a, sa, b, sb, **kw):
    from layer_mhc_seam_amd.seam import mxfp8_gemm
    out = mxfp8_gemm(to_dev(a), to_dev(sa), to_dev(b), to_dev(sb), **kw)
    torch.cuda.synchronize()
    return to_host(out)


def row_max(codes, scales):
    """max_k |value| per row of an MXFP8 operand (torch's float8_e4m3fn decode)."""
    v = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = v * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    return np.abs(v).max(axis=1)


def check_gemm(got_bits, want, a, sa, b, sb):
    K = a.shape[1]
    got = bf16_to_f32(got_bits).astype(np.float64)
    bound = 2.0 ** -8 * np.abs(want) + K * 2.0 ** -14 * np.outer(row_max(a, sa), row_max(b, sb))
    err = np.abs(got - want)
    bad = np.nonzero(err > bound)
    assert bad[0].size == 0, (f"{bad[0].size} elements beyond the bound, first at "
                              f"{list(zip(*bad))[:4]}: got {got[bad][:4]}, want {want[bad][:4]}")
    same = (got_bits == oracle.f32_to_bf16(want.astype(np.float32))).mean()
    assert same >= 0.90, f"only {same:.4f} equal to bf16(exact)"
    return same


@pytest.mark.parametrize("T,N,K", [(1, 16, 128), (17, 64, 256), (4, 5120, 5120), (16, 200, 640),
                                   (32, 300, 2048), (64, 5120, 1024), (33, 100, 8192),
                                   (130, 200, 384),
                                   (300, 128, 1024), (129, 129, 128), (256, 384, 5120),
                                   # ragged row and column blocks in several groups of
                                   # the block order, the last group partial
                                   (600, 300, 512), (1100, 260, 256),
                                   (2100, 300, 384), (4096, 517, 640),
                                   # more 128 x 128 blocks than CUs, one round of
                                   # 128 x 256 blocks
                                   (2100, 2000, 256), (1030, 4100, 128),
                                   # more weight columns than one round of the
                                   # smallest blocks covers, ragged last columns
                                   (4, 8200, 256), (20, 8200, 384),
                                   # 64 x 64, 128 x 64 and 128 x 128 blocks in one round
                                   (150, 3000, 256), (300, 3000, 256), (300, 5000, 384),
                                   (512, 5120, 256)])
def test_gemm_matches_oracle(T, N, K):
    a, sa, b, sb = mx_operands(T, N, K, seed=T + N + K)
    want, _ = oracle.mxfp8_gemm(a, sa, b, sb)
    check_gemm(gpu_gemm(a, sa, b, sb), want, a, sa, b, sb)


def test_gemm_consumes_the_seam_output():
    """The seam's mxfp8 codes and scales, as written, are the GEMM's A
    operand: the GPU chain seam -> GEMM against the oracle GEMM of the
    same codes and scales (themselves checked against the oracle quantiser
    of the GPU norm)."""
    T, H, N = 384, 5120, 256
    c = host_case(T, H, seed=80, y_boost_every=64)
    s = make_seam(c, T)
    o = s.run(**dev_inputs(c), out_dtype="mxfp8")
    torch.cuda.synchronize()
    got = {k: to_host(v) for k, v in o.items()}
    check_quant(got, "mxfp8")
    _, _, b, sb = mx_operands(1, N, H, seed=81)
    from layer_mhc_seam_amd.seam import mxfp8_gemm
    out = mxfp8_gemm(o["codes"], o["scales"], to_dev(b), to_dev(sb))
    torch.cuda.synchronize()
    want, _ = oracle.mxfp8_gemm(got["codes"], got["scales"], b, sb)
    check_gemm(to_host(out), want, got["codes"], got["scales"], b, sb)
    s.close()


def test_gemm_large_sampled():
    """T = 16384 activations against 512 weight rows at K = 5120; the oracle
    recomputes sampled rows, including the first and last row blocks."""
    T, N, K = 16384, 512, 5120
    a, sa, b, sb = mx_operands(T, N, K, seed=82)
    got = gpu_gemm(a, sa, b, sb)
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([np.arange(4), np.arange(T - 4, T),
                                    rng.choice(T, 40, replace=False)]))
    want, _ = oracle.mxfp8_gemm(a[idx], sa[idx], b, sb)
    check_gemm(got[idx], want, a[idx], sa[idx], b, sb)


@pytest.mark.parametrize("T,N,K", [(16000, 2044, 256), (16384, 2048, 256), (12288, 2560, 128),
                                   (4100, 5110, 256)])
def test_gemm_large_tiles_sampled(T, N, K):
    """Shapes with enough blocks that the launch takes the 256 x 256 blocks
    (chosen when their rounds of the CUs cost less than those of 128 x 128
    blocks two per CU), and one (4100 x 5110) that takes the latter: ragged
    last row and column blocks, N not a multiple of 8, several XCD groups of
    the block order.  The oracle recomputes sampled rows, including the
    first and last row blocks."""
    a, sa, b, sb = mx_operands(T, N, K, seed=T + N + K)
    got = gpu_gemm(a, sa, b, sb)
    rng = np.random.default_rng(T)
    idx = np.unique(np.concatenate([np.arange(4), np.arange(252, 260), np.arange(T - 12, T),
                                    rng.choice(T, 40, replace=False)]))
    want, _ = oracle.mxfp8_gemm(a[idx], sa[idx], b, sb)
    check_gemm(got[idx], want, a[idx], sa[idx], b, sb)


# (T, N, K) taking each launch instance: 16 x 32, 32 x 32, 64 x 32, 64 x 64,
# 128 x 64 and 128 x 128 blocks in one round, 128 x 256 blocks, 16 x 32 and
# 32 x 32 blocks in more than one round (128 x 128 blocks two per CU and
# 256 x 256 blocks: the sampled tests further down)
INSTANCE_SHAPES = [(12, 48, 256), (32, 5120, 256), (64, 5120, 256), (150, 3000, 256),
                   (300, 5000, 256), (512, 5120, 256), (2100, 2000, 256), (8, 8200, 256),
                   (20, 16400, 128)]


@pytest.mark.parametrize("T,N,K", INSTANCE_SHAPES)
def test_gemm_nan_code_propagates(T, N, K):
    a, sa, b, sb = mx_operands(T, N, K, seed=83)
    a[5, 77] = 0x7f
    got = bf16_to_f32(gpu_gemm(a, sa, b, sb))
    assert np.isnan(got[5]).all()
    assert not np.isnan(np.delete(got, 5, axis=0)).any()


def _full(v, r, K):
    return np.full((r, K // 32), v, np.uint8)


@pytest.mark.parametrize("T,N,K", [(48, 40, 256), (100, 40, 512), (20, 8200, 256),
                                   (150, 3000, 256), (300, 5000, 256)])
@pytest.mark.parametrize("sa,sb", [(0, 254), (254, 0), (1, 253), (2, 252), (57, 57)])
def test_gemm_extreme_scale_bytes(sa, sb, T, N, K):
    """Scale bytes at both ends of the ue8m0 range.  The block-scaled MFMA
    adds the two exponents before it scales, so 0 / 254 and 1 / 253 give the
    results of 127 / 127 with no intermediate underflow; 57 / 57 (2^-140)
    puts every result among binary32's subnormals, which are kept, not
    flushed.  All within the usual bar of the exact sum."""
    a, _, b, _ = mx_operands(T, N, K, seed=85)
    A, B = _full(sa, T, K), _full(sb, N, K)
    want, _ = oracle.mxfp8_gemm(a, A, b, B)
    check_gemm(gpu_gemm(a, A, b, B), want, a, A, b, B)


@pytest.mark.parametrize("T,N,K", [(64, 48, 256), (130, 48, 256), (130, 48, 512),
                                   (20, 8200, 256), (300, 5000, 256)])
def test_gemm_binary32_overflow(T, N, K):
    """Scales of 2^55 each push results up to the top of binary32.  The
    accumulator is binary32, so an output is +-inf only where its partial
    sums can leave that range (sum_k |a b| >= 2^127); every finite output is
    within the bar, and outputs whose exact value overflows bf16 are inf of
    the right sign."""
    a, _, b, _ = mx_operands(T, N, K, seed=86)
    A, B = _full(182, T, K), _full(182, N, K)
    want, absum = oracle.mxfp8_gemm(a, A, b, B)
    got = bf16_to_f32(gpu_gemm(a, A, b, B)).astype(np.float64)
    inf = ~np.isfinite(got)      # +-inf, or NaN where partial sums of both signs overflow
    assert inf.any() and (~inf).any()
    assert np.all(absum[inf] >= 2.0 ** 127)
    over = np.abs(want) >= 2.0 ** 128
    assert np.all(inf[over])
    # the sign is the exact sum's wherever the terms of the other sign cannot
    # take a partial sum out of range the other way (their total < 2^127)
    va = torch.from_numpy(a.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vb = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ap, an, bp, bn = (np.maximum(va, 0), np.maximum(-va, 0), np.maximum(vb, 0),
                      np.maximum(-vb, 0))
    f = 2.0 ** (2 * (182 - 127))
    pos, neg = (ap @ bp.T + an @ bn.T) * f, (ap @ bn.T + an @ bp.T) * f
    against = np.where(want > 0, neg, pos)
    signed = over & np.isinf(got) & (against < 2.0 ** 127)
    assert signed.any()
    assert np.all(np.sign(got[signed]) == np.sign(want[signed]))
    bound = 2.0 ** -8 * np.abs(want) + K * 2.0 ** -14 * np.outer(row_max(a, A), row_max(b, B))
    assert np.all(np.abs(got[~inf] - want[~inf]) <= bound[~inf])


@pytest.mark.parametrize("T,N,K", INSTANCE_SHAPES)
def test_gemm_scale_ff_is_nan(T, N, K):
    """OCP MX defines the E8M0 byte 0xff as NaN: a 0xff activation scale
    makes its output row NaN and a 0xff weight scale its column, even over
    zero codes, as in the oracle; every other output is unchanged."""
    a, sa, b, sb = mx_operands(T, N, K, seed=87)
    a[7, 64:96] = 0
    sa[7, 2] = 0xFF
    sb[5, 0] = 0xFF
    got = bf16_to_f32(gpu_gemm(a, sa, b, sb))
    want, _ = oracle.mxfp8_gemm(a, sa, b, sb)
    nan = np.isnan(want)
    assert nan[7].all() and nan[:, 5].all() and nan.sum() == N + T - 1
    assert np.array_equal(np.isnan(got), nan)
    keep = np.ones(T, bool)
    keep[7] = False
    cols = np.delete(np.arange(N), 5)
    check_gemm(gpu_gemm(a[keep], sa[keep], b[cols], sb[cols]), want[keep][:, cols], a[keep],
               sa[keep], b[cols], sb[cols])


@pytest.mark.parametrize("T,N,K", [(16384, 2048, 256), (4096, 5120, 256), (1500, 4000, 256)])
def test_gemm_large_tiles_special_values_sampled(T, N, K):
    """The 256 x 256 kernel (16384 x 2048), the 128 x 128 blocks two per CU
    (4096 x 5120) and the 128 x 256 blocks (1500 x 4000) with a NaN code, a
    0xff activation scale and a 0xff weight scale: the NaN rows and column,
    and sampled rows against the oracle."""
    r0, r1 = 3 * T // 16, 9 * T // 16
    a, sa, b, sb = mx_operands(T, N, K, seed=88)
    a[r0, 17] = 0x7f            # NaN code: row r0
    sa[r1, 5] = 0xFF            # NaN scale: row r1
    sb[1500, 2] = 0xFF          # NaN scale: column 1500
    bits = gpu_gemm(a, sa, b, sb)
    got = bf16_to_f32(bits)
    for row in (r0, r1):
        assert np.isnan(got[row]).all()
    assert np.isnan(got[:, 1500]).all()
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([[0, 255, 256, r0, r1, T - 1],
                                    rng.choice(T, 24, replace=False)]))
    want, _ = oracle.mxfp8_gemm(a[idx], sa[idx], b, sb)
    assert np.array_equal(np.isnan(got[idx]), np.isnan(want))
    ok = ~np.isin(idx, [r0, r1])
    cols = np.delete(np.arange(N), 1500)
    sel = idx[ok]
    check_gemm(bits[sel][:, cols], want[ok][:, cols], a[sel], sa[sel], b[cols], sb[cols])


# T on both sides of each change of launch instance at N = 5120 (with 256
# CUs): 16 x 32 | 32 x 32 | 64 x 32 | 64 x 64 | 128 x 64 | 128 x 128 |
# 128 x 256 | 256 x 256 | 128 x 128 two per CU
BOUNDARY_T = [16, 17, 32, 33, 64, 65, 192, 193, 384, 385, 768, 769, 1536, 1537, 4095, 4097]


@pytest.mark.parametrize("T", BOUNDARY_T)
def test_gemm_dispatch_boundaries_sampled(T):
    """Ragged T at each side of a change of block shape, N = 5120, K = 256:
    the first and last 16 rows (the ragged last block) and 16 more against
    the oracle."""
    N, K = 5120, 256
    a, sa, b, sb = mx_operands(T, N, K, seed=90 + T)
    got = gpu_gemm(a, sa, b, sb)
    rng = np.random.default_rng(T)
    idx = np.unique(np.concatenate([np.arange(min(16, T)), np.arange(max(0, T - 16), T),
                                    rng.choice(T, min(16, T), replace=False)]))
    want, _ = oracle.mxfp8_gemm(a[idx], sa[idx], b, sb)
    check_gemm(got[idx], want, a[idx], sa[idx], b, sb)


def test_gemm_empty_and_bad_arguments():
    from layer_mhc_seam_amd.seam import mxfp8_gemm
    z = lambda *s: torch.zeros(s, dtype=torch.uint8, device="cuda")
    assert mxfp8_gemm(z(0, 128), z(0, 4), z(16, 128), z(16, 4)).shape == (0, 16)
    with pytest.raises(RuntimeError):
        mxfp8_gemm(z(4, 96), z(4, 3), z(16, 96), z(16, 3))      # K not a multiple of 128
    with pytest.raises(ValueError):
        mxfp8_gemm(z(4, 128), z(4, 3), z(16, 128), z(16, 4))    # scales shape


def test_gemm_graph_replays_match_eager():
    from layer_mhc_seam_amd.seam import mxfp8_gemm
    a, sa, b, sb = mx_operands(200, 256, 1024, seed=84)
    da, dsa, db, dsb = to_dev(a), to_dev(sa), to_dev(b), to_dev(sb)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = mxfp8_gemm(da, dsa, db, dsb, stream=stream).clone()
        out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        mxfp8_gemm(da, dsa, db, dsb, out=out, stream=stream)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
