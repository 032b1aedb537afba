"""Pins of the CPU oracle against facts that do not come from the oracle:
library routines (torch), closed forms, invariants and brute force.

Every part of the oracle has at least one pin chosen so that a plausible
mistake there (a dropped term, a wrong sign, index or stream, a transposed
operand, a misplaced epsilon, the wrong Sinkhorn order, a wrong rounding
point) fails a test here.  The seam's steps and their order follow
"[FlyDSL] Single-launch Mega-mHC on gfx950", Motivation and Kernel
Architecture; the quantiser's crafted groups follow its Test Plan.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from layer_mhc_seam_amd import synth
from bits import bf16_to_f32, exact_bf16, ulp_diff

EPS = 1e-6


# ---------------------------------------------------------------- helpers --

def make_case(T, H, seed=1, xs=None):
    rng = np.random.default_rng(seed)
    x = oracle.f32_to_bf16(rng.standard_normal((T, 4, H)).astype(np.float32))
    y = oracle.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    fn = (rng.standard_normal((4 * H, 24)) / np.sqrt(4 * H)).astype(np.float32)
    gamma = oracle.f32_to_bf16((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    bias = (0.1 * rng.standard_normal(24)).astype(np.float32)
    pre, post, res = oracle.gate_inputs(rng.standard_normal((T, 4)),
                                        rng.standard_normal((T, 4)),
                                        rng.standard_normal((T, 4, 4)))
    return dict(x=x, y=y, pre=pre, post=post, res=res, fn=fn, gamma=gamma,
                bias=bias)


def run(c, **kw):
    return oracle.seam(c["x"], c["y"], c["pre"], c["post"], c["res"], c["fn"],
                       c["gamma"], c["bias"], **kw)


def ident(T):
    return np.broadcast_to(np.eye(4, dtype=np.float32), (T, 4, 4)).copy()


def rms_norm_lib(u_f32, gamma_bits, eps=EPS):
    """torch's RMSNorm (library routine) in float64, rounded to bf16 bits."""
    u = torch.from_numpy(np.asarray(u_f32, np.float64))
    w = torch.from_numpy(bf16_to_f32(gamma_bits).astype(np.float64))
    out = torch.nn.functional.rms_norm(u, (u.shape[-1],), w, eps)
    return oracle.f32_to_bf16(out.numpy().astype(np.float32))


def rn32(q: Fraction) -> Fraction:
    """Exact binary32 round-to-nearest-even of a rational (brute force)."""
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * ulp


def rn_bf16(q: Fraction) -> Fraction:
    """Exact bfloat16 round-to-nearest-even of a binary32 value."""
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 7)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * ulp


# ------------------------------------------------------ bf16 conversion ---

def test_oracle_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    # exact ties of both parities, signed zeros, subnormals, overflow to inf
    ties = (rng.integers(0, 2**16, 4096).astype(np.uint32) << 16) | 0x8000
    extra = np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                      1e-45, -1e-45, 1e-40, 3.3895314e38], np.float32)
    f = np.concatenate([f, ties.view(np.float32), extra])
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(f)
    assert np.array_equal(got, want)
    nan = oracle.f32_to_bf16(np.array([np.nan], np.float32))
    assert np.isnan(bf16_to_f32(nan)[0])


# ------------------------------------------------------------ post-mix ----

def test_oracle_postmix_identity_keeps_residual():
    T, H = 6, 64
    c = make_case(T, H)
    c["res"] = ident(T)
    c["post"] = np.zeros((T, 4), np.float32)
    o = run(c)
    assert np.array_equal(o["residual_out"], c["x"])


def test_oracle_postmix_permutation_not_transposed():
    T, H = 5, 64
    c = make_case(T, H, seed=2)
    P = np.zeros((4, 4), np.float32)
    for j in range(4):
        P[j, (j + 1) % 4] = 1.0          # x'[j] = x[(j+1) % 4]; not symmetric
    c["res"] = np.broadcast_to(P, (T, 4, 4)).copy()
    c["post"] = np.zeros((T, 4), np.float32)
    o = run(c)
    for j in range(4):
        assert np.array_equal(o["residual_out"][:, j], c["x"][:, (j + 1) % 4])


def test_oracle_postmix_layer_output_term():
    T, H = 8, 64
    c = make_case(T, H, seed=3)
    c["res"] = np.zeros((T, 4, 4), np.float32)
    post = np.zeros((T, 4), np.float32)
    post[np.arange(T), np.arange(T) % 4] = 1.0
    c["post"] = post
    o = run(c)
    for t in range(T):
        for j in range(4):
            if j == t % 4:
                assert np.array_equal(o["residual_out"][t, j], c["y"][t])
            else:   # 0 * x rounds to a signed zero: compare values
                assert not bf16_to_f32(o["residual_out"][t, j]).any()


def test_oracle_postmix_integer_closed_form():
    """Small integers keep every fp32 step exact, so x' = res x + post y."""
    T, H = 7, 96
    rng = np.random.default_rng(4)
    xi = rng.integers(-4, 5, (T, 4, H))
    yi = rng.integers(-4, 5, (T, H))
    ri = rng.integers(-2, 3, (T, 4, 4))
    pi = rng.integers(-2, 3, (T, 4))
    c = make_case(T, H, seed=4)
    c.update(x=exact_bf16(xi), y=exact_bf16(yi), res=ri.astype(np.float32),
             post=pi.astype(np.float32))
    o = run(c)
    want = np.einsum("tji,tih->tjh", ri, xi) + pi[:, :, None] * yi[:, None, :]
    assert np.array_equal(o["residual_out"], exact_bf16(want))


def test_oracle_postmix_rounding_points_brute_force():
    """The chain is one rounded product then fused multiply-adds, left to
    right, then one bf16 rounding; checked with exact rational arithmetic."""
    T, H = 3, 32
    c = make_case(T, H, seed=5)
    o = run(c)
    x = bf16_to_f32(c["x"]).astype(np.float64)
    y = bf16_to_f32(c["y"]).astype(np.float64)
    for t in range(T):
        for j in range(4):
            for h in range(0, H, 3):
                r = [Fraction(float(v)) for v in c["res"][t, j]]
                a = rn32(r[0] * Fraction(x[t, 0, h]))
                for i in range(1, 4):
                    a = rn32(r[i] * Fraction(x[t, i, h]) + a)
                a = rn32(Fraction(float(c["post"][t, j])) * Fraction(y[t, h]) + a)
                want = rn_bf16(a)
                got = Fraction(float(bf16_to_f32(o["residual_out"][t, j, h])))
                assert got == want, (t, j, h)


# ---------------------------------------------- collapse and the RMSNorm ---

def test_oracle_collapse_one_hot_pre_is_library_rmsnorm():
    """pre = e_k selects stream k; the norm is then torch's RMSNorm of x'[k]."""
    T, H = 8, 256
    c = make_case(T, H, seed=6)
    c["res"] = ident(T)
    c["post"] = np.zeros((T, 4), np.float32)
    pre = np.zeros((T, 4), np.float32)
    ks = (np.arange(T) * 3 + 1) % 4
    pre[np.arange(T), ks] = 1.0
    c["pre"] = pre
    o = run(c)
    for t in range(T):
        want = rms_norm_lib(bf16_to_f32(c["x"][t, ks[t]]), c["gamma"])
        d = ulp_diff(o["norm"][t], want)
        assert d.max() <= 1 and (d == 0).mean() > 0.97, t


def test_oracle_collapse_integer_closed_form():
    """Integer pre and streams make u exact; the norm is torch's RMSNorm(u)."""
    T, H = 6, 128
    rng = np.random.default_rng(7)
    xi = rng.integers(-8, 9, (T, 4, H))
    pi = rng.integers(-3, 4, (T, 4))
    c = make_case(T, H, seed=7)
    c.update(x=exact_bf16(xi), res=ident(T), post=np.zeros((T, 4), np.float32),
             pre=pi.astype(np.float32))
    o = run(c)
    u = np.einsum("ti,tih->th", pi, xi)          # |u| <= 96: exact in bf16
    for t in range(T):
        want = rms_norm_lib(u[t].astype(np.float64), c["gamma"])
        d = ulp_diff(o["norm"][t], want)
        assert d.max() <= 1 and (d == 0).mean() > 0.97, t


def test_oracle_identity_pre_on_copied_streams():
    """identity_pre with four identical streams collapses to that stream."""
    T, H = 4, 128
    c = make_case(T, H, seed=8)
    c["x"] = np.repeat(c["x"][:, :1], 4, axis=1)
    c["res"] = ident(T)
    c["post"] = np.zeros((T, 4), np.float32)
    o_id = run(c, identity_pre=True)
    pre = np.zeros((T, 4), np.float32)
    pre[:, 0] = 1.0
    c["pre"] = pre
    o_e0 = run(c)
    assert np.array_equal(o_id["norm"], o_e0["norm"])
    for t in range(T):
        want = rms_norm_lib(bf16_to_f32(c["x"][t, 0]), c["gamma"])
        assert ulp_diff(o_id["norm"][t], want).max() <= 1


def test_oracle_rmsnorm_epsilon_inside_the_root_and_mean():
    """u == c with c^2 ~ eps: norm = c / sqrt(c^2 + eps) * gamma."""
    T, H = 3, 64
    c = make_case(T, H, seed=9)
    cs = np.array([2.0 ** -10, -3 * 2.0 ** -11, 2.0 ** -8], np.float32)
    c["x"] = np.repeat(exact_bf16(cs)[:, None, None], 4, axis=1).repeat(H, axis=2)
    c["res"] = ident(T)
    c["post"] = np.zeros((T, 4), np.float32)
    o = run(c, identity_pre=True)
    g = bf16_to_f32(c["gamma"]).astype(np.float64)
    for t in range(T):
        v = float(cs[t])
        want = oracle.f32_to_bf16((v / np.sqrt(v * v + EPS) * g).astype(np.float32))
        assert ulp_diff(o["norm"][t], want).max() <= 1


def test_oracle_rmsnorm_zero_row():
    T, H = 2, 64
    c = make_case(T, H, seed=10)
    c["x"] = np.zeros((T, 4, H), np.uint16)
    c["res"] = ident(T)
    c["post"] = np.zeros((T, 4), np.float32)
    o = run(c)
    assert np.array_equal(bf16_to_f32(o["norm"]), np.zeros((T, H), np.float32))


# ----------------------------------------------------- gate projection ----

def doubly_stochastic():
    """A non-symmetric doubly stochastic 4x4 matrix with positive entries."""
    w = np.array([0.4, 0.3, 0.2, 0.1])
    K = np.zeros((4, 4))
    for j in range(4):
        for i in range(4):
            K[j, i] = w[(i - j) % 4]                # circulant
    K = 0.5 * K + 0.5 * K[[1, 2, 3, 0]][:, [0, 2, 1, 3]]
    assert np.allclose(K.sum(0), 1) and np.allclose(K.sum(1), 1)
    assert not np.allclose(K, K.T)
    return K


def test_oracle_gates_with_zero_fn_are_library_functions_of_bias():
    T, H = 3, 64
    c = make_case(T, H, seed=11)
    K = doubly_stochastic()
    bias = c["bias"].copy()
    bias[8:] = np.log(K).reshape(16)
    c["bias"] = bias.astype(np.float32)
    c["fn"] = np.zeros_like(c["fn"])
    o = run(c)
    b = torch.from_numpy(c["bias"].astype(np.float64))
    pre = torch.sigmoid(b[:4]).numpy()
    post = 2 * torch.sigmoid(b[4:8]).numpy()
    for t in range(T):
        np.testing.assert_allclose(o["pre_out"][t], pre, rtol=0, atol=1e-7)
        np.testing.assert_allclose(o["post_out"][t], post, rtol=0, atol=2e-7)
        # f32(log K) moves the fixed point by < 1e-7
        np.testing.assert_allclose(o["res_out"][t], K, rtol=0, atol=1e-6)


def test_oracle_gate_projection_flattened_index_closed_form():
    """Streams held at constants v_i make every dot a closed form; one-hot
    fn columns pin r = i*H + h, the [4H,24] layout and the mean over 4H."""
    T, H = 2, 64
    v = np.array([1.0, -2.0, 3.0, 0.5], np.float32)
    c = make_case(T, H, seed=12)
    c["x"] = np.broadcast_to(exact_bf16(v)[None, :, None], (T, 4, H)).copy()
    c["res"] = ident(T)
    c["post"] = np.zeros((T, 4), np.float32)
    fn = np.zeros((4 * H, 24), np.float32)
    picks = [(0, 0), (1, 5), (2, 63), (3, 17), (3, 63), (2, 0), (1, 33), (0, 40)]
    for k, (i0, h0) in enumerate(picks):
        fn[i0 * H + h0, k] = 1.0
    c["fn"] = fn
    c["bias"] = np.zeros(24, np.float32)
    o = run(c)
    rstd = 1.0 / np.sqrt(np.sum(v.astype(np.float64) ** 2) * H / (4 * H) + EPS)
    lk = np.array([rstd * v[i0] for (i0, _) in picks])
    sig = 1 / (1 + np.exp(-lk))
    for t in range(T):
        np.testing.assert_allclose(o["pre_out"][t], sig[:4], rtol=0, atol=1e-7)
        np.testing.assert_allclose(o["post_out"][t], 2 * sig[4:8], rtol=0, atol=2e-7)


def test_oracle_res_logits_row_major_not_transposed():
    """Rank-1 logit offsets from fn leave the Sinkhorn limit at K, the
    matrix bias[8:] encodes row-major; a transposed layout would give K^T."""
    T, H = 2, 64
    rng = np.random.default_rng(13)
    c = make_case(T, H, seed=13)
    K = doubly_stochastic()
    fn = np.zeros((4 * H, 24), np.float32)
    alpha = rng.standard_normal(4) * 0.05
    beta = rng.standard_normal(4) * 0.05
    for j in range(4):
        for i in range(4):
            fn[0:H, 8 + 4 * j + i] = alpha[j]          # stream 0 rows
            fn[H:2 * H, 8 + 4 * j + i] = beta[i]       # stream 1 rows
    c["fn"] = fn
    bias = np.zeros(24, np.float32)
    bias[8:] = np.log(K).reshape(16)
    c["bias"] = bias
    o = run(c)
    for t in range(T):
        np.testing.assert_allclose(o["res_out"][t], K, rtol=0, atol=1e-6)


def test_oracle_gates_invariant_to_residual_scale():
    """Doubling x' (res = 2I) doubles the residual exactly and leaves the
    gates unchanged up to eps: the logits are rstd-normalised."""
    T, H = 4, 128
    c = make_case(T, H, seed=14)
    c["post"] = np.zeros((T, 4), np.float32)
    c["res"] = ident(T)
    o1 = run(c)
    c["res"] = 2 * ident(T)
    o2 = run(c)
    np.testing.assert_array_equal(bf16_to_f32(o2["residual_out"]),
                                  2 * bf16_to_f32(o1["residual_out"]))
    for k in ("pre_out", "post_out", "res_out"):
        np.testing.assert_allclose(o1[k], o2[k], rtol=0, atol=2e-6)


def test_oracle_no_post_equals_identity_mix():
    T, H = 5, 128
    c = make_case(T, H, seed=15)
    o_np = run(c, post_form=False)
    assert "residual_out" not in o_np
    c["res"] = ident(T)
    c["post"] = np.zeros((T, 4), np.float32)
    o_p = run(c)
    for k in ("norm", "pre_out", "post_out", "res_out"):
        assert np.array_equal(o_np[k], o_p[k]), k


def test_oracle_token_range_matches_full_run():
    T, H = 9, 64
    c = make_case(T, H, seed=16)
    full = run(c)
    part = run(c, t0=3, t1=7)
    for k, v in full.items():
        assert np.array_equal(part[k][3:7], v[3:7]), k
        assert not part[k][:3].any() and not part[k][7:].any(), k


def test_oracle_gate_projection_brute_force_fp64():
    """Gate logits recovered from pre/post agree with an fp64 brute force
    over the stored residual (small case)."""
    T, H = 3, 32
    c = make_case(T, H, seed=17)
    o = run(c)
    xb = bf16_to_f32(o["residual_out"]).astype(np.float64).reshape(T, 4 * H)
    for t in range(T):
        ss = sum(float(v) * float(v) for v in xb[t])
        r = 1.0 / np.sqrt(ss / (4 * H) + EPS)
        for k in range(8):
            d = sum(float(xb[t, q]) * float(c["fn"][q, k]) for q in range(4 * H))
            lk = r * d + float(c["bias"][k])
            g = 1 / (1 + np.exp(-lk))
            got = o["pre_out"][t, k] if k < 4 else o["post_out"][t, k - 4] / 2
            assert abs(got - g) < 1e-7


# ------------------------------------------------------------ Sinkhorn ----

def test_oracle_sinkhorn_rank_one_logits_one_iteration():
    rng = np.random.default_rng(18)
    a = rng.standard_normal((50, 4, 1))
    b = rng.standard_normal((50, 1, 4))
    out = oracle.sinkhorn(a + b, iters=1)
    np.testing.assert_allclose(out, 0.25, rtol=0, atol=1e-15)


def test_oracle_sinkhorn_row_then_column_order():
    """diag(a) K: one row pass gives K exactly and the column pass keeps it;
    a column-first iteration would not."""
    K = doubly_stochastic()
    rng = np.random.default_rng(19)
    a = rng.standard_normal((20, 4, 1)) * 2
    out = oracle.sinkhorn(np.log(K)[None] + a, iters=1)
    np.testing.assert_allclose(out, np.broadcast_to(K, out.shape), rtol=0, atol=1e-14)


def test_oracle_sinkhorn_fixed_point_and_marginals():
    K = doubly_stochastic()
    rng = np.random.default_rng(20)
    a = rng.standard_normal((20, 4, 1))
    b = rng.standard_normal((20, 1, 4))
    out = oracle.sinkhorn(np.log(K)[None] + a + b, iters=20)
    np.testing.assert_allclose(out, np.broadcast_to(K, out.shape), rtol=0, atol=1e-9)
    z = rng.standard_normal((2000, 4, 4))
    m = oracle.sinkhorn(z, iters=20)
    np.testing.assert_allclose(m.sum(-2), 1, rtol=0, atol=1e-12)   # columns last
    # rows converge: typical error after 20 iterations is small, and more
    # iterations drive every row sum to 1
    assert np.quantile(np.abs(m.sum(-1) - 1), 0.99) < 1e-4
    m = oracle.sinkhorn(z, iters=2000)
    np.testing.assert_allclose(m.sum(-1), 1, rtol=0, atol=1e-9)


def test_oracle_sinkhorn_permutation_equivariant():
    rng = np.random.default_rng(21)
    z = rng.standard_normal((10, 4, 4))
    pr, pc = [2, 0, 3, 1], [1, 3, 0, 2]
    a = oracle.sinkhorn(z[:, pr][:, :, pc])
    b = oracle.sinkhorn(z)[:, pr][:, :, pc]
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def triangular_block_logits(blocks):
    """4x4 logits, block diagonal with upper-triangular 2x2 blocks
    [[a, b], [0, d]] (zeros as logits of -1000, whose exp is exactly 0)."""
    L = np.full((4, 4), -1000.0)
    for k, (a, b, d) in enumerate(blocks):
        r = 2 * k
        L[r, r], L[r, r + 1], L[r + 1, r + 1] = np.log(a), np.log(b), np.log(d)
    return L


def triangular_block_closed_form(blocks, n):
    """Row-then-column Sinkhorn of each block [[a, b], [0, d]] after n >= 1
    iterations:
        [[1, b / (a + 2 n b)], [0, (a + (2 n - 1) b) / (a + 2 n b)]].
    By induction: the first row pass gives [[a, b] / (a + b), [0, 1]] and the
    column pass turns that into the n = 1 form; from the n form, the row
    pass divides the first row by (a + (2 n + 1) b) / (a + 2 n b) and leaves
    [0, 1], and the column pass then gives the n + 1 form.  It converges
    like 1/n, so every iteration count gives another value."""
    M = np.zeros((4, 4))
    for k, (a, b, d) in enumerate(blocks):
        r = 2 * k
        M[r, r] = 1.0
        M[r, r + 1] = b / (a + 2 * n * b)
        M[r + 1, r + 1] = (a + (2 * n - 1) * b) / (a + 2 * n * b)
    return M


@pytest.mark.parametrize("n", [1, 2, 3, 7, 19, 20, 21])
def test_oracle_sinkhorn_iteration_count_closed_form(n):
    """The iteration count is pinned: a matrix without a doubly stochastic
    scaling (triangular support) converges like 1/n, with a closed form at
    every n.  An extra or a missing iteration moves M[0][1] by ~1e-3 at
    n = 20."""
    blocks = [(0.7, 1.9, 3.1), (2.0, 0.25, 5.0)]
    got = oracle.sinkhorn(triangular_block_logits(blocks)[None], iters=n)[0]
    np.testing.assert_allclose(got, triangular_block_closed_form(blocks, n), rtol=1e-13,
                               atol=0)


def test_oracle_sinkhorn_iterations_compose():
    """n iterations, then m more on the logarithm of the result, equal n + m
    iterations (a row pass on a matrix whose columns sum to one starts where
    the previous iteration stopped).  An off-by-one count breaks this."""
    rng = np.random.default_rng(22)
    z = 2.0 * rng.standard_normal((200, 4, 4))
    for n, m in ((1, 1), (1, 2), (2, 3), (5, 15)):
        a = oracle.sinkhorn(np.log(oracle.sinkhorn(z, iters=n)), iters=m)
        b = oracle.sinkhorn(z, iters=n + m)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_oracle_sinkhorn_zero_iterations_is_exp():
    z = np.random.default_rng(23).standard_normal((5, 4, 4))
    np.testing.assert_allclose(oracle.sinkhorn(z, iters=0), np.exp(z), rtol=4e-16, atol=0)


def test_oracle_seam_sinkhorn_iteration_count_through_bias():
    """fn = 0 makes the res logits equal bias[8:24] exactly, so the seam's
    res_out is the closed form at the seam's iteration count."""
    blocks = [(0.7, 1.9, 3.1), (2.0, 0.25, 5.0)]
    T, H = 3, 64
    c = synth.draw(T, H, seed=24)
    pre, post, res = oracle.gate_inputs(c["z_pre"], c["z_post"], c["z_res"])
    bias = np.zeros(24, np.float32)
    bias[8:] = triangular_block_logits(blocks).reshape(16)
    for n in (1, 2, 20):
        o = oracle.seam(c["x"], c["y"], pre, post, res, np.zeros((4 * H, 24), np.float32),
                        c["gamma"], bias, iters=n)
        want = triangular_block_closed_form(blocks, n).astype(np.float32)
        np.testing.assert_allclose(o["res_out"], np.broadcast_to(want, (T, 4, 4)), rtol=1e-6,
                                   atol=0)


def test_oracle_sigmoid_matches_torch():
    v = np.linspace(-30, 30, 10001)
    np.testing.assert_allclose(oracle.sigmoid(v),
                               torch.sigmoid(torch.from_numpy(v)).numpy(),
                               rtol=1e-15, atol=1e-300)


# ----------------------------------------------------------- quantiser ----

def e4m3_table():
    """All positive finite e4m3fn values by code (0..126), from the format's
    definition: bias 7, 3 mantissa bits, subnormals at exponent field 0."""
    vals = []
    for cde in range(127):
        e, m = cde >> 3, cde & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def brute_force_encode(s):
    """Nearest e4m3fn code of float64 values |s| <= 448, ties to even code."""
    tab = e4m3_table()
    a = np.abs(s)
    idx = np.searchsorted(tab, a, side="right") - 1          # tab[idx] <= a
    idx = np.clip(idx, 0, 126)
    hi = np.minimum(idx + 1, 126)
    dlo, dhi = a - tab[idx], tab[hi] - a
    up = (hi != idx) & ((dhi < dlo) | ((dhi == dlo) & (idx % 2 == 1)))
    code = np.where(up, hi, idx)
    return (code | (np.signbit(s) << 7)).astype(np.uint8)


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[np.isfinite(bf16_to_f32(b))]


@pytest.mark.slow
def test_oracle_e4m3_encode_exhaustive_brute_force():
    v = all_finite_bf16()
    vf = bf16_to_f32(v).astype(np.float64)
    for k in range(-127, 128):
        s = np.ldexp(vf, -k)
        ok = np.abs(s) <= 448
        got = oracle.e4m3_encode_scaled(v[ok], k)
        assert np.array_equal(got, brute_force_encode(s[ok])), k


def test_oracle_e4m3_encode_matches_torch_float8():
    v = all_finite_bf16()
    vf = bf16_to_f32(v).astype(np.float64)
    for k in (-127, -100, -20, -8, -3, 0, 1, 5, 40, 120):
        s = np.ldexp(vf, -k)
        ok = (np.abs(s) <= 448) & ((np.abs(s) >= 2.0 ** -60) | (s == 0))
        want = torch.from_numpy(s[ok].astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = oracle.e4m3_encode_scaled(v[ok], k)
        assert np.array_equal(got, want), k


def test_oracle_e4m3_decode_matches_torch_float8():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_oracle_scale_exponent_brute_force():
    v = all_finite_bf16()
    a = np.unique(np.abs(bf16_to_f32(v).astype(np.float64)))
    got = oracle.scale_exp(a)
    # brute force: walk k upward from -127 and keep the first k that covers
    # amax (448 * 2^k and amax are both exact in float64)
    want = np.full(a.shape, 127, np.int64)
    done = np.zeros(a.shape, bool)
    for k in range(-127, 128):
        hit = ~done & (448.0 * 2.0 ** k >= a)
        want[hit] = k
        done |= hit
    want[a == 0] = -127
    assert np.array_equal(got, want)
    edge = oracle.scale_exp(np.array([448.0, 446.0, 448.0 * 2 ** -5, 450.0, 0.0]))
    assert list(edge) == [0, 0, -5, 1, -127]


def crafted_groups():
    """Quantiser edge groups of 32 (Mega-mHC page, Test Plan): amax exactly
    448 * 2^k and its bf16 neighbours, zeros, signed zeros, subnormals,
    near-max values."""
    rng = np.random.default_rng(22)
    groups = []
    for k in (-127, -126, -125, -120, -60, -9, -1, 0, 1, 7, 60, 119, 120):
        top = 448.0 * 2.0 ** k
        if not np.isfinite(np.float32(top)) or top >= 3.3e38:
            continue
        tb = exact_bf16([top])[0] if top >= 2.0 ** -133 else None
        if tb is None:
            continue
        for nb in (-1, 0, 1):
            body = oracle.f32_to_bf16((rng.standard_normal(32) * top / 3).astype(np.float32))
            body[rng.integers(32)] = np.uint16(int(tb) + nb)
            groups.append(body)
    groups.append(np.zeros(32, np.uint16))
    groups.append(np.full(32, 0x8000, np.uint16))
    groups.append(np.arange(1, 33, dtype=np.uint16))                 # subnormals
    groups.append((np.arange(1, 33, dtype=np.uint16) | 0x8000).astype(np.uint16))
    groups.append(np.full(32, 0x7F7F, np.uint16))                     # bf16 max
    return np.stack(groups)


def test_oracle_quantize_crafted_groups():
    g = crafted_groups()
    codes, scales, grid = oracle.quantize(g.reshape(-1, 32))
    vf = bf16_to_f32(g).astype(np.float64)
    for n in range(g.shape[0]):
        amax = np.abs(vf[n]).max()
        k = int(scales[n, 0]) - 127
        if amax == 0:
            assert k == -127
        else:
            assert 448.0 * 2.0 ** k >= amax
            assert k == -127 or 448.0 * 2.0 ** (k - 1) < amax
        s = np.ldexp(vf[n], -k)
        assert np.array_equal(codes[n], brute_force_encode(s))
        dq = oracle.e4m3_decode(codes[n]) * 2.0 ** k
        # the dequantised value is exact in bf16 except 2^128 and above at
        # k = 120 (near bf16's max), which round to inf as IEEE rounding does
        with np.errstate(over="ignore"):
            dq32 = dq.astype(np.float32)
        assert np.array_equal(bf16_to_f32(grid[n]), dq32)
        assert np.array_equal(bf16_to_f32(grid[n][np.isfinite(dq32)]).astype(np.float64),
                              dq[np.isfinite(dq32)])
        assert np.array_equal(np.signbit(bf16_to_f32(grid[n])), np.signbit(dq))
    # a group whose amax is exactly 448 * 2^k stores that element as code 0x7E
    k0 = 5
    grp = np.zeros(32, np.uint16)
    grp[3] = exact_bf16([448.0 * 2 ** k0])[0]
    codes, scales, grid = oracle.quantize(grp[None])
    assert scales[0, 0] == k0 + 127 and codes[0, 3] == 0x7E


def test_oracle_quantize_dequant_error_bound():
    rng = np.random.default_rng(23)
    norm = oracle.f32_to_bf16((rng.standard_normal((16, 256)) *
                               np.exp(rng.standard_normal((16, 1)) * 4)).astype(np.float32))
    codes, scales, grid = oracle.quantize(norm)
    v = bf16_to_f32(norm).astype(np.float64).reshape(16, 8, 32)
    q = bf16_to_f32(grid).astype(np.float64).reshape(16, 8, 32)
    k = scales.astype(np.int64) - 127
    a = np.abs(v) * 2.0 ** -k[..., None]
    # e4m3 half-ulp at the scaled value's binade (2^-10 in the subnormal range)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half = 2.0 ** (e - 4) * 2.0 ** k[..., None]
    assert np.all(np.abs(q - v) <= half)


# ------------------------------------------- rounding points, brute force --

def test_oracle_collapse_rounds_u_to_bf16_brute_force():
    """u is the bf16 rounding of the exact-rational fma chain over the stored
    residual; torch's RMSNorm of that u matches the norm (<= 1 ulp, almost
    always bitwise).  An unrounded u would flip about a quarter of them."""
    T, H = 3, 64
    c = make_case(T, H, seed=24)
    o = run(c)
    xb = bf16_to_f32(o["residual_out"]).astype(np.float64)
    bitwise = []
    for t in range(T):
        p = [Fraction(float(v)) for v in c["pre"][t]]
        u = np.empty(H)
        for h in range(H):
            a = rn32(p[0] * Fraction(xb[t, 0, h]))
            for i in range(1, 4):
                a = rn32(p[i] * Fraction(xb[t, i, h]) + a)
            u[h] = float(rn_bf16(a))
        want = rms_norm_lib(u, c["gamma"])
        d = ulp_diff(o["norm"][t], want)
        assert d.max() <= 1
        bitwise.append((d == 0).mean())
    assert np.mean(bitwise) > 0.97


def fused_vs_split_cases(n_want=24, seed=25):
    """Search (x0, x3, r0, r3) with r1 = r2 = 0 where the fused chain
    RN(r3 x3 + RN(r0 x0)) and the split chain RN(RN(r3 x3) + RN(r0 x0)) give
    different bf16 results; every candidate is confirmed in exact rationals."""
    rng = np.random.default_rng(seed)
    found = []
    while len(found) < n_want:
        x0 = oracle.f32_to_bf16(rng.standard_normal(200_000).astype(np.float32))
        x3 = oracle.f32_to_bf16(rng.standard_normal(200_000).astype(np.float32))
        r0 = rng.random(200_000).astype(np.float32)
        r3 = rng.random(200_000).astype(np.float32)
        f0, f3 = bf16_to_f32(x0).astype(np.float64), bf16_to_f32(x3).astype(np.float64)
        a = (r0.astype(np.float64) * f0).astype(np.float32).astype(np.float64)
        fused = (r3.astype(np.float64) * f3 + a).astype(np.float32)
        split = ((r3.astype(np.float64) * f3).astype(np.float32).astype(np.float64)
                 + a).astype(np.float32)
        cand = np.nonzero(oracle.f32_to_bf16(fused) != oracle.f32_to_bf16(split))[0]
        for n in cand[:n_want - len(found)]:
            A = rn32(Fraction(float(r0[n])) * Fraction(float(f0[n])))
            fu = rn_bf16(rn32(Fraction(float(r3[n])) * Fraction(float(f3[n])) + A))
            sp = rn_bf16(rn32(rn32(Fraction(float(r3[n])) * Fraction(float(f3[n]))) + A))
            if fu != sp:
                found.append((x0[n], x3[n], r0[n], r3[n], fu))
    return found


def test_oracle_postmix_is_fused_multiply_add():
    cases = fused_vs_split_cases()
    T, H = len(cases), 32
    c = make_case(T, H, seed=26)
    res = np.zeros((T, 4, 4), np.float32)
    for t, (x0, x3, r0, r3, _) in enumerate(cases):
        c["x"][t, 0, :] = x0
        c["x"][t, 3, :] = x3
        res[t, 0, 0], res[t, 0, 3] = r0, r3
    c["res"] = res
    c["post"] = np.zeros((T, 4), np.float32)
    o = run(c)
    for t, (*_, fu) in enumerate(cases):
        got = bf16_to_f32(o["residual_out"][t, 0]).astype(np.float64)
        assert np.all(got == float(fu)), t


# ------------------------------------------------------ unshifted ordering --
# The other ordering of the method ("[FlyDSL] Single-launch Mega-mHC on
# gfx950", Test Result, notes on what each compared kernel computes): gates
# from x' first, then the collapse with the fresh pre.

def test_oracle_unshifted_zero_fn_collapses_with_sigmoid_of_bias():
    """fn = 0 makes every token's fresh pre sigmoid(bias[0:4]) (a library
    routine), so the unshifted norm is the delayed seam's with that pre."""
    T, H = 5, 128
    c = make_case(T, H, seed=21)
    c["fn"] = np.zeros_like(c["fn"])
    sig = torch.sigmoid(torch.from_numpy(c["bias"][:4].astype(np.float64))).numpy()
    p = np.tile(sig.astype(np.float32), (T, 1))
    un = oracle.seam(c["x"], c["y"], None, c["post"], c["res"], c["fn"], c["gamma"],
                     c["bias"], unshifted=True)
    assert np.array_equal(un["pre_out"], p)
    ref = run(dict(c, pre=p))
    assert np.array_equal(un["norm"], ref["norm"])
    assert np.array_equal(un["residual_out"], ref["residual_out"])


def test_oracle_unshifted_collapses_with_its_own_fresh_pre():
    T, H = 6, 256
    c = make_case(T, H, seed=22)
    un = oracle.seam(c["x"], c["y"], None, c["post"], c["res"], c["fn"], c["gamma"],
                     c["bias"], unshifted=True)
    delayed = run(c)
    # same x', so the same gates as the delayed seam
    for k in ("pre_out", "post_out", "res_out", "residual_out"):
        assert np.array_equal(un[k], delayed[k]), k
    # the norm is the delayed seam's with the carried pre replaced by pre_out
    again = run(dict(c, pre=un["pre_out"]))
    assert np.array_equal(un["norm"], again["norm"])
    assert not np.array_equal(un["norm"], delayed["norm"])


def test_oracle_unshifted_no_post_form():
    T, H = 4, 128
    c = make_case(T, H, seed=23)
    un = oracle.seam(c["x"], None, None, None, None, c["fn"], c["gamma"], c["bias"],
                     post_form=False, unshifted=True)
    again = oracle.seam(c["x"], None, un["pre_out"], None, None, c["fn"], c["gamma"],
                        c["bias"], post_form=False)
    assert np.array_equal(un["norm"], again["norm"])


# ------------------------------------------------------ 128-wide groups --
# The 128-wide grouping "[FlyDSL] Single-launch Mega-mHC on gfx950" lists as
# missing (Limitations), read as the same ue8m0 rule over 128 elements.

def test_oracle_g128_scale_is_max_of_its_four_g32_scales():
    """scale_exp is monotone in amax and the amax of 128 elements is the
    largest of its four 32-element amaxes: k128 = max of the four k32."""
    rng = np.random.default_rng(51)
    T, H = 6, 1024
    v = rng.standard_normal((T, H // 32, 32)) * np.exp2(rng.integers(-20, 20, (T, H // 32, 1)))
    norm = oracle.f32_to_bf16(v.reshape(T, H).astype(np.float32))
    norm[0, :32] = 0                                 # a zero subgroup
    norm[1, :128] = 0                                # a zero 128-group
    _, s32, _ = oracle.quantize(norm, 32)
    codes, s128, grid = oracle.quantize(norm, 128)
    assert np.array_equal(s128, s32.reshape(T, H // 128, 4).max(axis=-1))
    # codes are the scaled encode (pinned exhaustively above) at k128
    k = s128.astype(np.int64) - 127
    for t in range(T):
        for g in range(H // 128):
            piece = norm[t, 128 * g:128 * (g + 1)]
            assert np.array_equal(codes[t, 128 * g:128 * (g + 1)],
                                  oracle.e4m3_encode_scaled(piece, int(k[t, g])))


def test_oracle_g128_equals_g32_when_subgroups_share_a_scale():
    rng = np.random.default_rng(52)
    T, H = 4, 512
    v = rng.uniform(-1, 1, (T, H))
    v[:, ::32] = 1.5                                 # every 32-group has amax 1.5
    norm = oracle.f32_to_bf16(v.astype(np.float32))
    a = oracle.quantize(norm, 32)
    b = oracle.quantize(norm, 128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    assert np.array_equal(a[1].reshape(T, -1, 4)[..., 0], b[1])


def test_oracle_g128_rejects_bad_widths():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 96), np.uint16), 128)


# ------------------------------------------------- head reduce (n -> 1) --
# "[Triton/Gluon] [gfx950] [dsv4.1-flash] mHC fused kernel", description:
# an HC head reduce/store kernel is named among the unfused per-seam
# kernels and not described.  Reading: the collapse step on its own over the
# stored streams, bf16(sum_i w_i x_i), w == None for weights of 1/4.

def test_oracle_head_reduce_one_hot_weights_select_a_stream():
    T, H = 8, 96
    x = make_case(T, H, seed=40)["x"]
    w = np.zeros((T, 4), np.float32)
    ks = (np.arange(T) * 3 + 2) % 4
    w[np.arange(T), ks] = 1.0
    out = oracle.head_reduce(x, w)
    assert np.array_equal(out, x[np.arange(T), ks])


def test_oracle_head_reduce_integer_closed_form():
    """Small integer weights and streams make the sum exact in bf16."""
    T, H = 5, 64
    rng = np.random.default_rng(41)
    xi = rng.integers(-8, 9, (T, 4, H))
    wi = rng.integers(-3, 4, (T, 4))
    out = oracle.head_reduce(exact_bf16(xi), wi.astype(np.float32))
    want = (wi[:, :, None] * xi).sum(axis=1)          # |sum| <= 96
    assert np.array_equal(bf16_to_f32(out), want.astype(np.float32))


def test_oracle_head_reduce_identity_weights_are_a_quarter():
    """No weights means 1/4 each: four copies of a stream give it back, and
    a mean of dyadic streams is exact."""
    T, H = 4, 128
    x = make_case(T, H, seed=42)["x"]
    same = np.repeat(x[:, :1], 4, axis=1)
    assert np.array_equal(oracle.head_reduce(same), x[:, 0])
    q = np.full((T, 4), 0.25, np.float32)
    assert np.array_equal(oracle.head_reduce(x), oracle.head_reduce(x, q))
    xi = np.random.default_rng(43).integers(-16, 17, (T, 4, H)) * 4
    out = oracle.head_reduce(exact_bf16(xi))
    assert np.array_equal(bf16_to_f32(out), (xi.sum(axis=1) / 4).astype(np.float32))


def test_oracle_head_reduce_brute_force_exact_chain():
    """Every element is the bf16 rounding of the exact-rational chain
    RN(w0 x0), then RN(w_i x_i + a) for i = 1..3 (one rounding per step)."""
    T, H = 3, 48
    c = make_case(T, H, seed=44)
    w = c["pre"]
    out = oracle.head_reduce(c["x"], w)
    xf = bf16_to_f32(c["x"]).astype(np.float64)
    for t in range(T):
        p = [Fraction(float(v)) for v in w[t]]
        for h in range(H):
            a = rn32(p[0] * Fraction(xf[t, 0, h]))
            for i in range(1, 4):
                a = rn32(p[i] * Fraction(xf[t, i, h]) + a)
            assert Fraction(float(bf16_to_f32(out[t, h]))) == rn_bf16(a), (t, h)


def test_oracle_head_reduce_is_fused_multiply_add():
    """Inputs where a split multiply-add rounds to another bf16 value."""
    cases = fused_vs_split_cases(n_want=16, seed=45)
    T, H = len(cases), 16
    x = make_case(T, H, seed=46)["x"]
    w = np.zeros((T, 4), np.float32)
    for t, (x0, x3, r0, r3, _) in enumerate(cases):
        x[t, 0, :], x[t, 3, :] = x0, x3
        w[t, 0], w[t, 3] = r0, r3
    out = oracle.head_reduce(x, w)
    for t, (*_, fu) in enumerate(cases):
        assert np.all(bf16_to_f32(out[t]).astype(np.float64) == float(fu)), t


def test_oracle_head_reduce_is_the_seam_collapse():
    """The no_post seam normalises exactly this u: torch's RMSNorm of the
    head reduce of x with the carried pre matches the seam's norm."""
    T, H = 6, 256
    c = make_case(T, H, seed=47)
    o = oracle.seam(c["x"], None, c["pre"], None, None, c["fn"], c["gamma"], c["bias"],
                    post_form=False)
    u = oracle.head_reduce(c["x"], c["pre"])
    for t in range(T):
        d = ulp_diff(o["norm"][t], rms_norm_lib(bf16_to_f32(u[t]), c["gamma"]))
        assert d.max() <= 1 and (d == 0).mean() > 0.97, t


def test_oracle_head_reduce_rejects_bad_sizes():
    with pytest.raises(AssertionError):
        oracle.head_reduce(np.zeros((2, 3, 8), np.uint16))
    assert oracle.head_reduce(np.zeros((0, 4, 8), np.uint16)).shape == (0, 8)


# ------------------------------------------------ consumer GEMM (MXFP8) --
# "[FlyDSL] Single-launch Mega-mHC on gfx950", Kernel Architecture and Test
# Result: the ue8m0/e4m3 norm feeds the next layer's GEMM.  Reading: both
# operands MXFP8 along K (one ue8m0 scale per 32 K elements), out = a b^T.

def mx_case(T, N, K, seed, scale_lo=124, scale_hi=131):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], np.uint8)
    a = rng.choice(finite, (T, K))
    b = rng.choice(finite, (N, K))
    sa = rng.integers(scale_lo, scale_hi, (T, K // 32)).astype(np.uint8)
    sb = rng.integers(scale_lo, scale_hi, (N, K // 32)).astype(np.uint8)
    return a, sa, b, sb


def dequant_torch(codes, scales):
    """Library decode: torch's float8_e4m3fn cast, times 2^(s - 127)."""
    v = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))


def test_oracle_mxfp8_gemm_matches_library_matmul():
    a, sa, b, sb = mx_case(7, 24, 256, seed=50)
    out, absum = oracle.mxfp8_gemm(a, sa, b, sb)
    want = dequant_torch(a, sa) @ dequant_torch(b, sb).T
    assert np.allclose(out, want, rtol=0, atol=1e-12 * np.abs(want).max())
    assert np.all(absum >= np.abs(out))
    ref_abs = np.abs(dequant_torch(a, sa)) @ np.abs(dequant_torch(b, sb)).T
    assert np.allclose(absum, ref_abs, rtol=1e-12)


def test_oracle_mxfp8_gemm_one_hot_weights_select_columns():
    """Weight row n = 1.0 at column k_n (code 0x38, scale 127): out[:, n] is
    the dequantised activation column k_n."""
    T, N, K = 5, 12, 128
    a, sa, _, _ = mx_case(T, N, K, seed=51)
    ks = (np.arange(N) * 37 + 5) % K
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), ks] = 0x38
    sb = np.full((N, K // 32), 127, np.uint8)
    out, _ = oracle.mxfp8_gemm(a, sa, b, sb)
    assert np.array_equal(out, dequant_torch(a, sa)[:, ks])


def test_oracle_mxfp8_gemm_integer_closed_form():
    """Codes of small integers and unit scales: an exact integer matmul."""
    T, N, K = 4, 6, 96
    rng = np.random.default_rng(52)
    vals = np.array([-3, -2, -1, 0, 1, 2, 3])
    codes = {-3: 0xc4, -2: 0xc0, -1: 0xb8, 0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44}
    ai, bi = rng.choice(vals, (T, K)), rng.choice(vals, (N, K))
    enc = np.vectorize(lambda v: codes[int(v)])
    one = lambda r: np.full((r, K // 32), 127, np.uint8)
    out, absum = oracle.mxfp8_gemm(enc(ai).astype(np.uint8), one(T), enc(bi).astype(np.uint8),
                                   one(N))
    assert np.array_equal(out, (ai @ bi.T).astype(np.float64))
    assert np.array_equal(absum, (np.abs(ai) @ np.abs(bi).T).astype(np.float64))


def test_oracle_mxfp8_gemm_scale_applies_to_its_32_columns():
    """Raising one activation scale by one doubles exactly that block's
    share of the sum and nothing else."""
    T, N, K = 3, 8, 128
    a, sa, b, sb = mx_case(T, N, K, seed=53)
    out, _ = oracle.mxfp8_gemm(a, sa, b, sb)
    sa2 = sa.copy()
    sa2[1, 2] += 1
    out2, _ = oracle.mxfp8_gemm(a, sa2, b, sb)
    A, B = dequant_torch(a, sa), dequant_torch(b, sb)
    block = A[1, 64:96] @ B[:, 64:96].T
    assert np.allclose(out2[1] - out[1], block, rtol=0, atol=1e-12 * np.abs(block).max())
    assert np.array_equal(out2[[0, 2]], out[[0, 2]])


def test_oracle_mxfp8_gemm_scale_ff_is_nan():
    """OCP MX: the E8M0 byte 0xff encodes NaN (bytes 0..254 are 2^(s-127)).
    A 0xff activation scale makes its row NaN, a 0xff weight scale its
    column, even over zero codes; every other output is unchanged."""
    T, N, K = 4, 6, 128
    a, sa, b, sb = mx_case(T, N, K, seed=54)
    a[2, 32:64] = 0
    sa[2, 1] = 0xFF
    sb[4, 3] = 0xFF
    out, _ = oracle.mxfp8_gemm(a, sa, b, sb)
    nan = np.zeros((T, N), bool)
    nan[2, :] = nan[:, 4] = True
    assert np.isnan(out[nan]).all() and not np.isnan(out[~nan]).any()
    sa[2, 1], sb[4, 3] = 127, 127
    ok, _ = oracle.mxfp8_gemm(a, sa, b, sb)
    assert np.array_equal(out[~nan], ok[~nan])


def test_oracle_mxfp8_gemm_extreme_scales_multiply():
    """The two scales multiply: 2^(sa-127) 2^(sb-127) depends on sa + sb
    only, so scale bytes 0 / 254, 1 / 253 and 254 / 0 give the result of
    127 / 127 exactly (no intermediate underflow or overflow); 254 / 254
    overflows every non-zero output past binary32 and bf16."""
    T, N, K = 3, 5, 64
    a, _, b, _ = mx_case(T, N, K, seed=55)
    full = lambda v, r: np.full((r, K // 32), v, np.uint8)
    ref, _ = oracle.mxfp8_gemm(a, full(127, T), b, full(127, N))
    for x, y in ((0, 254), (1, 253), (254, 0), (100, 154)):
        out, _ = oracle.mxfp8_gemm(a, full(x, T), b, full(y, N))
        assert np.array_equal(out, ref), (x, y)
    big, _ = oracle.mxfp8_gemm(a, full(254, T), b, full(254, N))
    assert np.all(np.abs(big[ref != 0]) > 2.0 ** 128)


def test_oracle_mxfp8_gemm_rejects_bad_sizes():
    with pytest.raises(AssertionError):
        oracle.mxfp8_gemm(np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8),
                          np.zeros((3, 48), np.uint8), np.zeros((3, 1), np.uint8))
