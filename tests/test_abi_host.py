"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/mhc_seam.h declares, and its argument rules and launch
plan behave as documented.  Pointers passed to mhc_seam_validate are fake
addresses: validation never dereferences them."""
import ctypes
import os
import re

import pytest

from layer_mhc_seam_amd import seam as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc_seam.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mhc_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mhc_seam_create", "mhc_seam_run", "mhc_seam_destroy"):
        assert n in names
    assert set(names) == set(S.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = S.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_struct_layouts_match_header_sizes():
    # 4 int32 + 3 pointers + int64 + 2 int32 + 7 int32 (with padding)
    assert ctypes.sizeof(S.Desc) == 4 * 4 + 3 * 8 + 8 + 4 * 9 + 4   # ksplit, spin_polls, 6 reserved
    assert ctypes.sizeof(S.Args) == 8 + 4 * 4 + 13 * 8
    assert ctypes.sizeof(S.Plan) == 8 * 4


BASE = 0x7f0000000000


def desc(H=512, max_tokens=64, **kw):
    d = S.Desc()
    d.H, d.n, d.eps, d.sinkhorn_iters = H, 4, 1e-6, 20
    d.fn, d.gamma, d.bias = BASE, BASE + (1 << 24), BASE + (2 << 24)
    d.max_tokens = max_tokens
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def args(T=8, H=512, form="post", out="bf16", identity_pre=False, **kw):
    a = S.Args()
    a.T, a.form, a.out_dtype, a.identity_pre = T, S.FORMS[form], S.OUT_DTYPES[out], int(identity_pre)
    slot = [BASE + (k << 28) for k in range(3, 20)]
    a.x, a.norm, a.pre_out, a.post_out, a.res_out = slot[0], slot[1], slot[2], slot[3], slot[4]
    if not identity_pre:
        a.pre = slot[5]
    if form == "post":
        a.y, a.post, a.res, a.residual_out = slot[6], slot[7], slot[8], slot[9]
    if out == "fp8_grid":
        a.grid = slot[10]
    if out in ("mxfp8", "mxfp8_g128"):
        a.codes, a.scales = slot[11], slot[12]
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def validate(d, a):
    return S.lib().mhc_seam_validate(ctypes.byref(d), None if a is None else ctypes.byref(a))


@pytest.mark.parametrize("form", ["post", "no_post"])
@pytest.mark.parametrize("out", ["bf16", "fp8_grid", "mxfp8"])
@pytest.mark.parametrize("idp", [False, True])
def test_complete_pointer_sets_are_accepted(form, out, idp):
    assert validate(desc(), args(form=form, out=out, identity_pre=idp)) == S.OK


def test_desc_rules():
    assert validate(desc(), None) == S.OK
    assert validate(desc(H=500), None) == S.INVALID_ARG          # not a multiple of 64
    assert validate(desc(H=96), None) == S.INVALID_ARG
    assert validate(desc(n=3), None) == S.INVALID_ARG
    assert validate(desc(fn=None), None) == S.INVALID_ARG
    assert validate(desc(eps=-1.0), None) == S.INVALID_ARG
    assert validate(desc(H=5120, max_tokens=52429), None) == S.INVALID_ARG  # 2^31 bytes
    assert validate(desc(H=5120, max_tokens=52428), None) == S.OK
    assert validate(desc(ksplit=9), None) == S.INVALID_ARG       # > H/64 for H=512
    assert validate(desc(spin_polls=-2), None) == S.INVALID_ARG
    assert validate(desc(spin_polls=-1), None) == S.OK


@pytest.mark.parametrize("field", ["y", "post", "res", "residual_out"])
def test_incomplete_post_mix_inputs_are_errors(field):
    assert validate(desc(), args(**{field: None})) == S.INVALID_ARG
    assert b"required" in S.lib().mhc_seam_last_error()


@pytest.mark.parametrize("field", ["y", "post", "res", "residual_out"])
def test_no_post_rejects_post_mix_inputs(field):
    assert validate(desc(), args(form="no_post", **{field: BASE + (30 << 28)})) == S.INVALID_ARG
    assert b"must be NULL" in S.lib().mhc_seam_last_error()


def test_pre_presence_follows_identity_pre():
    assert validate(desc(), args(pre=None)) == S.INVALID_ARG
    assert validate(desc(), args(identity_pre=True, pre=BASE + (30 << 28))) == S.INVALID_ARG


def test_unshifted_takes_no_pre():
    """The unshifted ordering collapses with the fresh pre: no carried pre,
    no identity_pre."""
    assert validate(desc(), args(unshifted=1, pre=None)) == S.OK
    assert validate(desc(), args(unshifted=1, form="no_post", pre=None)) == S.OK
    assert validate(desc(), args(unshifted=1)) == S.INVALID_ARG            # pre given
    assert validate(desc(), args(unshifted=1, identity_pre=True)) == S.INVALID_ARG
    assert validate(desc(), args(unshifted=2, pre=None)) == S.INVALID_ARG


def test_g128_needs_h_multiple_of_128():
    assert validate(desc(H=512), args(H=512, out="mxfp8_g128")) == S.OK
    assert validate(desc(H=576), args(H=576, out="mxfp8_g128")) == S.INVALID_ARG
    assert validate(desc(H=576), args(H=576, out="mxfp8")) == S.OK


def test_output_pointers_follow_out_dtype():
    assert validate(desc(), args(out="bf16", grid=BASE + (30 << 28))) == S.INVALID_ARG
    assert validate(desc(), args(out="mxfp8", scales=None)) == S.INVALID_ARG
    assert validate(desc(), args(out="fp8_grid", codes=BASE + (30 << 28))) == S.INVALID_ARG


def test_alignment_overlap_and_sizes():
    assert validate(desc(), args(x=BASE + (3 << 28) + 8)) == S.INVALID_ARG
    a = args()
    a.norm = a.x + 64                                   # output inside an input
    assert validate(desc(), a) == S.INVALID_ARG
    assert b"overlaps" in S.lib().mhc_seam_last_error()
    a = args()
    a.pre_out = a.post_out                              # two outputs alias
    assert validate(desc(), a) == S.INVALID_ARG
    a = args()
    a.y = a.x                                           # inputs may alias each other
    assert validate(desc(), a) == S.OK
    assert validate(desc(), args(T=65)) == S.INVALID_ARG           # > max_tokens
    assert validate(desc(), args(T=-1)) == S.INVALID_ARG
    assert validate(desc(), args(T=0)) == S.OK
    assert validate(desc(), args(T=0, x=None, norm=None, y=None)) == S.OK
    assert validate(desc(), args(T=0, form="no_post", y=BASE)) == S.INVALID_ARG
    bad = args()
    bad.form = 7
    assert validate(desc(), bad) == S.INVALID_ARG


def test_status_strings():
    L = S.lib()
    for st in range(6):
        assert L.mhc_seam_status_string(st)
    assert b"unknown" in L.mhc_seam_status_string(99)


def test_plan_modes():
    # decode: one 16-token block split over up to 20 workgroups
    p = S.plan(5120, 4, 256)
    assert p["blocks"] == 1 and p["ksplit"] == 20 and p["row_segs"] == 0
    # half the CUs or fewer: split so that every CU has work
    p = S.plan(5120, 2048, 256)
    assert p["blocks"] == 128 and p["ksplit"] == 2 and p["grid"] == 256 and p["row_segs"] == 0
    assert p["ksplit"] * p["segs_per_split"] >= 80
    # large prefill: whole rows, u on chip
    p = S.plan(5120, 16384, 256)
    assert p == dict(blocks=1024, ksplit=1, segs_per_split=80, grid=1024, row_segs=10,
                     rows_blocks=1024)
    # a short tail after full rounds of the CUs runs split in the same launch
    p = S.plan(5120, 4160, 256)
    assert p["row_segs"] == 10 and p["rows_blocks"] == 256 and p["blocks"] == 260
    assert p["ksplit"] * p["segs_per_split"] >= 80 and p["segs_per_split"] <= 8
    assert p["grid"] == 256 + 4 * p["ksplit"]
    p = S.plan(5120, 16400, 256)
    assert p["rows_blocks"] == 1024 and p["grid"] == 1024 + p["ksplit"]
    # a tail splits into as many workgroups as fit on the CUs at once, at
    # least two per block: 25 x 10 splits of 8 segments (in the whole-row
    # launch), 26 x 9 of 9 segments, 128 x 2 of 40 (in a launch after it)
    p = S.plan(5120, 16 * (256 + 25), 256)
    assert p["rows_blocks"] == 256 and p["ksplit"] == 10 and p["grid"] == 256 + 250
    p = S.plan(5120, 16 * (256 + 26), 256)
    assert p["rows_blocks"] == 256 and p["ksplit"] == 9 and p["segs_per_split"] == 9
    assert p["grid"] == 256 + 26 * 9
    p = S.plan(5120, 6144, 256)
    assert p["rows_blocks"] == 256 and p["ksplit"] == 2 and p["segs_per_split"] == 40
    assert p["grid"] == 512
    # a tail of more than half the CUs stays whole
    p = S.plan(5120, 16 * (256 + 200), 256)
    assert p["rows_blocks"] == p["blocks"] == p["grid"] == 456 and p["ksplit"] == 1
    p = S.plan(512, 8, 256)
    assert p["blocks"] == 1
    # widths without a compiled whole-row kernel take split mode, even unsplit
    p = S.plan(192, 16384, 256)
    assert p["row_segs"] == 0 and p["ksplit"] == 1
    p = S.plan(512, 16384, 256)
    assert p["row_segs"] == 1 and p["ksplit"] == 1
    # split grid: block b, split s is workgroup b * ksplit + s, at most one per CU
    p = S.plan(5120, 384, 256)
    assert p["ksplit"] > 1 and p["grid"] == p["blocks"] * p["ksplit"] <= 256
    # overrides
    p = S.plan(5120, 16384, 256, ksplit=4)
    assert p["ksplit"] == 4 and p["segs_per_split"] == 20 and p["row_segs"] == 0
    p = S.plan(5120, 16384, 256, ksplit=1)
    assert p["ksplit"] == 1 and p["row_segs"] == 10
    p = S.plan(5120, 4160, 256, ksplit=1)          # override: no split tail
    assert p["grid"] == p["rows_blocks"] == 260
    # H whose rows have no whole-row kernel falls back to splits
    p = S.plan(8192, 16384, 256)
    assert p["row_segs"] == 0
    with pytest.raises(S.SeamError):
        S.plan(96, 4, 256)


# ------------------------------------------------------- head reduce rules --

def head_reduce(x, w, T, H, out):
    return S.lib().mhc_head_reduce(x, w, T, H, out, None)


@pytest.mark.parametrize("T,H", [(-1, 512), (4, 0), (4, -8), (4, 12), (4, 100)])
def test_head_reduce_rejects_sizes(T, H):
    assert head_reduce(BASE, None, T, H, BASE + (1 << 30), ) == 1


def test_head_reduce_pointer_rules():
    x, w, out = BASE, BASE + (1 << 28), BASE + (2 << 28)
    assert head_reduce(None, w, 4, 512, out) == 1
    assert head_reduce(x, w, 4, 512, None) == 1
    assert head_reduce(x + 8, w, 4, 512, out) == 1
    assert head_reduce(x, w + 4, 4, 512, out) == 1
    assert head_reduce(x, w, 4, 512, out + 2) == 1
    assert head_reduce(x, w, 4, 512, x + 4 * 512 * 8 - 16) == 1      # out inside x
    assert head_reduce(x, w, 4, 512, w - 16) == 1                     # out over w
    assert "overlaps" in S.lib().mhc_seam_last_error().decode()
    assert head_reduce(x, w, (1 << 62), 512, out) == 1
    assert head_reduce(None, None, 0, 512, None) == 0                 # nothing to do


# ------------------------------------------------------------- gemm rules --

def gemm(a, sa, b, sb, T, N, K, out):
    return S.lib().mhc_mxfp8_gemm(a, sa, b, sb, T, N, K, out, None)


@pytest.mark.parametrize("T,N,K", [(-1, 16, 128), (4, 0, 128), (4, 16, 0), (4, 16, 96),
                                   (4, 16, 8320)])
def test_gemm_rejects_sizes(T, N, K):
    assert gemm(BASE, BASE + (1 << 28), BASE + (2 << 28), BASE + (3 << 28), T, N, K,
                BASE + (4 << 28)) == 1


def test_gemm_pointer_rules():
    a, sa, b, sb, out = (BASE + (k << 28) for k in range(5))
    assert gemm(a, sa, b, sb, 0, 16, 128, None) == 0                 # nothing to do
    assert gemm(None, sa, b, sb, 4, 16, 128, out) == 1
    assert gemm(a + 8, sa, b, sb, 4, 16, 128, out) == 1              # a not 16-byte aligned
    assert gemm(a, sa + 2, b, sb, 4, 16, 128, out) == 1              # scales not 4-byte aligned
    assert gemm(a, sa, b, sb, 4, 16, 128, a + 64) == 1               # out over a
    assert "overlaps" in S.lib().mhc_seam_last_error().decode()


def test_gemm_blocks_by_token_count():
    """The consumer GEMM's output blocks and LDS stages by token count at
    N = K = 5120 on 256 CUs: the shapes measured fastest there, across every
    change of shape (16 x 32 up to 128 x 128 where one round of 128 x 128
    blocks covers the output, chosen by the bytes each CU streams; 128 x 256
    in one round; then 256 x 256, or 128 x 128 two per CU)."""
    want = {1: (16, 32, 6), 16: (16, 32, 6), 17: (32, 32, 6), 32: (32, 32, 6),
            33: (64, 32, 3), 64: (64, 32, 3), 65: (64, 64, 3), 192: (64, 64, 3),
            193: (128, 64, 3), 384: (128, 64, 3), 385: (128, 128, 3), 768: (128, 128, 3),
            769: (128, 256, 3), 1536: (128, 256, 3), 1537: (256, 256, 2), 2048: (256, 256, 2),
            3072: (256, 256, 2), 4096: (128, 128, 2), 6144: (256, 256, 2),
            16384: (256, 256, 2)}
    for T, shape in want.items():
        assert S.gemm_blocks(T, 5120, 256) == shape, T


def test_gemm_blocks_few_tokens_many_columns():
    """T <= 32 keeps the smallest blocks past one round of the CUs (measured
    faster there than one workgroup per 16 weight columns), and fewer CUs
    move the choice to smaller blocks earlier."""
    assert S.gemm_blocks(4, 32768, 256) == (16, 32, 6)
    assert S.gemm_blocks(20, 16400, 256) == (32, 32, 6)
    assert S.gemm_blocks(384, 5120, 256) == (128, 64, 3)
    assert S.gemm_blocks(384, 5120, 128) != (128, 64, 3)


@pytest.mark.parametrize("T,N,cus", [(0, 5120, 256), (4, 0, 256), (4, 5120, 0),
                                     (1 << 31, 5120, 256)])
def test_gemm_blocks_rejects(T, N, cus):
    with pytest.raises(S.SeamError):
        S.gemm_blocks(T, N, cus)
