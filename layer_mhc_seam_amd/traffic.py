"""Algorithmic HBM bytes of one seam (each tensor read or written once).

Reads: x (8TH), y (2TH, post form), the carried gates (pre 16T unless
identity_pre; post 16T and res 64T in the post form), fn (384H), gamma (2H),
bias (96).  Writes: residual_out (8TH, post form), norm (2TH), grid (2TH,
fp8_grid) or codes + scales (TH + TH/32, mxfp8), next gates (96T).

The pages' own convention counts only x, y, residual_out and norm: 20TH for
a bf16 post seam and 22TH with the fp8 grid ("[FlyDSL] Single-launch
Mega-mHC on gfx950", Realistic Bandwidth Ceiling); ``page_bytes`` gives it.
"""


def seam_bytes(T, H, form="post", out_dtype="bf16", identity_pre=False, unshifted=False):
    """(read_bytes, write_bytes) of one seam.

    unshifted: the collapse needs the whole row's fresh pre, and a block's x'
    does not fit on chip, so x' (8TH) and the fresh pre (16T) are read back
    once more; no carried pre is read.
    """
    post = form == "post"
    rd = 8 * T * H + 384 * H + 2 * H + 96
    if post:
        rd += 2 * T * H + 16 * T + 64 * T
    if unshifted:
        rd += 8 * T * H + 16 * T
    elif not identity_pre:
        rd += 16 * T
    wr = 2 * T * H + 96 * T
    if post:
        wr += 8 * T * H
    if out_dtype == "fp8_grid":
        wr += 2 * T * H
    elif out_dtype == "mxfp8":
        wr += T * H + T * (H // 32)
    elif out_dtype == "mxfp8_g128":
        wr += T * H + T * (H // 128)
    return rd, wr


def total_bytes(T, H, form="post", out_dtype="bf16", identity_pre=False, unshifted=False):
    r, w = seam_bytes(T, H, form, out_dtype, identity_pre, unshifted)
    return r + w


def page_bytes(T, H, form="post", out_dtype="bf16"):
    """The pages' convention: x, y, residual_out, norm (and the grid)."""
    b = (20 if form == "post" else 10) * T * H
    if out_dtype == "fp8_grid":
        b += 2 * T * H
    return b
