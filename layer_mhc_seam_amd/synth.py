"""Seeded synthetic seam inputs, shared by the tests, the smoke check and the
benchmark.

This module only draws random numbers and rounds them to the storage types;
it holds none of the seam's arithmetic.  The carried gates are returned as
the raw normal draws ``z_pre``, ``z_post`` and ``z_res``: the consumer turns
them into pre = sigmoid(z), post = 2 sigmoid(z) and res = Sinkhorn(exp(z)),
which is how a previous seam produces them.

Recipe (one CPU ``torch.Generator`` seeded with ``seed``; draw order x, y,
z_pre, z_post, z_res, gamma, fn, bias; every tensor is drawn for every form
so the stream of numbers does not depend on the form):
  x     = bf16(N(0,1))              [T,4,H]
  y     = bf16(N(0,1))              [T,H]   (x 2^8 on tokens t % 64 == 0 when
                                             ``y_boost_every`` is 64)
  z_pre, z_post ~ N(0,1) [T,4];  z_res ~ N(0,1) [T,4,4]
  gamma = bf16(1 + 0.1 N(0,1))      [H]
  fn    = f32(N(0,1) / sqrt(4H))    [4H,24]
  bias  = f32(0.1 N(0,1))           [24]

The workloads are the seam shapes the Mega-mHC pages measure at H = 5120
("[FlyDSL] Single-launch Mega-mHC on gfx950", performance tables), plus a
small H = 512 case for the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    form: str          # "post" | "no_post"
    out_dtype: str     # "bf16" | "fp8_grid" | "mxfp8"
    y_boost_every: int = 0
    identity_pre: bool = False


WORKLOADS = {
    "tiny_post_bf16": Workload("tiny_post_bf16", 8, 512, "post", "bf16"),
    "decode_post_bf16": Workload("decode_post_bf16", 4, 5120, "post", "bf16"),
    "prefill384_post_mxfp8": Workload("prefill384_post_mxfp8", 384, 5120,
                                      "post", "mxfp8", y_boost_every=64),
    "tail4160_nopost_bf16": Workload("tail4160_nopost_bf16", 4160, 5120,
                                     "no_post", "bf16"),
    "prefill16k_post_fp8grid": Workload("prefill16k_post_fp8grid", 16384,
                                        5120, "post", "fp8_grid"),
}


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def draw(T: int, H: int, seed: int = 0, y_boost_every: int = 0) -> dict:
    """Seeded inputs for one seam; bf16 tensors as uint16 bit patterns."""
    g = torch.Generator().manual_seed(seed)
    x = _bf16_bits(torch.randn(T, 4, H, generator=g))
    yf = torch.randn(T, H, generator=g)
    if y_boost_every:
        yf[::y_boost_every] *= 256.0          # exact in bf16
    y = _bf16_bits(yf)
    z_pre = torch.randn(T, 4, generator=g).numpy()
    z_post = torch.randn(T, 4, generator=g).numpy()
    z_res = torch.randn(T, 4, 4, generator=g).numpy()
    gamma = _bf16_bits(1.0 + 0.1 * torch.randn(H, generator=g))
    fn = (torch.randn(4 * H, 24, generator=g) / math.sqrt(4 * H)).numpy()
    bias = (0.1 * torch.randn(24, generator=g)).numpy()
    return dict(x=x, y=y, z_pre=z_pre, z_post=z_post, z_res=z_res,
                gamma=gamma, fn=fn.astype(np.float32),
                bias=bias.astype(np.float32))


def draw_workload(w: Workload, seed: int = 0) -> dict:
    return draw(w.T, w.H, seed=seed, y_boost_every=w.y_boost_every)
