"""CPU oracle for the fused, delayed mHC seam -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
built from ``mhc_oracle.c`` by ``oracle/build.py``) with numpy marshalling;
all arithmetic happens in the C file, whose header states the definitions,
rounding points and the page passages they follow:

  "[FlyDSL] Single-launch Mega-mHC on gfx950": Motivation (the seam's steps),
  Kernel Architecture (their order, the out_dtype outputs), Limitations
  (inf/NaN groups unspecified), Test Plan (forms, crafted quantiser groups).

bf16 tensors are carried as ``numpy.uint16`` bit patterns, fp8 codes and
ue8m0 scales as ``numpy.uint8``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB lets the mutation tests load a deliberately broken build
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_seam.argtypes = [_I64, _I32, _I64, _I64, _I32, _I32, _I32,
                                ctypes.c_float, _I32] + [_P] * 14
    lib.oracle_seam.restype = ctypes.c_int
    lib.oracle_quantize.argtypes = [_I64, _I32, _P, _P, _P, _P]
    lib.oracle_quantize.restype = ctypes.c_int
    lib.oracle_quantize_groups.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P]
    lib.oracle_quantize_groups.restype = ctypes.c_int
    lib.oracle_head_reduce.argtypes = [_I64, _I32, _P, _P, _P]
    lib.oracle_mxfp8_gemm.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P, _P]
    lib.oracle_mxfp8_gemm.restype = ctypes.c_int
    lib.oracle_head_reduce.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [_I32]
    lib.oracle_f32_to_bf16.argtypes = [_I64, _P, _P]
    lib.oracle_e4m3_encode_scaled.argtypes = [_I64, _P, _I32, _P]
    lib.oracle_e4m3_decode.argtypes = [_I64, _P, _P]
    lib.oracle_scale_exp.argtypes = [_I64, _P, _P]
    lib.oracle_sinkhorn.argtypes = [_I64, _P, _I32, _P]
    lib.oracle_sigmoid.argtypes = [_I64, _P, _P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's following calls (CPU-baseline timing)."""
    _load().oracle_set_threads(int(n))


def seam(x, y, pre, post, res, fn, gamma, bias, *, post_form=True,
         identity_pre=False, unshifted=False, eps=1e-6, iters=20, t0=0, t1=None):
    """One seam over tokens [t0, t1) (default: all).

    x [T,4,H] u16 (bf16 bits), y [T,H] u16 or None, pre/post [T,4] f32,
    res [T,4,4] f32, fn [4H,24] f32, gamma [H] u16, bias [24] f32.
    unshifted: gates first, then the collapse with the fresh pre (pre_out)
    instead of the carried one; pre must be None.
    Returns a dict with residual_out (post form only), norm, pre_out,
    post_out, res_out; rows outside [t0, t1) are zero.
    """
    lib = _load()
    x = _c(x, np.uint16)
    T, n, H = x.shape
    assert n == 4
    t1 = T if t1 is None else t1
    fn = _c(fn, np.float32)
    assert fn.shape == (4 * H, 24)
    gamma = _c(gamma, np.uint16)
    bias = _c(bias, np.float32)
    if post_form:
        y, post, res = _c(y, np.uint16), _c(post, np.float32), _c(res, np.float32)
        assert y.shape == (T, H) and post.shape == (T, 4) and res.shape == (T, 4, 4)
        resid = np.zeros((T, 4, H), np.uint16)
    else:
        y = post = res = resid = None
    if unshifted:
        assert pre is None and not identity_pre, "unshifted takes no pre"
    elif not identity_pre:
        pre = _c(pre, np.float32)
        assert pre.shape == (T, 4)
    else:
        pre = None
    norm = np.zeros((T, H), np.uint16)
    pre_out = np.zeros((T, 4), np.float32)
    post_out = np.zeros((T, 4), np.float32)
    res_out = np.zeros((T, 4, 4), np.float32)
    work = np.zeros(lib.oracle_max_threads() * 5 * H, np.float32)
    rc = lib.oracle_seam(T, H, t0, t1, int(bool(post_form)),
                         int(bool(identity_pre)), int(bool(unshifted)), float(eps), int(iters),
                         _ptr(x), _ptr(y), _ptr(pre), _ptr(post), _ptr(res),
                         _ptr(fn), _ptr(gamma), _ptr(bias), _ptr(resid),
                         _ptr(norm), _ptr(pre_out), _ptr(post_out),
                         _ptr(res_out), _ptr(work))
    if rc != 0:
        raise ValueError("oracle_seam rejected its sizes")
    out = dict(norm=norm, pre_out=pre_out, post_out=post_out, res_out=res_out)
    if post_form:
        out["residual_out"] = resid
    return out


def head_reduce(x, w=None):
    """n -> 1 reduction of the streams: bf16(sum_i w[t,i] * x[t,i,:]) with the
    collapse's binary32 chain; x [T,4,H] u16 (bf16 bits), w [T,4] f32 or None
    for weights of 1/4.  Returns out [T,H] u16."""
    lib = _load()
    x = _c(x, np.uint16)
    T, n, H = x.shape
    assert n == 4
    w = _c(w, np.float32)
    if w is not None:
        assert w.shape == (T, 4)
    out = np.zeros((T, H), np.uint16)
    if lib.oracle_head_reduce(T, H, _ptr(x), _ptr(w), _ptr(out)) != 0:
        raise ValueError("oracle_head_reduce rejected its sizes")
    return out


def mxfp8_gemm(a_codes, a_scales, b_codes, b_scales):
    """The consumer GEMM of MXFP8 operands along K: out[t, n] = sum_k
    a[t, k] b[n, k] with a = e4m3(a_codes) 2^(a_scales[t, k/32] - 127) [T, K]
    and b likewise [N, K], in binary64.  Returns (out, absum) float64 [T, N],
    absum = sum_k |a b|."""
    lib = _load()
    a_codes, b_codes = _c(a_codes, np.uint8), _c(b_codes, np.uint8)
    a_scales, b_scales = _c(a_scales, np.uint8), _c(b_scales, np.uint8)
    T, K = a_codes.shape
    N = b_codes.shape[0]
    assert b_codes.shape == (N, K) and K % 32 == 0
    assert a_scales.shape == (T, K // 32) and b_scales.shape == (N, K // 32)
    out = np.zeros((T, N), np.float64)
    absum = np.zeros((T, N), np.float64)
    if lib.oracle_mxfp8_gemm(T, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(b_codes),
                             _ptr(b_scales), _ptr(out), _ptr(absum)) != 0:
        raise ValueError("oracle_mxfp8_gemm rejected its sizes")
    return out, absum


def quantize(norm, group=32):
    """ue8m0 + e4m3 quantisation of a bf16 norm [T,H] (u16 bits) in groups of
    `group` (32 or 128) contiguous elements.

    Returns (codes u8 [T,H], scales u8 [T,H/group], grid u16 [T,H]).
    """
    lib = _load()
    norm = _c(norm, np.uint16)
    T, H = norm.shape
    codes = np.zeros((T, H), np.uint8)
    scales = np.zeros((T, H // group), np.uint8)
    grid = np.zeros((T, H), np.uint16)
    if lib.oracle_quantize_groups(T, H, group, _ptr(norm), _ptr(codes), _ptr(scales),
                                  _ptr(grid)) != 0:
        raise ValueError("oracle_quantize_groups rejected its sizes")
    return codes, scales, grid


def f32_to_bf16(a):
    """binary32 -> bf16 bits, round to nearest even."""
    a = _c(a, np.float32)
    out = np.zeros(a.shape, np.uint16)
    _load().oracle_f32_to_bf16(a.size, _ptr(a), _ptr(out))
    return out


def e4m3_encode_scaled(v_bf16, k):
    """e4m3fn codes of bf16 values scaled by 2^-k."""
    v = _c(v_bf16, np.uint16)
    out = np.zeros(v.shape, np.uint8)
    _load().oracle_e4m3_encode_scaled(v.size, _ptr(v), int(k), _ptr(out))
    return out


def e4m3_decode(codes):
    c = _c(codes, np.uint8)
    out = np.zeros(c.shape, np.float64)
    _load().oracle_e4m3_decode(c.size, _ptr(c), _ptr(out))
    return out


def scale_exp(amax):
    a = _c(amax, np.float64)
    out = np.zeros(a.shape, np.int32)
    _load().oracle_scale_exp(a.size, _ptr(a), _ptr(out))
    return out


def sinkhorn(logits, iters=20):
    """Sinkhorn of exp(logits) for [..., 4, 4] logits (float64 result)."""
    lg = _c(logits, np.float64)
    shape = lg.shape
    assert shape[-2:] == (4, 4)
    out = np.zeros(shape, np.float64)
    _load().oracle_sinkhorn(lg.size // 16, _ptr(lg), int(iters), _ptr(out))
    return out


def sigmoid(v):
    v = _c(v, np.float64)
    out = np.zeros(v.shape, np.float64)
    _load().oracle_sigmoid(v.size, _ptr(v), _ptr(out))
    return out


def gate_inputs(z_pre, z_post, z_res, iters=20):
    """Carried gates from raw normal draws, as the previous seam makes them:
    pre = sigmoid(z), post = 2*sigmoid(z), res = Sinkhorn(exp(z)); f32."""
    pre = sigmoid(z_pre).astype(np.float32)
    post = (2.0 * sigmoid(z_post)).astype(np.float32)
    res = sinkhorn(np.asarray(z_res, np.float64).reshape(-1, 4, 4),
                   iters).astype(np.float32).reshape(np.shape(z_res))
    return pre, post, res
