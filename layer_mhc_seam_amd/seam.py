"""Thin ctypes binding of libmhc_seam.so (C ABI in include/mhc_seam.h).

Argument marshalling only: every step of the seam runs in the library's HIP
kernels.  PyTorch supplies device memory and the stream.  The library is
loaded on first use; if it is missing this raises instead of computing
anything another way.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MHC_SEAM_LIB") or os.path.join(HERE, "libmhc_seam.so")

OK, INVALID_ARG, UNSUPPORTED_DEVICE, OUT_OF_MEMORY, HIP_ERROR, CAPTURE_ALLOC = range(6)
FORMS = {"post": 0, "no_post": 1}
OUT_DTYPES = {"bf16": 0, "fp8_grid": 1, "mxfp8": 2, "mxfp8_g128": 3}

_P = ctypes.c_void_p


class Desc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("n", ctypes.c_int32), ("eps", ctypes.c_float),
                ("sinkhorn_iters", ctypes.c_int32), ("fn", _P), ("gamma", _P), ("bias", _P),
                ("max_tokens", ctypes.c_int64), ("device", ctypes.c_int32),
                ("ksplit", ctypes.c_int32), ("spin_polls", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 6)]


class Args(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("form", ctypes.c_int32),
                ("identity_pre", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("unshifted", ctypes.c_int32),
                ("x", _P), ("y", _P), ("pre", _P), ("post", _P), ("res", _P),
                ("residual_out", _P), ("norm", _P), ("grid", _P), ("codes", _P),
                ("scales", _P), ("pre_out", _P), ("post_out", _P), ("res_out", _P)]


class Plan(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_int32), ("ksplit", ctypes.c_int32),
                ("segs_per_split", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("row_segs", ctypes.c_int32), ("rows_blocks", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


EXPORTS = ("mhc_seam_create", "mhc_seam_run", "mhc_seam_run_noalloc", "mhc_seam_destroy",
           "mhc_seam_validate",
           "mhc_seam_plan_for", "mhc_seam_status_string", "mhc_seam_last_error",
           "mhc_seam_copy", "mhc_stream_mix", "mhc_seam_quantize", "mhc_head_reduce",
           "mhc_mxfp8_gemm", "mhc_mxfp8_gemm_blocks")

_lib = None


class SeamError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"mhc_seam status {status}: {message}")
        self.status = status


def lib():
    """Load libmhc_seam.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m layer_mhc_seam_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    L.mhc_seam_create.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(_P)]
    L.mhc_seam_run.argtypes = [_P, ctypes.POINTER(Args), _P]
    L.mhc_seam_run_noalloc.argtypes = [_P, ctypes.POINTER(Args), _P]
    L.mhc_seam_destroy.argtypes = [_P]
    L.mhc_seam_validate.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Args)]
    L.mhc_seam_plan_for.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.POINTER(Plan)]
    L.mhc_seam_status_string.argtypes = [ctypes.c_int]
    L.mhc_seam_status_string.restype = ctypes.c_char_p
    L.mhc_seam_last_error.restype = ctypes.c_char_p
    L.mhc_seam_copy.argtypes = [_P, _P, ctypes.c_size_t, _P]
    L.mhc_stream_mix.argtypes = [_P, ctypes.c_size_t, _P, ctypes.c_size_t, _P]
    L.mhc_head_reduce.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P]
    L.mhc_mxfp8_gemm.argtypes = [_P, _P, _P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 _P, _P]
    L.mhc_seam_quantize.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    _P, _P, _P, _P]
    L.mhc_mxfp8_gemm_blocks.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32)]
    for name in ("mhc_seam_create", "mhc_seam_run", "mhc_seam_run_noalloc", "mhc_seam_destroy",
                 "mhc_seam_validate",
                 "mhc_seam_plan_for", "mhc_seam_copy", "mhc_stream_mix", "mhc_seam_quantize",
                 "mhc_mxfp8_gemm_blocks"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status):
    if status != OK:
        raise SeamError(status, lib().mhc_seam_last_error().decode())


def plan(H, T, cu_count=256, ksplit=0):
    """Launch plan the library would use (host only)."""
    p = Plan()
    _check(lib().mhc_seam_plan_for(H, T, cu_count, ksplit, ctypes.byref(p)))
    return dict(blocks=p.blocks, ksplit=p.ksplit, segs_per_split=p.segs_per_split,
                grid=p.grid, row_segs=p.row_segs, rows_blocks=p.rows_blocks)


def gemm_blocks(T, N, cu_count=256):
    """Output blocks (TM, TN) and LDS stages mhc_mxfp8_gemm launches for
    T x N on cu_count CUs (host only)."""
    tm, tn, st = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().mhc_mxfp8_gemm_blocks(T, N, cu_count, ctypes.byref(tm), ctypes.byref(tn),
                                       ctypes.byref(st)))
    return tm.value, tn.value, st.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Seam:
    """A seam handle: packed fn, gamma and bias for one width H.

    fn f32 [4H,24], gamma bf16 [H], bias f32 [24]: device tensors, copied by
    the library at creation.
    """

    def __init__(self, fn, gamma, bias, *, max_tokens, eps=1e-6, sinkhorn_iters=20,
                 ksplit=0, spin_polls=0):
        import torch
        H = gamma.shape[0]
        self._check_tensor("fn", fn, torch.float32, (4 * H, 24))
        self._check_tensor("gamma", gamma, torch.bfloat16, (H,))
        self._check_tensor("bias", bias, torch.float32, (24,))
        d = Desc()
        d.H, d.n, d.eps, d.sinkhorn_iters = H, 4, eps, sinkhorn_iters
        d.fn, d.gamma, d.bias = fn.data_ptr(), gamma.data_ptr(), bias.data_ptr()
        d.max_tokens = max_tokens
        d.device = fn.device.index if fn.device.index is not None else torch.cuda.current_device()
        d.ksplit = ksplit
        d.spin_polls = spin_polls
        h = _P()
        _check(lib().mhc_seam_create(ctypes.byref(d), ctypes.byref(h)))
        self._h = h
        self.H, self.max_tokens, self.device = H, max_tokens, fn.device

    @staticmethod
    def _check_tensor(name, t, dtype, shape):
        if t is None:
            raise ValueError(f"{name} is required")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def run(self, x, y=None, pre=None, post=None, res=None, *, form="post",
            identity_pre=False, out_dtype="bf16", unshifted=False, out=None, stream=None,
            noalloc=False):
        """Enqueue one seam on `stream` (default: torch's current stream).

        noalloc: call mhc_seam_run_noalloc, whose split-mode scratch is the
        library's fixed per-GPU array (pass every output in `out` to keep
        the call free of allocations).

        unshifted: gates from x' first, then the collapse with the fresh pre
        (pre_out) instead of a carried one; takes no pre.
        Returns a dict of output tensors (allocated unless given in `out`):
        residual_out (post form), norm, grid (fp8_grid), codes and scales
        (mxfp8, uint8), pre_out, post_out, res_out.
        """
        import torch
        T, H = x.shape[0], self.H
        dev = x.device
        post_form = form == "post"
        self._check_tensor("x", x, torch.bfloat16, (T, 4, H))
        if post_form:
            self._check_tensor("y", y, torch.bfloat16, (T, H))
            self._check_tensor("post", post, torch.float32, (T, 4))
            self._check_tensor("res", res, torch.float32, (T, 4, 4))
        elif any(v is not None for v in (y, post, res)):
            raise ValueError("no_post form takes no y, post or res")
        if unshifted:
            if pre is not None or identity_pre:
                raise ValueError("unshifted takes no pre and no identity_pre")
        elif not identity_pre:
            self._check_tensor("pre", pre, torch.float32, (T, 4))
        elif pre is not None:
            raise ValueError("identity_pre takes no pre")
        o = dict(out or {})

        def want(name, shape, dtype):
            if name not in o:
                o[name] = torch.empty(shape, dtype=dtype, device=dev)
            self._check_tensor(name, o[name], dtype, shape)

        if post_form:
            want("residual_out", (T, 4, H), torch.bfloat16)
        want("norm", (T, H), torch.bfloat16)
        if out_dtype == "fp8_grid":
            want("grid", (T, H), torch.bfloat16)
        if out_dtype in ("mxfp8", "mxfp8_g128"):
            want("codes", (T, H), torch.uint8)
            want("scales", (T, H // (128 if out_dtype == "mxfp8_g128" else 32)), torch.uint8)
        want("pre_out", (T, 4), torch.float32)
        want("post_out", (T, 4), torch.float32)
        want("res_out", (T, 4, 4), torch.float32)
        a = Args()
        a.T, a.form, a.identity_pre = T, FORMS[form], int(bool(identity_pre))
        a.out_dtype = OUT_DTYPES[out_dtype]
        a.unshifted = int(bool(unshifted))
        a.x, a.y, a.pre, a.post, a.res = (_ptr(x), _ptr(y), _ptr(pre), _ptr(post), _ptr(res))
        a.residual_out = _ptr(o.get("residual_out"))
        a.norm, a.grid = _ptr(o["norm"]), _ptr(o.get("grid"))
        a.codes, a.scales = _ptr(o.get("codes")), _ptr(o.get("scales"))
        a.pre_out, a.post_out = _ptr(o["pre_out"]), _ptr(o["post_out"])
        a.res_out = _ptr(o["res_out"])
        entry = lib().mhc_seam_run_noalloc if noalloc else lib().mhc_seam_run
        _check(entry(self._h, ctypes.byref(a), _stream_handle(stream)))
        return o

    def close(self):
        if getattr(self, "_h", None):
            _check(lib().mhc_seam_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quantize(src, *, group=32, codes=True, grid=True, stream=None):
    """MXFP8 quantisation of a bf16 [rows, H] device tensor in groups of
    `group` (32 or 128) elements with the seam's device quantiser.  Returns
    (codes u8, scales u8 [rows, H/group], grid bf16); the parts not asked for
    are None."""
    import torch
    rows, H = src.shape
    if src.dtype != torch.bfloat16 or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous bf16 device tensor")
    c = torch.empty((rows, H), dtype=torch.uint8, device=src.device) if codes else None
    sc = torch.empty((rows, H // group), dtype=torch.uint8, device=src.device) if codes else None
    g = torch.empty_like(src) if grid else None
    _check(lib().mhc_seam_quantize(_ptr(src), rows, H, group, _ptr(c), _ptr(sc), _ptr(g),
                                   _stream_handle(stream)))
    return c, sc, g


def copy(dst, src, nbytes, stream=None):
    """The library's 16-byte non-temporal device copy (bandwidth ceiling)."""
    _check(lib().mhc_seam_copy(_ptr(dst), _ptr(src), nbytes, _stream_handle(stream)))


def stream_mix(dst, dst_bytes, src, src_bytes, stream=None):
    """The library's read-src_bytes / write-dst_bytes streaming kernel (the
    copy ceiling at another read/write mix)."""
    _check(lib().mhc_stream_mix(_ptr(dst), dst_bytes, _ptr(src), src_bytes,
                                _stream_handle(stream)))


def head_reduce(x, w=None, *, out=None, stream=None):
    """n -> 1 reduction of the streams, stored: out[t, h] = bf16(sum_i
    w[t, i] * x[t, i, h]) (the seam's collapse chain) on the device.
    x bf16 [T, 4, H], w f32 [T, 4] or None for weights of 1/4.  Returns
    out bf16 [T, H] (allocated unless given)."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 3 \
            or x.shape[1] != 4:
        raise ValueError("x must be a contiguous bf16 [T, 4, H] device tensor")
    T, _, H = x.shape
    if w is not None and (w.dtype != torch.float32 or tuple(w.shape) != (T, 4)
                          or not w.is_contiguous() or w.device != x.device):
        raise ValueError("w must be a contiguous f32 [T, 4] tensor on x's device")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (T, H) or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("out must be a contiguous bf16 [T, H] tensor on x's device")
    _check(lib().mhc_head_reduce(_ptr(x), _ptr(w), T, H, _ptr(out), _stream_handle(stream)))
    return out


def mxfp8_gemm(a, a_scales, b, b_scales, *, out=None, stream=None):
    """Consumer GEMM of MXFP8 operands along K on the device: out[t, n] =
    bf16(sum_k a(t, k) b(n, k)).  a u8 [T, K] e4m3fn codes with a_scales u8
    [T, K/32] ue8m0 (the seam's mxfp8 output as it is), b u8 [N, K] and
    b_scales u8 [N, K/32] (weights).  Returns out bf16 [T, N]."""
    import torch
    T, K = a.shape
    N = b.shape[0]
    for name, t, shape in (("a", a, (T, K)), ("a_scales", a_scales, (T, K // 32)),
                           ("b", b, (N, K)), ("b_scales", b_scales, (N, K // 32))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous() \
                or t.device != a.device or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous u8 {shape} device tensor")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=a.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (T, N) or not out.is_contiguous() \
            or out.device != a.device:
        raise ValueError("out must be a contiguous bf16 [T, N] tensor on a's device")
    _check(lib().mhc_mxfp8_gemm(_ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales), T, N, K,
                                _ptr(out), _stream_handle(stream)))
    return out
