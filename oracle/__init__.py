"""CPU oracle for NVFP4 block-scaled quantization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, see its header for the
sources and the precision rules); this module only marshals numpy arrays.
Inputs are bfloat16 bit patterns (``uint16``) or float32 arrays; bf16 is
widened to float32 exactly (the bits shifted into the high half).

The UE5M3 scale format is pinned to what the "UE5M3" blog fixes (unsigned,
5 exponent and 3 mantissa bits, its emulation's bias and mantissa rounding);
its subnormals, NaN code and largest code remain a reading (the E4M3FN
conventions carried over).
"""
import ctypes
import os

import numpy as np

from . import build as _build

FMT_E4M3, FMT_UE5M3 = 0, 1
SELECT_6, SELECT_4OVER6 = 0, 1
SELECT_4OVER6_MAE, SELECT_4OVER6_MAXERR, SELECT_SWEEP = 2, 3, 4
ROUND_RNE, ROUND_SR = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# NVFP4_ORACLE_LIB names another build of nvfp4_oracle.c to load instead: the
# test that plants a mistake in a copy of the oracle runs the pins against it
_LIB_OVERRIDE = os.environ.get("NVFP4_ORACLE_LIB")
_LIB_PATH = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "nvfp4_oracle.c")
    if not _LIB_OVERRIDE and (not os.path.exists(_LIB_PATH) or
                              os.path.getmtime(_LIB_PATH) < os.path.getmtime(src)):
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.or_e2m1_value.restype = ctypes.c_double
    lib.or_e2m1_value.argtypes = [ctypes.c_int]
    lib.or_e2m1_code.restype = ctypes.c_int
    lib.or_e2m1_code.argtypes = [ctypes.c_float]
    lib.or_e2m1_code_sr.restype = ctypes.c_int
    lib.or_e2m1_code_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
    lib.or_scale_decode.restype = ctypes.c_double
    lib.or_scale_decode.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.or_scale_encode.restype = ctypes.c_int
    lib.or_scale_encode.argtypes = [ctypes.c_int, ctypes.c_float]
    lib.or_scale_nan_code.restype = ctypes.c_int
    lib.or_scale_nan_code.argtypes = [ctypes.c_int]
    lib.or_fmix32.restype = ctypes.c_uint32
    lib.or_fmix32.argtypes = [ctypes.c_uint32]
    lib.or_sr_hash.restype = ctypes.c_uint32
    lib.or_sr_hash.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.or_tensor_amax.restype = ctypes.c_float
    lib.or_tensor_amax.argtypes = [_f32p, _i64]
    lib.or_alpha.restype = ctypes.c_float
    lib.or_alpha.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.or_quantize.restype = ctypes.c_int
    lib.or_quantize.argtypes = [_f32p, _i64, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                _u8p, _u8p, _u64p, _f32p, _f32p]
    lib.or_dequantize.restype = ctypes.c_int
    lib.or_dequantize.argtypes = [_u8p, _u8p, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                  ctypes.c_int, _f32p, _u16p, _f32p]
    lib.or_sse.restype = ctypes.c_double
    lib.or_sse.argtypes = [_f32p, _f32p, _i64]
    lib.or_f32_to_bf16.restype = ctypes.c_uint16
    lib.or_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.or_fakequant_fwd.restype = ctypes.c_int
    lib.or_fakequant_fwd.argtypes = [_f32p, _i64, _i64, _f32p, _f32p, _f32p]
    lib.or_fakequant_bwd.restype = ctypes.c_int
    lib.or_fakequant_bwd.argtypes = [_f32p, _f32p, _i64, _i64, _f32p, _f32p, _f32p, _f32p, _f32p]
    lib.or_fakequant_fwd_amax.restype = ctypes.c_int
    lib.or_fakequant_fwd_amax.argtypes = [_f32p, _i64, _i64, _f32p, _f32p, _f32p]
    lib.or_fakequant_bwd_amax.restype = ctypes.c_int
    lib.or_fakequant_bwd_amax.argtypes = [_f32p, _f32p, _i64, _i64, _f32p, _f32p, _f32p, _f32p,
                                          _f32p]
    lib.or_row_amax.restype = ctypes.c_int
    lib.or_row_amax.argtypes = [_f32p, _i64, _i64, _f32p]
    lib.or_quantize_rowscaled.restype = ctypes.c_int
    lib.or_quantize_rowscaled.argtypes = [_f32p, _i64, _i64, _i64, _f32p, ctypes.c_float,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_uint64, _u8p, _u8p, _u64p]
    lib.or_dequantize_rowscaled.restype = ctypes.c_int
    lib.or_dequantize_rowscaled.argtypes = [_u8p, _u8p, _i64, _i64, _f32p, ctypes.c_float,
                                            ctypes.c_int, _f32p, _u16p, _f32p]
    lib.or_quantize_2d.restype = ctypes.c_int
    lib.or_quantize_2d.argtypes = [_f32p, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_int, _u8p, _u8p, _u8p, _u8p]
    lib.or_dequantized_amax.restype = ctypes.c_float
    lib.or_dequantized_amax.argtypes = [_u8p, _u8p, _i64, _i64, ctypes.c_float, _f32p,
                                        ctypes.c_float, ctypes.c_int]
    lib.or_requant_nvfp4_t.restype = ctypes.c_int
    lib.or_requant_nvfp4_t.argtypes = [_u8p, _u8p, _i64, _i64, ctypes.c_float, _f32p,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_uint64, _i64, _u8p,
                                       _u8p]
    lib.or_requant_mxfp8_t.restype = ctypes.c_int
    lib.or_requant_mxfp8_t.argtypes = [_u8p, _u8p, _i64, _i64, ctypes.c_float, _f32p,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_uint64, _i64, _u8p,
                                       _u8p]
    lib.or_e4m3_code_sr.restype = ctypes.c_int
    lib.or_e4m3_code_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
    lib.or_mxfp8_quantize_sr.restype = ctypes.c_int
    lib.or_mxfp8_quantize_sr.argtypes = [_f32p, _i64, _i64, _i64, ctypes.c_uint64, _u8p, _u8p]
    lib.or_mxfp8_dequantize.restype = ctypes.c_int
    lib.or_mxfp8_dequantize.argtypes = [_u8p, _u8p, _i64, _i64, _f32p]
    lib.or_rht_signs.restype = ctypes.c_uint32
    lib.or_rht_signs.argtypes = [ctypes.c_uint64]
    lib.or_rht16.restype = None
    lib.or_rht16.argtypes = [_f32p, ctypes.c_uint32, _f32p]
    lib.or_irht16.restype = None
    lib.or_irht16.argtypes = [_f32p, ctypes.c_uint32, _f32p]
    lib.or_rht_amax.restype = ctypes.c_float
    lib.or_rht_amax.argtypes = [_f32p, _i64, _i64, ctypes.c_int, ctypes.c_uint64]
    lib.or_quantize_rht.restype = ctypes.c_int
    lib.or_quantize_rht.argtypes = [_f32p, _i64, _i64, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.c_int, _i64, _u8p, _u8p, _u64p]
    lib.or_dequantize_rht.restype = ctypes.c_int
    lib.or_dequantize_rht.argtypes = [_u8p, _u8p, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_uint64, _f32p]
    lib.or_num_threads.restype = ctypes.c_int
    lib.or_num_threads.argtypes = []
    lib.or_set_num_threads.restype = None
    lib.or_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a, t):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(t)


def as_f32(x):
    """bf16 bits (uint16) -> float32 exactly; float32 passes through."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    if x.dtype == np.float32:
        return np.ascontiguousarray(x)
    raise TypeError(f"oracle input must be bf16 bits (uint16) or float32, got {x.dtype}")


def _fmt(fmt):
    if isinstance(fmt, str):
        return {"e4m3": FMT_E4M3, "ue5m3": FMT_UE5M3}[fmt]
    return int(fmt)


# ---------------------------------------------------------------- scalars
def e2m1_value(code):
    return _load().or_e2m1_value(int(code))


def e2m1_code(y):
    return _load().or_e2m1_code(float(y))


def e2m1_code_sr(y, h):
    return _load().or_e2m1_code_sr(float(y), int(h) & 0xFFFFFFFF)


def scale_decode(fmt, code):
    return _load().or_scale_decode(_fmt(fmt), int(code))


def scale_encode(fmt, s):
    return _load().or_scale_encode(_fmt(fmt), float(s))


def scale_nan_code(fmt):
    return _load().or_scale_nan_code(_fmt(fmt))


def fmix32(h):
    return _load().or_fmix32(int(h) & 0xFFFFFFFF)


def sr_hash(seed, idx):
    return _load().or_sr_hash(int(seed), int(idx))


def alpha(amax, sg):
    return _load().or_alpha(float(amax), float(sg))


def f32_to_bf16(f):
    return _load().or_f32_to_bf16(float(f))


def num_threads():
    return _load().or_num_threads()


def set_num_threads(n):
    """OpenMP threads of the oracle's parallel loops (results do not depend
    on it)."""
    _load().or_set_num_threads(int(n))


def default_global_max(fmt, select):
    """The FP8 maximum S_g the outer scale maps the tensor amax to."""
    fmt = _fmt(fmt)
    if fmt == FMT_UE5M3:
        return 114688.0
    four = (SELECT_4OVER6, SELECT_4OVER6_MAE, SELECT_4OVER6_MAXERR)
    return 256.0 if int(select) in four else 448.0


# ---------------------------------------------------------------- tensors
def tensor_amax(x):
    xf = as_f32(x).ravel()
    return _load().or_tensor_amax(_ptr(xf, _f32p), xf.size)


def quantize(x, amax, *, fmt=FMT_E4M3, select=SELECT_4OVER6, rounding=ROUND_RNE, seed=0,
             global_max=None, row0=0, want_sse=False):
    """Row-wise quantization of a 2-D array.  Returns (codes, scales, count4)
    or, with want_sse, (codes, scales, count4, sse_chosen, sse_six)."""
    xf = as_f32(x)
    assert xf.ndim == 2
    rows, cols = xf.shape
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, select) if global_max is None else float(global_max)
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    cnt = np.zeros(1, np.uint64)
    sse_sel = np.empty((rows, cols // 16), np.float32) if want_sse else None
    sse6 = np.empty((rows, cols // 16), np.float32) if want_sse else None
    st = _load().or_quantize(_ptr(xf, _f32p), rows, cols, int(row0), float(amax), sg, fmt,
                             int(select), int(rounding), int(seed), _ptr(codes, _u8p),
                             _ptr(scales, _u8p), _ptr(cnt, _u64p), _ptr(sse_sel, _f32p),
                             _ptr(sse6, _f32p))
    if st != 0:
        raise ValueError(f"oracle quantize rejected the arguments (status {st})")
    if want_sse:
        return codes, scales, int(cnt[0]), sse_sel, sse6
    return codes, scales, int(cnt[0])


def quantize_cols(x, amax, *, col0=0, **kw):
    """Column-wise quantization: blocks of 16 consecutive rows of one column,
    i.e. the row-wise quantization of the transpose (output is X^T's)."""
    xt = np.ascontiguousarray(as_f32(x).T)
    return quantize(xt, amax, row0=col0, **kw)


def dequantize(codes, scales, amax, *, fmt=FMT_E4M3, select=SELECT_4OVER6, global_max=None,
               want_bf16=False, want_block_scale=False):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, select) if global_max is None else float(global_max)
    out = np.empty((rows, cols), np.float32)
    ob = np.empty((rows, cols), np.uint16) if want_bf16 else None
    bs = np.empty((rows, cols // 16), np.float32) if want_block_scale else None
    st = _load().or_dequantize(_ptr(codes, _u8p), _ptr(scales, _u8p), rows, cols, float(amax),
                               sg, fmt, _ptr(out, _f32p), _ptr(ob, _u16p), _ptr(bs, _f32p))
    if st != 0:
        raise ValueError(f"oracle dequantize rejected the arguments (status {st})")
    res = [out]
    if want_bf16:
        res.append(ob)
    if want_block_scale:
        res.append(bs)
    return res[0] if len(res) == 1 else tuple(res)


def sse(x, xhat):
    xf = np.ascontiguousarray(as_f32(x)).ravel()
    xh = np.ascontiguousarray(xhat, dtype=np.float32).ravel()
    assert xf.size == xh.size
    return _load().or_sse(_ptr(xf, _f32p), _ptr(xh, _f32p), xf.size)


def fakequant_fwd(x, s_pre, s_post=None, *, amax=False):
    """x~ per block; with amax=True the per-block parameters are amaxes and
    s = fl(a / 6)."""
    xf = as_f32(x)
    rows, cols = xf.shape
    sp = np.ascontiguousarray(s_pre, dtype=np.float32)
    so = None if s_post is None else np.ascontiguousarray(s_post, dtype=np.float32)
    out = np.empty((rows, cols), np.float32)
    fn = _load().or_fakequant_fwd_amax if amax else _load().or_fakequant_fwd
    st = fn(_ptr(xf, _f32p), rows, cols, _ptr(sp, _f32p), _ptr(so, _f32p), _ptr(out, _f32p))
    if st != 0:
        raise ValueError(f"oracle fakequant_fwd rejected the arguments (status {st})")
    return out


def fakequant_bwd(x, g, s_pre, s_post=None, *, amax=False):
    """Returns (dx, ds) for tied scales, (dx, ds_pre, ds_post) for dual; with
    amax=True the parameters are amaxes (s = a / 6) and the gradients are
    with respect to them."""
    xf = as_f32(x)
    rows, cols = xf.shape
    gf = np.ascontiguousarray(g, dtype=np.float32)
    sp = np.ascontiguousarray(s_pre, dtype=np.float32)
    so = None if s_post is None else np.ascontiguousarray(s_post, dtype=np.float32)
    dx = np.empty((rows, cols), np.float32)
    dpre = np.empty(sp.shape, np.float32)
    dpost = None if s_post is None else np.empty(sp.shape, np.float32)
    fn = _load().or_fakequant_bwd_amax if amax else _load().or_fakequant_bwd
    st = fn(_ptr(xf, _f32p), _ptr(gf, _f32p), rows, cols, _ptr(sp, _f32p), _ptr(so, _f32p),
            _ptr(dx, _f32p), _ptr(dpre, _f32p), _ptr(dpost, _f32p))
    if st != 0:
        raise ValueError(f"oracle fakequant_bwd rejected the arguments (status {st})")
    if s_post is None:
        return dx, dpre
    return dx, dpre, dpost


def unpack_codes(codes):
    """[rows, cols/2] bytes -> [rows, cols] 4-bit codes (low nibble first)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


# ---------------------------------------------------------------- per-row outer scales
def row_amax(x):
    """A_r = max |x| over each row of a 2-D array (float32 per row)."""
    xf = as_f32(x)
    assert xf.ndim == 2
    out = np.empty(xf.shape[0], np.float32)
    st = _load().or_row_amax(_ptr(xf, _f32p), xf.shape[0], xf.shape[1], _ptr(out, _f32p))
    if st != 0:
        raise ValueError(f"oracle row_amax rejected the arguments (status {st})")
    return out


def quantize_rowscaled(x, row_amaxes, *, fmt=FMT_E4M3, select=SELECT_4OVER6,
                       rounding=ROUND_RNE, seed=0, global_max=None, row0=0):
    """Row-wise quantization with a per-row outer scale alpha_r from
    row_amaxes[r].  Returns (codes, scales, count4)."""
    xf = as_f32(x)
    assert xf.ndim == 2
    rows, cols = xf.shape
    ra = np.ascontiguousarray(np.asarray(row_amaxes, np.float32))
    assert ra.shape == (rows,)
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, select) if global_max is None else float(global_max)
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    cnt = np.zeros(1, np.uint64)
    st = _load().or_quantize_rowscaled(_ptr(xf, _f32p), rows, cols, int(row0), _ptr(ra, _f32p),
                                       sg, fmt, int(select), int(rounding), int(seed),
                                       _ptr(codes, _u8p), _ptr(scales, _u8p), _ptr(cnt, _u64p))
    if st != 0:
        raise ValueError(f"oracle quantize_rowscaled rejected the arguments (status {st})")
    return codes, scales, int(cnt[0])


def dequantize_rowscaled(codes, scales, row_amaxes, *, fmt=FMT_E4M3, select=SELECT_4OVER6,
                         global_max=None, want_bf16=False, want_block_scale=False):
    """x_hat under per-row outer scales; returns float32 [rows, cols] (and the
    bf16 bits and/or block scales when asked)."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, half = codes.shape
    cols = half * 2
    ra = np.ascontiguousarray(np.asarray(row_amaxes, np.float32))
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, select) if global_max is None else float(global_max)
    out = np.empty((rows, cols), np.float32)
    bf = np.empty((rows, cols), np.uint16) if want_bf16 else None
    bs = np.empty((rows, cols // 16), np.float32) if want_block_scale else None
    st = _load().or_dequantize_rowscaled(_ptr(codes, _u8p), _ptr(scales, _u8p), rows, cols,
                                         _ptr(ra, _f32p), sg, fmt, _ptr(out, _f32p),
                                         _ptr(bf, _u16p), _ptr(bs, _f32p))
    if st != 0:
        raise ValueError(f"oracle dequantize_rowscaled rejected the arguments (status {st})")
    res = [out]
    if want_bf16:
        res.append(bf)
    if want_block_scale:
        res.append(bs)
    return res[0] if len(res) == 1 else tuple(res)


# ---------------------------------------------------------------- 16x16 tile scales
def quantize_2d(x, amax, *, fmt=FMT_E4M3, global_max=None, want_t=True):
    """16x16-tile-scaled quantization (max->6, RNE).  Returns (codes, scales)
    in the row-wise layout and, with want_t, also (codes_t, scales_t) in the
    column-wise layout of X^T."""
    xf = as_f32(x)
    assert xf.ndim == 2
    rows, cols = xf.shape
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, SELECT_6) if global_max is None else float(global_max)
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    codes_t = np.zeros((cols, rows // 2), np.uint8) if want_t else None
    scales_t = np.empty((cols, rows // 16), np.uint8) if want_t else None
    st = _load().or_quantize_2d(_ptr(xf, _f32p), rows, cols, float(amax), sg, fmt,
                                _ptr(codes, _u8p), _ptr(scales, _u8p), _ptr(codes_t, _u8p),
                                _ptr(scales_t, _u8p))
    if st != 0:
        raise ValueError(f"oracle quantize_2d rejected the arguments (status {st})")
    return (codes, scales, codes_t, scales_t) if want_t else (codes, scales)


# ---------------------------------------------------------------- re-quantization
def _source(codes, scales, amax, row_amaxes, fmt, select, global_max):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, half = codes.shape
    assert (amax is None) != (row_amaxes is None), "one outer amax or one per row"
    ra = None if row_amaxes is None else np.ascontiguousarray(np.asarray(row_amaxes, np.float32))
    assert ra is None or ra.shape == (rows,)
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, select) if global_max is None else float(global_max)
    return codes, scales, rows, half * 2, (0.0 if amax is None else float(amax)), ra, sg, fmt


def dequantized_amax(codes, scales, *, amax=None, row_amaxes=None, fmt=FMT_E4M3,
                     select=SELECT_4OVER6, global_max=None):
    """max |x_hat| of an NVFP4 tensor (per-tensor amax, or one per row)."""
    codes, scales, rows, cols, a, ra, sg, fmt = _source(codes, scales, amax, row_amaxes, fmt,
                                                         select, global_max)
    return _load().or_dequantized_amax(_ptr(codes, _u8p), _ptr(scales, _u8p), rows, cols, a,
                                       _ptr(ra, _f32p), sg, fmt)


def requant_t(codes, scales, *, amax=None, row_amaxes=None, fmt=FMT_E4M3, select=SELECT_4OVER6,
              global_max=None, target="nvfp4", dst_amax=None, dst_fmt=FMT_E4M3,
              dst_global_max=None, seed=0, col0=0):
    """Dequantize an NVFP4 tensor, transpose, re-quantize with stochastic
    rounding.  target "nvfp4": returns (codes_t [cols, rows/2], scales_t
    [cols, rows/16]) under outer amax dst_amax; "mxfp8": returns (elems_t
    [cols, rows] E4M3 bytes, scales_t [cols, rows/32] E8M0 bytes).  col0:
    the source is the strip of columns col0.. of a wider tensor (SR indices
    of the wider output)."""
    codes, scales, rows, cols, a, ra, sg, fmt = _source(codes, scales, amax, row_amaxes, fmt,
                                                         select, global_max)
    lib = _load()
    if target == "nvfp4":
        dfmt = _fmt(dst_fmt)
        dsg = default_global_max(dfmt, SELECT_6) if dst_global_max is None else float(dst_global_max)
        ct = np.empty((cols, rows // 2), np.uint8)
        st_ = np.empty((cols, rows // 16), np.uint8)
        st = lib.or_requant_nvfp4_t(_ptr(codes, _u8p), _ptr(scales, _u8p), rows, cols, a,
                                    _ptr(ra, _f32p), sg, fmt, float(dst_amax), dsg, dfmt,
                                    int(seed), int(col0), _ptr(ct, _u8p), _ptr(st_, _u8p))
    elif target == "mxfp8":
        ct = np.empty((cols, rows), np.uint8)
        st_ = np.empty((cols, rows // 32), np.uint8)
        st = lib.or_requant_mxfp8_t(_ptr(codes, _u8p), _ptr(scales, _u8p), rows, cols, a,
                                    _ptr(ra, _f32p), sg, fmt, int(seed), int(col0), _ptr(ct, _u8p),
                                    _ptr(st_, _u8p))
    else:
        raise ValueError(f"unknown target {target!r}")
    if st != 0:
        raise ValueError(f"oracle requant_t rejected the arguments (status {st})")
    return ct, st_


def e4m3_code_sr(y, h):
    return _load().or_e4m3_code_sr(float(y), int(h) & 0xFFFFFFFF)


def mxfp8_quantize_sr(x, *, seed=0, row0=0):
    """MXFP8 (blocks of 32 along rows, E8M0 scale, E4M3 elements) with
    stochastic rounding.  Returns (elems [rows, cols], scales [rows, cols/32])."""
    xf = as_f32(x)
    assert xf.ndim == 2
    rows, cols = xf.shape
    el = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    st = _load().or_mxfp8_quantize_sr(_ptr(xf, _f32p), rows, cols, int(row0), int(seed),
                                      _ptr(el, _u8p), _ptr(sc, _u8p))
    if st != 0:
        raise ValueError(f"oracle mxfp8_quantize_sr rejected the arguments (status {st})")
    return el, sc


def mxfp8_dequantize(elems, scales):
    el = np.ascontiguousarray(elems, np.uint8)
    sc = np.ascontiguousarray(scales, np.uint8)
    rows, cols = el.shape
    out = np.empty((rows, cols), np.float32)
    st = _load().or_mxfp8_dequantize(_ptr(el, _u8p), _ptr(sc, _u8p), rows, cols, _ptr(out, _f32p))
    if st != 0:
        raise ValueError(f"oracle mxfp8_dequantize rejected the arguments (status {st})")
    return out


# ---------------------------------------------------------------- random Hadamard transform
AXIS_ROW, AXIS_COL = 1, 2


def rht_signs(sign_seed):
    """Bit j set: s_j = -1 (the tensor's sign vector)."""
    return _load().or_rht_signs(int(sign_seed))


def rht16(x16, sign_seed=0, *, inverse=False):
    x = np.ascontiguousarray(np.asarray(x16, np.float32).reshape(16))
    y = np.empty(16, np.float32)
    fn = _load().or_irht16 if inverse else _load().or_rht16
    fn(_ptr(x, _f32p), rht_signs(sign_seed), _ptr(y, _f32p))
    return y


def rht_amax(x, *, axis=AXIS_ROW, sign_seed=0):
    xf = as_f32(x)
    return _load().or_rht_amax(_ptr(xf, _f32p), xf.shape[0], xf.shape[1], int(axis), int(sign_seed))


def quantize_rht(x, amax, *, axis=AXIS_ROW, sign_seed=0, fmt=FMT_E4M3, select=SELECT_4OVER6,
                 rounding=ROUND_RNE, seed=0, global_max=None, out_row0=0):
    """Quantization of the block-wise transformed tensor.  axis ROW: row-wise
    layout; COL: the column-wise layout (of the transpose).  out_row0: the
    first output row's position in a larger output (x a strip of a larger
    tensor: its first row for ROW, its first column for COL), for the SR
    indices.  Returns (codes, scales, count4)."""
    xf = as_f32(x)
    rows, cols = xf.shape
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, select) if global_max is None else float(global_max)
    R, C = (rows, cols) if axis == AXIS_ROW else (cols, rows)
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // 16), np.uint8)
    cnt = np.zeros(1, np.uint64)
    st = _load().or_quantize_rht(_ptr(xf, _f32p), rows, cols, float(amax), sg, fmt, int(select),
                                 int(rounding), int(seed), int(sign_seed), int(axis), int(out_row0),
                                 _ptr(codes, _u8p), _ptr(scales, _u8p), _ptr(cnt, _u64p))
    if st != 0:
        raise ValueError(f"oracle quantize_rht rejected the arguments (status {st})")
    return codes, scales, int(cnt[0])


def dequantize_rht(codes, scales, amax, *, sign_seed=0, fmt=FMT_E4M3, select=SELECT_4OVER6,
                   global_max=None):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, half = codes.shape
    fmt = _fmt(fmt)
    sg = default_global_max(fmt, select) if global_max is None else float(global_max)
    out = np.empty((rows, half * 2), np.float32)
    st = _load().or_dequantize_rht(_ptr(codes, _u8p), _ptr(scales, _u8p), rows, half * 2,
                                   float(amax), sg, fmt, int(sign_seed), _ptr(out, _f32p))
    if st != 0:
        raise ValueError(f"oracle dequantize_rht rejected the arguments (status {st})")
    return out
