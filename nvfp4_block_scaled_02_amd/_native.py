"""ctypes loader for libnvfp4.so (the C ABI of include/nvfp4.h).

The library is built in-tree by ``nvfp4_block_scaled_02_amd.build`` (or
``__graft_entry__.build()``).  There is no fallback: if the library is
missing or cannot be loaded, every call raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")
ABI_VERSION = 8  # NVFP4_ABI_VERSION of include/nvfp4.h that these signatures follow

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
SCALE_E4M3, SCALE_UE5M3 = 0, 1
SELECT_6, SELECT_4OVER6 = 0, 1
SELECT_4OVER6_MAE, SELECT_4OVER6_MAXERR, SELECT_SWEEP = 2, 3, 4
ROUND_RNE, ROUND_SR = 0, 1
AXIS_ROW, AXIS_COL = 1, 2
TARGET_NVFP4, TARGET_MXFP8 = 0, 1

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float


class QuantArgs(ctypes.Structure):
    """nvfp4_quant_args of include/nvfp4.h (same field order, so the same
    C layout)."""
    _fields_ = [("x", _vp), ("rows", _i64), ("cols", _i64), ("amax", _vp),
                ("global_fp8_max", _f32), ("scale_fmt", _int), ("select", _int),
                ("rounding", _int), ("axes", _int), ("seed", _u64), ("codes", _vp),
                ("scales", _vp), ("codes_t", _vp), ("scales_t", _vp), ("count4", _vp),
                ("workspace", _vp)]


_qa = ctypes.POINTER(QuantArgs)
# name -> (restype, argtypes); the exported surface of include/nvfp4.h and
# include/nvfp4_testing.h (hipStream_t travels as a pointer)
SIGNATURES = {
    "nvfp4_abi_version": (_int, []),
    "nvfp4_status_string": (ctypes.c_char_p, [_int]),
    "nvfp4_workspace_bytes": (ctypes.c_size_t, []),
    "nvfp4_tensor_amax": (_int, [_vp, _i64, _vp, _vp, _vp]),
    "nvfp4_tensor_amax_noalloc": (_int, [_vp, _i64, _vp, _vp]),
    "nvfp4_quantize": (_int, [_qa, _vp]),
    "nvfp4_dequantize": (_int, [_vp, _vp, _i64, _i64, _vp, _f32, _int, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp]),
    "nvfp4_row_amax": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "nvfp4_quantize_rowscaled": (_int, [_qa, _vp]),
    "nvfp4_quantize_pertoken": (_int, [_qa, _vp, _vp]),
    "nvfp4_dequantize_rowscaled": (_int, [_vp, _vp, _i64, _i64, _vp, _f32, _int, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp]),
    "nvfp4_quantize_2d": (_int, [_qa, _vp]),
    "nvfp4_fakequant_fwd": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_fakequant_bwd": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "nvfp4_fakequant_fwd_amax": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_fakequant_bwd_amax": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "nvfp4_dequantized_amax": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _f32, _int, _vp, _vp, _vp]),
    "nvfp4_requantize_t": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _f32, _int, _int, _vp, _f32,
                                  _int, _u64, _vp, _vp, _vp]),
    "nvfp4_rht_amax": (_int, [_vp, _i64, _i64, _int, _u64, _vp, _vp, _vp]),
    "nvfp4_quantize_rht": (_int, [_qa, _u64, _vp]),
    "nvfp4_dequantize_rht": (_int, [_vp, _vp, _i64, _i64, _vp, _f32, _int, _u64, _vp, _vp]),
    "nvfp4_test_e2m1_rne_range": (_int, [_u32, _i64, _vp, _vp]),
    "nvfp4_test_e2m1_sr": (_int, [_vp, _vp, _i64, _vp, _vp]),
    "nvfp4_test_scale_encode_range": (_int, [_int, _u32, _i64, _vp, _vp]),
    "nvfp4_test_sr_hash": (_int, [_u64, _u64, _i64, _vp, _vp]),
    "nvfp4_test_e4m3_sr": (_int, [_vp, _vp, _i64, _vp, _vp]),
}

WORKSPACE_BYTES = 66688  # NVFP4_WORKSPACE_BYTES of include/nvfp4.h

_lib = None


class NativeError(RuntimeError):
    pass


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NativeError(
            f"{LIB_PATH} is not built; run `python -m nvfp4_block_scaled_02_amd.build` "
            "(hipcc, gfx950) first. There is no non-native fallback.")
    l = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(l, name)
        f.restype = res
        f.argtypes = args
    if l.nvfp4_abi_version() != ABI_VERSION or l.nvfp4_workspace_bytes() != WORKSPACE_BYTES:
        raise NativeError(
            f"{LIB_PATH} has ABI version {l.nvfp4_abi_version()}, the binding expects "
            f"{ABI_VERSION}; rebuild with `python -m nvfp4_block_scaled_02_amd.build`.")
    _lib = l
    return l


def check(status, what):
    if status != OK:
        msg = lib().nvfp4_status_string(status).decode()
        raise NativeError(f"{what} failed with status {status} ({msg})")
