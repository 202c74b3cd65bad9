"""Torch-facing wrappers over the C ABI of libnvfp4.so (include/nvfp4.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  Torch supplies device memory and the current stream.  Inputs must
be contiguous tensors on a GPU device; bf16 inputs are passed as their 16-bit
patterns.  Every tensor handed to the library is checked here against the
size the kernels index (the C ABI sees only pointers), so a wrongly sized
buffer raises before anything is launched.

Calls that combine one value per workgroup across a launch (the amax calls,
the 4/6 count, the squared-error report) need a workspace: by default one
zero-filled buffer per (device, stream) is created on first use and reused
(every call leaves it zeroed); ``workspace=`` passes another one.

``prepare(fn, ...)`` runs any single-launch call with its arguments checked
and its outputs allocated, but returns the launch (a ``Launch``) instead of
issuing it: loops that launch the same call many times (serving, timing,
graph capture) then pay one ctypes call per launch.
"""
import ctypes
import threading
from dataclasses import dataclass
from typing import Optional

import torch

from . import _native as N

_FMT = {"e4m3": N.SCALE_E4M3, "ue5m3": N.SCALE_UE5M3}
_SELECT = {"6": N.SELECT_6, "4over6": N.SELECT_4OVER6, "4over6-mae": N.SELECT_4OVER6_MAE,
           "4over6-maxerr": N.SELECT_4OVER6_MAXERR, "sweep": N.SELECT_SWEEP}
_ROUND = {"rne": N.ROUND_RNE, "sr": N.ROUND_SR}
_AXES = {"row": N.AXIS_ROW, "col": N.AXIS_COL, "both": N.AXIS_ROW | N.AXIS_COL}
_U64 = 0xFFFFFFFFFFFFFFFF


def default_global_max(fmt: str = "e4m3", select: str = "4over6") -> float:
    """FP8 maximum S_g the outer scale maps the tensor amax to."""
    if fmt == "ue5m3":
        return 114688.0
    return 256.0 if select.startswith("4over6") else 448.0


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, dtype, name, numel: Optional[int] = None):
    """t is a contiguous GPU tensor of dtype, holding exactly numel elements
    (when given): the extent the kernels read or write."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()} "
                         f"(shape {tuple(t.shape)})")


def _need_2d(x: torch.Tensor, dtype, name):
    _need(x, dtype, name)
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, cols]")
    return x.shape


_WORKSPACES = {}


def workspace(device=None) -> torch.Tensor:
    """The zero-filled workspace this binding uses for the current stream of
    `device` (created on first use; calls leave it zeroed)."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    key = (dev.index, _stream(dev))
    ws = _WORKSPACES.get(key)
    if ws is None:
        ws = torch.zeros(N.WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def _ws(given: Optional[torch.Tensor], dev):
    if given is None:
        return workspace(dev)
    _need(given, torch.uint8, "workspace", N.WORKSPACE_BYTES)
    return given


class Launch:
    """One entry point with its arguments checked once: each call issues the
    launch again on `stream` (default: the current stream of the device)
    without re-checking anything.  It keeps its tensors alive.  Made by
    prepare()."""

    def __init__(self, entry: str, args: tuple, device, keep):
        self._fn = getattr(N.lib(), entry)
        self._entry = entry
        self._args = args
        self._device = device
        self._keep = keep

    def __call__(self, stream=None):
        s = stream if stream is not None else _stream(self._device)
        st = self._fn(*self._args, s)
        if st != N.OK:
            N.check(st, self._entry)


_CAPTURE = threading.local()


def _invoke(entry: str, args: tuple, device, keep):
    """Issues entry(*args, stream) on the current stream of `device` now, or,
    inside prepare(), records it as a Launch instead."""
    launch = Launch(entry, args, device, keep)
    rec = getattr(_CAPTURE, "launches", None)
    if rec is not None:
        rec.append(launch)
    else:
        launch()


def prepare(fn, *args, **kwargs):
    """Runs fn(*args, **kwargs) -- a call of this module that issues exactly
    one library call -- with its arguments checked and its outputs allocated,
    but without launching.  Returns (launch, result): calling `launch()`
    issues the call, writing the outputs in `result`."""
    prev = getattr(_CAPTURE, "launches", None)
    _CAPTURE.launches = []
    try:
        result = fn(*args, **kwargs)
        launches = _CAPTURE.launches
    finally:
        _CAPTURE.launches = prev
    if len(launches) != 1:
        raise ValueError(f"{getattr(fn, '__name__', fn)} issues {len(launches)} library calls "
                         "with these arguments; prepare() needs exactly one (pass the amax it "
                         "would otherwise compute)")
    return launches[0], result


def tensor_amax(x: torch.Tensor, out: Optional[torch.Tensor] = None, *,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """max |x| over a bf16 tensor, as a 1-element float32 device tensor."""
    _need(x, torch.bfloat16, "x")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "out", 1)
    ws = _ws(workspace, x.device)
    _invoke("nvfp4_tensor_amax", (_ptr(x), x.numel(), _ptr(out), _ptr(ws)), x.device,
            (x, out, ws))
    return out


def prepare_tensor_amax(x: torch.Tensor, out: torch.Tensor, *,
                        workspace: Optional[torch.Tensor] = None) -> Launch:
    """tensor_amax(x, out) as a Launch."""
    return prepare(tensor_amax, x, out, workspace=workspace)[0]


@dataclass
class Quantized:
    """NVFP4 tensor: packed codes [rows, cols/2] (uint8, low nibble = even
    element), scale bytes [rows, cols/16], and the outer-scale inputs."""
    codes: Optional[torch.Tensor]
    scales: Optional[torch.Tensor]
    codes_t: Optional[torch.Tensor]
    scales_t: Optional[torch.Tensor]
    amax: torch.Tensor
    global_max: float
    fmt: str
    count4: Optional[torch.Tensor]


def _quant_outputs(out, rows, cols, ax, count4, dev):
    """Preallocated or new outputs, each checked against its layout."""
    out = dict(out or {})
    if ax & N.AXIS_ROW:
        out.setdefault("codes", torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev))
        out.setdefault("scales", torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev))
        _need(out["codes"], torch.uint8, "codes", rows * (cols // 2))
        _need(out["scales"], torch.uint8, "scales", rows * (cols // 16))
    if ax & N.AXIS_COL:
        out.setdefault("codes_t", torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev))
        out.setdefault("scales_t", torch.empty((cols, rows // 16), dtype=torch.uint8, device=dev))
        _need(out["codes_t"], torch.uint8, "codes_t", cols * (rows // 2))
        _need(out["scales_t"], torch.uint8, "scales_t", cols * (rows // 16))
    if count4 and "count4" not in out:
        out["count4"] = torch.zeros(1, dtype=torch.int64, device=dev)
    if "count4" in out:
        _need(out["count4"], torch.int64, "count4", 1)
    return out


def _quant_args(x, rows, cols, amax, global_max, fmt, select, rounding, ax, seed, out, ws):
    return N.QuantArgs(
        x=_ptr(x), rows=rows, cols=cols, amax=_ptr(amax), global_fp8_max=float(global_max),
        scale_fmt=_FMT[fmt], select=_SELECT[select], rounding=_ROUND[rounding], axes=ax,
        seed=int(seed) & _U64, codes=_ptr(out.get("codes")), scales=_ptr(out.get("scales")),
        codes_t=_ptr(out.get("codes_t")), scales_t=_ptr(out.get("scales_t")),
        count4=_ptr(out.get("count4")), workspace=_ptr(ws) if "count4" in out else None)


def quantize(x: torch.Tensor, amax: Optional[torch.Tensor] = None, *, fmt: str = "e4m3",
             select: str = "4over6", rounding: str = "rne", axes: str = "row", seed: int = 0,
             global_max: float = 0.0, count4: bool = False, out: Optional[dict] = None,
             workspace: Optional[torch.Tensor] = None) -> Quantized:
    """NVFP4-quantize a 2-D bf16 tensor.  amax: 1-element float32 device
    tensor (default: the fresh tensor amax).  axes: "row", "col" or "both".
    out: optional preallocated {"codes", "scales", "codes_t", "scales_t",
    "count4"} tensors (count4 is added to, not cleared)."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    if amax is None:
        amax = tensor_amax(x, workspace=workspace)
    _need(amax, torch.float32, "amax", 1)
    ax = _AXES[axes]
    out = _quant_outputs(out, rows, cols, ax, count4, x.device)
    ws = _ws(workspace, x.device) if "count4" in out else None
    args = _quant_args(x, rows, cols, amax, global_max, fmt, select, rounding, ax, seed, out, ws)
    _invoke("nvfp4_quantize", (ctypes.byref(args),), x.device, (x, amax, out, ws, args))
    gm = float(global_max) if global_max else default_global_max(fmt, select)
    return Quantized(out.get("codes"), out.get("scales"), out.get("codes_t"), out.get("scales_t"),
                     amax, gm, fmt, out.get("count4"))


def prepare_quantize(x: torch.Tensor, amax: torch.Tensor, **kwargs):
    """quantize() as a Launch: returns (launch, Quantized) with the outputs
    the launch writes."""
    return prepare(quantize, x, amax, **kwargs)


def dequantize(codes: torch.Tensor, scales: torch.Tensor, amax: torch.Tensor, *,
               global_max: float, fmt: str = "e4m3", out_dtype=torch.float32,
               want_block_scale: bool = False, x_ref: Optional[torch.Tensor] = None,
               sse: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, _entry: str = "nvfp4_dequantize"):
    """x_hat = q * D[scale] * alpha.  Returns x_hat (or None if out_dtype is
    None), plus the per-block effective scales if asked, plus the binary64
    SSE tensor if x_ref is given (sse, if passed, is overwritten)."""
    rows, half = _need_2d(codes, torch.uint8, "codes")
    cols = 2 * half
    _need(scales, torch.uint8, "scales", rows * (cols // 16))
    _need(amax, torch.float32, "amax", rows if _entry == "nvfp4_dequantize_rowscaled" else 1)
    dev = codes.device
    of32 = ob16 = None
    if out_dtype is not None:
        if out is None:
            out = torch.empty((rows, cols), dtype=out_dtype, device=dev)
        _need(out, out_dtype, "out", rows * cols)
        if out_dtype == torch.float32:
            of32 = out
        elif out_dtype == torch.bfloat16:
            ob16 = out
        else:
            raise TypeError("out_dtype must be float32, bfloat16 or None")
    bs = torch.empty((rows, cols // 16), dtype=torch.float32, device=dev) if want_block_scale else None
    ws = None
    if x_ref is not None:
        _need(x_ref, torch.bfloat16, "x_ref", rows * cols)
        if sse is None:
            sse = torch.empty(1, dtype=torch.float64, device=dev)
        _need(sse, torch.float64, "sse", 1)
        ws = _ws(workspace, dev)
    args = (_ptr(codes), _ptr(scales), rows, cols, _ptr(amax), ctypes.c_float(float(global_max)),
            _FMT[fmt], _ptr(of32), _ptr(ob16), _ptr(bs), _ptr(x_ref),
            _ptr(sse) if x_ref is not None else None, _ptr(ws))
    res = [out]
    if want_block_scale:
        res.append(bs)
    if x_ref is not None:
        res.append(sse)
    _invoke(_entry, args, dev, (codes, scales, amax, out, bs, x_ref, sse, ws))
    return res[0] if len(res) == 1 else tuple(res)


def prepare_dequantize(codes: torch.Tensor, scales: torch.Tensor, amax: torch.Tensor, **kwargs):
    """dequantize() as a Launch: returns (launch, result) with the result
    dequantize() would return."""
    return prepare(dequantize, codes, scales, amax, **kwargs)


# ---------------------------------------------------------------- per-row outer scales
def row_amax(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """max |x| over each row of a 2-D bf16 tensor, as float32 [rows]."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "out", rows)
    _invoke("nvfp4_row_amax", (_ptr(x), rows, cols, _ptr(out)), x.device, (x, out))
    return out


def quantize_rowscaled(x: torch.Tensor, row_amaxes: Optional[torch.Tensor] = None, *,
                       fmt: str = "e4m3", select: str = "4over6", rounding: str = "rne",
                       seed: int = 0, global_max: float = 0.0, count4: bool = False,
                       out: Optional[dict] = None,
                       workspace: Optional[torch.Tensor] = None) -> Quantized:
    """Row-wise NVFP4 quantization with a per-row outer scale (per-token
    scaling); row_amaxes defaults to row_amax(x).  Quantized.amax holds the
    per-row amaxes."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    if row_amaxes is None:
        row_amaxes = row_amax(x)
    _need(row_amaxes, torch.float32, "row_amaxes", rows)
    out = _quant_outputs(out, rows, cols, N.AXIS_ROW, count4, x.device)
    ws = _ws(workspace, x.device) if "count4" in out else None
    args = _quant_args(x, rows, cols, row_amaxes, global_max, fmt, select, rounding, N.AXIS_ROW,
                       seed, out, ws)
    _invoke("nvfp4_quantize_rowscaled", (ctypes.byref(args),), x.device,
            (x, row_amaxes, out, ws, args))
    gm = float(global_max) if global_max else default_global_max(fmt, select)
    return Quantized(out["codes"], out["scales"], None, None, row_amaxes, gm, fmt,
                     out.get("count4"))


def quantize_pertoken(x: torch.Tensor, *, fmt: str = "e4m3", select: str = "4over6",
                      rounding: str = "rne", seed: int = 0, global_max: float = 0.0,
                      count4: bool = False, out: Optional[dict] = None,
                      row_amaxes: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> Quantized:
    """row_amax(x) and quantize_rowscaled(x, ...) in one launch: the row
    amaxes are computed on the device and written to row_amaxes (new if not
    given), which Quantized.amax holds."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    if row_amaxes is None:
        row_amaxes = torch.empty(rows, dtype=torch.float32, device=x.device)
    _need(row_amaxes, torch.float32, "row_amaxes", rows)
    out = _quant_outputs(out, rows, cols, N.AXIS_ROW, count4, x.device)
    ws = _ws(workspace, x.device) if "count4" in out else None
    args = _quant_args(x, rows, cols, None, global_max, fmt, select, rounding, N.AXIS_ROW, seed,
                       out, ws)
    _invoke("nvfp4_quantize_pertoken", (ctypes.byref(args), _ptr(row_amaxes)), x.device,
            (x, row_amaxes, out, ws, args))
    gm = float(global_max) if global_max else default_global_max(fmt, select)
    return Quantized(out["codes"], out["scales"], None, None, row_amaxes, gm, fmt,
                     out.get("count4"))


def dequantize_rowscaled(codes: torch.Tensor, scales: torch.Tensor, row_amaxes: torch.Tensor, *,
                         global_max: float, fmt: str = "e4m3", out_dtype=torch.float32,
                         want_block_scale: bool = False, x_ref: Optional[torch.Tensor] = None,
                         sse: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """dequantize() with per-row outer scales (row_amaxes [rows])."""
    return dequantize(codes, scales, row_amaxes, global_max=global_max, fmt=fmt,
                      out_dtype=out_dtype, want_block_scale=want_block_scale, x_ref=x_ref,
                      sse=sse, out=out, workspace=workspace, _entry="nvfp4_dequantize_rowscaled")


# ---------------------------------------------------------------- 16x16 tile scales
def quantize_2d(x: torch.Tensor, amax: Optional[torch.Tensor] = None, *, fmt: str = "e4m3",
                global_max: float = 0.0, transpose: bool = True,
                out: Optional[dict] = None) -> Quantized:
    """NVFP4 with one block scale per 16x16 tile (max->6, RNE): the row-wise
    layout and, with transpose, the column-wise layout of X^T, whose codes are
    the transpose of the row-wise ones."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    if amax is None:
        amax = tensor_amax(x)
    _need(amax, torch.float32, "amax", 1)
    ax = N.AXIS_ROW | (N.AXIS_COL if transpose else 0)
    out = _quant_outputs(out, rows, cols, ax, False, x.device)
    out.pop("count4", None)
    args = _quant_args(x, rows, cols, amax, global_max, fmt, "6", "rne", ax, 0, out, None)
    _invoke("nvfp4_quantize_2d", (ctypes.byref(args),), x.device, (x, amax, out, args))
    gm = float(global_max) if global_max else default_global_max(fmt, "6")
    return Quantized(out["codes"], out["scales"], out.get("codes_t"), out.get("scales_t"), amax,
                     gm, fmt, None)


# ---------------------------------------------------------------- re-quantization
_TARGET = {"nvfp4": N.TARGET_NVFP4, "mxfp8": N.TARGET_MXFP8}


def _rq_source(codes, scales, amax, row_amaxes):
    rows, half = _need_2d(codes, torch.uint8, "codes")
    cols = 2 * half
    _need(scales, torch.uint8, "scales", rows * (cols // 16))
    if (amax is None) == (row_amaxes is None):
        raise ValueError("pass exactly one of amax (per tensor) and row_amaxes (per row)")
    if amax is not None:
        _need(amax, torch.float32, "amax", 1)
    else:
        _need(row_amaxes, torch.float32, "row_amaxes", rows)
    return rows, cols


def dequantized_amax(codes: torch.Tensor, scales: torch.Tensor, *,
                     amax: Optional[torch.Tensor] = None,
                     row_amaxes: Optional[torch.Tensor] = None, global_max: float,
                     fmt: str = "e4m3", out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """max |x_hat| of an NVFP4 tensor (one outer amax, or one per row), as a
    1-element float32 device tensor."""
    rows, cols = _rq_source(codes, scales, amax, row_amaxes)
    dev = codes.device
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=dev)
    _need(out, torch.float32, "out", 1)
    ws = _ws(workspace, dev)
    _invoke("nvfp4_dequantized_amax",
            (_ptr(codes), _ptr(scales), rows, cols, _ptr(amax), _ptr(row_amaxes),
             ctypes.c_float(float(global_max)), _FMT[fmt], _ptr(out), _ptr(ws)),
            dev, (codes, scales, amax, row_amaxes, out, ws))
    return out


def requantize_t(codes: torch.Tensor, scales: torch.Tensor, *,
                 amax: Optional[torch.Tensor] = None, row_amaxes: Optional[torch.Tensor] = None,
                 global_max: float, fmt: str = "e4m3", target: str = "mxfp8",
                 dst_amax: Optional[torch.Tensor] = None, dst_fmt: str = "e4m3",
                 dst_global_max: float = 0.0, seed: int = 0, out: Optional[dict] = None):
    """Dequantize an NVFP4 tensor, transpose it and re-quantize it with
    stochastic rounding.  target "mxfp8": returns (elems_t [cols, rows]
    E4M3 bytes, scales_t [cols, rows/32] E8M0 bytes).  target "nvfp4":
    returns (codes_t [cols, rows/2], scales_t [cols, rows/16]) under the outer
    amax dst_amax (default: the dequantized tensor's amax)."""
    rows, cols = _rq_source(codes, scales, amax, row_amaxes)
    dev = codes.device
    out = dict(out or {})
    if target == "nvfp4":
        if dst_amax is None:
            dst_amax = dequantized_amax(codes, scales, amax=amax, row_amaxes=row_amaxes,
                                        global_max=global_max, fmt=fmt)
        _need(dst_amax, torch.float32, "dst_amax", 1)
        out.setdefault("out_t", torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev))
        out.setdefault("scales_t", torch.empty((cols, rows // 16), dtype=torch.uint8, device=dev))
        n_t, n_s = cols * (rows // 2), cols * (rows // 16)
    elif target == "mxfp8":
        out.setdefault("out_t", torch.empty((cols, rows), dtype=torch.uint8, device=dev))
        out.setdefault("scales_t", torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev))
        n_t, n_s = cols * rows, cols * (rows // 32)
    else:
        raise ValueError(f"unknown target {target!r}")
    _need(out["out_t"], torch.uint8, "out_t", n_t)
    _need(out["scales_t"], torch.uint8, "scales_t", n_s)
    _invoke("nvfp4_requantize_t",
            (_ptr(codes), _ptr(scales), rows, cols, _ptr(amax), _ptr(row_amaxes),
             ctypes.c_float(float(global_max)), _FMT[fmt], _TARGET[target], _ptr(dst_amax),
             ctypes.c_float(float(dst_global_max)), _FMT[dst_fmt], int(seed) & _U64,
             _ptr(out["out_t"]), _ptr(out["scales_t"])),
            dev, (codes, scales, amax, row_amaxes, dst_amax, out))
    return out["out_t"], out["scales_t"]


# ---------------------------------------------------------------- random Hadamard transform
_AXIS1 = {"row": N.AXIS_ROW, "col": N.AXIS_COL}


def rht_amax(x: torch.Tensor, *, axis: str = "row", sign_seed: int = 0,
             out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """max |y| of the tensor with every block (row blocks or column blocks)
    transformed by the 16-point random Hadamard transform."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "out", 1)
    ws = _ws(workspace, x.device)
    _invoke("nvfp4_rht_amax",
            (_ptr(x), rows, cols, _AXIS1[axis], int(sign_seed) & _U64, _ptr(out), _ptr(ws)),
            x.device, (x, out, ws))
    return out


def quantize_rht(x: torch.Tensor, amax: Optional[torch.Tensor] = None, *, axis: str = "row",
                 sign_seed: int = 0, fmt: str = "e4m3", select: str = "4over6",
                 rounding: str = "rne", seed: int = 0, global_max: float = 0.0,
                 count4: bool = False, out: Optional[dict] = None,
                 workspace: Optional[torch.Tensor] = None) -> Quantized:
    """NVFP4 quantization of the block-wise transformed tensor along one axis
    ("row": row-wise layout; "col": the column-wise layout of the transpose,
    returned in .codes / .scales).  amax defaults to the transformed tensor's
    amax."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    if amax is None:
        amax = rht_amax(x, axis=axis, sign_seed=sign_seed, workspace=workspace)
    _need(amax, torch.float32, "amax", 1)
    ax = _AXIS1[axis]
    given = dict(out or {})
    if ax == N.AXIS_COL:  # the transpose's layout travels as codes_t / scales_t
        given = {{"codes": "codes_t", "scales": "scales_t"}.get(k, k): v for k, v in given.items()}
    o = _quant_outputs(given, rows, cols, ax, count4, x.device)
    ws = _ws(workspace, x.device) if "count4" in o else None
    args = _quant_args(x, rows, cols, amax, global_max, fmt, select, rounding, ax, seed, o, ws)
    _invoke("nvfp4_quantize_rht", (ctypes.byref(args), int(sign_seed) & _U64), x.device,
            (x, amax, o, ws, args))
    gm = float(global_max) if global_max else default_global_max(fmt, select)
    c, s = (o["codes"], o["scales"]) if ax == N.AXIS_ROW else (o["codes_t"], o["scales_t"])
    return Quantized(c, s, None, None, amax, gm, fmt, o.get("count4"))


def dequantize_rht(codes: torch.Tensor, scales: torch.Tensor, amax: torch.Tensor, *,
                   global_max: float, fmt: str = "e4m3", sign_seed: int = 0,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x_hat followed by the inverse transform of every row block (float32)."""
    rows, half = _need_2d(codes, torch.uint8, "codes")
    cols = 2 * half
    _need(scales, torch.uint8, "scales", rows * (cols // 16))
    _need(amax, torch.float32, "amax", 1)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=codes.device)
    _need(out, torch.float32, "out", rows * cols)
    _invoke("nvfp4_dequantize_rht",
            (_ptr(codes), _ptr(scales), rows, cols, _ptr(amax), ctypes.c_float(float(global_max)),
             _FMT[fmt], int(sign_seed) & _U64, _ptr(out)),
            codes.device, (codes, scales, amax, out))
    return out


# ---------------------------------------------------------------- fake quantization
def fakequant_fwd(x: torch.Tensor, s_pre: torch.Tensor, s_post: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, *, amax: bool = False) -> torch.Tensor:
    """x~ = s_post * clamp(round_E2M1(x / s_pre), -6, 6) per 16-element block.
    amax=True: s_pre / s_post hold block amaxes and s = a / 6."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    nb = rows * (cols // 16)
    _need(s_pre, torch.float32, "s_pre", nb)
    if s_post is not None:
        _need(s_post, torch.float32, "s_post", nb)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "out", rows * cols)
    entry = "nvfp4_fakequant_fwd_amax" if amax else "nvfp4_fakequant_fwd"
    _invoke(entry, (_ptr(x), rows, cols, _ptr(s_pre), _ptr(s_post), _ptr(out)), x.device,
            (x, s_pre, s_post, out))
    return out


def fakequant_bwd(x: torch.Tensor, grad: torch.Tensor, s_pre: torch.Tensor,
                  s_post: Optional[torch.Tensor] = None, out: Optional[dict] = None, *,
                  amax: bool = False):
    """Straight-through backward.  Returns (dx, ds) for tied scales and
    (dx, ds_pre, ds_post) for dual scales.  amax=True: the parameters are
    block amaxes (s = a / 6) and the gradients are with respect to them."""
    rows, cols = _need_2d(x, torch.bfloat16, "x")
    nb = rows * (cols // 16)
    _need(grad, torch.float32, "grad", rows * cols)
    _need(s_pre, torch.float32, "s_pre", nb)
    if s_post is not None:
        _need(s_post, torch.float32, "s_post", nb)
    dev = x.device
    out = dict(out or {})
    dx = out.get("dx")
    if dx is None:
        dx = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    _need(dx, torch.float32, "dx", rows * cols)
    dpre = out.get("ds_pre")
    if dpre is None:
        dpre = torch.empty(s_pre.shape, dtype=torch.float32, device=dev)
    _need(dpre, torch.float32, "ds_pre", nb)
    dpost = None
    if s_post is not None:
        dpost = out.get("ds_post")
        if dpost is None:
            dpost = torch.empty(s_post.shape, dtype=torch.float32, device=dev)
        _need(dpost, torch.float32, "ds_post", nb)
    entry = "nvfp4_fakequant_bwd_amax" if amax else "nvfp4_fakequant_bwd"
    _invoke(entry, (_ptr(x), _ptr(grad), rows, cols, _ptr(s_pre), _ptr(s_post), _ptr(dx),
                    _ptr(dpre), _ptr(dpost)), dev, (x, grad, s_pre, s_post, dx, dpre, dpost))
    return (dx, dpre) if s_post is None else (dx, dpre, dpost)
