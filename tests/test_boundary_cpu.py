"""The C-ABI library loads, exports every symbol its headers declare, and
rejects bad arguments on the host before any launch.  No GPU needed: every
call here either fails validation or has nothing to do (an empty tensor)."""
import ctypes
import os
import re

import pytest

from nvfp4_block_scaled_02_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("nvfp4.h", "nvfp4_testing.h")]

FAKE = 0x100000  # aligned non-null address that is never dereferenced
FAKE_ODD = 0x100004


def _declared():
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nvfp4_\w+)\s*\(", src, flags=re.M)
    return names


def test_library_loads_and_version():
    """The library, the binding and the header agree on the ABI version."""
    lib = N.lib()
    hdr = int(re.search(r"#define NVFP4_ABI_VERSION (\d+)", open(HEADERS[0]).read()).group(1))
    assert lib.nvfp4_abi_version() == N.ABI_VERSION == hdr


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 11
    lib = ctypes.CDLL(N.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
        assert n in N.SIGNATURES, f"{n} has no Python binding"
    assert set(N.SIGNATURES) == set(names)


def test_status_strings():
    lib = N.lib()
    for s, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported request"),
                    (3, b"HIP launch error"), (99, b"unknown status")]:
        assert lib.nvfp4_status_string(s) == text


def _qargs(**kw):
    a = dict(x=FAKE, rows=16, cols=32, amax=FAKE, gmax=0.0, fmt=0, select=1, rnd=0, axes=1,
             seed=0, codes=FAKE, scales=FAKE, codes_t=FAKE, scales_t=FAKE, count4=None, ws=None)
    a.update(kw)
    return N.QuantArgs(x=a["x"], rows=a["rows"], cols=a["cols"], amax=a["amax"],
                       global_fp8_max=a["gmax"], scale_fmt=a["fmt"], select=a["select"],
                       rounding=a["rnd"], axes=a["axes"], seed=a["seed"], codes=a["codes"],
                       scales=a["scales"], codes_t=a["codes_t"], scales_t=a["scales_t"],
                       count4=a["count4"], workspace=a["ws"])


def _q(**kw):
    return N.lib().nvfp4_quantize(_qargs(**kw), None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(amax=None), dict(rows=-1), dict(cols=-16), dict(cols=24),
    dict(fmt=2), dict(select=5), dict(select=-1), dict(rnd=2), dict(axes=0), dict(axes=4),
    dict(rnd=1, select=1), dict(rnd=1, select=2), dict(rnd=1, select=3), dict(rnd=1, select=4),
    dict(gmax=-1.0), dict(gmax=float("inf")), dict(gmax=float("nan")),
    dict(codes=None), dict(scales=None), dict(axes=2, rows=24), dict(axes=2, codes_t=None),
    dict(axes=3, scales_t=None), dict(axes=2, cols=20, rows=16), dict(x=FAKE_ODD),
    dict(codes=FAKE_ODD), dict(scales=FAKE + 2), dict(count4=FAKE_ODD, ws=FAKE),
    dict(rows=1 << 40, cols=1 << 40),
    # more than NVFP4_MAX_ELEMENTS = 2^44 elements
    dict(rows=(1 << 40) + 1, cols=16), dict(rows=1 << 31, cols=1 << 31),
    # the 4/6 count needs a workspace, 16-byte aligned
    dict(count4=FAKE), dict(count4=FAKE, ws=FAKE_ODD),
])
def test_quantize_rejects(kw):
    assert _q(**kw) == N.ERR_INVALID


def test_quantize_rejects_null_args():
    assert N.lib().nvfp4_quantize(None, None) == N.ERR_INVALID


def test_quantize_empty_is_ok_without_launch():
    assert _q(rows=0) == N.OK
    assert _q(cols=0) == N.OK
    assert _q(rows=0, axes=3) == N.OK
    assert _q(rows=0, count4=FAKE, ws=FAKE) == N.OK


def test_quant_args_layout_matches_the_header(tmp_path):
    """ctypes' QuantArgs has the C layout of nvfp4_quant_args: a host program
    built from the header prints every field's offset and the size."""
    fields = [f for f, _ in N.QuantArgs._fields_]
    c_name = {"global_fp8_max": "global_fp8_max"}
    src = tmp_path / "layout.c"
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "nvfp4.h"', "int main(void) {"]
    for f in fields:
        lines.append(f'  printf("%zu\\n", offsetof(nvfp4_quant_args, {c_name.get(f, f)}));')
    lines += ['  printf("%zu\\n", sizeof(nvfp4_quant_args));', "  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    import subprocess
    r = subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                        "-I/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"cannot build a host program against the HIP headers: {r.stderr[:200]}")
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [getattr(N.QuantArgs, f).offset for f in fields] + [ctypes.sizeof(N.QuantArgs)]
    assert got == want


def test_workspace_size_agrees():
    hdr = open(HEADERS[0]).read()
    n = int(re.search(r"#define NVFP4_WORKSPACE_BYTES (\d+)", hdr).group(1))
    assert N.lib().nvfp4_workspace_bytes() == N.WORKSPACE_BYTES == n


def _dq(**kw):
    a = dict(codes=FAKE, scales=FAKE, rows=16, cols=32, amax=FAKE, gmax=448.0, fmt=0,
             f32=FAKE, b16=None, bs=None, xref=None, sse=None, ws=None)
    a.update(kw)
    return N.lib().nvfp4_dequantize(a["codes"], a["scales"], a["rows"], a["cols"], a["amax"],
                                    a["gmax"], a["fmt"], a["f32"], a["b16"], a["bs"], a["xref"],
                                    a["sse"], a["ws"], None)


@pytest.mark.parametrize("kw", [
    dict(codes=None), dict(scales=None), dict(amax=None), dict(cols=8), dict(rows=-2),
    dict(fmt=5), dict(gmax=0.0), dict(gmax=-3.0), dict(xref=FAKE, ws=FAKE), dict(sse=FAKE, ws=FAKE),
    dict(f32=FAKE_ODD), dict(sse=FAKE_ODD, xref=FAKE, ws=FAKE),
    # the error report needs a workspace, 16-byte aligned
    dict(sse=FAKE, xref=FAKE), dict(sse=FAKE, xref=FAKE, ws=FAKE_ODD),
])
def test_dequantize_rejects(kw):
    assert _dq(**kw) == N.ERR_INVALID


def test_dequantize_empty_ok():
    assert _dq(rows=0) == N.OK
    assert _dq(rows=0, sse=FAKE, xref=FAKE, ws=FAKE) == N.OK


def test_amax_rejects():
    lib = N.lib()
    assert lib.nvfp4_tensor_amax(FAKE, -1, FAKE, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax(None, 16, FAKE, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax(FAKE, 16, None, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax(FAKE_ODD, 16, FAKE, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax(FAKE, 16, FAKE, None, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax(FAKE, 16, FAKE, FAKE_ODD, None) == N.ERR_INVALID
    # more than NVFP4_MAX_ELEMENTS = 2^44 elements
    assert lib.nvfp4_tensor_amax(FAKE, (1 << 44) + 1, FAKE, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax(FAKE, (1 << 63) - 1, FAKE, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax_noalloc(FAKE, (1 << 44) + 16, FAKE, None) == N.ERR_INVALID


def test_fakequant_rejects():
    lib = N.lib()
    f = lib.nvfp4_fakequant_fwd
    assert f(None, 16, 16, FAKE, None, FAKE, None) == N.ERR_INVALID
    assert f(FAKE, 16, 8, FAKE, None, FAKE, None) == N.ERR_INVALID
    assert f(FAKE, 16, 16, None, None, FAKE, None) == N.ERR_INVALID
    assert f(FAKE, 16, 16, FAKE, None, None, None) == N.ERR_INVALID
    assert f(FAKE, 0, 16, FAKE, None, FAKE, None) == N.OK
    b = lib.nvfp4_fakequant_bwd
    # dual scales need grad_s_post and tied scales must not get one
    assert b(FAKE, FAKE, 16, 16, FAKE, FAKE, FAKE, FAKE, None, None) == N.ERR_INVALID
    assert b(FAKE, FAKE, 16, 16, FAKE, None, FAKE, FAKE, FAKE, None) == N.ERR_INVALID
    assert b(FAKE, None, 16, 16, FAKE, None, FAKE, FAKE, None, None) == N.ERR_INVALID
    assert b(FAKE, FAKE, 16, 16, FAKE, None, FAKE, None, None, None) == N.ERR_INVALID
    assert b(FAKE, FAKE, 0, 16, FAKE, None, FAKE, FAKE, None, None) == N.OK


def test_row_amax_rejects():
    f = N.lib().nvfp4_row_amax
    assert f(FAKE, -1, 16, FAKE, None) == N.ERR_INVALID
    assert f(FAKE, 16, 24, FAKE, None) == N.ERR_INVALID
    assert f(None, 16, 16, FAKE, None) == N.ERR_INVALID
    assert f(FAKE, 16, 16, None, None) == N.ERR_INVALID
    assert f(FAKE_ODD, 16, 16, FAKE, None) == N.ERR_INVALID
    assert f(FAKE, 16, 16, FAKE + 2, None) == N.ERR_INVALID
    assert f(None, 0, 16, None, None) == N.OK


def _qrs(**kw):
    kw.setdefault("ra", FAKE)
    kw["amax"] = kw.pop("ra")
    return N.lib().nvfp4_quantize_rowscaled(_qargs(**kw), None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(ra=None), dict(rows=-1), dict(cols=24), dict(fmt=2), dict(select=5),
    dict(rnd=2), dict(rnd=1, select=1), dict(rnd=1, select=4), dict(gmax=-1.0), dict(gmax=float("nan")),
    dict(codes=None), dict(scales=None), dict(codes=FAKE_ODD), dict(scales=FAKE + 2),
    dict(x=FAKE_ODD), dict(ra=FAKE + 2), dict(count4=FAKE_ODD, ws=FAKE), dict(count4=FAKE),
    dict(axes=2), dict(axes=3),
])
def test_quantize_rowscaled_rejects(kw):
    assert _qrs(**kw) == N.ERR_INVALID


def test_quantize_rowscaled_empty_ok():
    assert _qrs(rows=0) == N.OK and _qrs(cols=0) == N.OK


def _qpt(**kw):
    ra = kw.pop("ra", FAKE)
    kw.setdefault("amax", None)  # not read: the call computes the row amaxes
    return N.lib().nvfp4_quantize_pertoken(_qargs(**kw), ra, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(ra=None), dict(ra=FAKE + 2), dict(rows=-1), dict(cols=24), dict(fmt=2),
    dict(select=5), dict(rnd=2), dict(rnd=1, select=1), dict(gmax=-1.0), dict(codes=None),
    dict(scales=None), dict(codes=FAKE_ODD), dict(x=FAKE_ODD), dict(count4=FAKE),
    dict(axes=2), dict(axes=3),
])
def test_quantize_pertoken_rejects(kw):
    assert _qpt(**kw) == N.ERR_INVALID


def test_quantize_pertoken_empty_ok():
    # no rows: nothing to write and no launch (cols == 0 with rows launches
    # the row amax, which writes the empty rows' zeros; GPU tests cover it)
    assert _qpt(rows=0) == N.OK


def _dqrs(**kw):
    a = dict(codes=FAKE, scales=FAKE, rows=16, cols=32, ra=FAKE, gmax=448.0, fmt=0,
             f32=FAKE, b16=None, bs=None, xref=None, sse=None, ws=None)
    a.update(kw)
    return N.lib().nvfp4_dequantize_rowscaled(a["codes"], a["scales"], a["rows"], a["cols"],
                                              a["ra"], a["gmax"], a["fmt"], a["f32"], a["b16"],
                                              a["bs"], a["xref"], a["sse"], a["ws"], None)


@pytest.mark.parametrize("kw", [
    dict(codes=None), dict(ra=None), dict(cols=8), dict(fmt=3), dict(gmax=0.0),
    dict(xref=FAKE, ws=FAKE), dict(f32=FAKE_ODD), dict(ra=FAKE + 2), dict(xref=FAKE, sse=FAKE),
])
def test_dequantize_rowscaled_rejects(kw):
    assert _dqrs(**kw) == N.ERR_INVALID


def _q2d(**kw):
    a = dict(rows=32, cols=32, select=0, axes=3)
    a.update(kw)
    return N.lib().nvfp4_quantize_2d(_qargs(**a), None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(amax=None), dict(rows=24), dict(cols=8), dict(fmt=2), dict(gmax=-2.0),
    dict(codes=None), dict(scales=None), dict(codes_t=None), dict(scales_t=None),
    dict(codes_t=FAKE_ODD), dict(codes=FAKE_ODD), dict(x=FAKE_ODD), dict(amax=FAKE + 2),
    dict(select=1), dict(rnd=1), dict(axes=2),
])
def test_quantize_2d_rejects(kw):
    assert _q2d(**kw) == N.ERR_INVALID


def test_quantize_2d_empty_ok():
    assert _q2d(rows=0) == N.OK
    assert _q2d(codes_t=None, scales_t=None, rows=0, axes=1) == N.OK


def _rq(**kw):
    a = dict(codes=FAKE, scales=FAKE, rows=64, cols=32, amax=FAKE, ra=None, gmax=448.0, fmt=0,
             target=1, dst=FAKE, dgmax=0.0, dfmt=0, seed=0, out=FAKE, out_s=FAKE)
    a.update(kw)
    return N.lib().nvfp4_requantize_t(a["codes"], a["scales"], a["rows"], a["cols"], a["amax"],
                                      a["ra"], a["gmax"], a["fmt"], a["target"], a["dst"],
                                      a["dgmax"], a["dfmt"], a["seed"], a["out"], a["out_s"], None)


@pytest.mark.parametrize("kw", [
    dict(codes=None), dict(scales=None), dict(amax=None), dict(ra=FAKE), dict(cols=24),
    dict(rows=-32), dict(fmt=5), dict(gmax=0.0), dict(gmax=float("inf")), dict(target=2),
    dict(rows=48), dict(target=0, rows=40), dict(target=0, dst=None), dict(target=0, dfmt=3),
    dict(target=0, dgmax=-1.0), dict(out=None), dict(out_s=None), dict(out=FAKE_ODD),
    dict(codes=FAKE_ODD), dict(amax=FAKE + 2), dict(amax=None, ra=FAKE + 2),
    dict(scales=FAKE + 1),
])
def test_requantize_t_rejects(kw):
    assert _rq(**kw) == N.ERR_INVALID


def test_requantize_t_empty_ok():
    assert _rq(rows=0) == N.OK
    assert _rq(cols=0, target=0, rows=48) == N.OK
    assert _rq(amax=None, ra=FAKE, rows=0) == N.OK


@pytest.mark.parametrize("kw", [
    dict(codes=None), dict(amax=None), dict(ra=FAKE), dict(cols=8), dict(fmt=4), dict(gmax=-1.0),
    dict(out=None), dict(out=FAKE + 1), dict(ws=None), dict(ws=FAKE_ODD),
])
def test_dequantized_amax_rejects(kw):
    a = dict(codes=FAKE, scales=FAKE, rows=16, cols=32, amax=FAKE, ra=None, gmax=448.0, fmt=0,
             out=FAKE, ws=FAKE)
    a.update(kw)
    assert N.lib().nvfp4_dequantized_amax(a["codes"], a["scales"], a["rows"], a["cols"],
                                          a["amax"], a["ra"], a["gmax"], a["fmt"], a["out"],
                                          a["ws"], None) == N.ERR_INVALID


def test_rht_calls_reject():
    lib = N.lib()
    f = lib.nvfp4_rht_amax
    assert f(FAKE, 16, 32, 1, 0, FAKE, None, None) == N.ERR_INVALID  # no workspace
    assert f(FAKE, 16, 32, 3, 0, FAKE, FAKE, None) == N.ERR_INVALID  # one axis only
    assert f(FAKE, 16, 24, 1, 0, FAKE, FAKE, None) == N.ERR_INVALID
    assert f(FAKE, 24, 32, 2, 0, FAKE, FAKE, None) == N.ERR_INVALID
    q = lib.nvfp4_quantize_rht
    assert q(_qargs(axes=3), 0, None) == N.ERR_INVALID
    assert q(_qargs(axes=2, rows=24), 0, None) == N.ERR_INVALID
    assert q(_qargs(count4=FAKE), 0, None) == N.ERR_INVALID
    assert q(None, 0, None) == N.ERR_INVALID
    assert q(_qargs(rows=0), 0, None) == N.OK


@pytest.mark.parametrize("entry", ["nvfp4_fakequant_fwd_amax", "nvfp4_fakequant_bwd_amax"])
def test_fakequant_amax_rejects(entry):
    lib = N.lib()
    if entry.endswith("fwd_amax"):
        f = lambda **k: lib.nvfp4_fakequant_fwd_amax(k.get("x", FAKE), 16, k.get("cols", 32),
                                                     k.get("a", FAKE), None, k.get("o", FAKE), None)
    else:
        f = lambda **k: lib.nvfp4_fakequant_bwd_amax(k.get("x", FAKE), FAKE, 16, k.get("cols", 32),
                                                     k.get("a", FAKE), None, k.get("o", FAKE),
                                                     FAKE, None, None)
    for kw in (dict(x=None), dict(a=None), dict(cols=24), dict(o=FAKE_ODD), dict(x=FAKE_ODD)):
        assert f(**kw) == N.ERR_INVALID, kw


def test_test_hooks_reject():
    lib = N.lib()
    assert lib.nvfp4_test_e2m1_rne_range(1, (1 << 32), FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_test_scale_encode_range(0, 0x7FFFFFFF, 2, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_test_scale_encode_range(7, 0, 2, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_test_e2m1_sr(None, FAKE, 4, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_test_sr_hash(0, 0, -1, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_test_e4m3_sr(FAKE, FAKE, 6, FAKE, None) == N.ERR_INVALID
    assert lib.nvfp4_test_e4m3_sr(FAKE, None, 4, FAKE, None) == N.ERR_INVALID


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(N, "_lib", None)
    monkeypatch.setattr(N, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(N.NativeError):
        N.lib()
