"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code.

- The CPU oracle (oracle/nvfp4_oracle.c), driven by
  tests/sanitize/oracle_driver.c over shapes, options and special values
  on exact-size heap buffers.
- The library's host side: every source compiled host-only (no device
  code), linked with host stand-ins for the HIP runtime
  (tests/sanitize/hip_runtime_stubs.c).  tests/sanitize/abi_driver.c drives
  every C ABI entry point through validation, defaults and launch-shape
  arithmetic with valid, invalid and extreme-size arguments.

Both run here, without a GPU; a sanitizer report or an unexpected status
fails the test.  The function sanitizer is left out of the library build:
its check on indirect calls does not apply to kernel launch stubs.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_02_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize=function",
             "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _have(*tools):
    return all(os.path.exists(t) or shutil.which(t) for t in tools)


@pytest.mark.skipif(not _have("gcc"), reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"] + SAN_FLAGS[:1] +
         SAN_FLAGS[2:] + ["-o", exe, os.path.join(SAN_DIR, "oracle_driver.c"),
                          os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-lm"])
    r = _run([exe], env=ENV, timeout=600)
    assert "all calls returned as expected" in r.stdout


@pytest.mark.skipif(not _have(HIPCC, CLANG, CLANGXX), reason="ROCm compilers not found")
def test_c_abi_host_side_under_asan_ubsan(tmp_path):
    objs = []
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith(".hip"):
            continue
        o = str(tmp_path / (f[:-4] + ".o"))
        # host-only: no device code is built, so the sanitizer flags apply to
        # host code alone (each is also marked for the host explicitly)
        cmd = [HIPCC, "--offload-host-only", "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, f),
               "-o", o, "-fno-omit-frame-pointer", "-g", "-O1"]
        for flag in SAN_FLAGS[:3]:
            cmd += ["-Xarch_host", flag]
        _run(cmd)
        objs.append(o)
    # the host-only objects name their (absent) device images; empty stand-ins
    nm = _run(["nm", "-u"] + objs).stdout
    fatbins = sorted(set(re.findall(r"__hip_fatbin_[0-9a-f]+", nm)))
    fb_c = tmp_path / "fatbins.c"
    fb_c.write_text("".join(f"const unsigned char {s}[16] = {{0}};\n" for s in fatbins))
    inc = ["-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROCM, "include")]
    extra = []
    for src, flags in ((str(fb_c), []), (os.path.join(SAN_DIR, "hip_runtime_stubs.c"), ["-std=c11"]),
                       (os.path.join(SAN_DIR, "abi_driver.c"), ["-std=c11"] + inc)):
        o = str(tmp_path / (os.path.basename(src)[:-2] + ".o"))
        _run([CLANG] + SAN_FLAGS + flags + ["-c", src, "-o", o])
        extra.append(o)
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX] + SAN_FLAGS + ["-o", exe] + extra + objs)
    r = _run([exe], env=ENV, timeout=600)
    assert "every status as expected" in r.stdout
