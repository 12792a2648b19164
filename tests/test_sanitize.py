"""CPU builds of the host code under AddressSanitizer and
UndefinedBehaviorSanitizer:

* both fp64 oracles (``oracle/*.c``, gcc), driven on small cases and on
  their argument checks by ``tests/native/oracle_sanitize.c``;
* the host layer of libsdattn (``sdattn_api.hip``: validation, device check,
  dispatch, operand layouts, launch-status mapping), compiled host-only and
  linked with ``tests/native/abi_sanitize.cpp``, which stands in for the
  three HIP runtime calls it makes and for the kernel launchers.

No GPU and no HIP runtime library are involved; sanitizers instrument host
code only.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def _check_clean(rc, out, what):
    assert rc == 0, f"{what} failed ({rc}):\n{out[-4000:]}"
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_oracles_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc missing")
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(NATIVE, "oracle_sanitize.c"),
                    os.path.join(ROOT, "oracle", "attn_oracle.c"),
                    os.path.join(ROOT, "oracle", "group_norm_oracle.c"), "-lm", "-o", exe])
    assert rc == 0, out
    _check_clean(*_run([exe], env=ENV), "oracle sanitizer run")


def test_host_abi_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ missing")
    flags = ["--cuda-host-only", "-O1", "-g", "-std=c++17",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
             "-I", os.path.join(ROOT, "unet_attention_amd", "csrc")]
    api_o, drv_o = str(tmp_path / "api.o"), str(tmp_path / "drv.o")
    rc, out = _run([HIPCC, *flags, "-c",
                    os.path.join(ROOT, "unet_attention_amd", "csrc", "sdattn_api.hip"),
                    "-o", api_o])
    assert rc == 0, out
    rc, out = _run([HIPCC, *flags, "-x", "hip", "-c", os.path.join(NATIVE, "abi_sanitize.cpp"),
                    "-o", drv_o])
    assert rc == 0, out
    exe = str(tmp_path / "abi_san")
    rc, out = _run([CLANGXX, "-fsanitize=address,undefined", api_o, drv_o, "-o", exe])
    assert rc == 0, out
    _check_clean(*_run([exe], env=ENV), "host ABI sanitizer run")
