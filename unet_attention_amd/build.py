"""Build libsdattn.so for gfx950 with hipcc (in-tree, no JIT cache).

Every source under csrc/ is compiled to an object in parallel, then linked
into ``unet_attention_amd/libsdattn.so``.  Packed-fp32 instructions are
disabled on the device side (``-packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsdattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str, extra: list[str]) -> None:
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


# Sources compiled once per head-dim class (-DSDATTN_DK=<dk>) so that the
# many kernel instantiations build in parallel; 0 is the dispatcher object.
PER_DK = {"attn_mfma.hip": [0] + list(range(16, 257, 16))}


def _units(srcs: list[str]) -> list[tuple[str, str, list[str]]]:
    """(source, object, extra flags) for every object of the library."""
    units = []
    for s in srcs:
        base = os.path.basename(s)
        if base in PER_DK:
            for dk in PER_DK[base]:
                units.append((s, os.path.join(BUILD_DIR, f"{base}.dk{dk}.o"),
                              [f"-DSDATTN_DK={dk}"]))
        else:
            units.append((s, os.path.join(BUILD_DIR, base + ".o"), []))
    return units


def build(extra: list[str] | None = None, jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every csrc/*.hip file and link libsdattn.so; return its path."""
    extra = list(extra or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    units = _units(srcs)
    objs = [o for _, o, _ in units]
    jobs = jobs or max(1, min(len(units), os.cpu_count() or 2, 16))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, o, extra + fl) for s, o, fl in units]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                    "-o", tmp], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    build_peak(verbose=verbose)
    return LIB


PEAK_SRC = os.path.join(PKG, "peak", "peak.hip")
PEAK_LIB = os.path.join(PKG, "libsdattn_peak.so")


def build_peak(verbose: bool = True) -> str:
    """The attainable-peak microbenchmarks (a separate library, not part of
    libsdattn's interface) used by the benchmark's peak leg."""
    tmp = PEAK_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", PEAK_SRC, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on peak.hip:\n{r.stdout}")
    os.replace(tmp, PEAK_LIB)
    if verbose:
        print(f"built {PEAK_LIB}", file=sys.stderr)
    return PEAK_LIB


if __name__ == "__main__":
    build()
