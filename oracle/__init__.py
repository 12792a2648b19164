"""Plain fp64 CPU oracles for scaled dot-product attention and GroupNorm.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and imports nothing from it.

The arithmetic lives in C: ``attn_oracle.c`` (the plain definition of
``O = softmax(sigma * Q K^T) V`` from the page "Diffusion inference engine
from scratch: Rust + wgpu", section 3.2, evaluated row by row in IEEE double
with sequential sums) and ``group_norm_oracle.c`` (the same page's section
3.1 GroupNorm, two-pass mean and variance per group, optional SiLU).  This
module only compiles them with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "attn_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
GN_SRC = os.path.join(_HERE, "group_norm_oracle.c")
GN_LIB = os.path.join(_HERE, "liboracle_gn.so")

# -O2, no -ffast-math and no FP contraction: sequential, reproducible sums.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
          "-ffp-contract=off", "-fno-fast-math"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc into a shared library; return its path."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)


def _as_f64(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError("oracle tensors are [B, H, L, d]")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


class Oracle:
    """ctypes handle on one compiled copy of ``attn_oracle.c``."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_attn_f64.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                        _i64, _i64, ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_rows_f64.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64,
                                             _i64, _i64, ctypes.c_double, _lp,
                                             _i64, _dp, ctypes.c_int]
        lib.oracle_attn_probs_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64,
                                              _i64, _i64, _i64, _i64,
                                              ctypes.c_double]
        lib.oracle_max_threads.argtypes = []
        for fn in (lib.oracle_attn_f64, lib.oracle_attn_rows_f64,
                   lib.oracle_attn_probs_f64, lib.oracle_max_threads):
            fn.restype = ctypes.c_int
        self._lib = lib

    @staticmethod
    def _shapes(q, k, v):
        B, H, Lq, d = q.shape
        if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
            raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
        return B, H, Lq, k.shape[2], d

    def max_threads(self) -> int:
        return int(self._lib.oracle_max_threads())

    def attn(self, q, k, v, scale: float, nthreads: int = 0) -> np.ndarray:
        """O[B,H,Lq,d] in float64 for every query row."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, H, Lq, Lk, d = self._shapes(q, k, v)
        out = np.empty((B, H, Lq, d), dtype=np.float64)
        rc = self._lib.oracle_attn_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                       B, H, Lq, Lk, d, float(scale), nthreads)
        if rc:
            raise RuntimeError(f"oracle_attn_f64 failed with code {rc}")
        return out

    def attn_rows(self, q, k, v, scale: float, rows, nthreads: int = 0) -> np.ndarray:
        """O for the flattened query rows ``(b*H + h)*Lq + i``; shape [n, d]."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, H, Lq, Lk, d = self._shapes(q, k, v)
        rows = np.ascontiguousarray(rows, dtype=np.int64).ravel()
        out = np.empty((rows.size, d), dtype=np.float64)
        rc = self._lib.oracle_attn_rows_f64(_ptr(q), _ptr(k), _ptr(v), B, H, Lq,
                                            Lk, d, float(scale),
                                            rows.ctypes.data_as(_lp), rows.size,
                                            _ptr(out), nthreads)
        if rc:
            raise RuntimeError(f"oracle_attn_rows_f64 failed with code {rc}")
        return out

    def attn_probs(self, q, k, v, scale: float):
        """(O[B,H,Lq,d], P[B,H,Lq,Lk]) for small cases."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, H, Lq, Lk, d = self._shapes(q, k, v)
        out = np.empty((B, H, Lq, d), dtype=np.float64)
        probs = np.empty((B, H, Lq, Lk), dtype=np.float64)
        rc = self._lib.oracle_attn_probs_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                             _ptr(probs), B, H, Lq, Lk, d,
                                             float(scale))
        if rc:
            raise RuntimeError(f"oracle_attn_probs_f64 failed with code {rc}")
        return out, probs


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from this directory's source (compiled if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default


def attn(q, k, v, scale, nthreads=0):
    return get().attn(q, k, v, scale, nthreads)


def attn_rows(q, k, v, scale, rows, nthreads=0):
    return get().attn_rows(q, k, v, scale, rows, nthreads)


def attn_probs(q, k, v, scale):
    return get().attn_probs(q, k, v, scale)


# ---------------------------------------------------------------------------
# GroupNorm (+ SiLU)

class GroupNormOracle:
    """ctypes handle on one compiled copy of ``group_norm_oracle.c``."""

    def __init__(self, path: str = GN_LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_group_norm_f64.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64,
                                              ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.oracle_group_norm_f64.restype = ctypes.c_int
        self._lib = lib

    def group_norm(self, x, gamma, beta, groups: int, eps: float, silu: bool = False,
                   nthreads: int = 0) -> np.ndarray:
        """x: [N, C, ...] (trailing dims flattened); gamma, beta: [C]."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        N, C = x.shape[0], x.shape[1]
        S = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
        g = np.ascontiguousarray(gamma, dtype=np.float64).reshape(-1)
        b = np.ascontiguousarray(beta, dtype=np.float64).reshape(-1)
        if g.size != C or b.size != C:
            raise ValueError("gamma and beta must have C entries")
        y = np.empty_like(x)
        rc = self._lib.oracle_group_norm_f64(_ptr(x), _ptr(g), _ptr(b), _ptr(y), N, C, S,
                                             groups, float(eps), int(bool(silu)), nthreads)
        if rc != 0:
            raise ValueError(f"oracle_group_norm_f64 failed ({rc})")
        return y


_default_gn: GroupNormOracle | None = None


def get_gn() -> GroupNormOracle:
    """The GroupNorm oracle built from this directory's source."""
    global _default_gn
    if _default_gn is None:
        if not os.path.exists(GN_LIB) or os.path.getmtime(GN_LIB) < os.path.getmtime(GN_SRC):
            build(GN_SRC, GN_LIB)
        _default_gn = GroupNormOracle(GN_LIB)
    return _default_gn


def group_norm(x, gamma, beta, groups, eps, silu=False, nthreads=0):
    return get_gn().group_norm(x, gamma, beta, groups, eps, silu, nthreads)
