"""Helpers for the GPU parity tests: move seeded inputs to the device, call
the HIP library through its C ABI, and apply the parity gates."""
from __future__ import annotations

import sys

import numpy as np

# Gates from the accuracy target: bf16 inputs with fp32 accumulation must
# match the fp64 oracle within max-abs 1e-2 and mean-abs 1e-3; the fp32 path
# within 1e-4.
BF16_MAX, BF16_MEAN = 1e-2, 1e-3
F32_MAX = 1e-4


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault can be traced."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x, device="cuda"):
    """Inputs -> (q, k, v) torch tensors holding exactly the stored values."""
    import torch
    if x.w.dtype in ("bf16", "f16"):
        tdt = torch.bfloat16 if x.w.dtype == "bf16" else torch.float16
        cv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(
            tdt).to(device)
        return cv(x.q_bits), cv(x.k_bits), cv(x.v_bits)
    return tuple(torch.from_numpy(np.ascontiguousarray(t)).to(device) for t in (x.q, x.k, x.v))


def tensors_from_f32(q, k, v, dtype: str, device="cuda"):
    """float32 numpy arrays (already representable in `dtype`) -> device tensors."""
    import torch
    from workloads import round_to_bf16_bits
    if dtype == "bf16":
        cv = lambda a: torch.from_numpy(round_to_bf16_bits(a).view(np.int16)).view(
            torch.bfloat16).to(device)
        return cv(q), cv(k), cv(v)
    if dtype == "f16":
        cv = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.float16)).to(device)
        return cv(q), cv(k), cv(v)
    return tuple(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
                 for a in (q, k, v))


def run(entry: str, q, k, v, scale: float, out_dtype=None):
    """Call one C entry point (through the ctypes binding) and return the
    output as float64 numpy."""
    import torch
    import unet_attention_amd as sd
    fn = {"auto": sd.fwd, "cross": sd.cross_fwd, "stream": sd.stream_fwd}[entry]
    out = fn(q, k, v, scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def errors(got, want):
    e = np.abs(got - want)
    return float(e.max()), float(e.mean())


def assert_f32_gate(got, want, what=""):
    mx, mean = errors(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= F32_MAX, f"{what}: fp32 max-abs {mx:.3e} > {F32_MAX}"


def assert_bf16_gate(got, want, what=""):
    mx, mean = errors(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= BF16_MAX, f"{what}: max-abs {mx:.3e} > {BF16_MAX}"
    assert mean <= BF16_MEAN, f"{what}: mean-abs {mean:.3e} > {BF16_MEAN}"


def half_ulp_bf16(x):
    """Half a bf16 unit in the last place of each value (8 significant bits)."""
    m, e = np.frexp(np.abs(x))   # |x| = m * 2^e, m in [0.5, 1)
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def half_ulp_f16(x):
    """Half an fp16 unit in the last place (11 significant bits; subnormal
    spacing 2^-24 below 2^-14)."""
    m, e = np.frexp(np.abs(x))
    return np.where(x == 0, 0.0, np.maximum(np.ldexp(1.0, e - 12), 2.0 ** -25))


def assert_bf16_out_gate(got, want, what="", out="bf16"):
    """A 16-bit output adds its own rounding: allow half an ulp of the output
    type (bf16 or fp16) of the exact value on top of the bf16 gate,
    elementwise and on the mean."""
    h = half_ulp_bf16(want) if out == "bf16" else half_ulp_f16(want)
    e = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    worst = float((e - h).max())
    assert worst <= BF16_MAX, f"{what}: max(|err| - ulp/2) {worst:.3e} > {BF16_MAX}"
    assert float(e.mean()) <= BF16_MEAN + float(h.mean()), \
        f"{what}: mean {e.mean():.3e} > {BF16_MEAN} + {h.mean():.3e}"
