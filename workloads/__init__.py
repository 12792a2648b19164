"""Seeded synthetic inputs for the UNet attention workloads.

This module serves both the HIP path's tests/benchmark and the CPU oracle.
It holds no attention arithmetic: it only names the workload shapes and
draws their Q, K, V tensors.

Shapes follow the diffusion pages: queries come from the latent feature map
flattened to HW tokens (64x64 latent for a 512x512 image, 8x VAE
compression), keys/values either from the same map (self-attention) or from
the 77-token CLIP text context (cross-attention); classifier-free guidance
doubles the batch (uncond + cond), so B = 2 with per-batch contexts.
Values are N(0, 1) stand-ins for activations; no dataset or weights exist
here and none are needed.

Recipe (identical for every consumer):
  * rng = numpy.random.default_rng(seed); q, k, v are drawn in that order,
    each as float32 standard normals in C order of [B, H, L, d];
  * bf16 (fp16) workloads round each float32 to bf16 (fp16) with
    round-to-nearest-even; both sides then see exactly the rounded values;
  * heavy-key workloads pick, per (b, h) in order, round(frac * Lk) key rows
    without replacement from the same generator (after v) and multiply those
    rows by a power of two (exact in bf16 and fp16 at these magnitudes), to
    stress running-max tracking.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "self" or "cross"
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: str           # "f32" or "bf16" (input storage type)
    seed: int
    heavy_frac: float = 0.0
    heavy_mult: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32: the exact value both sides use."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> int:
        """4*B*H*Lq*Lk*d: the two matrix products, softmax not counted."""
        return 4 * self.B * self.H * self.Lq * self.Lk * self.d

    def bytes_alg(self, out_bytes: int | None = None) -> int:
        """Compulsory HBM bytes: Q, K, V read once and O written once."""
        elt = 4 if self.dtype == "f32" else 2
        ob = elt if out_bytes is None else out_bytes
        return (elt * (self.B * self.H * self.Lq * self.d
                       + 2 * self.B * self.H * self.Lk * self.d)
                + ob * self.B * self.H * self.Lq * self.d)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads at their full sizes (64x64 latent = SD 1.5 at 512^2;
# 32x32 and 16x16 are the lower-resolution UNet levels; 128x128 is a
# 1024^2 image).  Head counts and widths follow C = H*d of the SD-1.5 UNet
# (320 = 8x40, 640 = 8x80, 1280 = 8x160).
WORKLOADS = {
    "1": Workload("1", "cross", 1, 1, 64, 77, 40, "f32", 1000,
                  note="single-head cross-attention, 8x8 latent, fp32"),
    "2": Workload("2", "self", 2, 8, 4096, 4096, 40, "bf16", 2000,
                  note="self-attention, 64x64 latent, CFG batch 2"),
    "3": Workload("3", "cross", 2, 8, 4096, 77, 40, "bf16", 3000,
                  note="cross-attention, 64x64 latent, 77-token context"),
    "4a": Workload("4a", "self", 2, 8, 1024, 1024, 80, "bf16", 4001,
                   note="self-attention, 32x32 latent"),
    "4b": Workload("4b", "cross", 2, 8, 1024, 77, 80, "bf16", 4002,
                   note="cross-attention, 32x32 latent"),
    "4c": Workload("4c", "self", 2, 8, 256, 256, 160, "bf16", 4003,
                   note="self-attention, 16x16 latent"),
    "4d": Workload("4d", "cross", 2, 8, 256, 77, 160, "bf16", 4004,
                   note="cross-attention, 16x16 latent"),
    "5": Workload("5", "self", 8, 10, 16384, 16384, 64, "bf16", 5000,
                  heavy_frac=0.01, heavy_mult=8.0,
                  note="self-attention, 128x128 latent, 1% of keys x8"),
    # fp16 storage of the 64x64-latent pair and of the heavy-key workload.
    "2h": Workload("2h", "self", 2, 8, 4096, 4096, 40, "f16", 2100,
                   note="self-attention, 64x64 latent, fp16"),
    "3h": Workload("3h", "cross", 2, 8, 4096, 77, 40, "f16", 3100,
                   note="cross-attention, 64x64 latent, 77-token context, fp16"),
    "5h": Workload("5h", "self", 8, 10, 16384, 16384, 64, "f16", 5100,
                   heavy_frac=0.01, heavy_mult=8.0,
                   note="self-attention, 128x128 latent, 1% of keys x8, fp16"),
    # Longer text contexts than CLIP's 77 tokens (several concatenated prompt
    # chunks, or larger text encoders), 64x64 latent.
    "6a": Workload("6a", "cross", 2, 8, 4096, 256, 40, "bf16", 6001,
                   note="cross-attention, 64x64 latent, 256-token context"),
    "6b": Workload("6b", "cross", 2, 8, 4096, 512, 40, "bf16", 6002,
                   note="cross-attention, 64x64 latent, 512-token context"),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite standard normals, so the NaN case does not arise.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """Q, K, V as float32 values (exactly the stored values) and, for bf16
    and fp16 workloads, their 16-bit patterns."""
    w: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    heavy_rows: np.ndarray | None = None   # [B, H, n] key rows that were scaled


def make_inputs(w: Workload) -> Inputs:
    """Draw the workload's Q, K, V from its seed (see the module recipe)."""
    rng = np.random.default_rng(w.seed)
    qs = (w.B, w.H, w.Lq, w.d)
    ks = (w.B, w.H, w.Lk, w.d)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    heavy = None
    if w.dtype == "bf16":
        qb, kb, vb = (round_to_bf16_bits(t) for t in (q, k, v))
        q, k, v = (bf16_bits_to_f32(t) for t in (qb, kb, vb))
    elif w.dtype == "f16":
        q, k, v = (t.astype(np.float16).astype(np.float32) for t in (q, k, v))
    if w.heavy_frac > 0.0:
        n = int(round(w.heavy_frac * w.Lk))
        heavy = np.empty((w.B, w.H, n), dtype=np.int64)
        for b in range(w.B):
            for h in range(w.H):
                heavy[b, h] = rng.choice(w.Lk, size=n, replace=False)
                k[b, h, heavy[b, h], :] *= np.float32(w.heavy_mult)
    if w.dtype == "bf16":
        # Re-derive the bit patterns after the (exact) power-of-two scaling.
        qb, kb, vb = (round_to_bf16_bits(t) for t in (q, k, v))
        assert np.array_equal(bf16_bits_to_f32(kb), k)
        return Inputs(w, q, k, v, qb, kb, vb, heavy)
    if w.dtype == "f16":
        qb, kb, vb = (t.astype(np.float16).view(np.uint16) for t in (q, k, v))
        assert np.array_equal(kb.view(np.float16).astype(np.float32), k)
        return Inputs(w, q, k, v, qb, kb, vb, heavy)
    return Inputs(w, q, k, v, heavy_rows=heavy)


def sample_rows(w: Workload, n: int, seed: int = 7) -> np.ndarray:
    """Flattened query rows (b*H + h)*Lq + i for sampled parity checks.

    Every (b, h) contributes its first and last row, the rows on both sides
    of each 32- and 128-row boundary it crosses, and random rows, so that
    tiles, tile edges and the ragged tail are all covered.
    """
    rng = np.random.default_rng(seed)
    rows = set()
    per = max(1, n // (w.B * w.H))
    for bh in range(w.B * w.H):
        base = bh * w.Lq
        cand = {0, w.Lq - 1}
        for edge in (32, 128):
            t = (w.Lq // edge) * edge
            for e in (t - 1, t, edge - 1, edge):
                if 0 <= e < w.Lq:
                    cand.add(e)
        cand |= set(int(x) for x in rng.integers(0, w.Lq, size=per))
        rows |= {base + c for c in cand}
    return np.array(sorted(rows), dtype=np.int64)


# ---------------------------------------------------------------------------
# GroupNorm (+ SiLU) workloads: the UNet's resnet-block activations at each
# level of SD 1.5 at 512x512 (CFG batch 2, 32 groups), and a 128x128 level
# (1024x1024 images) whose groups exceed what one workgroup holds on chip.
# Recipe: rng = default_rng(seed); x = 1.5 + 2 * N(0, 1) as float32 in C
# order of [N, C, H, W] (a non-zero mean, as activations have), rounded to
# the storage type like the attention inputs; then gamma = 1 + 0.25 * N(0, 1)
# and beta = 0.5 * N(0, 1), float32, C values each.

@dataclass(frozen=True)
class GnWorkload:
    name: str
    N: int
    C: int
    H: int
    W: int
    G: int
    dtype: str           # "f32", "bf16" or "f16"
    seed: int
    eps: float = 1e-5
    silu: bool = True
    note: str = field(default="", compare=False)

    @property
    def HW(self) -> int:
        return self.H * self.W

    def bytes_alg(self, out_bytes: int | None = None) -> int:
        """x read once and y written once, plus gamma and beta."""
        e = 4 if self.dtype == "f32" else 2
        o = e if out_bytes is None else out_bytes
        return self.N * self.C * self.HW * (e + o) + 8 * self.C

    def with_(self, **kw) -> "GnWorkload":
        return replace(self, **kw)


GN_WORKLOADS = {
    "gn64": GnWorkload("gn64", 2, 320, 64, 64, 32, "bf16", 7001,
                       note="64x64 level, 320 channels"),
    "gn32": GnWorkload("gn32", 2, 640, 32, 32, 32, "bf16", 7002,
                       note="32x32 level, 640 channels"),
    "gn16": GnWorkload("gn16", 2, 1280, 16, 16, 32, "bf16", 7003,
                       note="16x16 level, 1280 channels"),
    "gn8": GnWorkload("gn8", 2, 1280, 8, 8, 32, "bf16", 7004,
                      note="8x8 level, 1280 channels"),
    "gn128": GnWorkload("gn128", 2, 320, 128, 128, 32, "bf16", 7005,
                        note="128x128 level (1024x1024 image): 163840-element groups"),
}


@dataclass
class GnInputs:
    w: GnWorkload
    x: np.ndarray                 # float32 values (exactly the stored ones)
    x_bits: np.ndarray | None     # 16-bit patterns for bf16/f16
    gamma: np.ndarray
    beta: np.ndarray


def make_gn_inputs(w: GnWorkload) -> GnInputs:
    rng = np.random.default_rng(w.seed)
    x = (1.5 + 2.0 * rng.standard_normal((w.N, w.C, w.H, w.W), dtype=np.float32)).astype(np.float32)
    bits = None
    if w.dtype == "bf16":
        bits = round_to_bf16_bits(x)
        x = bf16_bits_to_f32(bits)
    elif w.dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)
        bits = x.astype(np.float16).view(np.uint16)
    gamma = (1.0 + 0.25 * rng.standard_normal(w.C)).astype(np.float32)
    beta = (0.5 * rng.standard_normal(w.C)).astype(np.float32)
    return GnInputs(w, x, bits, gamma, beta)
