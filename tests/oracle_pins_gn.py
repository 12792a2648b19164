"""Pins of the GroupNorm (+ SiLU) oracle to facts that do not come from the
oracle itself: closed forms derived by hand, invariants of normalisation,
special values of SiLU, and torch's own fp64 group_norm on the CPU.

Each pin takes a ``GroupNormOracle``-like object and raises AssertionError
when the oracle disagrees.  ``tests/test_oracle_gn.py`` runs them, and also
runs them against deliberately broken copies of the oracle source.
"""
from __future__ import annotations

import math

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def pin_constant_groups(orc):
    """Every group constant (different constants per group, equal inside a
    group of consecutive channels): x - mu is exactly 0, so y = beta[c]."""
    N, C, S, G = 2, 6, 5, 3
    x = np.empty((N, C, S))
    for n in range(N):
        for c in range(C):
            x[n, c, :] = 1.5 + 2.0 * (c // (C // G)) + 10.0 * n
    gamma = _rng(1).standard_normal(C)
    beta = _rng(2).standard_normal(C)
    y = orc.group_norm(x, gamma, beta, G, 1e-5)
    _close(y, np.broadcast_to(beta[None, :, None], y.shape), 0.0, "constant groups")


def pin_two_values(orc):
    """A group holding a and b equally often: mu = (a+b)/2, every deviation is
    +-h with h = (a-b)/2, var = h^2, so y = +-h / sqrt(h^2 + eps)."""
    a, b, eps = 3.25, -1.75, 0.5
    S = 8
    x = np.empty((1, 2, S))
    x[0, 0, :] = a
    x[0, 1, :] = b
    y = orc.group_norm(x, np.ones(2), np.zeros(2), 1, eps)
    h = (a - b) / 2.0
    want = h / math.sqrt(h * h + eps)
    _close(y[0, 0], np.full(S, want), 1e-15, "two values (a)")
    _close(y[0, 1], np.full(S, -want), 1e-15, "two values (b)")


def pin_unit_moments(orc):
    """eps = 0, gamma = 1, beta = 0: every group's outputs have mean 0 and
    mean square 1 (population variance)."""
    N, C, S, G = 3, 8, 37, 4
    x = 4.0 + 3.0 * _rng(3).standard_normal((N, C, S))
    y = orc.group_norm(x, np.ones(C), np.zeros(C), G, 0.0).reshape(N, G, -1)
    _close(y.mean(-1), np.zeros((N, G)), 1e-13, "group mean")
    _close((y * y).mean(-1), np.ones((N, G)), 1e-12, "group mean square")


def pin_shift_invariance(orc):
    """Adding a constant to a whole group leaves its output unchanged."""
    N, C, S, G = 2, 6, 11, 3
    x = _rng(4).standard_normal((N, C, S))
    gamma, beta = _rng(5).standard_normal(C), _rng(6).standard_normal(C)
    t = np.repeat(np.array([[100.0, -7.0, 0.5], [3.0, 40.0, -60.0]]), C // G, axis=1)
    y0 = orc.group_norm(x, gamma, beta, G, 1e-5)
    y1 = orc.group_norm(x + t[:, :, None], gamma, beta, G, 1e-5)
    _close(y1, y0, 1e-11, "shift invariance")


def pin_scale_invariance(orc):
    """eps = 0: scaling a group by s > 0 leaves the normalised values
    unchanged; s < 0 negates them."""
    N, C, S, G = 1, 4, 16, 2
    x = _rng(7).standard_normal((N, C, S))
    y0 = orc.group_norm(x, np.ones(C), np.zeros(C), G, 0.0)
    _close(orc.group_norm(x * 8.0, np.ones(C), np.zeros(C), G, 0.0), y0, 1e-13, "scale 8")
    _close(orc.group_norm(x * -0.25, np.ones(C), np.zeros(C), G, 0.0), -y0, 1e-13, "scale -1/4")


def pin_group_independence(orc):
    """Changing one group's input changes no other group's output."""
    N, C, S, G = 2, 8, 9, 4
    x = _rng(8).standard_normal((N, C, S))
    gamma, beta = _rng(9).standard_normal(C), _rng(10).standard_normal(C)
    y0 = orc.group_norm(x, gamma, beta, G, 1e-5)
    x2 = x.copy()
    x2[1, 4, :3] += 2.0   # part of sample 1, group 2 (a whole-group affine map would not show)
    y1 = orc.group_norm(x2, gamma, beta, G, 1e-5)
    mask = np.ones_like(y0, dtype=bool)
    mask[1, 4:6, :] = False
    _close(y1[mask], y0[mask], 0.0, "other groups")
    assert np.abs(y1[1, 4:6] - y0[1, 4:6]).max() > 1e-3, "changed group did not change"


def pin_per_channel_affine(orc):
    """y(gamma, beta) = gamma[c] * y(1, 0) + beta[c], channel by channel."""
    N, C, S, G = 2, 6, 7, 2
    x = _rng(11).standard_normal((N, C, S)) + 2.0
    gamma, beta = _rng(12).standard_normal(C), _rng(13).standard_normal(C)
    y1 = orc.group_norm(x, np.ones(C), np.zeros(C), G, 1e-3)
    y = orc.group_norm(x, gamma, beta, G, 1e-3)
    _close(y, gamma[None, :, None] * y1 + beta[None, :, None], 1e-14, "affine")


def pin_silu_special_values(orc):
    """Constant groups give y = beta before SiLU; sigmoid(ln 3) = 3/4 and
    sigmoid(-ln 3) = 1/4, so SiLU(+-ln 3) = 3 ln 3 / 4 and -ln 3 / 4;
    SiLU(0) = 0."""
    L3 = math.log(3.0)
    x = np.full((1, 3, 4), 2.0)
    beta = np.array([L3, -L3, 0.0])
    y = orc.group_norm(x, np.ones(3), beta, 3, 1e-5, silu=True)
    _close(y[0, 0], np.full(4, 0.75 * L3), 1e-15, "silu(ln 3)")
    _close(y[0, 1], np.full(4, -0.25 * L3), 1e-15, "silu(-ln 3)")
    _close(y[0, 2], np.zeros(4), 0.0, "silu(0)")


def pin_torch_group_norm(orc):
    """torch.nn.functional.group_norm (+ silu) in fp64 on the CPU."""
    import torch
    import torch.nn.functional as F
    for (N, C, H, W, G, eps, seed) in ((2, 32, 5, 7, 8, 1e-5, 14), (1, 12, 3, 3, 12, 1e-6, 15),
                                       (3, 10, 4, 1, 1, 1e-2, 16)):
        r = _rng(seed)
        x = 1.5 + 2.0 * r.standard_normal((N, C, H, W))
        gamma, beta = r.standard_normal(C), r.standard_normal(C)
        ref = F.group_norm(torch.from_numpy(x), G, torch.from_numpy(gamma),
                           torch.from_numpy(beta), eps)
        _close(orc.group_norm(x, gamma, beta, G, eps), ref.numpy(), 1e-12, f"torch G={G}")
        _close(orc.group_norm(x, gamma, beta, G, eps, silu=True), F.silu(ref).numpy(), 1e-12,
               f"torch silu G={G}")


ALL_PINS = [pin_constant_groups, pin_two_values, pin_unit_moments, pin_shift_invariance,
            pin_scale_invariance, pin_group_independence, pin_per_channel_affine,
            pin_silu_special_values, pin_torch_group_norm]
