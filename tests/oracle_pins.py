"""Pins that tie the CPU oracle to mathematics rather than to itself.

The pages print no worked numbers for attention, so every pin comes from
the definition of softmax attention (page "Diffusion inference engine from
scratch: Rust + wgpu", section 3.2) and from exact mathematics:

* brute force in 50-digit decimal arithmetic on tiny cases;
* closed forms (hand-derived fixtures, Lk = 1, equal keys, scale 0,
  constant values, one dominant score);
* invariants (rows of P sum to 1, query permutation equivariance, joint
  key/value permutation invariance, key-shift invariance, (b, h)
  independence, rows entry point == full entry point);
* library special cases (torch's fp64 SDPA on the CPU, numpy two-pass).

Each pin is a plain function of an ``oracle.Oracle`` handle that raises
AssertionError on failure, so the same pins can be run against deliberately
broken copies of the oracle (see test_oracle.py's mutation test).
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# brute force


def decimal_attention(q, k, v, scale, digits=50):
    """Attention for one (b, h) slice evaluated in `digits`-digit decimals.

    Inputs are converted exactly (Decimal(float) is exact), so the only
    error left is the decimal rounding at 50 digits."""
    getcontext().prec = digits
    sig = Decimal(float(scale))
    Lq, d = q.shape
    Lk = k.shape[0]
    out = np.empty((Lq, d))
    for i in range(Lq):
        s = [sig * sum(Decimal(float(q[i, c])) * Decimal(float(k[j, c]))
                       for c in range(d)) for j in range(Lk)]
        m = max(s)
        e = [(x - m).exp() for x in s]
        tot = sum(e)
        for c in range(d):
            out[i, c] = float(sum(e[j] / tot * Decimal(float(v[j, c]))
                                  for j in range(Lk)))
    return out


def pin_brute_force(orc):
    """Oracle == 50-digit decimal attention to 1e-13 on tiny cases."""
    for seed, (Lq, Lk, d) in enumerate([(1, 1, 1), (2, 3, 2), (3, 4, 4),
                                        (4, 2, 3), (4, 4, 4)]):
        q = _rand((1, 1, Lq, d), 10 + seed)
        k = _rand((1, 1, Lk, d), 20 + seed, 2.0)
        v = _rand((1, 1, Lk, d), 30 + seed)
        scale = 1.0 / math.sqrt(d) * (1.0 + 0.5 * seed)
        got = orc.attn(q, k, v, scale)[0, 0]
        want = decimal_attention(q[0, 0], k[0, 0], v[0, 0], scale)
        err = np.abs(got - want).max()
        assert err <= 1e-13, f"brute force Lq={Lq} Lk={Lk} d={d}: {err}"


# --------------------------------------------------------------------------
# closed forms


def pin_golden_closed_forms(orc):
    """Hand-derived cases stored under tests/golden/ with their derivations."""
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    assert cases
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        got = orc.attn(q, k, v, c["scale"])[0, 0]
        want = np.array(c["expected"], dtype=np.float64)
        err = np.abs(got - want).max()
        assert err <= c["tol"], f"golden case {c['name']}: err {err}"


def pin_single_key(orc):
    """Lk = 1: softmax over one key is 1, so O = v_0 exactly."""
    q = _rand((2, 3, 5, 8), 1)
    k = _rand((2, 3, 1, 8), 2)
    v = _rand((2, 3, 1, 8), 3)
    got = orc.attn(q, k, v, 0.35)
    assert np.array_equal(got, np.broadcast_to(v, got.shape)), "Lk=1 not exact"


def pin_identical_keys(orc):
    """All keys equal: every score in a row is equal, P is uniform, O = mean(V)."""
    q = _rand((1, 2, 6, 8), 4)
    k = np.broadcast_to(_rand((1, 2, 1, 8), 5), (1, 2, 9, 8)).copy()
    v = _rand((1, 2, 9, 8), 6)
    got = orc.attn(q, k, v, 0.4)
    want = np.broadcast_to(v.mean(axis=2, keepdims=True), got.shape)
    assert np.abs(got - want).max() <= 1e-14, "identical keys != mean(V)"


def pin_zero_scale(orc):
    """scale = 0: all scores zero, O = mean(V) whatever Q and K are."""
    q = _rand((1, 1, 4, 8), 7, 10.0)
    k = _rand((1, 1, 11, 8), 8, 10.0)
    v = _rand((1, 1, 11, 8), 9)
    got = orc.attn(q, k, v, 0.0)
    want = np.broadcast_to(v.mean(axis=2, keepdims=True), got.shape)
    assert np.abs(got - want).max() <= 1e-14, "scale 0 != mean(V)"


def pin_constant_values(orc):
    """Every value row equal to u: O = u since P rows sum to 1."""
    q = _rand((1, 1, 5, 8), 10)
    k = _rand((1, 1, 7, 8), 11)
    u = _rand((1, 1, 1, 8), 12)
    v = np.broadcast_to(u, (1, 1, 7, 8)).copy()
    got = orc.attn(q, k, v, 0.3)
    assert np.abs(got - np.broadcast_to(u, got.shape)).max() <= 1e-14


def pin_dominant_score(orc):
    """q = a*e_1, k_{j*} = e_1, other keys orthogonal to e_1: the score
    a*scale for j* exceeds the others (all 0) by a*scale, so
    O = v_{j*} + O(Lk * exp(-a*scale)).  With a*scale = 50 the residual is
    ~1e-20; with 1000 it underflows to exactly zero, and any oracle that
    does not subtract the row maximum overflows."""
    Lk, d, jstar = 13, 8, 5
    k = _rand((1, 1, Lk, d), 13)
    k[..., 0] = 0.0
    k[0, 0, jstar] = 0.0
    k[0, 0, jstar, 0] = 1.0
    v = _rand((1, 1, Lk, d), 14)
    scale = 0.25
    for gap in (50.0, 1000.0):
        q = np.zeros((1, 1, 1, d))
        q[..., 0] = gap / scale
        got = orc.attn(q, k, v, scale)[0, 0, 0]
        assert np.all(np.isfinite(got)), f"non-finite at gap {gap}"
        assert np.abs(got - v[0, 0, jstar]).max() <= 1e-14, f"gap {gap}"


# --------------------------------------------------------------------------
# invariants


def pin_rows_sum_to_one(orc):
    """Every row of P sums to 1 and P >= 0; O = P V."""
    q = _rand((2, 2, 7, 8), 15)
    k = _rand((2, 2, 19, 8), 16, 3.0)
    v = _rand((2, 2, 19, 8), 17)
    out, p = orc.attn_probs(q, k, v, 0.5)
    assert np.all(p >= 0.0)
    assert np.abs(p.sum(axis=-1) - 1.0).max() <= 1e-14, "P rows do not sum to 1"
    assert np.abs(np.einsum("bhij,bhjc->bhic", p, v) - out).max() <= 1e-14


def pin_query_permutation(orc):
    """Permuting query rows permutes output rows (rows are independent)."""
    q = _rand((1, 2, 12, 8), 18)
    k = _rand((1, 2, 10, 8), 19)
    v = _rand((1, 2, 10, 8), 20)
    perm = np.random.default_rng(21).permutation(12)
    a = orc.attn(q, k, v, 0.4)
    b = orc.attn(q[:, :, perm], k, v, 0.4)
    assert np.array_equal(a[:, :, perm], b), "query permutation not equivariant"


def pin_key_value_permutation(orc):
    """Permuting key and value rows together leaves O unchanged."""
    q = _rand((1, 2, 6, 8), 22)
    k = _rand((1, 2, 17, 8), 23, 2.0)
    v = _rand((1, 2, 17, 8), 24)
    perm = np.random.default_rng(25).permutation(17)
    a = orc.attn(q, k, v, 0.4)
    b = orc.attn(q, k[:, :, perm], v[:, :, perm], 0.4)
    assert np.abs(a - b).max() <= 1e-13, "joint K/V permutation changed O"


def pin_key_shift(orc):
    """k_j -> k_j + u for every j adds the same q_i.u*scale to row i's
    scores, which softmax ignores."""
    q = _rand((1, 1, 5, 8), 26)
    k = _rand((1, 1, 9, 8), 27)
    v = _rand((1, 1, 9, 8), 28)
    u = _rand((1, 1, 1, 8), 29, 40.0)
    a = orc.attn(q, k, v, 0.5)
    b = orc.attn(q, k + u, v, 0.5)
    assert np.abs(a - b).max() <= 1e-11, "key shift changed O"


def pin_head_independence(orc):
    """Each (b, h) slice computed alone equals that slice of the batch."""
    q = _rand((2, 3, 5, 8), 30)
    k = _rand((2, 3, 7, 8), 31)
    v = _rand((2, 3, 7, 8), 32)
    full = orc.attn(q, k, v, 0.45)
    for b in range(2):
        for h in range(3):
            one = orc.attn(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                           v[b:b + 1, h:h + 1], 0.45)
            assert np.array_equal(one[0, 0], full[b, h]), f"(b,h)=({b},{h})"


def pin_rows_entry(orc):
    """attn_rows on any row subset == the same rows of attn."""
    q = _rand((2, 2, 9, 8), 33)
    k = _rand((2, 2, 6, 8), 34)
    v = _rand((2, 2, 6, 8), 35)
    full = orc.attn(q, k, v, 0.3).reshape(-1, 8)
    rows = np.array([0, 5, 8, 9, 17, 20, 35], dtype=np.int64)
    got = orc.attn_rows(q, k, v, 0.3, rows)
    assert np.array_equal(got, full[rows]), "rows entry disagrees"


# --------------------------------------------------------------------------
# library special cases


def _numpy_two_pass(q, k, v, scale):
    s = np.einsum("bhid,bhjd->bhij", q, k) * scale
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return np.einsum("bhij,bhjd->bhid", e / e.sum(axis=-1, keepdims=True), v)


def pin_library_cross_check(orc):
    """torch's fp64 SDPA on the CPU and a numpy two-pass softmax agree with
    the oracle to 1e-12 on the fp32 cross-attention shape (1x1x64x77, d=40)
    and on ragged tiny shapes."""
    import torch
    import torch.nn.functional as F
    for seed, shape in enumerate([(1, 1, 64, 77, 40), (2, 3, 5, 3, 8),
                                  (1, 2, 33, 65, 16)]):
        B, H, Lq, Lk, d = shape
        q = _rand((B, H, Lq, d), 40 + seed)
        k = _rand((B, H, Lk, d), 50 + seed)
        v = _rand((B, H, Lk, d), 60 + seed)
        scale = 1.0 / math.sqrt(d)
        got = orc.attn(q, k, v, scale)
        ref_t = F.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            scale=scale).numpy()
        ref_n = _numpy_two_pass(q, k, v, scale)
        assert np.abs(got - ref_t).max() <= 1e-12, f"torch SDPA {shape}"
        assert np.abs(got - ref_n).max() <= 1e-12, f"numpy two-pass {shape}"


ALL_PINS = [
    pin_brute_force, pin_golden_closed_forms, pin_single_key,
    pin_identical_keys, pin_zero_scale, pin_constant_values,
    pin_dominant_score, pin_rows_sum_to_one, pin_query_permutation,
    pin_key_value_permutation, pin_key_shift, pin_head_independence,
    pin_rows_entry, pin_library_cross_check,
]
