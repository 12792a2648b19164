"""CPU tests of the fp64 oracle against its pins (no GPU needed)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import oracle_pins
from workloads import WORKLOADS, bf16_bits_to_f32, make_inputs, round_to_bf16_bits


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


# A plausible mistake anywhere in the oracle must trip at least one pin.
# Each mutant is a textual edit of attn_oracle.c, compiled on the CPU into a
# scratch directory; the real oracle is never modified.
MUTANTS = {
    "dropped_scale": ("s[j] = sigma * dot;", "s[j] = dot;"),
    "transposed_k": ("dot += q_row[c] * k_row[c];",
                     "dot += q_row[c] * k_bh[c * Lk + j];"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "no_normalise": ("for (int64_t j = 0; j < Lk; ++j) s[j] = s[j] / l;",
                     "for (int64_t j = 0; j < Lk; ++j) s[j] = s[j] / 2.0;"),
    "transposed_v": ("o_row[c] += pj * v_row[c];",
                     "o_row[c] += pj * v_bh[c * Lk + j];"),
    "min_not_max": ("if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    "head_zero_kv": ("attend_row(q + r * d, k + bh * Lk * d, v + bh * Lk * d, Lk, d, scale, s,\n                 out + r * d, NULL);",
                     "attend_row(q + r * d, k, v, Lk, d, scale, s,\n                 out + r * d, NULL);"),
    "scale_on_values": ("const double pj = s[j];", "const double pj = s[j] * sigma;"),
    "dropped_last_key": ("for (int64_t j = 0; j < Lk; ++j) {\n    s[j] = exp(s[j] - m);",
                         "for (int64_t j = 0; j < Lk; ++j) {\n    if (j == Lk - 1 && Lk > 1) { s[j] = 0.0; continue; }\n    s[j] = exp(s[j] - m);"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(oracle.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    lib = oracle.build(str(path), str(tmp_path / f"libmut_{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_oracle_threads_do_not_change_result(oracle_lib):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 2, 37, 16))
    k = rng.standard_normal((2, 2, 29, 16))
    v = rng.standard_normal((2, 2, 29, 16))
    a = oracle_lib.attn(q, k, v, 0.25, nthreads=1)
    b = oracle_lib.attn(q, k, v, 0.25, nthreads=4)
    assert np.array_equal(a, b)


def test_oracle_rejects_bad_shapes(oracle_lib):
    q = np.zeros((1, 1, 2, 4))
    with pytest.raises(ValueError):
        oracle_lib.attn(q, np.zeros((1, 1, 3, 5)), np.zeros((1, 1, 3, 5)), 1.0)
    with pytest.raises(ValueError):
        oracle_lib.attn(q[0], q[0], q[0], 1.0)


# --------------------------------------------------------------------------
# the seeded input generator (shared by both sides, no attention arithmetic)


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # ties
    ours = round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_are_deterministic_and_rounded():
    w = WORKLOADS["4d"].with_(B=1, H=2, Lq=8)
    a, b = make_inputs(w), make_inputs(w)
    for t in ("q", "k", "v", "q_bits", "k_bits", "v_bits"):
        assert np.array_equal(getattr(a, t), getattr(b, t))
    assert np.array_equal(bf16_bits_to_f32(a.k_bits), a.k)
    assert a.q.shape == (1, 2, 8, 160) and a.k.shape == (1, 2, 77, 160)


def test_heavy_keys_recipe():
    w = WORKLOADS["5"].with_(B=1, H=2, Lq=4, Lk=1000)
    x = make_inputs(w)
    assert x.heavy_rows.shape == (1, 2, 10)
    plain = make_inputs(w.with_(heavy_frac=0.0))
    for h in range(2):
        rows = x.heavy_rows[0, h]
        assert len(set(rows.tolist())) == 10
        np.testing.assert_array_equal(x.k[0, h, rows], 8 * plain.k[0, h, rows])
        mask = np.ones(1000, bool)
        mask[rows] = False
        np.testing.assert_array_equal(x.k[0, h, mask], plain.k[0, h, mask])
