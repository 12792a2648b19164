"""The GroupNorm (+ SiLU) oracle against its pins, and the pins against
plausible mistakes compiled into copies of the oracle (CPU only)."""
from __future__ import annotations

import shutil

import numpy as np
import pytest

import oracle
from tests import oracle_pins_gn


@pytest.fixture(scope="module")
def gn():
    return oracle.get_gn()


@pytest.mark.parametrize("pin", oracle_pins_gn.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(gn, pin):
    pin(gn)


MUTANTS = {
    "unbiased_variance": ("const double var = ss / (double)M;",
                          "const double var = ss / (double)(M - 1);"),
    "no_eps": ("1.0 / sqrt(var + eps)", "1.0 / sqrt(var)"),
    "eps_outside_sqrt": ("1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    "gamma_of_first_channel": ("const double ga = gamma[c0 + cc]", "const double ga = gamma[c0]"),
    "no_beta": ("* inv_std * ga + be;", "* inv_std * ga;"),
    "affine_before_normalising": ("double y = (xg[i] - mu) * inv_std * ga + be;",
                                  "double y = (xg[i] * ga + be - mu) * inv_std;"),
    "uncentred_variance": ("const double t = xg[i] - mu;", "const double t = xg[i];"),
    "silu_sign": ("y = y / (1.0 + exp(-y));", "y = y / (1.0 + exp(y));"),
    "silu_always": ("if (silu) y = y / (1.0 + exp(-y));", "y = y / (1.0 + exp(-y));"),
    "mean_drops_last": ("for (int64_t i = 0; i < M; ++i) sum += xg[i];",
                        "for (int64_t i = 0; i + 1 < M; ++i) sum += xg[i];"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(oracle.GN_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    path = tmp_path / "mut_gn.c"
    path.write_text(src.replace(old, new))
    orc = oracle.GroupNormOracle(oracle.build(str(path), str(tmp_path / f"libgn_{name}.so")))
    failed = []
    for pin in oracle_pins_gn.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_threads_do_not_change_result(gn):
    x = np.random.default_rng(3).standard_normal((4, 32, 9, 9))
    g, b = np.ones(32), np.zeros(32)
    assert np.array_equal(gn.group_norm(x, g, b, 8, 1e-5, nthreads=1),
                          gn.group_norm(x, g, b, 8, 1e-5, nthreads=4))


def test_rejects_bad_groups(gn):
    with pytest.raises(ValueError):
        gn.group_norm(np.zeros((1, 6, 4)), np.ones(6), np.zeros(6), 4, 1e-5)
    with pytest.raises(ValueError):
        gn.group_norm(np.zeros((1, 6, 4)), np.ones(5), np.zeros(6), 3, 1e-5)
