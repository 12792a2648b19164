"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Every test here needs an MI355X; all are marked ``gpu``.  Inputs come from
the seeded generator in ``workloads``; expected values come only from the
oracle (or from closed forms).
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import (assert_bf16_gate, assert_bf16_out_gate, assert_f32_gate,
                            errors, run, say, tensors_from_f32, to_device)
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

_ORACLE_CACHE = {}


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import unet_attention_amd as sd
    sd.load()
    return "cuda"


def oracle_full(name):
    if name not in _ORACLE_CACHE:
        w = WORKLOADS[name]
        x = make_inputs(w)
        _ORACLE_CACHE[name] = (x, oracle.attn(x.q, x.k, x.v, w.scale))
    return _ORACLE_CACHE[name]


# ---------------------------------------------------------------------------
# the workloads at full size


@pytest.mark.parametrize("name", ["1", "2", "3", "4a", "4b", "4c", "4d", "6a", "6b", "2h", "3h"])
def test_workload_parity(dev, name):
    import torch
    w = WORKLOADS[name]
    x, want = oracle_full(name)
    q, k, v = to_device(x)
    if w.dtype == "f32":
        for entry in ("auto", "stream", "cross"):
            say(f"workload {name} fp32 entry={entry} {w}")
            got = run(entry, q, k, v, w.scale)
            say(f"workload {name} {entry} f32 max/mean err %.3e %.3e" % errors(got, want))
            assert_f32_gate(got, want, f"{name}/{entry}")
        return
    import unet_attention_amd as sd
    in_cap = w.Lk <= sd.sdattn_cross_max_ctx(w.d, sd.SDATTN_DTYPE_BF16)
    entries = ["auto", "stream"] + (["cross"] if w.kind == "cross" and in_cap else [])
    outs = {}
    for entry in entries:
        say(f"workload {name} bf16->fp32 entry={entry} {w}")
        outs[entry] = got = run(entry, q, k, v, w.scale, out_dtype=torch.float32)
        say(f"workload {name} {entry} f32out max/mean err %.3e %.3e" % errors(got, want))
        assert_bf16_gate(got, want, f"{name}/{entry}/f32out")
        lo = torch.bfloat16 if w.dtype == "bf16" else torch.float16
        say(f"workload {name} {w.dtype}->{w.dtype} entry={entry}")
        gotb = run(entry, q, k, v, w.scale, out_dtype=lo)
        say(f"workload {name} {entry} {w.dtype} out max/mean err %.3e %.3e" % errors(gotb, want))
        assert_bf16_out_gate(gotb, want, f"{name}/{entry}/{w.dtype}out", out=w.dtype)
    if "cross" in outs:
        assert np.array_equal(outs["cross"], outs["auto"]), "cross entry != fwd entry"


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["5", "5h"])
def test_workload5_full(dev, name):
    """128x128 latent, B=8, H=10, L=16384, d=64, 1% of keys x8, bf16 (5) and
    fp16 (5h): the whole output (1.3 M rows of 64) in both output modes
    against the fp64 oracle, in the benchmark's launch configuration.  The
    oracle runs one batch element at a time (10 heads, ~0.7 TFLOP each);
    every element is compared and the worst (b, h, i) of each mode is
    reported."""
    import torch
    import unet_attention_amd as sd
    from tests.gpu_util import BF16_MAX, BF16_MEAN, half_ulp_bf16, half_ulp_f16
    w = WORKLOADS[name]
    lo = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    half_ulp = half_ulp_bf16 if w.dtype == "bf16" else half_ulp_f16
    x = make_inputs(w)
    q, k, v = to_device(x)
    got = {}
    for odt in (torch.float32, lo):
        say(f"workload {name} full size, out {odt}")
        out = sd.fwd(q, k, v, scale=w.scale, out_dtype=odt)
        torch.cuda.synchronize()
        got[odt] = out.float().cpu().numpy()
        del out
    del q, k, v
    st = {odt: {"max": 0.0, "sum": 0.0, "where": None, "hsum": 0.0} for odt in got}
    n = 0
    for b in range(w.B):
        want = oracle.attn(x.q[b:b + 1], x.k[b:b + 1], x.v[b:b + 1], w.scale)[0]
        n += want.size
        for odt, g in got.items():
            e = np.abs(g[b].astype(np.float64) - want)
            assert np.all(np.isfinite(g[b])), f"non-finite output in batch {b}"
            if odt == lo:
                h = half_ulp(want)
                st[odt]["hsum"] += float(h.sum())
                e_gate = e - h
            else:
                e_gate = e
            i = int(np.argmax(e_gate))
            if e_gate.flat[i] > st[odt]["max"]:
                hh, row, col = np.unravel_index(i, e_gate.shape)
                st[odt]["max"] = float(e_gate.flat[i])
                st[odt]["where"] = (b, int(hh), int(row), int(col))
            st[odt]["sum"] += float(e.sum())
        say(f"workload {name} batch {b}: f32out max {st[torch.float32]['max']:.3e} at "
            f"{st[torch.float32]['where']}; {w.dtype}out max(|err|-ulp/2) "
            f"{st[lo]['max']:.3e} at {st[lo]['where']}")
    m32 = st[torch.float32]["sum"] / n
    m16 = st[lo]["sum"] / n
    h16 = st[lo]["hsum"] / n
    say(f"workload {name} full: f32out max {st[torch.float32]['max']:.3e} mean {m32:.3e}; "
        f"{w.dtype}out max(|err|-ulp/2) {st[lo]['max']:.3e} mean {m16:.3e} "
        f"(+ulp/2 mean {h16:.3e})")
    assert st[torch.float32]["max"] <= BF16_MAX and m32 <= BF16_MEAN
    assert st[lo]["max"] <= BF16_MAX and m16 <= BF16_MEAN + h16


# ---------------------------------------------------------------------------
# ragged shapes and every head dim class


SHAPES = [(1, 1), (15, 2), (33, 63), (65, 64), (129, 65), (17, 77), (40, 127),
          (64, 128), (31, 129), (100, 200), (70, 333)]
DIMS = [8, 24, 40, 64, 80, 136, 160, 256]


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("Lq,Lk", SHAPES)
def test_ragged_bf16(dev, Lq, Lk, d):
    import torch
    import unet_attention_amd as sd
    w = Workload("ragged", "self", 1, 2, Lq, Lk, d, "bf16", 7000 + 31 * Lq + Lk + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    entries = ["auto", "stream"]
    if Lk <= sd.sdattn_cross_max_ctx(d, sd.SDATTN_DTYPE_BF16):
        entries.append("cross")
    for entry in entries:
        say(f"ragged bf16 Lq={Lq} Lk={Lk} d={d} entry={entry}")
        got = run(entry, q, k, v, w.scale, out_dtype=torch.float32)
        assert_bf16_gate(got, want, f"Lq={Lq} Lk={Lk} d={d} {entry}")
        gotb = run(entry, q, k, v, w.scale, out_dtype=torch.bfloat16)
        assert_bf16_out_gate(gotb, want, f"Lq={Lq} Lk={Lk} d={d} {entry} bf16out")


@pytest.mark.parametrize("d", [8, 40, 64, 80, 160, 256])
@pytest.mark.parametrize("Lq,Lk", [(1, 1), (33, 63), (17, 77), (64, 128), (31, 129), (100, 333)])
def test_ragged_f16(dev, Lq, Lk, d):
    import torch
    import unet_attention_amd as sd
    w = Workload("ragged16", "self", 1, 2, Lq, Lk, d, "f16", 9000 + 31 * Lq + Lk + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    entries = ["auto", "stream"]
    if Lk <= sd.sdattn_cross_max_ctx(d, sd.SDATTN_DTYPE_F16):
        entries.append("cross")
    for entry in entries:
        say(f"ragged f16 Lq={Lq} Lk={Lk} d={d} entry={entry}")
        got = run(entry, q, k, v, w.scale, out_dtype=torch.float32)
        assert_bf16_gate(got, want, f"f16 Lq={Lq} Lk={Lk} d={d} {entry}")
        goth = run(entry, q, k, v, w.scale, out_dtype=torch.float16)
        assert_bf16_out_gate(goth, want, f"f16 Lq={Lq} Lk={Lk} d={d} {entry} f16out", out="f16")


@pytest.mark.parametrize("d", [8, 40, 64, 200, 256])
@pytest.mark.parametrize("Lq,Lk", [(1, 1), (17, 77), (65, 64), (100, 333)])
def test_ragged_f32(dev, Lq, Lk, d):
    w = Workload("ragged32", "self", 2, 1, Lq, Lk, d, "f32", 8000 + 31 * Lq + Lk + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    say(f"ragged fp32 Lq={Lq} Lk={Lk} d={d}")
    assert_f32_gate(run("auto", q, k, v, w.scale), want, f"f32 Lq={Lq} Lk={Lk} d={d}")


# ---------------------------------------------------------------------------
# closed forms and invariants on the GPU


def _rand(shape, seed, s=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * s).astype(np.float32)


@pytest.mark.parametrize("dtype,d", [("f32", 40), ("bf16", 40), ("bf16", 64), ("bf16", 160)])
@pytest.mark.parametrize("entry", ["auto", "stream"])
def test_single_key_returns_value_row(dev, dtype, d, entry):
    """Lk = 1: the one weight is 1, so O = v_0.  Bitwise on the fp32 path and
    where the row sum comes from the matrix core (the bf16-rounded weight is
    exactly 1); where the row sum is an fp32 sum, the weight exp2(s*c - m) is
    1 up to the rounding residual of s*c, so O = v_0 to ~1e-6 relative."""
    import torch
    from workloads import bf16_bits_to_f32, round_to_bf16_bits
    q, k, v = _rand((2, 3, 50, d), 1, 3.0), _rand((2, 3, 1, d), 2, 3.0), _rand((2, 3, 1, d), 3)
    if dtype == "bf16":
        q, k, v = (bf16_bits_to_f32(round_to_bf16_bits(a)) for a in (q, k, v))
    tq, tk, tv = tensors_from_f32(q, k, v, dtype)
    say(f"single key {dtype} d={d} {entry}")
    got = run(entry, tq, tk, tv, 1 / math.sqrt(d),
              out_dtype=torch.float32 if dtype == "bf16" else None)
    want = np.broadcast_to(v.astype(np.float64), got.shape)
    ones_row = ((d + 15) // 16 * 16) % 32 == 16
    if dtype == "f32" or ones_row:
        assert np.array_equal(got, want)
    else:
        assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max()


@pytest.mark.parametrize("Lk", [77, 300])
def test_identical_keys_and_zero_scale_give_mean(dev, Lk):
    import torch
    from workloads import bf16_bits_to_f32, round_to_bf16_bits
    d = 40
    q = _rand((1, 2, 70, d), 4, 2.0)
    k = np.broadcast_to(_rand((1, 2, 1, d), 5, 2.0), (1, 2, Lk, d)).copy()
    v = _rand((1, 2, Lk, d), 6)
    q, k, v = (bf16_bits_to_f32(round_to_bf16_bits(a)) for a in (q, k, v))
    mean = np.broadcast_to(v.astype(np.float64).mean(axis=2, keepdims=True), (1, 2, 70, d))
    tq, tk, tv = tensors_from_f32(q, k, v, "bf16")
    for entry in ("auto", "stream"):
        say(f"identical keys Lk={Lk} {entry}")
        assert_bf16_gate(run(entry, tq, tk, tv, 0.3, torch.float32), mean, "identical keys")
        # scale 0 with distinct keys
        tk2 = tensors_from_f32(q, _rand((1, 2, Lk, d), 7, 5.0), v, "bf16")[1]
        say(f"zero scale Lk={Lk} {entry}")
        assert_bf16_gate(run(entry, tq, tk2, tv, 0.0, torch.float32), mean, "scale 0")


@pytest.mark.parametrize("entry", ["auto", "stream"])
def test_negative_scale_and_dominant_key(dev, entry):
    import torch
    from workloads import bf16_bits_to_f32, round_to_bf16_bits
    d, Lk = 64, 200
    q = _rand((1, 2, 40, d), 8)
    k = _rand((1, 2, Lk, d), 9)
    v = _rand((1, 2, Lk, d), 10)
    q, k, v = (bf16_bits_to_f32(round_to_bf16_bits(a)) for a in (q, k, v))
    tq, tk, tv = tensors_from_f32(q, k, v, "bf16")
    say(f"negative scale {entry}")
    want = oracle.attn(q, k, v, -0.125)
    assert_bf16_gate(run(entry, tq, tk, tv, -0.125, torch.float32), want, "negative scale")
    # one dominant key: q = a e_0 with a*scale = 50, k_j* = e_0, others orthogonal
    k2 = k.copy()
    k2[..., 0] = 0.0
    jstar = 137
    k2[:, :, jstar] = 0.0
    k2[:, :, jstar, 0] = 1.0
    q2 = np.zeros_like(q)
    q2[..., 0] = 400.0
    tq2, tk2, _ = tensors_from_f32(q2, k2, v, "bf16")
    say(f"dominant key {entry}")
    got = run(entry, tq2, tk2, tv, 0.125, torch.float32)
    want2 = np.broadcast_to(v[:, :, jstar:jstar + 1].astype(np.float64), got.shape)
    # residual of the other keys ~ 199 * 2^-72; the rest is fp32 rounding of l
    assert np.abs(got - want2).max() <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [40, 64])
def test_shifted_keys_stress_running_max(dev, d, dtype):
    """Keys shifted by a large common vector: scores reach |s| ~ 40 with a
    maximum that keeps growing along the keys (in fp16 the streaming kernel
    must move its reference up many times); compare with the oracle on the
    same (rounded) inputs."""
    import torch
    from workloads import bf16_bits_to_f32, round_to_bf16_bits
    Lk = 1500
    q = _rand((1, 2, 96, d), 11)
    k = _rand((1, 2, Lk, d), 12) + np.linspace(0, 6, Lk, dtype=np.float32)[None, None, :, None]
    v = _rand((1, 2, Lk, d), 13)
    if dtype == "f16":
        q, k, v = (a.astype(np.float16).astype(np.float32) for a in (q, k, v))
    else:
        q, k, v = (bf16_bits_to_f32(round_to_bf16_bits(a)) for a in (q, k, v))
    want = oracle.attn(q, k, v, 0.125)
    tq, tk, tv = tensors_from_f32(q, k, v, dtype)
    say(f"shifted keys d={d} {dtype}")
    assert_bf16_gate(run("auto", tq, tk, tv, 0.125, torch.float32), want,
                     f"shifted keys d={d} {dtype}")


def _aligned_key_case(d, seed, v_big=None, dtype="bf16"):
    """Every query close to one direction u (|q| ~ 6); key 250 = 24 u, the
    other keys small: key 250 scores ~144 above the rest (times scale).
    Values are rounded to `dtype` (bf16 or f16)."""
    from workloads import bf16_bits_to_f32, round_to_bf16_bits
    Lq, Lk, jstar = 70, 333, 250
    u = np.full(d, 1.0 / math.sqrt(d), dtype=np.float32)
    q = 6.0 * u + _rand((1, 2, Lq, d), seed, 0.3)
    k = _rand((1, 2, Lk, d), seed + 1, 0.5)
    k[:, :, jstar] = 24.0 * u
    v = _rand((1, 2, Lk, d), seed + 2)
    if v_big is not None:
        v[:, :, jstar] = v_big
    if dtype == "f16":
        return tuple(a.astype(np.float16).astype(np.float32) for a in (q, k, v))
    return tuple(bf16_bits_to_f32(round_to_bf16_bits(a)) for a in (q, k, v))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [40, 64, 80])
@pytest.mark.parametrize("scale", [1.0, 0.5])
def test_far_key_beyond_first_tile(dev, d, scale, dtype):
    """A key whose score exceeds every score of the first key tile by ~200
    (scale 1) or ~100 (scale 0.5) binary orders: weights taken relative to an
    early maximum overflow fp32 in the first case, and must still give the
    oracle's result."""
    import torch
    q, k, v = _aligned_key_case(d, 300 + d, dtype=dtype)
    want = oracle.attn(q, k, v, scale)
    tq, tk, tv = tensors_from_f32(q, k, v, dtype)
    for entry in ("auto", "stream"):
        say(f"far key {dtype} d={d} scale={scale} {entry}")
        got = run(entry, tq, tk, tv, scale, torch.float32)
        assert_bf16_gate(got, want, f"far key {dtype} d={d} scale={scale} {entry}")


@pytest.mark.parametrize("d", [40, 64])
def test_huge_values_far_key(dev, d):
    """Weights up to ~2^50 times values of 2^90: the unnormalised output
    passes fp32's range although every weight and the row sum stay finite.
    Compared relative to the output's size."""
    import torch
    q, k, v = _aligned_key_case(d, 400 + d, v_big=2.0 ** 90)
    scale = 0.25
    want = oracle.attn(q, k, v, scale)
    tq, tk, tv = tensors_from_f32(q, k, v, "bf16")
    say(f"huge values d={d}")
    got = run("auto", tq, tk, tv, scale, torch.float32)
    assert np.all(np.isfinite(got)), "non-finite output"
    rel = np.abs(got - want).max() / np.abs(want).max()
    assert rel <= 1e-2, f"relative max error {rel:.3e}"


def test_repeatable_bitwise(dev):
    import torch
    x, _ = oracle_full("2")
    q, k, v = to_device(x)
    say("repeatability workload 2")
    a = run("auto", q, k, v, WORKLOADS["2"].scale, torch.bfloat16)
    b = run("auto", q, k, v, WORKLOADS["2"].scale, torch.bfloat16)
    assert np.array_equal(a, b)


def test_non_default_stream(dev):
    import torch
    import unet_attention_amd as sd
    x, want = oracle_full("3")
    q, k, v = to_device(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("non-default stream workload 3")
    with torch.cuda.stream(s):
        out = sd.fwd(q, k, v, scale=WORKLOADS["3"].scale, out_dtype=torch.float32)
    s.synchronize()
    assert_bf16_gate(out.double().cpu().numpy(), want, "side stream")


def test_stream_argument_with_own_output(dev):
    """A stream handle passed as argument (not torch's current stream): the
    binding allocates the output on that stream and the kernel runs there."""
    import torch
    import unet_attention_amd as sd
    x, want = oracle_full("3")
    q, k, v = to_device(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("stream argument workload 3")
    outs = [sd.fwd(q, k, v, scale=WORKLOADS["3"].scale, out_dtype=torch.float32,
                   stream=s.cuda_stream) for _ in range(3)]
    s.synchronize()
    for out in outs:
        assert_bf16_gate(out.double().cpu().numpy(), want, "stream argument")


def test_errors_on_device(dev):
    import torch
    import unet_attention_amd as sd
    # q is large enough that K/V views of up to 512 rows at its start stay
    # inside it (so the overlap check does not fire before the one tested)
    q = torch.zeros(1, 1, 512, 40, dtype=torch.bfloat16, device=dev)
    out = torch.empty(1, 1, 256, 40, dtype=torch.bfloat16, device=dev)
    p = q.data_ptr()
    say("misaligned pointer on device")
    assert sd.sdattn_fwd(p + 2, p, p, out.data_ptr(), 1, 1, 63, 64, 40, 0.1, 1, None) == \
        sd.SDATTN_ERR_MISALIGNED
    assert sd.sdattn_fwd(p, p, p, p, 1, 1, 64, 64, 40, 0.1, 1, None) == sd.SDATTN_ERR_INVALID_ARG
    cap = sd.sdattn_cross_max_ctx(40, 1)
    assert sd.sdattn_cross_fwd(p, p, p, out.data_ptr(), 1, 1, 64, cap + 1, 40, 0.1, 1, None) == \
        sd.SDATTN_ERR_UNSUPPORTED
    with pytest.raises(sd.SdattnError):
        sd.cross_fwd(q, torch.zeros(1, 1, cap + 1, 40, dtype=torch.bfloat16, device=dev),
                     torch.zeros(1, 1, cap + 1, 40, dtype=torch.bfloat16, device=dev))


@pytest.mark.parametrize("d", [16, 32, 48, 56])
@pytest.mark.parametrize("Lq,Lk", [(31, 129), (100, 200), (70, 333), (64, 1000)])
def test_streaming_every_row_layout(dev, Lq, Lk, d):
    """The streaming kernel for d <= 64 lays out K and V rows per exact head
    dim (d = DK or DK - 8): the dims the ragged sweep above does not reach."""
    import torch
    w = Workload("layout", "self", 1, 2, Lq, Lk, d, "bf16", 7500 + 31 * Lq + Lk + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    say(f"streaming layout Lq={Lq} Lk={Lk} d={d}")
    assert_bf16_gate(run("stream", q, k, v, w.scale, out_dtype=torch.float32), want,
                     f"Lq={Lq} Lk={Lk} d={d}")
    assert_bf16_out_gate(run("stream", q, k, v, w.scale, out_dtype=torch.bfloat16), want,
                         f"Lq={Lq} Lk={Lk} d={d} bf16out")


@pytest.mark.parametrize("dtype,Lq,Lk,d", [
    ("bf16", 600, 333, 40), ("bf16", 600, 333, 64), ("f16", 600, 333, 40),
    ("bf16", 520, 64, 48), ("bf16", 700, 129, 64), ("f16", 600, 1000, 56),
    ("bf16", 1100, 200, 32)])
def test_fixed_reference_both_key_orders(dev, dtype, Lq, Lk, d):
    """Several 256-row query blocks per head: even blocks take the key tiles
    first to last, odd blocks last to first, so the ragged tile is processed
    last or first (and supplies the first reference)."""
    import torch
    w = Workload("keyorder", "self", 2, 2, Lq, Lk, d, dtype, 13000 + Lq + Lk + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    lo = torch.bfloat16 if dtype == "bf16" else torch.float16
    say(f"key orders {dtype} Lq={Lq} Lk={Lk} d={d}")
    assert_bf16_gate(run("stream", q, k, v, w.scale, out_dtype=torch.float32), want,
                     f"{dtype} Lq={Lq} Lk={Lk} d={d}")
    assert_bf16_out_gate(run("stream", q, k, v, w.scale, out_dtype=lo), want,
                         f"{dtype} Lq={Lq} Lk={Lk} d={d} 16-bit out", out=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [72, 80, 96, 136, 160])
@pytest.mark.parametrize("Lk", [100, 333, 1024])
def test_rescaling_key_split(dev, d, Lk, dtype):
    """Small grids of the rescaling kernel (d > 64): each 32-row query block
    is shared by four waves on 128-key tiles (head dims up to 96) or two on
    64-key tiles (wider), whose partial results are merged through LDS;
    ragged and whole key counts."""
    import torch
    w = Workload("ksplit", "self", 2, 2, 100, Lk, d, dtype, 14000 + Lk + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    lo = torch.bfloat16 if dtype == "bf16" else torch.float16
    say(f"key split {dtype} Lk={Lk} d={d}")
    assert_bf16_gate(run("stream", q, k, v, w.scale, out_dtype=torch.float32), want,
                     f"{dtype} Lk={Lk} d={d}")
    assert_bf16_out_gate(run("stream", q, k, v, w.scale, out_dtype=lo), want,
                         f"{dtype} Lk={Lk} d={d} 16-bit out", out=dtype)


@pytest.mark.parametrize("d", [80, 160])
def test_rescaling_unsplit_grid(dev, d):
    """d > 64 with enough query blocks for the whole chip: the rescaling
    kernel's plain form (small grids above run its split form)."""
    import torch
    w = Workload("unsplit", "self", 2, 8, 4096, 300, d, "bf16", 7700 + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    say(f"rescaling plain grid d={d}")
    assert_bf16_gate(run("auto", q, k, v, w.scale, out_dtype=torch.float32), want, f"d={d}")


# ---------------------------------------------------------------------------
# token-major operands (sdattn_fwd_strided)


def _to_tokens(a):
    """[B, H, L, d] -> [B, L, H*d] (numpy)."""
    B, H, L, d = a.shape
    return np.ascontiguousarray(a.transpose(0, 2, 1, 3).reshape(B, L, H * d))


STRIDED_CASES = [  # (dtype, H, Lq, Lk, d): short-key, fixed-reference, rescaling, fp32
    ("bf16", 2, 129, 77, 40), ("bf16", 3, 300, 300, 64), ("bf16", 2, 100, 333, 80),
    ("bf16", 3, 100, 300, 40), ("bf16", 2, 70, 200, 56),
    ("f16", 2, 65, 200, 40), ("f32", 2, 33, 77, 40),
]


@pytest.mark.parametrize("dtype,H,Lq,Lk,d", STRIDED_CASES)
def test_token_major_matches_head_major(dev, dtype, H, Lq, Lk, d):
    """Packed [B, L, C] operands give the oracle's result and exactly the
    head-major entry's output; also with an output of row stride 2C whose
    other columns must stay untouched."""
    import torch
    import unet_attention_amd as sd
    B = 2
    w = Workload("tok", "self", B, H, Lq, Lk, d, dtype, 11000 + Lq + Lk + d)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    odt = torch.float32
    ref = sd.fwd(q, k, v, scale=w.scale, out_dtype=odt)
    qt, kt, vt = (t.permute(0, 2, 1, 3).reshape(B, t.shape[2], H * d).contiguous()
                  for t in (q, k, v))
    say(f"token-major {dtype} H={H} Lq={Lq} Lk={Lk} d={d}")
    got = sd.fwd_tokens(qt, kt, vt, H, scale=w.scale, out_dtype=odt)
    torch.cuda.synchronize()
    got_hm = got.view(B, Lq, H, d).permute(0, 2, 1, 3).cpu().numpy().astype(np.float64)
    gate = assert_f32_gate if dtype == "f32" else assert_bf16_gate
    gate(got_hm, want, f"token-major {dtype}")
    assert np.array_equal(got_hm, ref.cpu().numpy().astype(np.float64)), \
        "token-major result differs from the head-major entry"
    wide = torch.full((B, Lq, 2 * H * d), 7.0, dtype=odt, device=dev)
    sd.fwd_tokens(qt, kt, vt, H, out=wide[:, :, :H * d], scale=w.scale, out_dtype=odt)
    torch.cuda.synchronize()
    assert torch.equal(wide[:, :, :H * d], got), "strided output differs"
    assert bool((wide[:, :, H * d:] == 7.0).all()), "columns outside the output were written"


@pytest.mark.parametrize("dtype,Lk", [("bf16", 77), ("bf16", 256), ("f16", 256)])
def test_fused_qkv_projection_slices(dev, dtype, Lk):
    """q, k, v as column slices of one [B, L, 3C] projection (row stride 3C)."""
    import torch
    import unet_attention_amd as sd
    B, H, d = 2, 4, 64
    L = Lk
    w = Workload("qkv", "self", B, H, L, L, d, dtype, 12000 + Lk)
    x = make_inputs(w)
    want = oracle.attn(x.q, x.k, x.v, w.scale)
    q, k, v = to_device(x)
    C = H * d
    qkv = torch.cat([t.permute(0, 2, 1, 3).reshape(B, L, C) for t in (q, k, v)], dim=2)
    qs, ks, vs = qkv[:, :, :C], qkv[:, :, C:2 * C], qkv[:, :, 2 * C:]
    assert qs.stride(1) == 3 * C
    say(f"fused qkv {dtype} L={L}")
    got = sd.fwd_tokens(qs, ks, vs, H, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got_hm = got.view(B, L, H, d).permute(0, 2, 1, 3).cpu().numpy().astype(np.float64)
    assert_bf16_gate(got_hm, want, f"fused qkv {dtype} L={L}")
