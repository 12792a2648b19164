"""C-ABI tests that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments with the documented status
before any HIP call."""
import math
import os
import re

import pytest

import unet_attention_amd as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdattn.h")

# Fake, 16-byte aligned addresses: validation fails before they are used.
Q, K, V, O = 0x100000, 0x200000, 0x300000, 0x400000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdattn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sd.LIB_PATH):
        pytest.skip("libsdattn.so not built")
    return sd.load()


def test_exports_every_header_symbol(lib):
    names = header_functions()
    assert "sdattn_fwd" in names and "sdattn_cross_fwd" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sdattn.h but not exported"
    assert set(names) == set(sd.EXPORTS), "binding and header disagree"


def test_version_and_strerror(lib):
    assert sd.sdattn_version() == 10300
    seen = set()
    for code in range(6):
        msg = sd.sdattn_strerror(code)
        assert msg and msg not in seen
        seen.add(msg)
    assert "unknown" in sd.sdattn_strerror(99)
    assert "unknown" in sd.sdattn_strerror(-1)


def test_cross_max_ctx(lib):
    for dt in (sd.SDATTN_DTYPE_F32, sd.SDATTN_DTYPE_BF16, sd.SDATTN_DTYPE_BF16_F32OUT,
               sd.SDATTN_DTYPE_F16, sd.SDATTN_DTYPE_F16_F32OUT):
        for d in (8, 40, 64, 80, 160, 256):
            assert sd.sdattn_cross_max_ctx(d, dt) >= 77
        for d in (0, 4, 41, 264, -8):
            assert sd.sdattn_cross_max_ctx(d, dt) == 0
    assert sd.sdattn_cross_max_ctx(40, 5) == 0
    assert sd.sdattn_cross_max_ctx(40, 7) == 0


def call(entry, **kw):
    args = dict(q=Q, k=K, v=V, out=O, B=2, H=8, Lq=64, Lk=77, d=40,
                scale=1 / math.sqrt(40), dtype=sd.SDATTN_DTYPE_BF16, stream=None)
    args.update(kw)
    fn = getattr(sd, entry)
    return fn(args["q"], args["k"], args["v"], args["out"], args["B"], args["H"],
              args["Lq"], args["Lk"], args["d"], args["scale"], args["dtype"],
              args["stream"])


ENTRIES = ["sdattn_fwd", "sdattn_cross_fwd", "sdattn_stream_fwd"]

BAD = [
    ("null_q", dict(q=None), sd.SDATTN_ERR_INVALID_ARG),
    ("null_k", dict(k=None), sd.SDATTN_ERR_INVALID_ARG),
    ("null_v", dict(v=None), sd.SDATTN_ERR_INVALID_ARG),
    ("null_out", dict(out=None), sd.SDATTN_ERR_INVALID_ARG),
    ("B0", dict(B=0), sd.SDATTN_ERR_INVALID_ARG),
    ("H0", dict(H=0), sd.SDATTN_ERR_INVALID_ARG),
    ("Lq0", dict(Lq=0), sd.SDATTN_ERR_INVALID_ARG),
    ("Lk0", dict(Lk=0), sd.SDATTN_ERR_INVALID_ARG),
    ("d0", dict(d=0), sd.SDATTN_ERR_INVALID_ARG),
    ("negB", dict(B=-1), sd.SDATTN_ERR_INVALID_ARG),
    ("dtype", dict(dtype=5), sd.SDATTN_ERR_INVALID_ARG),
    ("dtype_neg", dict(dtype=-1), sd.SDATTN_ERR_INVALID_ARG),
    ("nan_scale", dict(scale=float("nan")), sd.SDATTN_ERR_INVALID_ARG),
    ("inf_scale", dict(scale=float("inf")), sd.SDATTN_ERR_INVALID_ARG),
    ("too_big", dict(B=1 << 12, H=1 << 10, Lq=1 << 12), sd.SDATTN_ERR_INVALID_ARG),
    ("d_odd", dict(d=41), sd.SDATTN_ERR_UNSUPPORTED),
    ("d_12", dict(d=12), sd.SDATTN_ERR_UNSUPPORTED),
    ("d_264", dict(d=264), sd.SDATTN_ERR_UNSUPPORTED),
    ("misaligned_q", dict(q=Q + 2), sd.SDATTN_ERR_MISALIGNED),
    ("misaligned_k", dict(k=K + 8), sd.SDATTN_ERR_MISALIGNED),
    ("misaligned_v", dict(v=V + 4), sd.SDATTN_ERR_MISALIGNED),
    ("misaligned_out", dict(out=O + 2), sd.SDATTN_ERR_MISALIGNED),
    ("out_is_q", dict(out=Q), sd.SDATTN_ERR_INVALID_ARG),
    ("out_overlaps_k_tail", dict(out=K - 16), sd.SDATTN_ERR_INVALID_ARG),
    ("out_overlaps_v", dict(out=V + 64), sd.SDATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("case", BAD, ids=[b[0] for b in BAD])
def test_invalid_arguments(lib, entry, case):
    _, kw, want = case
    assert call(entry, **kw) == want


@pytest.mark.parametrize("dtype", [0, 1, 2, 3, 4])
def test_cross_rejects_long_context(lib, dtype):
    cap = sd.sdattn_cross_max_ctx(40, dtype)
    assert call("sdattn_cross_fwd", Lk=cap + 1, dtype=dtype) == sd.SDATTN_ERR_UNSUPPORTED


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("dtype", [1, 2, 3, 4])
def test_valid_call_without_gpu_reports_device(lib, entry, dtype):
    if _gpu_present():
        pytest.skip("a GPU is present; fake pointers must not reach a launch")
    assert call(entry, dtype=dtype) == sd.SDATTN_ERR_DEVICE


def test_torch_wrapper_checks_shapes(lib):
    import torch
    q = torch.zeros(1, 1, 4, 8)
    with pytest.raises(ValueError):
        sd.fwd(q, q, q)  # CPU tensors are refused before any call
    with pytest.raises(ValueError):
        sd.fwd(q.to(torch.float16), q, q)


def call_strided(**kw):
    args = dict(q=Q, k=K, v=V, out=O, B=2, H=8, Lq=64, Lk=77, d=40, ldq=320, ldkv=320,
                ldo=320, scale=1 / math.sqrt(40), dtype=sd.SDATTN_DTYPE_BF16, stream=None)
    args.update(kw)
    return sd.sdattn_fwd_strided(*(args[n] for n in (
        "q", "k", "v", "out", "B", "H", "Lq", "Lk", "d", "ldq", "ldkv", "ldo", "scale",
        "dtype", "stream")))


BAD_STRIDED = [
    ("ldq_small", dict(ldq=312), sd.SDATTN_ERR_INVALID_ARG),     # < H*d
    ("ldkv_small", dict(ldkv=8), sd.SDATTN_ERR_INVALID_ARG),
    ("ldo_small", dict(ldo=40), sd.SDATTN_ERR_INVALID_ARG),
    ("ldq_unaligned", dict(ldq=324), sd.SDATTN_ERR_INVALID_ARG),  # rows not 16-byte aligned
    ("ldo_zero", dict(ldo=0), sd.SDATTN_ERR_INVALID_ARG),
    ("ldkv_neg", dict(ldkv=-320), sd.SDATTN_ERR_INVALID_ARG),
    ("null_v", dict(v=None), sd.SDATTN_ERR_INVALID_ARG),
    ("dtype", dict(dtype=5), sd.SDATTN_ERR_INVALID_ARG),
    ("d_odd", dict(d=41, ldq=328, ldkv=328, ldo=328), sd.SDATTN_ERR_UNSUPPORTED),
    ("misaligned_k", dict(k=K + 8), sd.SDATTN_ERR_MISALIGNED),
    # out's rows span B*Lq*320 elements: starting inside q's span overlaps it
    ("out_overlaps_q", dict(out=Q + 2 * 320), sd.SDATTN_ERR_INVALID_ARG),
    ("too_big", dict(Lq=1 << 22, ldq=1024, ldo=1024), sd.SDATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("case", BAD_STRIDED, ids=[b[0] for b in BAD_STRIDED])
def test_strided_invalid_arguments(lib, case):
    _, kw, want = case
    assert call_strided(**kw) == want


@pytest.mark.parametrize("dtype", [0, 1, 2, 3, 4])
def test_strided_valid_call_without_gpu_reports_device(lib, dtype):
    if _gpu_present():
        pytest.skip("a GPU is present; fake pointers must not reach a launch")
    # fused projection layout: k and v are column slices of q's rows
    assert call_strided(k=Q + 2 * 320, v=Q + 4 * 320, ldq=960, ldkv=960, Lk=64,
                        dtype=dtype) == sd.SDATTN_ERR_DEVICE


# --------------------------------------------------------------------------
# GroupNorm entry: host-side validation

X, GA, BE, Y = 0x10000000, 0x70000000, 0x70010000, 0x40000000


def call_gn(**kw):
    args = dict(x=X, gamma=GA, beta=BE, y=Y, N=2, C=320, HW=4096, G=32, eps=1e-5, silu=1,
                dtype=sd.SDATTN_DTYPE_BF16, stream=None)
    args.update(kw)
    return sd.sdattn_group_norm(*(args[n] for n in (
        "x", "gamma", "beta", "y", "N", "C", "HW", "G", "eps", "silu", "dtype", "stream")))


BAD_GN = [
    ("null_x", dict(x=None), sd.SDATTN_ERR_INVALID_ARG),
    ("null_gamma", dict(gamma=None), sd.SDATTN_ERR_INVALID_ARG),
    ("null_y", dict(y=None), sd.SDATTN_ERR_INVALID_ARG),
    ("N0", dict(N=0), sd.SDATTN_ERR_INVALID_ARG),
    ("G0", dict(G=0), sd.SDATTN_ERR_INVALID_ARG),
    ("C_not_multiple_of_G", dict(C=330), sd.SDATTN_ERR_INVALID_ARG),
    ("eps_negative", dict(eps=-1e-5), sd.SDATTN_ERR_INVALID_ARG),
    ("eps_nan", dict(eps=float("nan")), sd.SDATTN_ERR_INVALID_ARG),
    ("silu_2", dict(silu=2), sd.SDATTN_ERR_INVALID_ARG),
    ("dtype", dict(dtype=9), sd.SDATTN_ERR_INVALID_ARG),
    ("too_big", dict(N=1 << 10, HW=1 << 20), sd.SDATTN_ERR_INVALID_ARG),
    ("HW_not_multiple_of_8", dict(HW=4092), sd.SDATTN_ERR_UNSUPPORTED),
    ("too_many_channels_per_group", dict(C=16384, G=1, HW=8), sd.SDATTN_ERR_UNSUPPORTED),
    ("misaligned_x", dict(x=X + 2), sd.SDATTN_ERR_MISALIGNED),
    ("misaligned_y", dict(y=Y + 8), sd.SDATTN_ERR_MISALIGNED),
    ("misaligned_gamma", dict(gamma=GA + 2), sd.SDATTN_ERR_MISALIGNED),
    ("y_overlaps_x", dict(y=X + 64), sd.SDATTN_ERR_INVALID_ARG),
    ("in_place_with_fp32_out", dict(y=X, dtype=sd.SDATTN_DTYPE_BF16_F32OUT),
     sd.SDATTN_ERR_INVALID_ARG),
    ("y_overlaps_beta", dict(y=BE - 16), sd.SDATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("case", BAD_GN, ids=[b[0] for b in BAD_GN])
def test_group_norm_invalid_arguments(lib, case):
    _, kw, want = case
    assert call_gn(**kw) == want


@pytest.mark.parametrize("dtype", [0, 1, 2, 3, 4])
def test_group_norm_valid_call_without_gpu_reports_device(lib, dtype):
    if _gpu_present():
        pytest.skip("a GPU is present; fake pointers must not reach a launch")
    assert call_gn(dtype=dtype) == sd.SDATTN_ERR_DEVICE
    if dtype in (0, 1, 3):   # same element size in and out: in place is allowed
        assert call_gn(dtype=dtype, y=X) == sd.SDATTN_ERR_DEVICE
