"""The lane layouts every 16-bit attention kernel relies on, probed on the
GPU with one wave (libsdattn_peak.so's peak_probe_layouts) and compared with
their documented form:

* v_mfma_f32_32x32x16_bf16: lane l supplies row (A) / column (B) l % 32 with
  k = 8 (l / 32) .. 8 (l / 32) + 7, and accumulator register i of lane l
  holds row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32;
* ds_read_b64_tr_b16: within each 16-lane group, lane i element j is
  element i % 4 of the 8 bytes that lane 4 j + i / 4 addresses;
* v_permlane32_swap(x, x): the first result of lane l is x of lane l % 32,
  the second x of lane 32 + l % 32.

Marked gpu; the values are integers, compared exactly.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from unet_attention_amd import build as hb
    lib = ctypes.CDLL(hb.PEAK_LIB)
    lib.peak_probe_layouts.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    out = torch.full((2432,), -1, dtype=torch.int32, device="cuda")
    rc = lib.peak_probe_layouts(out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_mfma_operand_and_accumulator_layout(probe):
    lanes, regs = np.meshgrid(np.arange(64), np.arange(16), indexing="ij")
    rows = 8 * (regs // 4) + 4 * (lanes // 32) + regs % 4
    assert np.array_equal(probe[:1024].reshape(64, 16), rows % 16)
    assert np.array_equal(probe[1024:2048].reshape(64, 16), np.broadcast_to(lanes % 32, (64, 16)))


def test_transposing_lds_read(probe):
    got = probe[2048:2304].reshape(64, 4)
    want = np.empty((64, 4), dtype=np.int64)
    for lane in range(64):
        g, i = divmod(lane, 16)
        for j in range(4):
            src = 16 * g + 4 * j + i // 4          # lane whose address is read
            want[lane, j] = 4 * src + i % 4        # halfword index = stored value
    assert np.array_equal(got, want)


def test_permlane32_swap_halves(probe):
    got = probe[2304:2432].reshape(64, 2)
    lanes = np.arange(64)
    assert np.array_equal(got[:, 0], 100 + lanes % 32)
    assert np.array_equal(got[:, 1], 100 + 32 + lanes % 32)
