"""CPU fragment model of the gfx950 MFMA layouts the kernels rely on, checked
against the hardware through a one-instruction probe (the INT8 QK page's first
validation layer, §7, redone for gfx950's instructions).

Model (lane l, element e of an operand register tuple, register r of the result):
  v_mfma_f32_16x16x32_bf16: A[i][k] = a[l][e] with i = l % 16, k = 8 (l // 16) + e;
                            B[k][j] = b[l][e] with j = l % 16, k = 8 (l // 16) + e;
                            D[i][j] = d[l][r] with i = 4 (l // 16) + r, j = l % 16.
  v_mfma_i32_16x16x64_i8:   the same with 16 elements per lane, k = 16 (l // 16) + e.
Integer-valued random inputs make every product and sum exact, so the check is
bit-exact. A different but identical-for-A-and-B order of k inside a lane would
still pass, which is exactly the property the kernels need.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from gqa_causal_prefill_amd import build as gqa_build

pytestmark = pytest.mark.gpu


def probe_lib():
    if not os.path.exists(gqa_build.PROBE_LIB):
        pytest.fail("probe library not built")
    return ctypes.CDLL(gqa_build.PROBE_LIB)


def model_product(a, b, kpl):
    """a, b: [64, kpl] lane fragments -> D as [64, 4] lane fragments."""
    A = np.zeros((16, 4 * kpl), np.int64)
    B = np.zeros((4 * kpl, 16), np.int64)
    for l in range(64):
        for e in range(kpl):
            A[l % 16, kpl * (l // 16) + e] = a[l, e]
            B[kpl * (l // 16) + e, l % 16] = b[l, e]
    D = A @ B
    d = np.zeros((64, 4), np.int64)
    for l in range(64):
        for r in range(4):
            d[l, r] = D[4 * (l // 16) + r, l % 16]
    return d


def test_bf16_16x16x32_layout():
    lib = probe_lib()
    rng = np.random.default_rng(0)
    a = rng.integers(-8, 9, (64, 8))
    b = rng.integers(-8, 9, (64, 8))
    ta = torch.tensor(a, dtype=torch.bfloat16, device="cuda")
    tb = torch.tensor(b, dtype=torch.bfloat16, device="cuda")
    td = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    print("probe: v_mfma_f32_16x16x32_bf16", flush=True)
    assert lib.gqa_probe_mfma_f32_16x16x32_bf16(ctypes.c_void_p(ta.data_ptr()),
                                                ctypes.c_void_p(tb.data_ptr()),
                                                ctypes.c_void_p(td.data_ptr()), None) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(td.cpu().numpy().astype(np.int64), model_product(a, b, 8))


def test_i8_16x16x64_layout():
    lib = probe_lib()
    rng = np.random.default_rng(1)
    a = rng.integers(-127, 128, (64, 16))
    b = rng.integers(-127, 128, (64, 16))
    ta = torch.tensor(a, dtype=torch.int8, device="cuda")
    tb = torch.tensor(b, dtype=torch.int8, device="cuda")
    td = torch.zeros((64, 4), dtype=torch.int32, device="cuda")
    print("probe: v_mfma_i32_16x16x64_i8", flush=True)
    assert lib.gqa_probe_mfma_i32_16x16x64_i8(ctypes.c_void_p(ta.data_ptr()),
                                              ctypes.c_void_p(tb.data_ptr()),
                                              ctypes.c_void_p(td.data_ptr()), None) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(td.cpu().numpy().astype(np.int64), model_product(a, b, 16))
