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


# ---------------------------------------------------------------- data-movement instructions

def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_ds_read_tr16_b64_model():
    """Model: within each group of 16 lanes, lane j's element k is element j % 4 of the
    8-byte chunk read by lane 4k + j // 4 of the same group."""
    lib = probe_lib()
    img = torch.arange(4096, dtype=torch.int16, device="cuda")
    rng = np.random.default_rng(2)
    patterns = [[8 * l for l in range(64)],
                [(l % 16) * 64 + (l // 16) * 8 for l in range(64)],
                list(8 * rng.permutation(1024)[:64])]
    for offs in patterns:
        host = (ctypes.c_int * 64)(*[int(o) for o in offs])
        dev_offs = torch.tensor(offs, dtype=torch.int32, device="cuda")
        out = torch.zeros((64, 4), dtype=torch.int16, device="cuda")
        print("probe: ds_read_b64_tr_b16", flush=True)
        assert lib.gqa_probe_ds_read_tr16_b64(_ptr(img), _ptr(dev_offs), host, _ptr(out), None) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        chunks = np.array([[o // 2 + e for e in range(4)] for o in offs])  # element values = indices
        for lane in range(64):
            grp, j = lane // 16, lane % 16
            want = [chunks[16 * grp + 4 * k + j // 4][j % 4] for k in range(4)]
            assert got[lane].tolist() == want, (lane, got[lane].tolist(), want)


def test_global_load_lds_dwordx4_model():
    """Model: lane t's 16 bytes land at the wave-uniform LDS base + 16 t."""
    lib = probe_lib()
    src = torch.arange(256, dtype=torch.int32, device="cuda") + 5000
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")
    print("probe: global_load_lds_dwordx4", flush=True)
    assert lib.gqa_probe_global_load_lds_dwordx4(_ptr(src), _ptr(out), None) == 0
    torch.cuda.synchronize()
    want = np.full(1024, -1)
    want[64:64 + 256] = np.arange(256) + 5000
    np.testing.assert_array_equal(out.cpu().numpy(), want)


def test_permlane_swaps_model():
    """Model: permlane16_swap(x, x) returns (x of lane l or l-16, x of lane l or l+16) so
    that their max/sum is the xor-16 reduction; permlane32_swap likewise for xor 32."""
    lib = probe_lib()
    out = torch.zeros((64, 4), dtype=torch.int32, device="cuda")
    print("probe: permlane swaps", flush=True)
    assert lib.gqa_probe_permlane_swaps(_ptr(out), None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    a = lambda l: 1000 + l  # noqa: E731  (old operand)
    b = lambda l: 2000 + l  # noqa: E731  (src operand)
    for l in range(64):
        row = l // 16
        want16 = (a(l), a(l + 16)) if row % 2 == 0 else (b(l - 16), b(l))
        want32 = (a(l), a(l + 32)) if l < 32 else (b(l - 32), b(l))
        assert tuple(got[l, :2]) == want16, (l, got[l])
        assert tuple(got[l, 2:]) == want32, (l, got[l])
