"""Histories of 2^22 keys (the K and V tensors 8.6 GB each, paged caches of 262,144
blocks): the path at sizes where every byte offset of K/V needs 64 bits.

The float64 oracle cannot take 4 million keys per row, so these tests use a property
that holds at any size. Q is zero except feature 0 (= 16) and K is zero except feature 0
of two spike keys: p1 far inside the history (score 30) and p2 inside the chunk itself
(score 40); every other score is exactly 0. A row's softmax then puts all but
n / e^30 < 4e-7 of its weight on the latest spike it sees (p2 outweighs p1 by e^10), so
its output is V[p1] for rows before p2's position and V[p2] from there on (the inclusive
causal boundary: query i sees key kv_len - q_len + i). V varies from row to row, so a
key read from the wrong position, a dropped tile or a wrong boundary gives the wrong V
row, far outside the bf16 tolerance. The spikes also lie far above the first tile's
reference maximum, so the workgroups that hold them take the restart with exact maxima.
"""

import numpy as np
import pytest
import torch

import gqa_causal_prefill_amd as gqa
from gqa_synth import BLOCK_SIZE, HKV, HQ, D

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
KV = 1 << 22
P1 = 1_234_567


def note(msg):
    print(msg, flush=True)


def spike_inputs(q_len):
    """Q, K, V on the GPU, and the two spike positions."""
    p2 = KV - q_len + q_len // 2          # seen by rows q_len // 2 .. q_len - 1
    q = torch.zeros((q_len, HQ, D), dtype=torch.bfloat16, device=DEV)
    q[:, :, 0] = 16.0
    k = torch.zeros((KV, HKV, D), dtype=torch.bfloat16, device=DEV)
    k[P1, :, 0] = 30.0                    # score = 16 * 30 / 16 = 30
    k[p2, :, 0] = 40.0                    # score 40
    # V[j, g, d] = ((7 j + 3 d + g) mod 11 - 5) / 8: multiples of 1/8, exact in bf16
    v = torch.empty((KV, HKV, D), dtype=torch.bfloat16, device=DEV)
    g = torch.arange(HKV, device=DEV, dtype=torch.int32).view(1, HKV, 1)
    d = torch.arange(D, device=DEV, dtype=torch.int32).view(1, 1, D)
    chunk = 1 << 20
    for j0 in range(0, KV, chunk):
        j = torch.arange(j0, j0 + chunk, device=DEV, dtype=torch.int32).view(chunk, 1, 1)
        v[j0:j0 + chunk] = (((7 * (j % 11) + 3 * d + g) % 11 - 5).to(torch.float32) / 8).to(torch.bfloat16)
    return q, k, v, p2


def expected(v, q_len, p2):
    """Row i, head h: V[p1, h // 6] before p2's position, V[p2, h // 6] from there on."""
    off = KV - q_len
    rows = np.arange(q_len)
    v1 = v[P1].float().cpu().numpy()            # [4, 256]
    v2 = v[p2].float().cpu().numpy()
    src = np.where((off + rows >= p2)[:, None, None], v2[None], v1[None])    # [q, 4, 256]
    return np.repeat(src, HQ // HKV, axis=1)                                 # [q, 24, 256]


def check(out, ref, what):
    e = np.abs(out.float().cpu().numpy().astype(np.float64) - ref)
    note(f"  {what}: max {e.max():.3e} mean {e.mean():.3e}")
    assert e.max() <= 1e-2 and e.mean() <= 1e-3


@pytest.mark.parametrize("q_len", [40, 1])
def test_max_history_contiguous(q_len):
    note(f"case max history contiguous {q_len}x{KV}")
    q, k, v, p2 = spike_inputs(q_len)
    out = gqa.gqa_attn_prefill_ws(q, k, v)
    torch.cuda.synchronize()
    check(out, expected(v, q_len, p2), gqa.gqa_attn_prefill_plan(q_len, KV).split()[4])
    if q_len > 1:
        out1 = gqa.gqa_attn_prefill(q, k, v)   # one workgroup per token block, no segments
        torch.cuda.synchronize()
        check(out1, expected(v, q_len, p2), "unsplit")
    del q, k, v
    torch.cuda.empty_cache()


def test_max_history_paged():
    q_len = 40
    note(f"case max history paged {q_len}x{KV}")
    q, k, v, p2 = spike_inputs(q_len)
    nb = KV // BLOCK_SIZE
    gen = torch.Generator(device="cpu").manual_seed(22)
    bt = torch.randperm(nb, generator=gen).to(torch.int32).to(DEV)
    # cache[bt[t // 16], g, t % 16, :] = x[t, g, :]
    def scatter(x):
        cache = torch.empty((nb, HKV, BLOCK_SIZE, D), dtype=x.dtype, device=DEV)
        cache[bt.long()] = x.view(nb, BLOCK_SIZE, HKV, D).permute(0, 2, 1, 3)
        return cache
    kc, vc = scatter(k), scatter(v)
    ref = expected(v, q_len, p2)
    del k
    out = gqa.gqa_attn_prefill_ws(q, kc, vc, block_table=bt, kv_len=KV)
    torch.cuda.synchronize()
    check(out, ref, "paged, 262144 blocks")
    del q, kc, vc, v
    torch.cuda.empty_cache()


def test_max_history_int8k():
    """INT8 keys: the spike rows quantise to code 127 with scale 30/127 or 40/127 (every
    other row is all zeros: scale 0, C11), Q quantises to 127 with scale 16/127, so the
    restored scores are 30 and 40 to fp32 rounding."""
    q_len = 40
    note(f"case max history int8k {q_len}x{KV}")
    q, k, v, p2 = spike_inputs(q_len)
    del k
    kq = torch.zeros((KV, HKV, D), dtype=torch.int8, device=DEV)
    kq[P1, :, 0] = 127
    kq[p2, :, 0] = 127
    ks = torch.zeros((KV, HKV), dtype=torch.float32, device=DEV)
    ks[P1] = 30.0 / 127.0
    ks[p2] = 40.0 / 127.0
    out = gqa.gqa_attn_prefill_ws(q, kq, v, k_scale=ks)
    torch.cuda.synchronize()
    check(out, expected(v, q_len, p2), "int8 keys")
    del q, kq, ks, v
    torch.cuda.empty_cache()
