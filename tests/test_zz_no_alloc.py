"""gqa_attn_prefill_noalloc through the C ABI: the KV-segment partials in the library's
scratch array instead of a caller's workspace.

Its plan is that of gqa_attn_prefill_ws, so its output must be bit for bit that of
gqa_attn_prefill_ws with a workspace, and within the tolerances of the oracle (bf16:
max |err| <= 1e-2, mean <= 1e-3). Two calls in a row share the array, the second with
a smaller input, so leftovers of the first must not leak into the second.
"""

import ctypes

import numpy as np
import pytest
import torch

import gqa_causal_prefill_amd as gqa
import oracle
from gqa_synth import WORKLOADS, make_qkv, make_workload
from tolerance import BF16_MAX, BF16_MEAN, INT8_MAX, errors

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)


def c_noalloc(q, k, v, out, block_table=None, k_scale=None, kv_len=None, num_blocks=0):
    """One call of the C entry point with raw device pointers on torch's current stream."""
    vp = ctypes.c_void_p
    kv_len = k.shape[0] if kv_len is None else kv_len
    st = gqa.library().gqa_attn_prefill_noalloc(
        vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()),
        vp(block_table.data_ptr()) if block_table is not None else None, num_blocks,
        vp(k_scale.data_ptr()) if k_scale is not None else None, q.shape[0], kv_len,
        vp(out.data_ptr()), vp(torch.cuda.current_stream(DEV).cuda_stream))
    assert st == 0, gqa.gqa_status_string(st)
    return out


def test_noalloc_two_calls_match_workspace_call():
    # call 1: the paged 512 x 32768 tail, 4 KV segments (50.7 MB of partials)
    w = WORKLOADS[4]
    need = gqa.gqa_attn_prefill_workspace_size(w.q_len, w.kv_len, paged=True)
    note(f"case noalloc {w.name}: {need} bytes of partials")
    assert 0 < need <= gqa.NOALLOC_SCRATCH_BYTES
    d = make_workload(w)
    q, kc, vc, bt = (d["q"].to(DEV), d["k_cache"].to(DEV), d["v_cache"].to(DEV),
                     d["block_table"].to(DEV))
    out1 = torch.full_like(q, float("nan"))
    c_noalloc(q, kc, vc, out1, block_table=bt, kv_len=w.kv_len, num_blocks=w.num_blocks)
    want1 = gqa.gqa_attn_prefill_ws(q, kc, vc, block_table=bt, kv_len=w.kv_len)
    torch.cuda.synchronize()
    assert torch.equal(out1, want1)
    mx, mean = errors(out1, oracle.attention(d["q"], oracle.gather_paged(d["k_cache"], d["block_table"], w.kv_len),
                                             oracle.gather_paged(d["v_cache"], d["block_table"], w.kv_len)))
    note(f"  max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN

    # call 2, right after: a smaller contiguous chunk, 5 KV segments
    q_len, kv_len = 40, 3000
    need2 = gqa.gqa_attn_prefill_workspace_size(q_len, kv_len)
    note(f"case noalloc {q_len}x{kv_len}: {need2} bytes of partials")
    assert 0 < need2 < need
    qs, ks, vs, _ = make_qkv(q_len, kv_len, seed=9100)
    qd, kd, vd = qs.to(DEV), ks.to(DEV), vs.to(DEV)
    out2 = torch.full_like(qd, float("nan"))
    c_noalloc(qd, kd, vd, out2)
    want2 = gqa.gqa_attn_prefill_ws(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(out2, want2)
    mx, mean = errors(out2, oracle.attention(qs, ks, vs))
    note(f"  max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_noalloc_int8k_partial_split_and_unsplit():
    """INT8 keys with only the longest token blocks cut (the 3072 x 16384 plan), then a
    chunk whose plan needs no partials at all."""
    w = WORKLOADS[5]
    note(f"case noalloc {w.name}")
    d = make_workload(w)
    kq, ks = oracle.quantize_rows_int8(d["k"])
    q, k, v, sk = d["q"].to(DEV), torch.from_numpy(kq).to(DEV), d["v"].to(DEV), torch.from_numpy(ks).to(DEV)
    out = torch.full_like(q, float("nan"))
    c_noalloc(q, k, v, out, k_scale=sk)
    want = gqa.gqa_attn_prefill_ws(q, k, v, k_scale=sk)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    mx, _ = errors(out, oracle.attention_int8k(d["q"], kq, ks, d["v"]))
    note(f"  max {mx:.3e}")
    assert mx <= INT8_MAX

    q_len, kv_len = 256, 1024
    assert gqa.gqa_attn_prefill_workspace_size(q_len, kv_len) == 0
    qs, kk, vv, _ = make_qkv(q_len, kv_len, seed=9200)
    out3 = torch.full((q_len, 24, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    c_noalloc(qs.to(DEV), kk.to(DEV), vv.to(DEV), out3)
    want3 = gqa.gqa_attn_prefill(qs.to(DEV), kk.to(DEV), vv.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out3, want3)
