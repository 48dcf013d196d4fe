"""Parity of the decode shape (q_len <= 4) with the CPU oracle.

A chunk of at most 4 query tokens runs with one token per wave and the 6 query heads
of a GQA group on 6 of the 16 columns of the matrix instruction ("gfx936 DCU上实现INT8
QK MMAC" §5.1 makes the same choice for decode), usually with the history cut into
KV segments. The arithmetic per column is the prefill one, so the same tolerances
apply: bf16 max |err| <= 1e-2 and mean <= 1e-3 against the float64 oracle; INT8 keys
within 2e-3 plus half a bf16 ulp of the output of the oracle that applies the same
quantisation. Every shape is compared element by element.
"""

import numpy as np
import pytest
import torch

import gqa_causal_prefill_amd as gqa
import oracle
from gqa_synth import (WORKLOADS, block_table_for, make_qkv, make_workload, scatter_paged,
                       scatter_paged_int8_splitd, scatter_paged_scales)
from tolerance import BF16_MAX, BF16_MEAN, INT8_MAX, errors, int8_excess  # noqa: F401

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)


def decode_plan(q_len, kv_len, paged=False, int8k=False):
    plan = gqa.gqa_attn_prefill_plan(q_len, kv_len, paged=paged, int8k=int8k)
    assert "decode_t4h6" in plan, plan
    return plan


@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (1, 63), (2, 100), (3, 517), (4, 4), (4, 2000),
                                          (1, 5000)])
def test_decode_contiguous_full(q_len, kv_len):
    note(f"case decode {q_len}x{kv_len}: {decode_plan(q_len, kv_len)}")
    q, k, v, _ = make_qkv(q_len, kv_len, seed=8000 + 7 * q_len + kv_len)
    ref = oracle.attention(q, k, v)
    for f in (gqa.gqa_attn_prefill, gqa.gqa_attn_prefill_ws):
        out = f(q.to(DEV), k.to(DEV), v.to(DEV))
        torch.cuda.synchronize()
        mx, mean = errors(out, ref)
        note(f"  {f.__name__}: max {mx:.3e} mean {mean:.3e}")
        assert mx <= BF16_MAX and mean <= BF16_MEAN


@pytest.mark.parametrize("q_len,kv_len,nb", [(1, 300, 25), (4, 1000, 70)])
def test_decode_paged_full_and_bitwise_equal_to_contiguous(q_len, kv_len, nb):
    note(f"case decode paged {q_len}x{kv_len}: {decode_plan(q_len, kv_len, paged=True)}")
    q, k, v, rng = make_qkv(q_len, kv_len, seed=8100 + kv_len)
    bt = block_table_for(rng, kv_len, nb)
    kc, vc = scatter_paged(k, bt, nb), scatter_paged(v, bt, nb)
    for f in (gqa.gqa_attn_prefill, gqa.gqa_attn_prefill_ws):
        out = f(q.to(DEV), kc.to(DEV), vc.to(DEV), block_table=bt.to(DEV), kv_len=kv_len)
        contig = f(q.to(DEV), k.to(DEV), v.to(DEV))
        torch.cuda.synchronize()
        mx, mean = errors(out, oracle.attention(q, k, v))
        assert mx <= BF16_MAX and mean <= BF16_MEAN
        assert torch.equal(out, contig)


@pytest.mark.parametrize("q_len,kv_len", [(1, 700), (3, 3000)])
def test_decode_int8k_full(q_len, kv_len):
    note(f"case decode int8k {q_len}x{kv_len}: {decode_plan(q_len, kv_len, int8k=True)}")
    q, k, v, _ = make_qkv(q_len, kv_len, seed=8200 + kv_len)
    kq, ks = oracle.quantize_rows_int8(k)
    ref = oracle.attention_int8k(q, kq, ks, v)
    for f in (gqa.gqa_attn_prefill, gqa.gqa_attn_prefill_ws):
        out = f(q.to(DEV), torch.from_numpy(kq).to(DEV), v.to(DEV),
                k_scale=torch.from_numpy(ks).to(DEV))
        torch.cuda.synchronize()
        assert int8_excess(out, ref) <= 0


def test_decode_paged_int8k_full():
    q_len, kv_len, nb = 2, 900, 60
    note(f"case decode paged int8k: {decode_plan(q_len, kv_len, paged=True, int8k=True)}")
    q, k, v, rng = make_qkv(q_len, kv_len, seed=8300)
    kq, ks = oracle.quantize_rows_int8(k)
    bt = block_table_for(rng, kv_len, nb)
    kc = scatter_paged_int8_splitd(torch.from_numpy(kq), bt, nb)
    sc = scatter_paged_scales(torch.from_numpy(ks), bt, nb)
    vc = scatter_paged(v, bt, nb)
    out = gqa.gqa_attn_prefill_ws(q.to(DEV), kc.to(DEV), vc.to(DEV), block_table=bt.to(DEV),
                                  k_scale=sc.to(DEV), kv_len=kv_len)
    torch.cuda.synchronize()
    assert int8_excess(out, oracle.attention_int8k(q, kq, ks, v)) <= 0


def test_decode_restart():
    """Keys from 900 on score 144 (log2 units) above the first tile's."""
    q_len, kv_len = 2, 2000
    note(f"case decode restart: {decode_plan(q_len, kv_len)}")
    q, k, v, _ = make_qkv(q_len, kv_len, seed=8400)
    q2, k2 = q.to(torch.float32).clone(), k.to(torch.float32).clone()
    q2[..., 0] += 40.0
    k2[900:, :, 0] = 40.0
    q, k = q2.to(torch.bfloat16), k2.to(torch.bfloat16)
    ref = oracle.attention(q, k, v)
    for f in (gqa.gqa_attn_prefill, gqa.gqa_attn_prefill_ws):
        out = f(q.to(DEV), k.to(DEV), v.to(DEV))
        torch.cuda.synchronize()
        mx, mean = errors(out, ref)
        assert mx <= BF16_MAX and mean <= BF16_MEAN


@pytest.mark.parametrize("idx", [8, 9])
def test_full_size_decode(idx):
    """The decode workloads the benchmark times (1 token over 32768 keys, contiguous and
    paged), every output."""
    w = WORKLOADS[idx]
    note(f"case {w.name}: {decode_plan(w.q_len, w.kv_len, paged=w.paged)}")
    d = make_workload(w)
    if w.paged:
        out = gqa.gqa_attn_prefill_ws(d["q"].to(DEV), d["k_cache"].to(DEV), d["v_cache"].to(DEV),
                                      block_table=d["block_table"].to(DEV), kv_len=w.kv_len)
    else:
        out = gqa.gqa_attn_prefill_ws(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV))
    torch.cuda.synchronize()
    mx, mean = errors(out, oracle.attention(d["q"], d["k"], d["v"]))
    note(f"  max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_full_size_paged_int8k_decode():
    """The INT8 QK page's decode case: one token over 32768 keys of a paged split-d INT8
    K cache, as the benchmark times it (KV segments through a workspace); every output
    against the oracle on the oracle's codes."""
    w = WORKLOADS[10]
    note(f"case {w.name}: {decode_plan(w.q_len, w.kv_len, paged=True, int8k=True)}")
    d = make_workload(w)
    kq, ks = oracle.quantize_rows_int8(d["k"])
    bt = d["block_table"]
    kc = scatter_paged_int8_splitd(torch.from_numpy(kq), bt, w.num_blocks)
    sc = scatter_paged_scales(torch.from_numpy(ks), bt, w.num_blocks)
    out = gqa.gqa_attn_prefill_ws(d["q"].to(DEV), kc.to(DEV), d["v_cache"].to(DEV),
                                  block_table=bt.to(DEV), k_scale=sc.to(DEV), kv_len=w.kv_len)
    torch.cuda.synchronize()
    ref = oracle.attention_int8k(d["q"], kq, ks, d["v"])
    e = np.abs(out.float().cpu().numpy().astype(np.float64) - ref)
    note(f"  max {e.max():.3e}")
    assert e.max() <= INT8_MAX
