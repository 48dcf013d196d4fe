"""Parity of gqa_attn_prefill_qint8 (Q quantised before the call) with the oracle.

"gfx936 DCU上实现INT8 QK MMAC" §4 moves the query quantisation out of the attention
into the producer of Q, so that every KV segment of a long history reads one set of
codes. The entry point takes those codes and scales. Two checks:

* against the oracle's attention_int8 on the same codes and scales (codes from the
  oracle's quantiser, and arbitrary codes with arbitrary float32 scales, which no
  quantiser would produce): the INT8 bound (2e-3, plus half a bf16 ulp of the output on
  short histories), element by element;
* against gqa_attn_prefill_ws on the bf16 Q those codes were quantised from: the kernel
  quantises each row with the same rule, so the outputs must be bitwise equal,
  unsplit, split into KV segments, paged and in the decode shape.
"""

import numpy as np
import pytest
import torch

import gqa_causal_prefill_amd as gqa
import oracle
from gqa_synth import (WORKLOADS, block_table_for, make_qkv, make_workload,
                       scatter_paged, scatter_paged_int8_splitd, scatter_paged_scales)
from tolerance import BF16_MAX, BF16_MEAN, INT8_MAX, errors, int8_excess  # noqa: F401

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)


def dev(x):
    return (torch.from_numpy(x) if isinstance(x, np.ndarray) else x).to(DEV)


# (q_len, kv_len): unsplit, split into KV segments, decode shape, ragged tails
SHAPES = [(200, 1500), (64, 3000), (2, 900), (37, 5000), (1, 70)]


@pytest.mark.parametrize("q_len,kv_len", SHAPES)
def test_qint8_matches_oracle_and_the_quantising_call(q_len, kv_len):
    plan = gqa.gqa_attn_prefill_plan(q_len, kv_len, int8k=True)
    note(f"case qint8 {q_len}x{kv_len}: {plan}")
    q, k, v, _ = make_qkv(q_len, kv_len, seed=9000 + q_len + kv_len)
    kq, ks = oracle.quantize_rows_int8(k)
    qq, sq = oracle.quantize_rows_int8(q)
    out = gqa.gqa_attn_prefill_qint8(dev(qq), dev(sq), dev(kq), dev(v), k_scale=dev(ks))
    ref_call = gqa.gqa_attn_prefill_ws(dev(q), dev(kq), dev(v), k_scale=dev(ks))
    torch.cuda.synchronize()
    assert int8_excess(out, oracle.attention_int8(qq, sq, kq, ks, v)) <= 0
    assert torch.equal(out, ref_call)


def test_qint8_arbitrary_codes_and_scales():
    """Codes and scales no quantiser would produce: the kernel must use the given
    scales, not recompute them from the codes."""
    q_len, kv_len = 96, 2500
    note(f"case qint8 arbitrary codes {q_len}x{kv_len}")
    rng = np.random.default_rng(91)
    qq = rng.integers(-127, 128, (q_len, 24, 256)).astype(np.int8)
    sq = (rng.random((q_len, 24)) * 4e-4).astype(np.float32)
    sq[5, 3] = 0.0                                   # a zero scale: uniform weights
    _, k, v, _ = make_qkv(q_len, kv_len, seed=92)
    kq, ks = oracle.quantize_rows_int8(k)
    out = gqa.gqa_attn_prefill_qint8(dev(qq), dev(sq), dev(kq), dev(v), k_scale=dev(ks))
    torch.cuda.synchronize()
    assert int8_excess(out, oracle.attention_int8(qq, sq, kq, ks, v)) <= 0


def test_qint8_paged_split_equals_contiguous():
    q_len, kv_len, nb = 64, 5000, 400
    note(f"case qint8 paged {q_len}x{kv_len}")
    q, k, v, rng = make_qkv(q_len, kv_len, seed=93)
    kq, ks = oracle.quantize_rows_int8(k)
    qq, sq = oracle.quantize_rows_int8(q)
    bt = block_table_for(rng, kv_len, nb)
    kc = scatter_paged_int8_splitd(torch.from_numpy(kq), bt, nb)
    sc = scatter_paged_scales(torch.from_numpy(ks), bt, nb)
    vc = scatter_paged(v, bt, nb)
    out = gqa.gqa_attn_prefill_qint8(dev(qq), dev(sq), dev(kc), dev(vc), block_table=dev(bt),
                                     k_scale=dev(sc), kv_len=kv_len)
    contig = gqa.gqa_attn_prefill_qint8(dev(qq), dev(sq), dev(kq), dev(v), k_scale=dev(ks))
    torch.cuda.synchronize()
    assert int8_excess(out, oracle.attention_int8(qq, sq, kq, ks, v)) <= 0
    assert torch.equal(out, contig)


def test_full_size_paged_int8k_with_quantised_q():
    """The paged INT8 512 x 32768 workload, which runs as KV segments: one set of query
    codes serves every segment; bitwise equal to the quantising call, and every row
    against the oracle."""
    w = WORKLOADS[7]
    note(f"case {w.name} with quantised Q: generating inputs")
    d = make_workload(w)
    kq, ks = oracle.quantize_rows_int8(d["k"])
    qq, sq = oracle.quantize_rows_int8(d["q"])
    bt = d["block_table"]
    kc = dev(scatter_paged_int8_splitd(torch.from_numpy(kq), bt, w.num_blocks))
    sc = dev(scatter_paged_scales(torch.from_numpy(ks), bt, w.num_blocks))
    vc = dev(d["v_cache"])
    assert gqa.gqa_attn_prefill_workspace_size(w.q_len, w.kv_len, paged=True, int8k=True) > 0
    note(f"case {w.name} with quantised Q: running")
    out = gqa.gqa_attn_prefill_qint8(dev(qq), dev(sq), kc, vc, block_table=dev(bt), k_scale=sc,
                                     kv_len=w.kv_len)
    ref_call = gqa.gqa_attn_prefill_ws(dev(d["q"]), kc, vc, block_table=dev(bt), k_scale=sc,
                                       kv_len=w.kv_len)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_call)
    note(f"case {w.name} with quantised Q: oracle")
    mx, mean = errors(out, oracle.attention_int8(qq, sq, kq, ks, d["v"]))
    note(f"  all {w.q_len} rows x 24 heads x 256: max {mx:.3e} mean {mean:.3e}")
    assert mx <= INT8_MAX
