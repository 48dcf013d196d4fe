"""Parity of paged INT8-K attention (split-d K cache, paged scales) with the oracle.

The K codes live in the split-d page layout of "gfx936 DCU上实现INT8 QK MMAC" §3 and
their scales in pages of the same blocks; every scale slot that no key uses holds NaN,
so reading one would poison the output. The oracle gathers codes and scales back into
logical order and applies the INT8 definition. The kernel runs the contiguous INT8
arithmetic in the same order, so paged and contiguous outputs must be bitwise equal;
against the oracle the INT8 bound applies (2e-3, plus half a bf16 ulp of the output on
short histories, as for the contiguous INT8 path).
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


def paged_inputs(q_len, kv_len, nb, seed, shift=None):
    q, k, v, rng = make_qkv(q_len, kv_len, seed=seed)
    if shift is not None:   # keys from `shift` on score far above the first tile's
        q2, k2 = q.to(torch.float32).clone(), k.to(torch.float32).clone()
        q2[..., 0] += 40.0
        k2[shift:, :, 0] = 40.0
        q, k = q2.to(torch.bfloat16), k2.to(torch.bfloat16)
    kq, ks = oracle.quantize_rows_int8(k)
    bt = block_table_for(rng, kv_len, nb)
    kq_t, ks_t = torch.from_numpy(kq), torch.from_numpy(ks)
    return dict(q=q, v=v, kq=kq, ks=ks, bt=bt,
                kc=scatter_paged_int8_splitd(kq_t, bt, nb), sc=scatter_paged_scales(ks_t, bt, nb),
                vc=scatter_paged(v, bt, nb))


def run_paged(d, kv_len, ws=False):
    f = gqa.gqa_attn_prefill_ws if ws else gqa.gqa_attn_prefill
    return f(d["q"].to(DEV), d["kc"].to(DEV), d["vc"].to(DEV), block_table=d["bt"].to(DEV),
             k_scale=d["sc"].to(DEV), kv_len=kv_len)


def run_contig(d, ws=False):
    f = gqa.gqa_attn_prefill_ws if ws else gqa.gqa_attn_prefill
    return f(d["q"].to(DEV), torch.from_numpy(d["kq"]).to(DEV), d["v"].to(DEV),
             k_scale=torch.from_numpy(d["ks"]).to(DEV))


def oracle_ref(d, kv_len, rows=None):
    kq = oracle.gather_paged_int8_splitd(d["kc"], d["bt"], kv_len)
    ks = oracle.gather_paged_scales(d["sc"], d["bt"], kv_len)
    return oracle.attention_int8k(d["q"], kq, ks, d["v"], rows=rows)


@pytest.mark.parametrize("q_len,kv_len,nb", [(1, 16, 1), (33, 70, 9), (64, 257, 40),
                                             (100, 1000, 70), (300, 1300, 90)])
def test_paged_int8k_full_and_bitwise_equal_to_contiguous(q_len, kv_len, nb):
    note(f"case paged int8k {q_len}x{kv_len} blocks {nb}")
    d = paged_inputs(q_len, kv_len, nb, seed=7000 + kv_len)
    out = run_paged(d, kv_len)
    contig = run_contig(d)
    torch.cuda.synchronize()
    assert int8_excess(out, oracle_ref(d, kv_len)) <= 0
    assert torch.equal(out, contig)


def test_paged_int8k_split_segments():
    q_len, kv_len, nb = 64, 5000, 400
    note(f"case paged int8k split {q_len}x{kv_len}")
    assert gqa.gqa_attn_prefill_workspace_size(q_len, kv_len, paged=True, int8k=True) > 0
    d = paged_inputs(q_len, kv_len, nb, seed=7100)
    out = run_paged(d, kv_len, ws=True)
    contig = run_contig(d, ws=True)
    torch.cuda.synchronize()
    assert int8_excess(out, oracle_ref(d, kv_len)) <= 0
    assert torch.equal(out, contig)


def test_paged_int8k_restart():
    q_len, kv_len, nb = 48, 600, 45
    note("case paged int8k restart")
    d = paged_inputs(q_len, kv_len, nb, seed=7200, shift=230)
    out = run_paged(d, kv_len)
    torch.cuda.synchronize()
    assert int8_excess(out, oracle_ref(d, kv_len)) <= 0


def test_full_size_paged_int8k():
    w = WORKLOADS[7]
    note(f"case {w.name}: generating inputs")
    data = make_workload(w)
    kq, ks = oracle.quantize_rows_int8(data["k"])   # the codes both sides read
    bt = data["block_table"]
    kc = scatter_paged_int8_splitd(torch.from_numpy(kq), bt, w.num_blocks)
    sc = scatter_paged_scales(torch.from_numpy(ks), bt, w.num_blocks)
    note(f"case {w.name}: running (the benchmark's launch: KV segments through a workspace)")
    out = gqa.gqa_attn_prefill_ws(data["q"].to(DEV), kc.to(DEV), data["v_cache"].to(DEV),
                                  block_table=bt.to(DEV), k_scale=sc.to(DEV), kv_len=w.kv_len)
    torch.cuda.synchronize()
    note(f"case {w.name}: oracle")
    ref = oracle.attention_int8k(data["q"], oracle.gather_paged_int8_splitd(kc, bt, w.kv_len),
                                 oracle.gather_paged_scales(sc, bt, w.kv_len), data["v"])
    mx, mean = errors(out, ref)
    note(f"  all {w.q_len} rows x 24 heads x 256: max {mx:.3e} mean {mean:.3e}")
    assert mx <= INT8_MAX
