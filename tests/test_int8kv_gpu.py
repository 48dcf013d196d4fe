"""Parity of the INT8-value path (gqa_attn_prefill_int8kv, gqa_quantize_v_int8) with the
oracle's reading of INT8 PV ("gfx936 DCU上实现INT8 QK MMAC" §6; oracle/int8pv.py).

* The V quantiser is integer work: codes and scales bitwise equal to the oracle's,
  padding positions written as 0.
* The attention output is held, element by element, to the INT8 bound (2e-3, plus half a
  bf16 ulp of the reference where the output reaches 0.5 and more) plus the allowance the
  oracle derives for P codes that lie within the kernel's float32 accuracy of a rounding
  boundary (tolerance.int8kv_code_slack): such a code is correct either way.
* Closed forms: equal scores with constant V give V exactly, up to the longest history
  the int32 sums allow; a row dominated by one key returns that key's value.
* Bitwise: Q codes handed in equal Q quantised inside; two runs; stored positions past
  kv_len never change the result.
"""

import numpy as np
import pytest
import torch

import gqa_causal_prefill_amd as gqa
import oracle
from gqa_synth import WORKLOADS, make_qkv, make_workload
from tolerance import as_f64, int8kv_code_slack, int8kv_excess

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)


def dev(x):
    return (torch.from_numpy(np.ascontiguousarray(x)) if isinstance(x, np.ndarray) else x).to(DEV)


def ld_for(kv_len, extra=0):
    return (kv_len + 15) // 16 * 16 + extra


def inputs(q_len, kv_len, seed, extra_ld=0, pad_code=0):
    """bf16 q, INT8 K codes and scales, feature-major INT8 V codes [4, 256, ld] and scales,
    all from the oracle's quantisers."""
    q, k, v, _ = make_qkv(q_len, kv_len, seed)
    kq, ks = oracle.quantize_rows_int8(k)
    vq, vs = oracle.quantize_v_int8(v)
    ld = ld_for(kv_len, extra_ld)
    stored = np.full((4, 256, ld), pad_code, np.int8)
    stored[:, :, :kv_len] = vq
    return q, kq, ks, stored, vs


def run(q, kq, ks, vq, vs, q_scale=None):
    out = gqa.gqa_attn_prefill_int8kv(dev(q), dev(kq), dev(ks), dev(vq), dev(vs),
                                      q_scale=None if q_scale is None else dev(q_scale))
    torch.cuda.synchronize()
    return out


def check(name, out, q, kq, ks, vq, vs, rows=None):
    ref, slack = oracle.attention_int8kv(q, kq, ks, vq, vs, rows=rows, code_slack=int8kv_code_slack)
    got = as_f64(out) if rows is None else as_f64(out)[rows]
    err = np.abs(got - ref)
    note(f"{name}: max err {err.max():.3e} mean {err.mean():.3e}; elements with a code "
         f"allowance {int((slack > 0).sum())} (largest {slack.max():.2e})")
    assert int8kv_excess(out if rows is None else out[torch.as_tensor(rows)], ref, slack) <= 0


@pytest.mark.parametrize("kv_len,extra", [(1, 0), (100, 0), (1000, 48), (3000, 0), (16384, 16)])
def test_v_quantizer_bit_exact(kv_len, extra):
    note(f"case v quantizer {kv_len} ld+{extra}")
    _, _, v, _ = make_qkv(1, kv_len, seed=7100 + kv_len)
    ld = ld_for(kv_len, extra)
    codes = torch.full((4, 256, ld), 77, dtype=torch.int8, device=DEV)
    scales = torch.full((4, 256), float("nan"), dtype=torch.float32, device=DEV)
    gqa.gqa_quantize_v_int8(v.to(DEV), v_ld=ld, v_codes=codes, v_scale=scales)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_v_int8(v)
    c = codes.cpu().numpy()
    np.testing.assert_array_equal(c[:, :, :kv_len], rq)
    assert np.all(c[:, :, kv_len:] == 0)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


# (q_len, kv_len): single key, no history, ragged token blocks and tiles, 1.5 rounds
SHAPES = [(1, 1), (5, 5), (33, 100), (64, 64), (100, 1000), (257, 3000), (40, 4100), (96, 2500),
          (1, 70), (300, 300)]


@pytest.mark.parametrize("q_len,kv_len", SHAPES)
def test_int8kv_matches_oracle(q_len, kv_len):
    plan = gqa.gqa_attn_prefill_plan(q_len, kv_len, int8k=2)
    note(f"case int8kv {q_len}x{kv_len}: {plan}")
    q, kq, ks, vq, vs = inputs(q_len, kv_len, seed=7200 + q_len + kv_len)
    out = run(q, kq, ks, vq, vs)
    check(f"int8kv {q_len}x{kv_len}", out, q, kq, ks, vq, vs)


def test_int8kv_q_codes_bitwise_and_deterministic():
    q_len, kv_len = 130, 2100
    note(f"case int8kv q codes {q_len}x{kv_len}")
    q, kq, ks, vq, vs = inputs(q_len, kv_len, seed=7301)
    a = run(q, kq, ks, vq, vs)
    b = run(q, kq, ks, vq, vs)
    qq, sq = oracle.quantize_rows_int8(q)
    c = run(qq, kq, ks, vq, vs, q_scale=sq)
    assert torch.equal(a, b)
    assert torch.equal(a, c)


def test_int8kv_positions_past_kv_len_are_not_read():
    q_len, kv_len = 70, 1111
    note(f"case int8kv padding {q_len}x{kv_len}")
    a = run(*inputs(q_len, kv_len, seed=7302))
    b = run(*inputs(q_len, kv_len, seed=7302, extra_ld=80, pad_code=127))
    c = run(*inputs(q_len, kv_len, seed=7302, extra_ld=16, pad_code=-127))
    assert torch.equal(a, b) and torch.equal(a, c)


def test_int8kv_zero_query_rows():
    q_len, kv_len = 48, 600
    note(f"case int8kv zero query rows {q_len}x{kv_len}")
    q, kq, ks, vq, vs = inputs(q_len, kv_len, seed=7303)
    q[::3] = 0
    check("int8kv zero rows", run(q, kq, ks, vq, vs), q, kq, ks, vq, vs)


def test_int8kv_dominant_key():
    # one key's score far above the rest for every query: its code is 127, the others 0,
    # and every output row is that key's dequantised value
    q_len, kv_len = 40, 900
    note(f"case int8kv dominant key {q_len}x{kv_len}")
    q, kq, ks, vq, vs = inputs(q_len, kv_len, seed=7304)
    q = torch.ones_like(q)
    kq[:] = 0
    kq[3] = 127
    ks[:] = 1.0 / 127
    out = run(q, kq, ks, vq, vs)
    expect = (vq[:, :, 3].astype(np.float64) * vs.astype(np.float64))   # [4, 256]
    exp_rows = np.repeat(expect, 6, axis=0)[None, :, :]
    np.testing.assert_allclose(as_f64(out), np.broadcast_to(exp_rows, out.shape), rtol=2 ** -8, atol=0)
    check("int8kv dominant key", out, q, kq, ks, vq, vs)


def test_int8kv_longest_history_equal_scores():
    # K codes 0: every visible key gets code 127; V constant 1.5: every code 127 with
    # sV = 1.5 / 127. The int32 sums reach 127 * 127 * kv_len at the largest kv_len the
    # call accepts, and the output is 1.5 exactly.
    kv_len = gqa.INT8KV_MAX_KV
    q_len = 40
    note(f"case int8kv longest history {q_len}x{kv_len}")
    q = torch.randn((q_len, 24, 256), generator=torch.Generator().manual_seed(7305)).to(torch.bfloat16)
    kq = np.zeros((kv_len, 4, 256), np.int8)
    ks = np.ones((kv_len, 4), np.float32)
    v = torch.full((kv_len, 4, 256), 1.5, dtype=torch.bfloat16, device=DEV)
    vq, vs = gqa.gqa_quantize_v_int8(v)
    torch.cuda.synchronize()
    assert torch.all(vq[:, :, :kv_len] == 127)
    out = gqa.gqa_attn_prefill_int8kv(dev(q), dev(kq), dev(ks), vq, vs)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 1.5)


def test_int8kv_full_size():
    """The INT8-key workload's shape and inputs (3072 new tokens over 16384 keys), V codes
    from the library's quantiser: every row against the oracle."""
    w = WORKLOADS[5]
    note(f"case int8kv full size {w.q_len}x{w.kv_len}")
    d = make_workload(w)
    kq, ks = gqa.gqa_quantize_rows_int8(d["k"].to(DEV))
    vq, vs = gqa.gqa_quantize_v_int8(d["v"].to(DEV))
    out = gqa.gqa_attn_prefill_int8kv(d["q"].to(DEV), kq, ks, vq, vs)
    torch.cuda.synchronize()
    rvq, rvs = oracle.quantize_v_int8(d["v"])
    np.testing.assert_array_equal(vq.cpu().numpy(), rvq)
    np.testing.assert_array_equal(vs.cpu().numpy(), rvs)
    check("int8kv full size", out, d["q"], kq.cpu().numpy(), ks.cpu().numpy(), rvq, rvs)
