"""Pins of the INT8 P·V oracle (oracle/int8pv.py) against facts it does not define itself.

The reading (INT8 V per (KV head, feature), P codes against the exact row maximum, row
sum from the codes) is checked against a hand-worked example (tests/golden), closed
forms (equal scores give code 127 everywhere, a row that sees one key returns that key's
value), an invariant (stored positions past kv_len are never read) and a bound against
float attention on the dequantised values. The last tests plant plausible mistakes in
the oracle and check that these pins catch them.
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import int8pv as int8pv_mod
from oracle import prefill as prefill_mod
from gqa_synth import make_qkv, HQ, HKV, D

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8pv_hand_example.txt")


def _heads(spec):
    if "-" in spec:
        a, b = spec.split("-")
        return range(int(a), int(b) + 1)
    return [int(spec)]


def load_example():
    ex = dict(codes={}, out=[], v={}, vcol_scales={}, vcodes={})
    with open(GOLDEN) as f:
        lines = [ln.split("#", 1)[0].split() for ln in f]
    lines = [t for t in lines if t]
    for t in lines:
        if t[0] in ("q_len", "kv_len", "ld", "vquant_kv_len"):
            ex[t[0]] = int(t[1])
    q_len, kv_len, ld = ex["q_len"], ex["kv_len"], ex["ld"]
    qq = np.zeros((q_len, HQ, D), np.int8)
    kq = np.zeros((kv_len, HKV, D), np.int8)
    ks = np.ones((kv_len, HKV), np.float32)
    vq = np.zeros((HKV, D, ld), np.int8)
    vs = np.zeros((HKV, D), np.float32)
    for t in lines:
        if t[0] == "qq":
            qq[int(t[1]), int(t[2]), int(t[3])] = int(t[4])
        elif t[0] == "kq":
            kq[int(t[1]), int(t[2]), int(t[3])] = int(t[4])
        elif t[0] == "k_scale_head0":
            ks[:, 0] = np.float32(float(t[1]))
        elif t[0] == "vq":
            vq[int(t[1]), int(t[2]), :] = [int(x) for x in t[3:]]
        elif t[0] == "v_scale":
            vs[int(t[1]), int(t[2])] = float(t[3])
        elif t[0] == "codes":
            ex["codes"][(int(t[1]), int(t[2]))] = [int(x) for x in t[3:]]
        elif t[0] == "out":
            for h in _heads(t[2]):
                ex["out"].append((int(t[1]), h, int(t[3]), int(t[4]) / int(t[5])))
        elif t[0] == "v":
            ex["v"][(int(t[1]), int(t[2]))] = [float(x) for x in t[3:]]
        elif t[0] == "vs":
            ex["vcol_scales"][(int(t[1]), int(t[2]))] = float(t[3])
        elif t[0] == "vcodes":
            ex["vcodes"][(int(t[1]), int(t[2]))] = [int(x) for x in t[3:]]
    ex.update(qq=qq, sq=np.ones((q_len, HQ), np.float32), kq=kq, ks=ks, vq=vq, vs=vs)
    return ex


def _run_example(ex):
    return oracle.attention_int8qkv(ex["qq"], ex["sq"], ex["kq"], ex["ks"], ex["vq"], ex["vs"])


# ----------------------------------------------------------------------------- golden

def test_golden_int8pv_hand_example():
    ex = load_example()
    out = _run_example(ex)
    expect = np.zeros_like(out)
    for t, h, f, val in ex["out"]:
        expect[t, h, f] = val
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-12)


def test_golden_int8pv_codes():
    ex = load_example()
    # the hand example's scores in natural units: s_j = d_j ln 2, key 5 masked for query 0
    d = ex["kq"][:, 0, 0].astype(np.float64)
    for (t, h), codes in ex["codes"].items():
        lim = ex["kv_len"] - ex["q_len"] + t
        s = np.where(np.arange(ex["kv_len"]) <= lim, d * math.log(2.0), -np.inf)[None, :]
        pq, _ = oracle.p_codes(s)
        np.testing.assert_array_equal(pq[0, :lim + 1], codes)
        assert np.all(pq[0, lim + 1:] == 0)


def test_golden_v_quantizer_hand_example():
    ex = load_example()
    n = ex["vquant_kv_len"]
    v = np.zeros((n, HKV, D), np.float32)
    for (g, f), vals in ex["v"].items():
        v[:, g, f] = vals
    vq, vs = oracle.quantize_v_int8(v)
    assert vq.shape == (HKV, D, n) and vq.dtype == np.int8 and vs.shape == (HKV, D)
    expect_q = np.zeros((HKV, D, n), np.int8)
    expect_s = np.zeros((HKV, D), np.float32)
    for (g, f), codes in ex["vcodes"].items():
        expect_q[g, f] = codes
        expect_s[g, f] = np.float32(ex["vcol_scales"][(g, f)])
    np.testing.assert_array_equal(vq, expect_q)
    np.testing.assert_array_equal(vs, expect_s)


# ----------------------------------------------------------------------------- closed forms

def _random_codes(q_len, kv_len, seed, ld=None):
    q, k, v, _ = make_qkv(q_len, kv_len, seed)
    qq, sq = oracle.quantize_rows_int8(q)
    kq, ks = oracle.quantize_rows_int8(k)
    vq, vs = oracle.quantize_v_int8(v)
    if ld is not None and ld > kv_len:
        pad = np.full((HKV, D, ld), 99, np.int8)
        pad[:, :, :kv_len] = vq
        vq = pad
    return qq, sq, kq, ks, vq, vs


def test_equal_scores_give_prefix_means():
    qq, sq, kq, ks, vq, vs = _random_codes(5, 13, seed=31)
    kq[:] = 0   # every score 0: every visible key gets code 127
    out = oracle.attention_int8qkv(qq, sq, kq, ks, vq, vs)
    csum = np.cumsum(vq.astype(np.float64), axis=2)   # [4, 256, kv_len]
    for i in range(5):
        n = 13 - 5 + i + 1
        for h in range(HQ):
            g = h // 6
            np.testing.assert_allclose(out[i, h], vs[g].astype(np.float64) * csum[g, :, n - 1] / n, rtol=0,
                                       atol=1e-12)


def test_row_that_sees_one_key_returns_its_value():
    qq, sq, kq, ks, vq, vs = _random_codes(4, 4, seed=32)   # no history: query 0 sees key 0
    out = oracle.attention_int8qkv(qq, sq, kq, ks, vq, vs)
    for h in range(HQ):
        np.testing.assert_allclose(out[0, h], vs[h // 6].astype(np.float64) * vq[h // 6, :, 0], rtol=0,
                                   atol=1e-12)


def test_positions_past_kv_len_are_not_read():
    a = _random_codes(7, 40, seed=33)
    b = _random_codes(7, 40, seed=33, ld=64)
    assert b[4].shape == (HKV, D, 64) and np.all(b[4][:, :, 40:] == 99)
    np.testing.assert_array_equal(oracle.attention_int8qkv(*a), oracle.attention_int8qkv(*b))


def test_within_code_rounding_bound_of_float_weights():
    # Pq = c + e with c = 127 exp(s - max s) and |e| <= 1/2, so against float attention
    # on the dequantised values (weights c / sum c) the output moves by at most
    # 0.5 sum_j |v_j - o_c| / sum_j Pq_j, and sum_j Pq_j >= sum_j c_j - n / 2.
    q_len, kv_len = 6, 50
    qq, sq, kq, ks, vq, vs = _random_codes(q_len, kv_len, seed=34)
    out = oracle.attention_int8qkv(qq, sq, kq, ks, vq, vs)
    vdeq = (vq.astype(np.float64) * vs[:, :, None].astype(np.float64)).transpose(2, 0, 1)
    ref = oracle.attention_int8(qq, sq, kq, ks, vdeq)
    worst = 0.0
    for i in range(q_len):
        n = kv_len - q_len + i + 1
        for h in range(HQ):
            g = h // 6
            s = oracle.score_matrix_int8k(qq.astype(np.float64), sq.astype(np.float64),
                                          kq.astype(np.float64), ks.astype(np.float64), h,
                                          np.array([i]), n)[0]
            c = 127.0 * np.exp(s - s.max())
            dev = np.abs(vdeq[:n, g, :] - ref[i, h][None, :]).sum(axis=0)
            bound = 0.5 * dev / (c.sum() - n / 2) + 1e-12
            err = np.abs(out[i, h] - ref[i, h])
            assert np.all(err <= bound), (i, h, float((err - bound).max()))
            worst = max(worst, float(err.max()))
    assert worst > 0.0   # the codes do round: the two differ


def test_code_slack_flags_only_keys_near_a_boundary():
    qq, sq, kq, ks, vq, vs = _random_codes(3, 30, seed=35)
    plain = oracle.attention_int8qkv(qq, sq, kq, ks, vq, vs)
    out0, slack0 = oracle.attention_int8qkv(qq, sq, kq, ks, vq, vs, code_slack=lambda c, t: 0.0 * c)
    np.testing.assert_array_equal(out0, plain)
    assert np.all(slack0 == 0.0)
    # a slack just under 1/2 makes nearly every key ambiguous (not the row maximum's: c = 127
    # lies exactly 1/2 from 126.5 and 127.5), so outputs get positive allowances
    _, slack = oracle.attention_int8qkv(qq, sq, kq, ks, vq, vs, code_slack=lambda c, t: 0.49 + 0.0 * c)
    assert np.all(slack[:, :, :] >= 0.0) and np.any(slack > 0.0)


# ----------------------------------------------------------------------------- planted mistakes

def _pin_battery():
    failed = []
    for name, fn in [("golden", test_golden_int8pv_hand_example),
                     ("prefix_means", test_equal_scores_give_prefix_means),
                     ("one_key", test_row_that_sees_one_key_returns_its_value),
                     ("padding", test_positions_past_kv_len_are_not_read),
                     ("bound", test_within_code_rounding_bound_of_float_weights)]:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_int8pv_pins_pass_on_the_real_oracle():
    assert _pin_battery() == []


@pytest.mark.parametrize("mutation", ["floor_codes", "sum_of_unrounded", "causal_exclusive",
                                      "causal_top_left", "v_token_major", "scale_of_other_head",
                                      "head_mod4"])
def test_int8pv_pins_catch_planted_mistakes(monkeypatch, mutation):
    m = int8pv_mod
    if mutation == "floor_codes":
        def floor_codes(s):
            mx = np.max(s, axis=1, keepdims=True)
            c = 127 * np.exp(s - mx)
            return np.floor(c), c
        monkeypatch.setattr(m, "p_codes", floor_codes)
    elif mutation == "sum_of_unrounded":
        def unrounded(s):
            mx = np.max(s, axis=1, keepdims=True)
            c = 127 * np.exp(s - mx)
            return c, c
        monkeypatch.setattr(m, "p_codes", unrounded)
    elif mutation == "causal_exclusive":
        monkeypatch.setattr(m, "causal_limit",
                            lambda i, q_len, kv_len: np.maximum(kv_len - q_len + np.asarray(i) - 1, 0))
    elif mutation == "causal_top_left":
        monkeypatch.setattr(m, "causal_limit", lambda i, q_len, kv_len: np.asarray(i))
    elif mutation == "v_token_major":
        real = m.attention_int8qkv

        def transposed(qq, q_scale, kq, k_scale, vq, v_scale, *a, **kw):
            vq = np.asarray(vq)
            n = vq.shape[2]
            flat = vq.reshape(HKV, -1)[:, :D * n].reshape(HKV, n, D).transpose(0, 2, 1)
            return real(qq, q_scale, kq, k_scale, np.ascontiguousarray(flat), v_scale, *a, **kw)
        monkeypatch.setattr(oracle, "attention_int8qkv", transposed)
    elif mutation == "scale_of_other_head":
        real = m.attention_int8qkv

        def wrong_scale(qq, q_scale, kq, k_scale, vq, v_scale, *a, **kw):
            return real(qq, q_scale, kq, k_scale, vq, np.asarray(v_scale)[::-1].copy(), *a, **kw)
        monkeypatch.setattr(oracle, "attention_int8qkv", wrong_scale)
    elif mutation == "head_mod4":
        monkeypatch.setattr(m, "kv_head_of", lambda h: h % 4)
    assert _pin_battery() != [], mutation
    assert prefill_mod.kv_head_of(7) == 1   # the other module is untouched
