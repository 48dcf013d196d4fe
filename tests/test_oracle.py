"""Pins of the CPU oracle against facts it does not define itself.

Each test checks the oracle against something other than its own formula:
hand-derived worked examples (tests/golden, each with its citation), brute
force on tiny inputs, closed forms (constant V, zero Q, saturation), invariants
(softmax weights, causal perturbation, chunk consistency, GQA symmetry), a
library routine (torch's scaled_dot_product_attention in float64) and the
INT8 bound printed by the INT8 QK page (§2.1). The mutation tests at the end
plant plausible mistakes in the oracle and check that the pins catch them.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import prefill as oracle_attention_mod
from gqa_synth import make_qkv, scatter_paged, block_table_for, HQ, HKV, D

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- golden parsers

def load_attention_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "attention_hand_examples.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                q_len, kv_len = int(tok[2]), int(tok[3])
                cur = dict(name=tok[1],
                           q=np.zeros((q_len, HQ, D)), k=np.zeros((kv_len, HKV, D)),
                           v=np.zeros((kv_len, HKV, D)), expect=np.zeros((q_len, HQ, D)))
            elif tok[0] == "end":
                cases.append(cur)
                cur = None
            else:
                t, h, d = int(tok[1]), int(tok[2]), int(tok[3])
                cur[tok[0]][t, h, d] = float(tok[4])
    return cases


def load_quant_rows():
    rows, bound, cur = [], None, None
    with open(os.path.join(GOLDEN, "quantize_int8_hand_examples.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "row":
                cur = dict(x=np.zeros(D, np.float32), xq=np.zeros(D, np.int8), s=None)
            elif tok[0] == "x":
                cur["x"][int(tok[1])] = float(tok[2])
            elif tok[0] == "xq":
                cur["xq"][int(tok[1])] = int(tok[2])
            elif tok[0] == "s":
                cur["s"] = float(tok[1])
            elif tok[0] == "end":
                rows.append(cur)
            elif tok[0] == "int32_dot_bound":
                bound = int(tok[1])
    return rows, bound


def load_gather_example():
    spec = {"keys": []}
    with open(os.path.join(GOLDEN, "paged_gather_hand_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "kv_len":
                spec["kv_len"] = int(tok[1])
            elif tok[0] == "num_blocks":
                spec["num_blocks"] = int(tok[1])
            elif tok[0] == "block_table":
                spec["block_table"] = [int(x) for x in tok[1:]]
            elif tok[0] == "key":
                spec["keys"].append((int(tok[1]), int(tok[3]), int(tok[5])))
    return spec


def f64(x):
    return x.to(torch.float64).numpy()


# ----------------------------------------------------------------------------- golden examples

@pytest.mark.parametrize("case", load_attention_cases(), ids=lambda c: c["name"])
def test_golden_attention_hand_examples(case):
    out = oracle.attention(case["q"], case["k"], case["v"])
    np.testing.assert_allclose(out, case["expect"], rtol=0, atol=1e-12)


def test_golden_quantizer_hand_examples():
    rows, _ = load_quant_rows()
    x = np.stack([r["x"] for r in rows])
    xq, s = oracle.quantize_rows_int8(x)
    for r, row in enumerate(rows):
        assert s[r] == np.float32(row["s"]), (r, s[r], row["s"])
        np.testing.assert_array_equal(xq[r], row["xq"])


def test_golden_int32_bound_from_page():
    _, bound = load_quant_rows()
    assert bound == 256 * 127 * 127
    # the extreme rows reach it exactly, and the INT8 score path keeps it exact
    qq = np.full((1, HQ, D), 127.0)
    kq = np.full((1, HKV, D), -127.0)
    s = oracle.score_matrix_int8k(qq, np.ones((1, HQ)), kq, np.ones((1, HKV)), h=0)
    assert s[0, 0] * 16 == -bound
    assert bound < 2**31 - 1


def test_golden_paged_gather_hand_example():
    spec = load_gather_example()
    nb, kv_len = spec["num_blocks"], spec["kv_len"]
    # a cache whose every entry encodes (block, kv head, slot, dim)
    code = (np.arange(nb)[:, None, None, None] * 1e6 + np.arange(HKV)[None, :, None, None] * 1e5
            + np.arange(16)[None, None, :, None] * 1e3 + np.arange(D)[None, None, None, :])
    got = oracle.gather_paged(code, np.array(spec["block_table"]), kv_len)
    for t, blk, slot in spec["keys"]:
        np.testing.assert_array_equal(got[t], code[blk, :, slot, :])
    assert len(spec["keys"]) == kv_len


def load_splitd_example():
    spec = {"k": [], "s": []}
    with open(os.path.join(GOLDEN, "paged_int8_splitd_hand_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] in ("kv_len", "num_blocks"):
                spec[tok[0]] = int(tok[1])
            elif tok[0] == "block_table":
                spec["block_table"] = [int(x) for x in tok[1:]]
            elif tok[0] == "k":
                spec["k"].append(tuple(int(x) for x in tok[1:]))
            elif tok[0] == "s":
                spec["s"].append(tuple(int(x) for x in tok[1:]))
    return spec


def test_golden_paged_int8_splitd_hand_example():
    """INT8 QK §3's split-d paged K layout and the paged scales, against positions
    worked out by hand."""
    spec = load_splitd_example()
    nb, kv_len, bt = spec["num_blocks"], spec["kv_len"], np.array(spec["block_table"])
    b, h, c, sl, e = np.meshgrid(np.arange(nb), np.arange(HKV), np.arange(D // 16), np.arange(16),
                                 np.arange(16), indexing="ij")
    kcache = b * 65536 + h * 4096 + c * 256 + sl * 16 + e
    b2, h2, s2 = np.meshgrid(np.arange(nb), np.arange(HKV), np.arange(16), indexing="ij")
    scache = (b2 * 100 + h2 * 10 + s2).astype(np.float64)
    k = oracle.gather_paged_int8_splitd(kcache, bt, kv_len)
    sc = oracle.gather_paged_scales(scache, bt, kv_len)
    assert k.shape == (kv_len, HKV, D) and sc.shape == (kv_len, HKV)
    for t, hh, f, want in spec["k"]:
        assert k[t, hh, f] == want, (t, hh, f)
    for t, hh, want in spec["s"]:
        assert sc[t, hh] == want, (t, hh)


def test_splitd_gather_equals_rowmajor_gather():
    """The split-d cache holds the same rows as a [block, head, slot, 256] cache whose row
    (block, head, slot) is the concatenation of its 16 chunks; both gathers agree."""
    rng = np.random.default_rng(7)
    nb, kv_len = 6, 83
    kc = rng.integers(-127, 128, (nb, HKV, D // 16, 16, 16)).astype(np.int8)
    rows = np.zeros((nb, HKV, 16, D), np.int8)
    for c in range(D // 16):
        rows[:, :, :, 16 * c:16 * c + 16] = kc[:, :, c, :, :]
    bt = rng.permutation(nb)
    got = oracle.gather_paged_int8_splitd(kc, bt, kv_len)
    want = oracle.gather_paged(rows, bt, kv_len)
    assert got.dtype == np.int8
    np.testing.assert_array_equal(got.astype(np.float64), want)


def test_splitd_generator_round_trip():
    """The input generator's split-d placement is what the oracle's gather reads back,
    and every scale slot the keys do not use is NaN."""
    from gqa_synth import scatter_paged_int8_splitd, scatter_paged_scales
    rng = np.random.default_rng(8)
    kv_len, nb = 37, 5
    kq = torch.from_numpy(rng.integers(-127, 128, (kv_len, HKV, D)).astype(np.int8))
    ks = torch.from_numpy(rng.random((kv_len, HKV), dtype=np.float32))
    bt = block_table_for(rng, kv_len, nb)
    kc, sc = scatter_paged_int8_splitd(kq, bt, nb), scatter_paged_scales(ks, bt, nb)
    assert kc.shape == (nb, HKV, D // 16, 16, 16) and kc.dtype == torch.int8
    np.testing.assert_array_equal(oracle.gather_paged_int8_splitd(kc, bt, kv_len), kq.numpy())
    np.testing.assert_array_equal(oracle.gather_paged_scales(sc, bt, kv_len), ks.numpy())
    assert int(torch.isnan(sc).sum()) == (nb * 16 - kv_len) * HKV


# ----------------------------------------------------------------------------- brute force

def brute_force(q, k, v):
    """Scalar loops over the statement: query i at position kv_len-q_len+i sees keys
    0..that position; head h reads KV head h//6; score = dot/sqrt(256)."""
    q_len, kv_len = len(q), len(k)
    out = [[[0.0] * D for _ in range(HQ)] for _ in range(q_len)]
    for i in range(q_len):
        pos = kv_len - q_len + i
        for h in range(HQ):
            g = h // (HQ // HKV)
            sc = []
            for j in range(pos + 1):
                acc = 0.0
                for d in range(D):
                    acc += q[i][h][d] * k[j][g][d]
                sc.append(acc / math.sqrt(D))
            top = max(sc)
            w = [math.exp(x - top) for x in sc]
            z = math.fsum(w)
            for d in range(D):
                out[i][h][d] = math.fsum(w[j] * v[j][g][d] for j in range(pos + 1)) / z
    return np.array(out)


@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (3, 3), (3, 8), (7, 7), (7, 12)])
def test_brute_force_tiny(q_len, kv_len):
    q, k, v, _ = make_qkv(q_len, kv_len, seed=100 + 10 * q_len + kv_len)
    want = brute_force(f64(q).tolist(), f64(k).tolist(), f64(v).tolist())
    got = oracle.attention(q, k, v)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- invariants / closed forms

def test_weights_sum_to_one_and_respect_causality():
    q, k, v, _ = make_qkv(5, 11, seed=7)
    _, w = oracle.attention(q, k, v, return_weights=True)
    for (i, h), p in w.items():
        lim = 11 - 5 + i
        assert abs(p.sum() - 1.0) < 1e-12
        assert np.all(p[lim + 1:] == 0.0)
        assert np.all(p[:lim + 1] > 0.0)


def test_constant_v_gives_v():
    q, k, _, _ = make_qkv(6, 9, seed=8)
    c = np.random.default_rng(0).standard_normal((HKV, D))
    v = np.broadcast_to(c, (9, HKV, D)).copy()
    out = oracle.attention(q, k, v)
    for h in range(HQ):
        np.testing.assert_allclose(out[:, h, :], np.broadcast_to(c[h // 6], (6, D)), atol=1e-12)


def test_zero_q_is_prefix_mean():
    _, k, v, _ = make_qkv(4, 10, seed=9)
    q = np.zeros((4, HQ, D))
    out = oracle.attention(q, k, v)
    vv = f64(v)
    for i in range(4):
        lim = 10 - 4 + i
        for h in range(HQ):
            np.testing.assert_allclose(out[i, h], vv[:lim + 1, h // 6].mean(axis=0), atol=1e-12)


def test_causal_perturbation_leaves_earlier_rows_unchanged():
    q, k, v, _ = make_qkv(6, 14, seed=10)
    for i in range(6):
        lim = 14 - 6 + i
        base = oracle.attention(q, k, v, rows=[i])
        k2, v2 = f64(k).copy(), f64(v).copy()
        k2[lim + 1:] += 5.0
        v2[lim + 1:] -= 3.0
        pert = oracle.attention(q, k2, v2, rows=[i])
        np.testing.assert_array_equal(pert, base)


def test_first_row_of_square_chunk_is_v0():
    q, k, v, _ = make_qkv(5, 5, seed=11)
    out = oracle.attention(q, k, v)
    vv = f64(v)
    for h in range(HQ):
        np.testing.assert_array_equal(out[0, h], vv[0, h // 6])


def test_chunk_consistency():
    """Full causal attention over N tokens equals the concatenation of chunked calls."""
    n = 40
    q, k, v, _ = make_qkv(n, n, seed=12)
    full = oracle.attention(q, k, v)
    parts = []
    for a, b in [(0, 13), (13, 29), (29, 40)]:
        parts.append(oracle.attention(q[a:b], k[:b], v[:b]))
    np.testing.assert_allclose(np.concatenate(parts), full, rtol=0, atol=1e-13)


def test_gqa_equal_heads_and_permutation():
    q, k, v, _ = make_qkv(4, 7, seed=13)
    qq = f64(q).copy()
    for g in range(HKV):
        qq[:, 6 * g:6 * g + 6] = qq[:, 6 * g:6 * g + 1]
    out = oracle.attention(qq, k, v)
    for g in range(HKV):
        for h in range(6 * g + 1, 6 * g + 6):
            np.testing.assert_array_equal(out[:, h], out[:, 6 * g])
    # permuting KV heads together with their query groups permutes the outputs
    perm = [2, 0, 3, 1]
    qp = np.concatenate([f64(q)[:, 6 * p:6 * p + 6] for p in perm], axis=1)
    kp, vp = f64(k)[:, perm], f64(v)[:, perm]
    base = oracle.attention(q, k, v)
    got = oracle.attention(qp, kp, vp)
    want = np.concatenate([base[:, 6 * p:6 * p + 6] for p in perm], axis=1)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_softmax_saturation_picks_the_dominant_key():
    """A score 1000 above all others puts all the weight on that key (needs max-subtraction)."""
    kv_len = 6
    k = np.zeros((kv_len, HKV, D))
    for j in range(kv_len):
        k[j, :, j] = 1.0
    v = np.random.default_rng(1).standard_normal((kv_len, HKV, D))
    q = np.zeros((1, HQ, D))
    q[0, :, 3] = 16000.0          # score 1000 on key 3, 0 on the others
    out = oracle.attention(q, k, v)
    assert np.all(np.isfinite(out))
    for h in range(HQ):
        np.testing.assert_allclose(out[0, h], v[3, h // 6], rtol=0, atol=1e-300)


def test_textbook_sdpa_reduction():
    """q_len == kv_len: standard causal GQA attention as torch computes it in float64."""
    n = 33
    q, k, v, _ = make_qkv(n, n, seed=14)
    got = oracle.attention(q, k, v)
    qt = q.to(torch.float64).permute(1, 0, 2)[None]
    kt = k.to(torch.float64).permute(1, 0, 2)[None]
    vt = v.to(torch.float64).permute(1, 0, 2)[None]
    try:
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                               enable_gqa=True)
    except TypeError:  # older torch: expand the groups by hand
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.repeat_interleave(6, dim=1), vt.repeat_interleave(6, dim=1), is_causal=True)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- paged

def test_paged_gather_reproduces_contiguous():
    rng = np.random.default_rng(3)
    _, k, v, _ = make_qkv(1, 70, seed=15)
    bt = block_table_for(rng, 70, num_blocks=9)
    kc, vc = scatter_paged(k, bt, 9), scatter_paged(v, bt, 9)
    np.testing.assert_array_equal(oracle.gather_paged(kc, bt, 70), f64(k))
    np.testing.assert_array_equal(oracle.gather_paged(vc, bt, 70), f64(v))


# ----------------------------------------------------------------------------- INT8

def test_quantizer_properties():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, D)).astype(np.float32) * rng.uniform(0.01, 50, (64, 1)).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    xq, s = oracle.quantize_rows_int8(x)
    assert xq.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(xq.astype(np.int32)) <= 127)
    # the largest element of each row maps to +/-127
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(xq[np.arange(64), am].astype(np.int32)) == 127)
    # reconstruction error at most half a step (plus float32 slack)
    err = np.abs(xq.astype(np.float64) * s[:, None] - x)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))


def test_int8_reduces_to_float_when_quantisation_is_exact():
    """Integer-valued Q rows with max 127 and K rows that are integers times 2^-3 with
    max 127*2^-3 are quantised exactly, so INT8-K attention equals float attention."""
    rng = np.random.default_rng(5)
    q_len, kv_len = 5, 12
    q = rng.integers(-120, 121, (q_len, HQ, D)).astype(np.float64)
    q[:, :, 0] = 127.0
    kint = rng.integers(-120, 121, (kv_len, HKV, D)).astype(np.float64)
    kint[:, :, 1] = -127.0
    k = kint * 0.125
    v = rng.standard_normal((kv_len, HKV, D))
    kq, ks = oracle.quantize_rows_int8(k)
    assert np.all(ks == np.float32(0.125))
    np.testing.assert_array_equal(kq.astype(np.float64) * ks[..., None].astype(np.float64), k)
    got = oracle.attention_int8k(q, kq, ks, v)
    want = oracle.attention(q, k, v)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_int8_codes_reduce_to_float_attention_on_dequantised_values():
    """attention_int8 on arbitrary codes and float32 scales (not the quantiser's) equals
    float attention on Qq·sQ and Kq·sK: the products are exact in float64, so only the
    order of the score arithmetic differs."""
    rng = np.random.default_rng(18)
    q_len, kv_len = 6, 23
    qq = rng.integers(-127, 128, (q_len, HQ, D)).astype(np.int8)
    kq = rng.integers(-127, 128, (kv_len, HKV, D)).astype(np.int8)
    sq = (rng.random((q_len, HQ)) * 0.02 + 1e-3).astype(np.float32)
    ks = (rng.random((kv_len, HKV)) * 0.02 + 1e-3).astype(np.float32)
    sq[2, 7] = 0.0   # a zero row: uniform weights over its keys
    v = rng.standard_normal((kv_len, HKV, D))
    got = oracle.attention_int8(qq, sq, kq, ks, v)
    q = qq.astype(np.float64) * sq[..., None].astype(np.float64)
    k = kq.astype(np.float64) * ks[..., None].astype(np.float64)
    np.testing.assert_allclose(got, oracle.attention(q, k, v), rtol=0, atol=1e-12)
    off = kv_len - q_len
    np.testing.assert_allclose(got[2, 7], v[:off + 3, 1].mean(0), atol=1e-12)
    # the quantising form is this one on the quantiser's codes
    qb, kb, vb, _ = make_qkv(4, 30, seed=19)
    kq2, ks2 = oracle.quantize_rows_int8(kb)
    qq2, sq2 = oracle.quantize_rows_int8(qb)
    np.testing.assert_array_equal(oracle.attention_int8k(qb, kq2, ks2, vb),
                                  oracle.attention_int8(qq2, sq2, kq2, ks2, vb))


def test_int8_scores_within_closed_form_bound():
    """|Sq - S| <= (sQ/2) sum|k| + (sK/2) sum|q| + 256 sQ sK / 4, all over 16."""
    q, k, _, _ = make_qkv(6, 20, seed=16)
    qf, kf = f64(q), f64(k)
    qq, sq = oracle.quantize_rows_int8(q)
    kq, ks = oracle.quantize_rows_int8(k)
    for h in (0, 5, 6, 13, 23):
        g = h // 6
        s_exact = oracle.score_matrix(qf, kf, h)
        s_int8 = oracle.score_matrix_int8k(qq.astype(np.float64), sq.astype(np.float64),
                                           kq.astype(np.float64), ks.astype(np.float64), h)
        bound = ((sq[:, h, None] / 2) * np.abs(kf[:, g]).sum(-1)[None, :]
                 + (ks[None, :, g] / 2) * np.abs(qf[:, h]).sum(-1)[:, None]
                 + D * sq[:, h, None] * ks[None, :, g] / 4) / 16
        assert np.all(np.abs(s_int8 - s_exact) <= bound * (1 + 1e-6))
        # the integer part really is an integer of bounded size
        s_int = s_int8 * 16 / (sq[:, h, None].astype(np.float64) * ks[None, :, g])
        assert np.all(np.abs(s_int - np.rint(s_int)) < 1e-6)
        assert np.all(np.abs(s_int) <= 256 * 127 * 127)


def test_int8_zero_query_row_gives_uniform_weights():
    _, k, v, _ = make_qkv(3, 9, seed=17)
    kq, ks = oracle.quantize_rows_int8(k)
    q = np.zeros((3, HQ, D))
    out = oracle.attention_int8k(q, kq, ks, v)
    vv = f64(v)
    for i in range(3):
        for h in range(HQ):
            np.testing.assert_allclose(out[i, h], vv[:9 - 3 + i + 1, h // 6].mean(0), atol=1e-12)


# ----------------------------------------------------------------------------- planted mistakes

def _pin_battery():
    """Run a subset of the pins; return the names of those that fail."""
    failed = []
    for case in load_attention_cases():
        out = oracle.attention(case["q"], case["k"], case["v"])
        if not np.allclose(out, case["expect"], rtol=0, atol=1e-9):
            failed.append("golden_" + case["name"])
    try:
        test_textbook_sdpa_reduction()
    except AssertionError:
        failed.append("sdpa")
    try:
        test_chunk_consistency()
    except AssertionError:
        failed.append("chunk")
    return failed


def test_pins_pass_on_the_real_oracle():
    assert _pin_battery() == []


@pytest.mark.parametrize("mutation", ["head_mod4", "scale_128", "causal_top_left",
                                      "causal_exclusive"])
def test_pins_catch_planted_mistakes(monkeypatch, mutation):
    m = oracle_attention_mod
    if mutation == "head_mod4":
        monkeypatch.setattr(m, "kv_head_of", lambda h: h % 4)
    elif mutation == "scale_128":
        monkeypatch.setattr(m, "SCALE", 1.0 / math.sqrt(128))
    elif mutation == "causal_top_left":
        monkeypatch.setattr(m, "causal_limit", lambda i, q_len, kv_len: np.asarray(i))
    elif mutation == "causal_exclusive":
        monkeypatch.setattr(m, "causal_limit",
                            lambda i, q_len, kv_len: np.maximum(kv_len - q_len + np.asarray(i) - 1, 0))
    assert _pin_battery() != [], mutation
