"""Float64 oracle of attention with INT8 values and INT8 P·V (test infrastructure only).

See the package docstring for who may use it; pages are cited as [INT8 QK §n].

[INT8 QK §6] names INT8 PV (V held in INT8 and the P·V product in integers) among the
pieces of the pages' final submission and defines nothing more: neither the granularity
of V's scales nor how the softmax weights P become 8-bit integers. The reading taken here
is the plainest one whose result does not depend on how a kernel cuts the keys into
tiles or segments:

* V codes per (KV head, feature) over the whole sequence. The per-row quantiser of
  [INT8 QK §1, §4] (``quantize_rows_int8``: s = max|x| / 127 in float32, codes
  round-half-even(x / s) clamped to [-127, 127], a zero row gives s = 0) is applied to
  each (KV head, feature) column of V along the tokens:
  sV[g, f] = max_t |V[t, g, f]| / 127 and Vq[g, f, t] = round(V[t, g, f] / sV[g, f]).
  One scale per feature then factors out of the whole key reduction, so the product
  over any set of keys is one integer dot product.
  The codes are stored feature-major, [4, 256, ld] with ld >= kv_len (token index
  fastest): the layout the producer writes for this call.
* P codes against each row's exact maximum over its visible keys:
  Pq_ij = round-half-even(127 * exp(s_ij - max_j s_ij)), 0 for masked keys, so every
  code lies in [0, 127] and the largest weight of a row is exactly 127.
* o_i = sV * (sum_j Pq_ij * Vq_j) / (sum_j Pq_ij): the row sum is taken from the same
  codes as the numerator, as the bf16 path takes its row sum from the same rounded P.

The scores s_ij are those of the INT8-key path (``score_matrix_int8k``, [INT8 QK §1]).
Everything is float64 and exact where it can be: the integer sums stay below 2^53.
"""

from __future__ import annotations

import numpy as np

from .prefill import D, HKV, HQ, _as_f64, causal_limit, kv_head_of, quantize_rows_int8, \
    score_matrix_int8k

P_LEVELS = 127   # largest P code: the top of the symmetric INT8 range [INT8 QK §2.1]


def quantize_v_int8(v):
    """INT8 codes of V per (KV head, feature) over the tokens (the reading above).

    v: [kv_len, 4, 256] (bf16 values or floats). Returns (vq int8 [4, 256, kv_len],
    vs float32 [4, 256]) with vq[g, f, t] the code of v[t, g, f]: the per-row quantiser
    applied to each (g, f) column along the tokens.
    """
    if hasattr(v, "detach"):
        import torch

        v = v.detach().to("cpu", torch.float32).numpy()
    x = np.asarray(v, dtype=np.float32)
    if x.ndim != 3 or x.shape[1:] != (HKV, D):
        raise ValueError(f"v must be [kv_len, {HKV}, {D}], got {x.shape}")
    return quantize_rows_int8(np.ascontiguousarray(x.transpose(1, 2, 0)))


def p_codes(s):
    """P codes of a block of masked scores (natural units, masked entries -inf).

    Each row's maximum over its finite entries is subtracted, then
    Pq = round-half-even(127 * exp(s - max)); masked entries give 0. Returns
    (codes float64, the unrounded 127 * exp(s - max)).
    """
    m = np.max(s, axis=1, keepdims=True)
    c = P_LEVELS * np.exp(s - m)
    return np.rint(c), c


def attention_int8kv(q, kq, k_scale, vq, v_scale, rows=None, heads=None, chunk=256,
                     code_slack=None):
    """INT8 keys and INT8 values with the query rows quantised once [INT8 QK §4].

    q: [q_len, 24, 256] bf16 values, quantised by ``quantize_rows_int8``; the rest as in
    ``attention_int8qkv``.
    """
    qq, sq = quantize_rows_int8(q)
    return attention_int8qkv(qq, sq, kq, k_scale, vq, v_scale, rows, heads, chunk, code_slack)


def attention_int8qkv(qq, q_scale, kq, k_scale, vq, v_scale, rows=None, heads=None, chunk=256,
                      code_slack=None):
    """Causal GQA prefill attention on INT8 query, key and value codes (the reading above).

    qq int8 [q_len, 24, 256] with q_scale [q_len, 24]; kq int8 [kv_len, 4, 256] with
    k_scale [kv_len, 4]; vq int8 [4, 256, ld] (feature-major, ld >= kv_len; codes at
    token positions >= kv_len are never read) with v_scale [4, 256].
    ``rows`` / ``heads`` restrict the computation as in ``attention``.
    Returns float64 [len(rows), len(heads), 256].

    code_slack: optional function (c, tmax) -> delta, where c [n, nk] holds the unrounded
    127 * exp(s - max) of n rows and tmax [n] the largest |s| * log2(e) of each row over its
    visible keys. A P code whose c lies within delta of a rounding boundary (k + 1/2) may be
    rounded either way by an implementation that computes c to that accuracy; then the
    function also returns, per output element, the largest change that any such choice
    can make: sum over those keys of |sV * Vq_j - o| / (sum of codes - their count).
    """
    qq = _as_f64(qq)
    kqf = _as_f64(kq)
    ks = _as_f64(k_scale)
    sq = _as_f64(q_scale)
    vqf = _as_f64(vq)
    vs = _as_f64(v_scale)
    q_len, kv_len = qq.shape[0], kqf.shape[0]
    if qq.shape[1:] != (HQ, D) or sq.shape != (q_len, HQ):
        raise ValueError("bad query shapes for the INT8 P·V oracle")
    if kqf.shape[1:] != (HKV, D) or ks.shape != (kv_len, HKV) or q_len > kv_len:
        raise ValueError("bad key shapes for the INT8 P·V oracle")
    if vqf.ndim != 3 or vqf.shape[:2] != (HKV, D) or vqf.shape[2] < kv_len or vs.shape != (HKV, D):
        raise ValueError("bad value shapes for the INT8 P·V oracle")
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(HQ)) if heads is None else list(heads)
    out = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    slack = np.zeros_like(out) if code_slack is not None else None
    log2e = 1.0 / np.log(2.0)
    for hi, h in enumerate(heads):
        g = kv_head_of(h)
        for a in range(0, len(rows), chunk):
            idx = rows[a:a + chunk]
            lim = causal_limit(idx, q_len, kv_len)
            nk = int(lim.max()) + 1
            s = score_matrix_int8k(qq, sq, kqf, ks, h, idx, nk)
            masked = np.arange(nk)[None, :] > lim[:, None]
            s = np.where(masked, -np.inf, s)
            pq, c = p_codes(s)
            l = pq.sum(axis=1)
            vcol = vqf[g, :, :nk]                                   # [256, nk] codes
            o = (pq @ vcol.T) * vs[g][None, :] / l[:, None]
            out[a:a + len(idx), hi, :] = o
            if code_slack is not None:
                tmax = np.max(np.where(masked, 0.0, np.abs(s)), axis=1) * log2e
                delta = code_slack(c, tmax)
                amb = (~masked) & (np.abs(c - (np.floor(c) + 0.5)) <= delta)
                for r in np.nonzero(amb.any(axis=1))[0]:
                    js = np.nonzero(amb[r])[0]
                    denom = l[r] - len(js)
                    dev = np.abs(vcol[:, js].T * vs[g][None, :] - o[r][None, :]).sum(axis=0)
                    slack[a + r, hi, :] = dev / denom if denom > 0 else np.inf
    return (out, slack) if code_slack is not None else out
