"""Plain float64 causal GQA prefill attention (the oracle's arithmetic).

Test infrastructure only; see the package docstring for who may use it and for
the page titles cited below as [DCU report §n] and [INT8 QK §n].

Definition (restated from the pages, not copied):

* shape: 24 query heads, 4 KV heads, head_dim 256, so each KV head serves six
  consecutive query heads, kv = h // 6 [DCU report §1], [INT8 QK §5.2];
* score s_ij = (q_i · k_j) / sqrt(256) = (q_i · k_j) / 16 [INT8 QK §1];
* chunked prefill with history: the q_len new queries are the last q_len
  positions of a kv_len-long sequence, so query i sits at position
  kv_len - q_len + i and sees keys 0 .. kv_len - q_len + i (inclusive)
  [DCU report §2 "causal mask"; the dispatch in §3 is keyed on the real
  q_len and kv_len of a chunk];
* weights p_ij = exp(s_ij - max_j s) / sum_j exp(s_ij - max_j s) over the
  visible keys, output o_i = sum_j p_ij v_j [DCU report §2].

The implementation is the definition written out with NumPy: one matmul for
the scores, an explicit boolean mask, a plain softmax, one matmul for the
output, per (query head, chunk of query rows). No blocking over keys, no online
softmax, no fusion.
"""

from __future__ import annotations

import numpy as np

HQ = 24          # query heads [DCU report §1]
HKV = 4          # KV heads [DCU report §1]
D = 256          # head_dim [DCU report §1]
GROUP = HQ // HKV  # GQA ratio 6
SCALE = 1.0 / 16.0  # 1/sqrt(head_dim) [INT8 QK §1]
BLOCK_SIZE = 16  # tokens per paged-cache block (paged layout [block, kv_head, 16, 256])


def kv_head_of(h: int) -> int:
    """KV head serving query head ``h``: consecutive groups of six [INT8 QK §5.2]."""
    return h // GROUP


def causal_limit(i, q_len: int, kv_len: int):
    """Index of the last key visible to query ``i`` of a chunk (inclusive).

    Query i sits at position kv_len - q_len + i of the sequence; it sees its own
    position and everything before it [DCU report §2].
    """
    return kv_len - q_len + np.asarray(i)


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (bf16 included): exact widening
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 3 or q.shape[1:] != (HQ, D):
        raise ValueError(f"q must be [q_len, {HQ}, {D}], got {q.shape}")
    if k.ndim != 3 or k.shape[1:] != (HKV, D) or v.shape != k.shape:
        raise ValueError(f"k and v must be [kv_len, {HKV}, {D}], got {k.shape} {v.shape}")
    if q.shape[0] > k.shape[0]:
        raise ValueError("q_len must not exceed kv_len")


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of a score block whose masked entries hold -inf."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=1, keepdims=True)


def _attend(score_fn, v, q_len, kv_len, rows, heads, chunk, return_weights):
    """Shared driver: masked softmax over scores from ``score_fn(h, rows)``, then PV.

    ``score_fn(h, idx)`` returns the float64 scores of query rows ``idx`` against
    keys 0 .. max visible key of those rows, already multiplied by the softmax
    scale.
    """
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(HQ)) if heads is None else list(heads)
    out = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    weights = {} if return_weights else None
    for hi, h in enumerate(heads):
        g = kv_head_of(h)
        for a in range(0, len(rows), chunk):
            idx = rows[a:a + chunk]
            lim = causal_limit(idx, q_len, kv_len)          # [n]
            nk = int(lim.max()) + 1
            s = score_fn(h, idx, nk)                          # [n, nk]
            keys = np.arange(nk)
            s = np.where(keys[None, :] > lim[:, None], -np.inf, s)
            p = _softmax_rows(s)
            out[a:a + len(idx), hi, :] = p @ v[:nk, g, :]
            if return_weights:
                full = np.zeros((len(idx), kv_len))
                full[:, :nk] = p
                for r, i in enumerate(idx):
                    weights[(int(i), h)] = full[r]
    return (out, weights) if return_weights else out


def score_matrix(q, k, h: int, idx=None, nk=None) -> np.ndarray:
    """Unmasked scores (q_i · k_j) / 16 of query head ``h`` [INT8 QK §1].

    q: [q_len, 24, 256], k: [kv_len, 4, 256] as float64 arrays; ``idx`` selects
    query rows, ``nk`` keeps keys 0 .. nk-1. Returns [len(idx), nk].
    """
    idx = np.arange(q.shape[0]) if idx is None else idx
    nk = k.shape[0] if nk is None else nk
    g = kv_head_of(h)
    return (q[idx, h, :] @ k[:nk, g, :].T) * SCALE


def attention(q, k, v, rows=None, heads=None, chunk=256, return_weights=False):
    """Causal GQA prefill attention in float64.

    q: [q_len, 24, 256]; k, v: [kv_len, 4, 256] (contiguous, logical order).
    Values are taken exactly (bf16 tensors are widened without rounding).
    ``rows`` / ``heads`` restrict the computation to those query indices /
    query heads (the result of any row does not depend on the others).
    Returns float64 [len(rows), len(heads), 256]; with ``return_weights`` also a
    dict {(i, h): p_i over all kv_len keys}.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check_shapes(q, k, v)
    q_len, kv_len = q.shape[0], k.shape[0]

    def scores(h, idx, nk):
        return score_matrix(q, k, h, idx, nk)

    return _attend(scores, v, q_len, kv_len, rows, heads, chunk, return_weights)


def gather_paged(cache, block_table, kv_len: int) -> np.ndarray:
    """Logical K (or V) [kv_len, 4, 256] read back from a paged cache.

    cache: [num_blocks, 4, 16, 256]; block_table: int [ceil(kv_len/16)].
    Logical key t lives in physical block block_table[t // 16] at slot t % 16
    [INT8 QK §3: block table -> physical block -> slot in the page].
    """
    cache = _as_f64(cache)
    bt = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                    dtype=np.int64)
    nb, hkv, bs, d = cache.shape
    if (hkv, bs, d) != (HKV, BLOCK_SIZE, D):
        raise ValueError(f"paged cache must be [blocks, {HKV}, {BLOCK_SIZE}, {D}]")
    out = np.empty((kv_len, HKV, D), dtype=np.float64)
    for t in range(kv_len):
        blk = bt[t // BLOCK_SIZE]
        if not 0 <= blk < nb:
            raise IndexError(f"block table entry {blk} out of range for {nb} blocks")
        out[t] = cache[blk, :, t % BLOCK_SIZE, :]
    return out


def gather_paged_int8_splitd(cache, block_table, kv_len: int) -> np.ndarray:
    """Logical INT8 K codes [kv_len, 4, 256] read back from the split-d paged cache.

    cache: [num_blocks, 4, 256 / 16, 16, 16] -- per (block, KV head) the 256 features
    of its 16 slots are stored as 16 chunks of 16 features, chunk-major, so that a
    chunk of all 16 slots is contiguous [INT8 QK §3: K cache [block, kv_head,
    head_dim / 16, block_size, 16]]. Feature f of logical key t, KV head h is
    cache[block_table[t // 16], h, f // 16, t % 16, f % 16]. Codes are returned in
    the cache's dtype (exact).
    """
    cache = np.asarray(cache.cpu() if hasattr(cache, "cpu") else cache)
    bt = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                    dtype=np.int64)
    nb = cache.shape[0]
    if cache.shape[1:] != (HKV, D // 16, BLOCK_SIZE, 16):
        raise ValueError(f"split-d cache must be [blocks, {HKV}, {D // 16}, {BLOCK_SIZE}, 16]")
    out = np.empty((kv_len, HKV, D), dtype=cache.dtype)
    for t in range(kv_len):
        blk = bt[t // BLOCK_SIZE]
        if not 0 <= blk < nb:
            raise IndexError(f"block table entry {blk} out of range for {nb} blocks")
        slot = t % BLOCK_SIZE
        for h in range(HKV):
            for c in range(D // 16):
                out[t, h, 16 * c:16 * c + 16] = cache[blk, h, c, slot, :]
    return out


def gather_paged_scales(scale_cache, block_table, kv_len: int) -> np.ndarray:
    """Per-token key scales [kv_len, 4] read back from a paged scale cache [num_blocks,
    4, 16]: the scale of logical key t, KV head h is scale_cache[block_table[t // 16],
    h, t % 16] (the scales live in the same pages as their keys' codes)."""
    sc = np.asarray(scale_cache.cpu() if hasattr(scale_cache, "cpu") else scale_cache)
    bt = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                    dtype=np.int64)
    nb = sc.shape[0]
    if sc.shape[1:] != (HKV, BLOCK_SIZE):
        raise ValueError(f"paged scale cache must be [blocks, {HKV}, {BLOCK_SIZE}]")
    out = np.empty((kv_len, HKV), dtype=sc.dtype)
    for t in range(kv_len):
        blk = bt[t // BLOCK_SIZE]
        if not 0 <= blk < nb:
            raise IndexError(f"block table entry {blk} out of range for {nb} blocks")
        out[t] = sc[blk, :, t % BLOCK_SIZE]
    return out


def quantize_rows_int8(x):
    """Symmetric dynamic INT8 quantisation of each 256-element row [INT8 QK §1, §4].

    s = max|x| / 127 and xq = round(x / s), clamped to [-127, 127] (the range of
    [INT8 QK §2.1]). The page leaves "round" and the arithmetic open; this
    oracle fixes them as: float32 arithmetic, max|x| exact, s = fl32(max|x| / 127)
    by IEEE division, xq = round-half-to-even(fl32(x / s)). A row of zeros has
    s = 0 and xq = 0 (so its scores are 0).
    Returns (xq int8 [..., 256], s float32 [...]).
    """
    if hasattr(x, "detach"):
        import torch

        x = x.detach().to("cpu", torch.float32).numpy()
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = (x32 / s[..., None]).astype(np.float32)
    r = np.where(s[..., None] == 0, np.float32(0.0), r)
    xq = np.clip(np.rint(r), -127, 127).astype(np.int8)
    return xq, s


def score_matrix_int8k(qq, sq, kq, k_scale, h: int, idx=None, nk=None) -> np.ndarray:
    """Scores of query head ``h`` from INT8 codes [INT8 QK §1].

    The integer dot product Qq·Kqᵀ (exact: every partial sum is an integer of
    magnitude at most 256·127·127, far inside float64's exact range) times
    sQ(query token, query head) · sK(key token, kv head) · 1/16, restored per
    score before any softmax. qq: [q_len, 24, 256] codes, sq: [q_len, 24],
    kq: [kv_len, 4, 256] codes, k_scale: [kv_len, 4]; all float64 arrays.
    """
    idx = np.arange(qq.shape[0]) if idx is None else idx
    nk = kq.shape[0] if nk is None else nk
    g = kv_head_of(h)
    s_int = qq[idx, h, :] @ kq[:nk, g, :].T
    return s_int * sq[idx, h][:, None] * k_scale[:nk, g][None, :] * SCALE


def attention_int8k(q, kq, k_scale, v, rows=None, heads=None, chunk=256,
                    return_weights=False):
    """Causal GQA prefill attention with INT8 keys [INT8 QK §1, §4].

    q: [q_len, 24, 256] (bf16 values); kq: int8 [kv_len, 4, 256];
    k_scale: float32 [kv_len, 4] (one scale per key token and KV head);
    v: [kv_len, 4, 256]. Each query row (token, head) is quantised once with
    ``quantize_rows_int8`` [INT8 QK §4: the query is quantised once, before the
    attention], then ``attention_int8`` runs on the codes.
    """
    qq, sq = quantize_rows_int8(q)
    return attention_int8(qq, sq, kq, k_scale, v, rows, heads, chunk, return_weights)


def attention_int8(qq, q_scale, kq, k_scale, v, rows=None, heads=None, chunk=256,
                   return_weights=False):
    """Causal GQA prefill attention on INT8 query and key codes [INT8 QK §1, §4].

    The form the pages arrive at in [INT8 QK §4], where the producer of Q has
    already quantised each query row: qq int8 [q_len, 24, 256] with q_scale
    float32 [q_len, 24], kq int8 [kv_len, 4, 256] with k_scale [kv_len, 4], and
    v [kv_len, 4, 256]. Scores come from ``score_matrix_int8k``; the rest is as
    in ``attention``. The codes need not come from ``quantize_rows_int8``.
    """
    qq = _as_f64(qq)
    kqf = _as_f64(kq)
    ks = _as_f64(k_scale)
    v = _as_f64(v)
    q_len, kv_len = qq.shape[0], kqf.shape[0]
    if qq.shape[1:] != (HQ, D) or kqf.shape[1:] != (HKV, D) or ks.shape != (kv_len, HKV):
        raise ValueError("bad shapes for the INT8-K oracle")
    if v.shape != (kv_len, HKV, D) or q_len > kv_len:
        raise ValueError("bad shapes for the INT8-K oracle")
    sq64 = _as_f64(q_scale)
    if sq64.shape != (q_len, HQ):
        raise ValueError("bad shapes for the INT8-K oracle")

    def scores(h, idx, nk):
        return score_matrix_int8k(qq, sq64, kqf, ks, h, idx, nk)

    return _attend(scores, v, q_len, kv_len, rows, heads, chunk, return_weights)
