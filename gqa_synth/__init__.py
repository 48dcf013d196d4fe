"""Seeded synthetic inputs for causal GQA prefill attention.

This module is shared by the tests, the benchmark and the smoke check. It
holds none of the attention arithmetic: it only draws numbers, rounds them to
bf16, draws a block-table permutation and places logical K/V rows into a paged
cache. Both the CPU oracle and the HIP library consume what it returns; it
imports neither.

Recipe (the workloads of the pages' microbenchmarks: query chunks of 4096,
3072 and 512 tokens against short, medium and long KV, 24 query heads over 4 KV
heads, head_dim 256, BF16):

* ``np.random.default_rng(seed)``; Q, K, V drawn in that order as float32
  standard normals, then rounded to bf16 (round-to-nearest-even, torch's
  float->bf16 conversion). The bf16 tensors are the ground truth for both sides.
* paged workloads then draw ``block_table = rng.permutation(num_blocks)[:n]``
  (n = ceil(kv_len / 16)) and place logical key t at
  ``cache[block_table[t // 16], :, t % 16, :]``. Physical blocks that the table
  does not use and slots past kv_len - 1 are filled with a large sentinel pattern
  (+/-64 and 0) so that a wrong gather shows up in the output.
* paged INT8 keys: the codes of the logical K go to the split-d cache
  ``[num_blocks, 4, 16, 16, 16]`` (feature f of key t at
  ``[block_table[t // 16], h, f // 16, t % 16, f % 16]``) and their scales to a paged
  scale cache ``[num_blocks, 4, 16]`` whose unused entries are NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

HQ, HKV, D, BLOCK_SIZE = 24, 4, 256, 16


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a prefill chunk of q_len queries over kv_len keys."""

    name: str
    q_len: int
    kv_len: int
    paged: bool = False
    int8k: bool = False
    int8v: bool = False   # INT8 values too (INT8 P·V); implies int8k
    num_blocks: int = 0   # paged only: physical blocks in the cache
    seed: int = 0

    @property
    def pairs_per_head(self) -> int:
        """Visible (query, key) pairs per head: sum over i of (kv_len - q_len + i + 1)."""
        off = self.kv_len - self.q_len
        return self.q_len * off + self.q_len * (self.q_len + 1) // 2


# The five workloads (tiny parity case, three contiguous chunks, a paged tail
# chunk, an INT8-K chunk) plus the pages' 4096 x 16K shape as an extra row.
WORKLOADS = {
    1: Workload("tiny_128x128", 128, 128, seed=1),
    2: Workload("chunk_4096x8192", 4096, 8192, seed=2),
    3: Workload("longkv_4096x32768", 4096, 32768, seed=3),
    4: Workload("paged_tail_512x32768", 512, 32768, paged=True, num_blocks=2048, seed=4),
    5: Workload("int8k_3072x16384", 3072, 16384, int8k=True, seed=5),
    6: Workload("chunk_4096x16384", 4096, 16384, seed=6),
    7: Workload("paged_int8k_512x32768", 512, 32768, paged=True, int8k=True, num_blocks=2048, seed=7),
    8: Workload("decode_1x32768", 1, 32768, seed=8),
    9: Workload("decode_paged_1x32768", 1, 32768, paged=True, num_blocks=2048, seed=9),
    10: Workload("decode_paged_int8k_1x32768", 1, 32768, paged=True, int8k=True, num_blocks=2048,
                 seed=10),
    # the INT8-K chunk's shape and inputs (seed 5) with bf16 keys: what INT8 keys save
    11: Workload("bf16k_3072x16384", 3072, 16384, seed=5),
    # the same chunk with INT8 values as well (INT8 P·V), same inputs
    12: Workload("int8kv_3072x16384", 3072, 16384, int8k=True, int8v=True, seed=5),
}


def bf16_normal(rng: np.random.Generator, shape) -> torch.Tensor:
    """float32 N(0, 1) draws rounded to bf16 (RNE), as a CPU tensor."""
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)


def make_qkv(q_len: int, kv_len: int, seed: int):
    """Q [q_len, 24, 256], K and V [kv_len, 4, 256], bf16 CPU tensors."""
    rng = np.random.default_rng(seed)
    q = bf16_normal(rng, (q_len, HQ, D))
    k = bf16_normal(rng, (kv_len, HKV, D))
    v = bf16_normal(rng, (kv_len, HKV, D))
    return q, k, v, rng


def sentinel_fill(shape, dtype=torch.bfloat16) -> torch.Tensor:
    """Deterministic +64 / -64 / 0 pattern used for cache memory no key may read."""
    n = int(np.prod(shape))
    pat = np.array([64.0, -64.0, 0.0], dtype=np.float32)[np.arange(n) % 3]
    return torch.from_numpy(pat.reshape(shape)).to(dtype)


def block_table_for(rng: np.random.Generator, kv_len: int, num_blocks: int) -> torch.Tensor:
    n = math.ceil(kv_len / BLOCK_SIZE)
    if num_blocks < n:
        raise ValueError(f"{num_blocks} blocks cannot hold {kv_len} keys")
    return torch.from_numpy(rng.permutation(num_blocks)[:n].astype(np.int32))


def scatter_paged(x: torch.Tensor, block_table: torch.Tensor, num_blocks: int) -> torch.Tensor:
    """Place logical rows x [kv_len, 4, 256] into a cache [num_blocks, 4, 16, 256]."""
    kv_len = x.shape[0]
    cache = sentinel_fill((num_blocks, HKV, BLOCK_SIZE, D), x.dtype)
    n = block_table.shape[0]
    padded = torch.zeros((n * BLOCK_SIZE, HKV, D), dtype=x.dtype)
    padded[:kv_len] = x
    # slots past kv_len - 1 of the last block keep the sentinel pattern
    tail = cache[block_table[-1].item()].clone()
    cache[block_table.long()] = padded.view(n, BLOCK_SIZE, HKV, D).permute(0, 2, 1, 3)
    last_used = kv_len - (n - 1) * BLOCK_SIZE
    cache[block_table[-1].item(), :, last_used:, :] = tail[:, last_used:, :]
    return cache


def scatter_paged_int8_splitd(kq: torch.Tensor, block_table: torch.Tensor,
                              num_blocks: int) -> torch.Tensor:
    """Place logical INT8 K codes [kv_len, 4, 256] into the split-d paged cache
    [num_blocks, 4, 16, 16, 16]: feature f of key t, head h goes to
    [block_table[t // 16], h, f // 16, t % 16, f % 16]. Unused memory holds the
    sentinel pattern."""
    rows = scatter_paged(kq, block_table, num_blocks)          # [nb, 4, 16 slots, 256]
    return rows.view(num_blocks, HKV, BLOCK_SIZE, D // 16, 16).permute(0, 1, 3, 2, 4).contiguous()


def scatter_paged_scales(ks: torch.Tensor, block_table: torch.Tensor,
                         num_blocks: int) -> torch.Tensor:
    """Place per-token key scales [kv_len, 4] (float32) into a paged scale cache
    [num_blocks, 4, 16]: the scale of key t, head h goes to
    [block_table[t // 16], h, t % 16]. Every other entry is NaN, so a scale that the
    computation should never use poisons the result if it is read."""
    kv_len = ks.shape[0]
    cache = torch.full((num_blocks, HKV, BLOCK_SIZE), float("nan"), dtype=torch.float32)
    for t0 in range(0, kv_len, BLOCK_SIZE):
        n = min(BLOCK_SIZE, kv_len - t0)
        cache[int(block_table[t0 // BLOCK_SIZE]), :, :n] = ks[t0:t0 + n].T
    return cache


def make_workload(w: Workload) -> dict:
    """All CPU tensors of a workload.

    Keys: q, k, v (logical bf16), plus for paged workloads block_table (int32),
    k_cache and v_cache (bf16 [num_blocks, 4, 16, 256]).
    INT8-K (and INT8-value) workloads return bf16 K and V here; quantising them is the
    caller's step.
    """
    q, k, v, rng = make_qkv(w.q_len, w.kv_len, w.seed)
    out = dict(q=q, k=k, v=v)
    if w.paged:
        bt = block_table_for(rng, w.kv_len, w.num_blocks)
        out["block_table"] = bt
        out["k_cache"] = scatter_paged(k, bt, w.num_blocks)
        out["v_cache"] = scatter_paged(v, bt, w.num_blocks)
    return out
