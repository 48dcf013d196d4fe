"""CPU oracle for causal grouped-query prefill attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use it. It shares no code with the HIP library.

Pages cited (by title and section; the code restates them, it copies nothing):

* "DCU使用技术报告（中篇）" (DCU technical report, part 2), cited as
  [DCU report §n]. §1 fixes the attention shape (24 query heads, 4 KV heads,
  head_dim 256, GQA ratio 6, BF16); §2 states what the dedicated prefill
  kernel computes (QK, causal mask, online softmax, PV, FP32 accumulation)
  and says the later query-reuse variants leave that math unchanged (§4).
* "gfx936 DCU上实现INT8 QK MMAC" (INT8 QK MMAC on gfx936), cited as
  [INT8 QK §n]. §1 gives the score S = Q·Kᵀ/sqrt(d), the symmetric dynamic
  quantisation Q ≈ Qq·sQ, K ≈ Kq·sK and the post-scale applied per score
  before softmax; §2.1 the [-127, 127] range and the INT32 bound; §3 the paged
  K cache walk (block table -> physical block -> slot); §4 the per-row
  quantiser sQ = max|Q|/127, Qq = round(Q/sQ); §5.2 the GQA map kv = head/6;
  §6 names INT8 PV (V in INT8) and defines nothing more: ``int8pv`` states the
  reading taken for it.

Everything here is float64 unless a page fixes another precision. The one
place that is not float64 is the INT8 quantiser, which runs in float32 (the
reading taken for the unspecified "round" of [INT8 QK §4]: IEEE float32
division and round-half-to-even), so that both sides of a comparison take the
same integer decisions.

Pin status: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` and ``tests/test_oracle_int8pv.py`` (brute force, closed forms, invariants, a library
reduction and hand-derived fixtures under ``tests/golden/``). None is
"parity unpinned".
"""

from .prefill import (  # noqa: F401
    D,
    GROUP,
    HKV,
    HQ,
    SCALE,
    BLOCK_SIZE,
    attention,
    attention_int8,
    attention_int8k,
    causal_limit,
    gather_paged,
    gather_paged_int8_splitd,
    gather_paged_scales,
    kv_head_of,
    quantize_rows_int8,
    score_matrix,
    score_matrix_int8k,
)
from .int8pv import (  # noqa: F401
    P_LEVELS,
    attention_int8kv,
    attention_int8qkv,
    p_codes,
    quantize_v_int8,
)
