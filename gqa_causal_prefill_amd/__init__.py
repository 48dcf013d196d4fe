"""MI355X-native causal grouped-query prefill attention (24Q / 4KV, head_dim 256).

The compute lives in libgqa_prefill.so (HIP kernels for gfx950 behind a C ABI,
include/gqa_prefill.h); this package is its Python binding. Importing the
package does not load the library; the first call does, and fails loudly if the
library has not been built.
"""

from .binding import (  # noqa: F401
    BLOCK_SIZE,
    HEAD_DIM,
    INT8KV_MAX_KV,
    NOALLOC_SCRATCH_BYTES,
    NUM_KV_HEADS,
    NUM_Q_HEADS,
    GqaError,
    gqa_abi_version,
    gqa_attn_prefill,
    gqa_attn_prefill_int8kv,
    gqa_attn_prefill_noalloc,
    gqa_attn_prefill_plan,
    gqa_attn_prefill_qint8,
    gqa_attn_prefill_workspace_size,
    gqa_attn_prefill_ws,
    gqa_quantize_rows_int8,
    gqa_quantize_v_int8,
    gqa_status_string,
    library,
)
