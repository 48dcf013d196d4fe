"""The C-ABI library on the host: it loads, exports what the header declares and
rejects bad arguments before touching the GPU (no compute call runs here)."""

import ctypes
import os
import re

import numpy as np
import pytest

from gqa_causal_prefill_amd import build as gqa_build
from gqa_causal_prefill_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")

OK, NULL, BADLEN, MISALIGNED, UNSUPPORTED, HIPERR, WORKSPACE, SCRATCH = range(8)


def _have_lib():
    return os.path.exists(gqa_build.LIB)


pytestmark = pytest.mark.skipif(not _have_lib(), reason="libgqa_prefill.so not built")


def declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gqa_\w+)\s*\(", text, flags=re.M)
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"gqa_attn_prefill", "gqa_attn_prefill_ws", "gqa_attn_prefill_workspace_size",
            "gqa_attn_prefill_qint8", "gqa_quantize_rows_int8", "gqa_attn_prefill_plan",
            "gqa_attn_prefill_noalloc", "gqa_attn_prefill_int8kv", "gqa_quantize_v_int8",
            "gqa_abi_version", "gqa_status_string"} <= set(names)
    lib = ctypes.CDLL(gqa_build.LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_loads():
    if not os.path.exists(gqa_build.PROBE_LIB):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(gqa_build.PROBE_LIB)
    assert hasattr(lib, "gqa_probe_mfma_f32_16x16x32_bf16")
    assert hasattr(lib, "gqa_probe_mfma_i32_16x16x64_i8")


def test_abi_version_and_status_strings():
    assert binding.gqa_abi_version() == 5
    for s in range(8):
        assert binding.gqa_status_string(s)
    assert binding.gqa_status_string(99) == "unknown status"


def call(q=16, k=16, v=16, bt=None, nb=0, ks=None, q_len=4, kv_len=8, out=16):
    lib = binding.library()
    vp = ctypes.c_void_p
    return lib.gqa_attn_prefill(vp(q), vp(k), vp(v), vp(bt), nb, vp(ks), q_len, kv_len, vp(out),
                                None)


def test_zero_queries_is_a_noop():
    # q_len == 0 returns OK without reading any pointer (even NULL ones)
    assert call(q=None, k=None, v=None, out=None, q_len=0, kv_len=0) == OK
    assert call(q=None, k=None, v=None, out=None, q_len=0, kv_len=100) == OK


@pytest.mark.parametrize("q_len,kv_len", [(-1, 4), (5, 4), (1, -3), (1, (1 << 24) + 1)])
def test_bad_lengths(q_len, kv_len):
    assert call(q_len=q_len, kv_len=kv_len) == BADLEN


@pytest.mark.parametrize("which", ["q", "k", "v", "out"])
def test_null_pointers(which):
    assert call(**{which: None}) == NULL


def test_paged_int8_argument_errors():
    # paged caches with INT8 keys are accepted; these argument errors return before any
    # launch: a misaligned scale cache, and too few blocks for kv_len
    assert call(bt=16, nb=1, ks=18) == MISALIGNED
    assert call(bt=16, nb=0, ks=16, kv_len=8) == BADLEN


@pytest.mark.parametrize("which", ["q", "k", "v", "out"])
def test_misaligned_tensors(which):
    assert call(**{which: 16 + 8}) == MISALIGNED


def test_misaligned_small_args():
    assert call(bt=16 + 2, nb=1) == MISALIGNED
    assert call(ks=16 + 1) == MISALIGNED


def test_too_few_blocks():
    # kv_len 40 needs ceil(40/16) = 3 blocks
    assert call(bt=16, nb=2, kv_len=40) == BADLEN
    assert call(bt=16, nb=0, kv_len=40) == BADLEN


def test_quantizer_argument_checks():
    lib = binding.library()
    vp = ctypes.c_void_p
    assert lib.gqa_quantize_rows_int8(None, 0, None, None, None) == OK
    assert lib.gqa_quantize_rows_int8(vp(16), -1, vp(16), vp(16), None) == BADLEN
    assert lib.gqa_quantize_rows_int8(None, 4, vp(16), vp(16), None) == NULL
    assert lib.gqa_quantize_rows_int8(vp(16 + 4), 4, vp(16), vp(16), None) == MISALIGNED
    assert lib.gqa_quantize_rows_int8(vp(16), 4, vp(16 + 1), vp(16), None) == MISALIGNED


def test_plan_describes_the_dispatch():
    plan = binding.gqa_attn_prefill_plan(4096, 32768)
    assert "variant=bf16_contiguous" in plan
    # one workgroup per (KV head, 32-token block) covering the 6 query heads of the
    # group: 4 * 128
    assert "workgroups=512" in plan and "threads=256" in plan
    assert "variant=bf16_paged" in binding.gqa_attn_prefill_plan(512, 32768, paged=True)
    assert "variant=int8k" in binding.gqa_attn_prefill_plan(3072, 16384, int8k=True)
    assert "workgroups=4" in binding.gqa_attn_prefill_plan(1, 1)
    assert "variant=int8k_paged_splitd" in binding.gqa_attn_prefill_plan(512, 32768, paged=True,
                                                                         int8k=True)
    with pytest.raises(binding.GqaError):
        binding.gqa_attn_prefill_plan(10, 5)


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(4, 24, 256, dtype=torch.bfloat16)
    k = torch.zeros(8, 4, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.gqa_attn_prefill(q, k, k)


# ------------------------------------------------------------------ KV segments and workspace

def ws_call(ws, ws_bytes, q_len=512, kv_len=32768, bt=None, nb=0):
    lib = binding.library()
    vp = ctypes.c_void_p
    return lib.gqa_attn_prefill_ws(vp(16), vp(16), vp(16), vp(bt), nb, None, q_len, kv_len,
                                   vp(16), vp(ws), ws_bytes, None)


SPLIT_512x32768 = 4 * 512 * 24 * (256 + 2) * 4   # 4 segments of fp32 (O, m, l) per row


def test_workspace_size():
    # grids that balance by their longest-first order run unsplit and need nothing
    assert binding.gqa_attn_prefill_workspace_size(4096, 32768) == 0
    assert binding.gqa_attn_prefill_workspace_size(4096, 8192) == 0
    assert binding.gqa_attn_prefill_workspace_size(2048, 32768) == 0   # one full round
    # 512 queries: 4 KV heads x 16 token blocks = 64 workgroups -> 4 segments of ~126 tiles
    assert binding.gqa_attn_prefill_workspace_size(512, 32768) == SPLIT_512x32768
    assert binding.gqa_attn_prefill_workspace_size(512, 32768, paged=True) == SPLIT_512x32768
    assert binding.gqa_attn_prefill_workspace_size(512, 32768, int8k=True) == SPLIT_512x32768
    # a grid that ends in a part-filled round (3072 queries: 384 workgroups) cuts only its
    # longest token blocks: the rows of 1024 tokens, in 2 segments
    assert binding.gqa_attn_prefill_workspace_size(3072, 16384, int8k=True) == 2 * 1024 * 24 * 258 * 4
    # short histories are not split below 8 tiles a segment
    assert binding.gqa_attn_prefill_workspace_size(32, 500) == 0
    # arguments the call would refuse
    assert binding.gqa_attn_prefill_workspace_size(10, 5) == 0
    assert binding.gqa_attn_prefill_workspace_size(512, 32768, paged=True, int8k=True) == \
        SPLIT_512x32768


def test_workspace_errors_return_before_launch():
    # every case below is refused on the host, so no kernel is launched
    assert ws_call(None, 0) == WORKSPACE
    assert ws_call(4096, SPLIT_512x32768 - 1) == WORKSPACE
    assert ws_call(4096 + 8, SPLIT_512x32768) == MISALIGNED
    assert ws_call(4096, SPLIT_512x32768, q_len=10, kv_len=5) == BADLEN
    lib = binding.library()
    vp = ctypes.c_void_p
    assert lib.gqa_attn_prefill_ws(None, vp(16), vp(16), None, 0, None, 512, 32768, vp(16),
                                   vp(4096), SPLIT_512x32768, None) == NULL
    # q_len == 0 is a no-op for the workspace form too
    assert lib.gqa_attn_prefill_ws(None, None, None, None, 0, None, 0, 100, None, None, 0,
                                   None) == OK


def test_plan_reports_segments():
    plan = binding.gqa_attn_prefill_plan(4096, 32768)
    assert "segments=1 whole_token_blocks=128 workspace_bytes=0" in plan
    plan = binding.gqa_attn_prefill_plan(512, 32768, paged=True)
    assert "workgroups=256" in plan and "segments=4 whole_token_blocks=0" in plan
    assert f"workspace_bytes={SPLIT_512x32768}" in plan


def test_plan_partial_split():
    """384 workgroups (1.5 rounds on 256 CUs): the 32 longest of the 96 token blocks of
    each KV head are cut in two, making 512 work units, two full rounds; the workspace
    holds only those blocks' rows (1024 tokens x 24 heads x (256 + 2) floats x 2)."""
    plan = binding.gqa_attn_prefill_plan(3072, 16384, int8k=True)
    assert "workgroups=512" in plan and "segments=2 whole_token_blocks=64" in plan
    assert f"workspace_bytes={2 * 1024 * 24 * 258 * 4}" in plan
    assert binding.gqa_attn_prefill_workspace_size(3072, 16384, int8k=True) == 2 * 1024 * 24 * 258 * 4
    # a grid of whole rounds is not cut
    assert "segments=1" in binding.gqa_attn_prefill_plan(4096, 8192)


def qint8_call(qc=16, qs=16, k=16, v=16, bt=None, nb=0, ks=16, q_len=4, kv_len=8, out=16,
               ws=None, ws_bytes=0):
    lib = binding.library()
    vp = ctypes.c_void_p
    return lib.gqa_attn_prefill_qint8(vp(qc), vp(qs), vp(k), vp(v), vp(bt), nb, vp(ks), q_len,
                                      kv_len, vp(out), vp(ws), ws_bytes, None)


def test_qint8_argument_errors_return_before_launch():
    # every case below is refused on the host, so no kernel is launched
    assert qint8_call(qc=None, qs=None, k=None, v=None, ks=None, out=None, q_len=0) == OK
    assert qint8_call(qs=None) == NULL
    assert qint8_call(ks=None) == NULL       # the codes are only meaningful with INT8 keys
    assert qint8_call(qc=None) == NULL
    assert qint8_call(qs=16 + 2) == MISALIGNED
    assert qint8_call(qc=16 + 8) == MISALIGNED
    assert qint8_call(ks=16 + 1) == MISALIGNED
    assert qint8_call(q_len=9, kv_len=8) == BADLEN
    assert qint8_call(bt=16, nb=0, kv_len=40) == BADLEN
    # a shape that splits needs the workspace gqa_attn_prefill_ws would need
    need = binding.gqa_attn_prefill_workspace_size(512, 32768, int8k=True)
    assert need > 0
    assert qint8_call(q_len=512, kv_len=32768) == WORKSPACE
    assert qint8_call(q_len=512, kv_len=32768, ws=4096, ws_bytes=need - 1) == WORKSPACE


def test_qint8_binding_checks_dtypes():
    import torch
    q = torch.zeros((4, 24, 256), dtype=torch.int8)
    with pytest.raises(ValueError):   # k_scale is required
        binding.gqa_attn_prefill_qint8(q, torch.zeros((4, 24)), torch.zeros((8, 4, 256),
                                       dtype=torch.int8), torch.zeros((8, 4, 256)))


def _plan_fields(q_len, kv_len, paged=False, int8k=False):
    plan = binding.gqa_attn_prefill_plan(q_len, kv_len, paged=paged, int8k=int8k)
    return {kv.split("=")[0]: kv.split("=")[1] for kv in plan.split()}


def test_plan_invariants_over_many_shapes():
    """What the kernel assumes of every plan, over a sweep of lengths: the grid holds
    one workgroup per whole token block and `segments` per cut one; the workspace holds
    the cut blocks' rows; every KV segment is at least 8 tiles of 64 keys long and
    starts at or before its token block's first query (position kv_len - q_len + the
    block's first token), so the first key of every segment is visible to every query
    of its workgroup."""
    rng = np.random.default_rng(0)
    shapes = [(q, q + h) for q in (1, 3, 4, 5, 31, 32, 33, 100, 512, 1000, 2048, 2080, 2112, 3000,
                                   3072, 4096, 5000, 6000, 8192, 9000)
              for h in (0, 1, 500, 4096, 30000)]
    shapes += [(int(q), int(q + h)) for q, h in zip(rng.integers(1, 12000, 60), rng.integers(0, 70000, 60))]
    cut_shapes = 0
    for q_len, kv_len in shapes:
        f = _plan_fields(q_len, kv_len)
        tok = 4 if q_len <= 4 else 32
        n_tblk = -(-q_len // tok)
        nseg, whole = int(f["segments"]), int(f["whole_token_blocks"])
        wg, ws = int(f["workgroups"]), int(f["workspace_bytes"])
        assert binding.gqa_attn_prefill_workspace_size(q_len, kv_len) == ws
        if nseg == 1:
            assert whole == n_tblk and wg == 4 * n_tblk and ws == 0, (q_len, kv_len, f)
            continue
        cut_shapes += 1
        assert 0 <= whole < n_tblk, (q_len, kv_len, f)
        assert wg == 4 * (whole + (n_tblk - whole) * nseg), (q_len, kv_len, f)
        assert ws == nseg * (q_len - tok * whole) * 24 * 258 * 4, (q_len, kv_len, f)
        off = kv_len - q_len
        for t in range(whole, n_tblk):
            last = min((t + 1) * tok, q_len)
            tiles = (off + last + 63) // 64
            starts = [tiles * s // nseg for s in range(nseg + 1)]
            assert min(b - a for a, b in zip(starts, starts[1:])) >= 8, (q_len, kv_len, t, f)
            assert starts[-2] * 64 <= off + t * tok, (q_len, kv_len, t, f)
    assert cut_shapes >= 20


def noalloc_call(q_len, kv_len, paged=False, int8k=False):
    lib = binding.library()
    vp = ctypes.c_void_p
    nb = (kv_len + 15) // 16 if paged else 0
    return lib.gqa_attn_prefill_noalloc(vp(16), vp(16), vp(16), vp(16) if paged else None, nb,
                                        vp(16) if int8k else None, q_len, kv_len, vp(16), None)


def test_header_scratch_size_matches_binding():
    text = open(os.path.join(HEADER_DIR, "gqa_prefill.h")).read()
    m = re.search(r"#define GQA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("paged,int8k", [(False, False), (True, False), (False, True), (True, True)])
def test_noalloc_refuses_plans_beyond_its_scratch(paged, int8k):
    """A call whose KV segments need more than the scratch array is refused on the host,
    before any device call (this runs without a GPU); lengths whose plan fits are not
    refused for their size."""
    big = (1840, 131072)
    need = binding.gqa_attn_prefill_workspace_size(*big, paged, int8k)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    assert noalloc_call(*big, paged, int8k) == SCRATCH
    # argument errors still come first
    assert noalloc_call(5, 4, paged, int8k) == BADLEN
    assert noalloc_call(0, 4, paged, int8k) == OK


def call_int8kv(q=16, qs=None, k=16, ks=16, v=16, vs=16, v_ld=16, q_len=4, kv_len=8, out=16):
    lib = binding.library()
    vp = ctypes.c_void_p
    return lib.gqa_attn_prefill_int8kv(vp(q), vp(qs), vp(k), vp(ks), vp(v), vp(vs), v_ld, q_len,
                                       kv_len, vp(out), None)


def test_int8kv_argument_errors_return_before_launch():
    # q_len == 0 is a no-op whatever the pointers
    assert call_int8kv(q=None, k=None, ks=None, v=None, vs=None, out=None, q_len=0) == OK
    assert call_int8kv(q_len=5, kv_len=4) == BADLEN
    for which in ("q", "k", "ks", "v", "vs", "out"):
        assert call_int8kv(**{which: None}) == NULL, which
    # v_ld: a multiple of 16, at least kv_len
    assert call_int8kv(v_ld=8) == BADLEN
    assert call_int8kv(v_ld=24) == BADLEN
    assert call_int8kv(kv_len=40, v_ld=32) == BADLEN
    assert call_int8kv(v_ld=-16) == BADLEN
    for which in ("q", "k", "v", "out", "vs"):
        assert call_int8kv(**{which: 16 + 4}) == MISALIGNED, which
    assert call_int8kv(ks=16 + 1) == MISALIGNED
    assert call_int8kv(qs=16 + 2) == MISALIGNED
    # the int32 sums bound the history
    lim = binding.INT8KV_MAX_KV
    assert call_int8kv(q_len=1, kv_len=lim + 1, v_ld=lim + 16) == UNSUPPORTED


def test_v_quantizer_argument_checks():
    lib = binding.library()
    vp = ctypes.c_void_p
    q = lib.gqa_quantize_v_int8
    assert q(vp(16), -1, 16, vp(16), vp(16), None) == BADLEN
    assert q(vp(16), 20, 16, vp(16), vp(16), None) == BADLEN
    assert q(vp(16), 8, 24, vp(16), vp(16), None) == BADLEN
    assert q(None, 8, 16, vp(16), vp(16), None) == NULL
    assert q(vp(16), 8, 16, None, vp(16), None) == NULL
    assert q(vp(16), 8, 16, vp(16), None, None) == NULL
    assert q(vp(16 + 8), 8, 16, vp(16), vp(16), None) == MISALIGNED
    assert q(vp(16), 8, 16, vp(16 + 4), vp(16), None) == MISALIGNED
    assert q(vp(16), 8, 16, vp(16), vp(16 + 2), None) == MISALIGNED


def test_plan_int8kv():
    plan = binding.gqa_attn_prefill_plan(3072, 16384, int8k=2)
    assert "variant=int8kv_contiguous_t32h6_kt64" in plan
    assert "segments=1" in plan and "workgroups=384" in plan and "workspace_bytes=0" in plan
    # every q_len runs the prefill shape (there is no decode shape for INT8 values)
    assert "workgroups=4 " in binding.gqa_attn_prefill_plan(1, 32768, int8k=2)
    assert binding.gqa_attn_prefill_workspace_size(3072, 16384, int8k=2) == 0
    with pytest.raises(binding.GqaError):
        binding.gqa_attn_prefill_plan(1, binding.INT8KV_MAX_KV + 1, int8k=2)
    with pytest.raises(binding.GqaError):
        binding.gqa_attn_prefill_plan(16, 64, paged=True, int8k=2)


def test_int8kv_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros((4, 24, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.gqa_attn_prefill_int8kv(q, None, None, None, None)
    with pytest.raises(ValueError):
        binding.gqa_quantize_v_int8(torch.zeros((8, 4, 256), dtype=torch.bfloat16))
