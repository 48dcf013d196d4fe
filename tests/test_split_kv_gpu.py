"""Parity of the KV-segment path (gqa_attn_prefill_ws) with the CPU oracle.

When q_len is short the call cuts every token block's history into KV segments; when
a larger grid would end in a part-filled round of workgroups, only its longest token
blocks are cut. Each cut workgroup writes an unnormalised partial output with its
reference maximum and row sum, and a merge kernel combines them by the log-sum-exp
rule. The result is the same softmax, so the bf16 tolerances of the unsplit path apply
unchanged (max |err| <= 1e-2, mean |err| <= 1e-3 against the float64 oracle; INT8 keys
2e-3), element by element over the whole output; rows of token blocks that are not
cut are bitwise those of the call without a workspace.
"""

import numpy as np
import pytest
import torch

import gqa_causal_prefill_amd as gqa
import oracle
from gqa_synth import block_table_for, make_qkv, scatter_paged
from tolerance import BF16_MAX, BF16_MEAN, INT8_MAX, errors

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)


def segments(q_len, kv_len, paged=False):
    plan = gqa.gqa_attn_prefill_plan(q_len, kv_len, paged=paged)
    return int(plan.split("segments=")[1].split()[0])


# (q_len, kv_len) -> segments: 8 KV segments for one token block, 5 for a ragged
# 4-block chunk, 16 for a single query, 3 for 17 token blocks with a ragged last one
SPLIT_SHAPES = [(32, 4096, 8), (100, 3000, 5), (1, 8192, 16), (513, 9000, 3)]


@pytest.mark.parametrize("q_len,kv_len,nseg", SPLIT_SHAPES)
def test_split_contiguous_full(q_len, kv_len, nseg):
    note(f"case split contiguous {q_len}x{kv_len}")
    assert segments(q_len, kv_len) == nseg
    q, k, v, _ = make_qkv(q_len, kv_len, seed=5000 + q_len)
    out = gqa.gqa_attn_prefill_ws(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    mx, mean = errors(out, oracle.attention(q, k, v))
    note(f"  {nseg} segments: max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_split_paged_full_and_bitwise_equal_to_contiguous():
    q_len, kv_len, nb = 64, 5000, 400
    note(f"case split paged {q_len}x{kv_len}")
    assert segments(q_len, kv_len, paged=True) > 1
    q, k, v, rng = make_qkv(q_len, kv_len, seed=5100)
    bt = block_table_for(rng, kv_len, nb)
    kc, vc = scatter_paged(k, bt, nb), scatter_paged(v, bt, nb)
    out = gqa.gqa_attn_prefill_ws(q.to(DEV), kc.to(DEV), vc.to(DEV), block_table=bt.to(DEV),
                                  kv_len=kv_len)
    contig = gqa.gqa_attn_prefill_ws(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    mx, mean = errors(out, oracle.attention(q, k, v))
    note(f"  max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN
    assert torch.equal(out, contig)


def test_split_restart_inside_a_segment():
    """Keys from 1500 on score 144 (log2 units) above the rest: segment 2 (keys
    1024..1535) must restart with its exact maxima, later segments take a high
    reference from their first tile, and the merge weighs the low segments by ~2^-144."""
    q_len, kv_len, start = 32, 4096, 1500
    note("case split restart")
    q, k, v, _ = make_qkv(q_len, kv_len, seed=5200)
    q2, k2 = q.to(torch.float32).clone(), k.to(torch.float32).clone()
    q2[..., 0] += 40.0
    k2[start:, :, 0] = 40.0
    q, k = q2.to(torch.bfloat16), k2.to(torch.bfloat16)
    out = gqa.gqa_attn_prefill_ws(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    mx, mean = errors(out, oracle.attention(q, k, v))
    note(f"  max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_split_deterministic_and_close_to_unsplit():
    note("case split determinism")
    q, k, v, _ = make_qkv(40, 6000, seed=5300)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = gqa.gqa_attn_prefill_ws(qd, kd, vd)
    b = gqa.gqa_attn_prefill_ws(qd, kd, vd)
    c = gqa.gqa_attn_prefill(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    d = (a.float() - c.float()).abs()
    note(f"  split vs unsplit: max {d.max().item():.3e}")
    assert d.max().item() <= 2 * BF16_MAX


def test_split_workspace_reused_for_a_smaller_call():
    """One workspace sized for a large call serves a smaller one; its previous
    contents do not leak into the result."""
    note("case split workspace reuse")
    big = gqa.gqa_attn_prefill_workspace_size(64, 8192)
    ws = torch.full((big,), 0x7F, dtype=torch.uint8, device=DEV)   # NaN-like fill pattern
    for q_len, kv_len, seed in [(64, 8192, 5400), (16, 2000, 5401)]:
        assert 0 < gqa.gqa_attn_prefill_workspace_size(q_len, kv_len) <= big
        q, k, v, _ = make_qkv(q_len, kv_len, seed=seed)
        out = gqa.gqa_attn_prefill_ws(q.to(DEV), k.to(DEV), v.to(DEV), workspace=ws)
        torch.cuda.synchronize()
        mx, mean = errors(out, oracle.attention(q, k, v))
        note(f"  {q_len}x{kv_len}: max {mx:.3e} mean {mean:.3e}")
        assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_unsplit_shapes_ignore_the_workspace():
    """A grid that fills the chip runs in one piece: the workspace form returns the
    plain call's bits."""
    note("case no split")
    q, k, v, _ = make_qkv(1024, 1500, seed=5500)
    assert gqa.gqa_attn_prefill_workspace_size(1024, 1500) == 0
    a = gqa.gqa_attn_prefill_ws(q.to(DEV), k.to(DEV), v.to(DEV))
    b = gqa.gqa_attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("q_len,kv_len", [(64, 3000), (200, 4000)])
def test_split_int8k_full(q_len, kv_len):
    """INT8 keys through KV segments: every segment quantises its query rows itself,
    with the same codes, so the INT8 bound of the unsplit path applies."""
    note(f"case split int8k {q_len}x{kv_len}")
    plan = gqa.gqa_attn_prefill_plan(q_len, kv_len, int8k=True)
    assert int(plan.split("segments=")[1].split()[0]) > 1
    q, k, v, _ = make_qkv(q_len, kv_len, seed=5600 + q_len)
    kq, ks = oracle.quantize_rows_int8(k)
    out = gqa.gqa_attn_prefill_ws(q.to(DEV), torch.from_numpy(kq).to(DEV), v.to(DEV),
                                  k_scale=torch.from_numpy(ks).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.attention_int8k(q, kq, ks, v)
    e = np.abs(out.float().cpu().numpy().astype(np.float64) - ref)
    note(f"  max {e.max():.3e}")
    assert e.max() <= 2e-3


# ------------------------------------------------------------------ partial splits

def plan_fields(q_len, kv_len, paged=False, int8k=False):
    plan = gqa.gqa_attn_prefill_plan(q_len, kv_len, paged=paged, int8k=int8k)
    return {kv.split("=")[0]: kv.split("=")[1] for kv in plan.split()}




# (q_len, kv_len, segments, whole token blocks of 32 tokens): grids of more than 256
# workgroups that would end in a part-filled round have only their longest token
# blocks cut into KV segments; the last shape has a ragged last token block
PARTIAL_SHAPES = [(3072, 8192, 2, 64), (2112, 6000, 3, 35), (5000, 20000, 2, 122)]


@pytest.mark.parametrize("q_len,kv_len,nseg,whole", PARTIAL_SHAPES)
def test_partial_split_contiguous(q_len, kv_len, nseg, whole):
    """Rows of the whole token blocks come from the same workgroup program as the
    call without a workspace (bitwise equal); rows of the split ones pass through the
    merge and match the oracle to the bf16 tolerance."""
    note(f"case partial split {q_len}x{kv_len}")
    f = plan_fields(q_len, kv_len)
    assert int(f["segments"]) == nseg and int(f["whole_token_blocks"]) == whole
    q0 = 32 * whole
    q, k, v, _ = make_qkv(q_len, kv_len, seed=5700 + q_len)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ws = torch.empty(gqa.gqa_attn_prefill_workspace_size(q_len, kv_len), dtype=torch.uint8, device=DEV)
    assert ws.numel() == nseg * (q_len - q0) * 24 * 258 * 4
    a = gqa.gqa_attn_prefill_ws(qd, kd, vd, workspace=ws)
    b = gqa.gqa_attn_prefill(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(a[:q0], b[:q0])
    mx, mean = errors(a, oracle.attention(q, k, v))
    note(f"  {nseg} segments from token {q0}, all {q_len} rows: max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN
    # the split rows stay within rounding of the unsplit call's
    assert (a[q0:].float() - b[q0:].float()).abs().max().item() <= 2e-2


def test_partial_split_int8k():
    q_len, kv_len = 3072, 8192
    note(f"case partial split int8k {q_len}x{kv_len}")
    f = plan_fields(q_len, kv_len, int8k=True)
    assert int(f["segments"]) == 2 and int(f["whole_token_blocks"]) == 64
    q0 = 32 * 64
    q, k, v, _ = make_qkv(q_len, kv_len, seed=5800)
    kq, ks = oracle.quantize_rows_int8(k)
    args = (q.to(DEV), torch.from_numpy(kq).to(DEV), v.to(DEV))
    a = gqa.gqa_attn_prefill_ws(*args, k_scale=torch.from_numpy(ks).to(DEV))
    b = gqa.gqa_attn_prefill(*args, k_scale=torch.from_numpy(ks).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(a[:q0], b[:q0])
    mx, mean = errors(a, oracle.attention_int8k(q, kq, ks, v))
    note(f"  all {q_len} rows: max {mx:.3e} mean {mean:.3e}")
    assert mx <= INT8_MAX


def test_partial_split_restart():
    """Keys from 2000 on score 144 (log2 units) above the first tile: every whole token
    block and the first segment of every cut one restarts with exact maxima; the second
    segments take a high reference from their first tile; the merge weighs each cut
    block's segments together."""
    q_len, kv_len, start = 3072, 8192, 2000
    note(f"case partial split restart {q_len}x{kv_len}")
    f = plan_fields(q_len, kv_len)
    assert int(f["segments"]) == 2 and int(f["whole_token_blocks"]) == 64
    q, k, v, _ = make_qkv(q_len, kv_len, seed=5900)
    q2, k2 = q.to(torch.float32).clone(), k.to(torch.float32).clone()
    q2[..., 0] += 40.0
    k2[start:, :, 0] = 40.0
    q, k = q2.to(torch.bfloat16), k2.to(torch.bfloat16)
    out = gqa.gqa_attn_prefill_ws(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    mx, mean = errors(out, oracle.attention(q, k, v))
    note(f"  all {q_len} rows: max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_partial_split_paged_bitwise_equal_to_contiguous():
    """A partially split grid over paged caches (bf16, and INT8 keys in the split-d page
    layout) runs the same arithmetic as over contiguous K/V: the outputs are bitwise
    equal, whole token blocks and cut ones alike."""
    from gqa_synth import scatter_paged_int8_splitd, scatter_paged_scales

    q_len, kv_len, nb = 3072, 8192, 600
    note(f"case partial split paged {q_len}x{kv_len}")
    for int8k in (False, True):
        f = plan_fields(q_len, kv_len, paged=True, int8k=int8k)
        assert int(f["segments"]) == 2 and int(f["whole_token_blocks"]) == 64, f
    q, k, v, rng = make_qkv(q_len, kv_len, seed=6000)
    bt = block_table_for(rng, kv_len, nb)
    qd, btd = q.to(DEV), bt.to(DEV)
    vc = scatter_paged(v, bt, nb).to(DEV)
    a = gqa.gqa_attn_prefill_ws(qd, scatter_paged(k, bt, nb).to(DEV), vc, block_table=btd,
                                kv_len=kv_len)
    b = gqa.gqa_attn_prefill_ws(qd, k.to(DEV), v.to(DEV))
    kq, ks = oracle.quantize_rows_int8(k)
    kq_t, ks_t = torch.from_numpy(kq), torch.from_numpy(ks)
    c = gqa.gqa_attn_prefill_ws(qd, scatter_paged_int8_splitd(kq_t, bt, nb).to(DEV), vc,
                                block_table=btd, kv_len=kv_len,
                                k_scale=scatter_paged_scales(ks_t, bt, nb).to(DEV))
    d = gqa.gqa_attn_prefill_ws(qd, kq_t.to(DEV), v.to(DEV), k_scale=ks_t.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(c, d)
    mx, mean = errors(a, oracle.attention(q, k, v))
    note(f"  bf16 all {q_len} rows: max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_side_stream_without_workspace():
    """A call on a stream other than torch's current one, with no workspace and no out
    given: the binding allocates both for that stream (so torch cannot hand their memory
    to work on the current stream while the kernels still use it), and the result is
    bitwise that of the same call on the current stream."""
    q_len, kv_len = 64, 3000
    note(f"case side stream {q_len}x{kv_len}")
    assert gqa.gqa_attn_prefill_workspace_size(q_len, kv_len) > 0
    q, k, v, _ = make_qkv(q_len, kv_len, seed=6100)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    want = gqa.gqa_attn_prefill_ws(qd, kd, vd)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(DEV)
    outs = [gqa.gqa_attn_prefill_ws(qd, kd, vd, stream=side) for _ in range(3)]
    # allocations on the current stream meanwhile must not reuse the side stream's blocks
    junk = [torch.full((q_len * 24 * 258 * 4 * 8,), 255, dtype=torch.uint8, device=DEV)
            for _ in range(3)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    for o in outs:
        assert torch.equal(o, want)
