"""ctypes binding of libgqa_prefill.so (argument marshalling only).

Every function has the name of the C entry point it calls. Tensors are torch
tensors on the GPU; torch supplies device memory and the current stream, the
HIP library does all the work. There is no fallback: if the library is missing
or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

from .build import LIB

NUM_Q_HEADS = 24
NUM_KV_HEADS = 4
HEAD_DIM = 256
BLOCK_SIZE = 16

GQA_OK = 0
_STATUS_NAMES = {
    0: "GQA_OK",
    1: "GQA_ERR_NULL_ARG",
    2: "GQA_ERR_BAD_LENGTH",
    3: "GQA_ERR_MISALIGNED",
    4: "GQA_ERR_UNSUPPORTED",
    5: "GQA_ERR_HIP",
    6: "GQA_ERR_WORKSPACE",
    7: "GQA_ERR_SCRATCH",
}
# bytes of device scratch memory gqa_attn_prefill_noalloc holds per GPU
NOALLOC_SCRATCH_BYTES = 64 << 20
# longest history gqa_attn_prefill_int8kv accepts (its int32 sums stay below 2^31)
INT8KV_MAX_KV = 1 << 17


class GqaError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS_NAMES.get(status, status)} "
                         f"({gqa_status_string(status)})")


_lib = None


def library() -> ctypes.CDLL:
    """Load libgqa_prefill.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with "
                               "`python -m gqa_causal_prefill_amd.build`")
        lib = ctypes.CDLL(LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.gqa_abi_version.restype = ctypes.c_int
        lib.gqa_abi_version.argtypes = []
        lib.gqa_status_string.restype = ctypes.c_char_p
        lib.gqa_status_string.argtypes = [ctypes.c_int]
        lib.gqa_attn_prefill.restype = ctypes.c_int
        lib.gqa_attn_prefill.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, vp]
        lib.gqa_attn_prefill_ws.restype = ctypes.c_int
        lib.gqa_attn_prefill_ws.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, vp,
                                            ctypes.c_size_t, vp]
        lib.gqa_attn_prefill_noalloc.restype = ctypes.c_int
        lib.gqa_attn_prefill_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, vp]
        lib.gqa_attn_prefill_qint8.restype = ctypes.c_int
        lib.gqa_attn_prefill_qint8.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp,
                                               ctypes.c_size_t, vp]
        lib.gqa_attn_prefill_workspace_size.restype = ctypes.c_size_t
        lib.gqa_attn_prefill_workspace_size.argtypes = [i32, i32, ctypes.c_int, ctypes.c_int]
        lib.gqa_quantize_rows_int8.restype = ctypes.c_int
        lib.gqa_quantize_rows_int8.argtypes = [vp, i64, vp, vp, vp]
        lib.gqa_attn_prefill_int8kv.restype = ctypes.c_int
        lib.gqa_attn_prefill_int8kv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp]
        lib.gqa_quantize_v_int8.restype = ctypes.c_int
        lib.gqa_quantize_v_int8.argtypes = [vp, i32, i32, vp, vp, vp]
        lib.gqa_attn_prefill_plan.restype = ctypes.c_int
        lib.gqa_attn_prefill_plan.argtypes = [i32, i32, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_char_p, ctypes.c_size_t]
        _lib = lib
    return _lib


def gqa_abi_version() -> int:
    return library().gqa_abi_version()


def gqa_status_string(status: int) -> str:
    return library().gqa_status_string(status).decode()


def gqa_attn_prefill_plan(q_len: int, kv_len: int, paged: bool = False, int8k: int = False) -> str:
    """The launch a call would choose; int8k: 0 bf16 keys, 1 INT8 keys, 2 INT8 keys and values."""
    buf = ctypes.create_string_buffer(256)
    st = library().gqa_attn_prefill_plan(q_len, kv_len, int(paged), int(int8k), buf, 256)
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_plan")
    return buf.value.decode()


def gqa_attn_prefill_workspace_size(q_len: int, kv_len: int, paged: bool = False,
                                    int8k: bool = False) -> int:
    """Bytes of workspace gqa_attn_prefill_ws needs (0: it runs unsplit)."""
    return int(library().gqa_attn_prefill_workspace_size(q_len, kv_len, int(paged), int(int8k)))


def _launch_stream(dev, stream):
    """The torch stream a call is enqueued on: `stream`, else torch's current stream."""
    if dev.type != "cuda":
        raise ValueError("the library runs on the GPU; the first tensor is on " + str(dev))
    return torch.cuda.current_stream(dev) if stream is None else stream


def _stream_handle(stream):
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream, shape, dtype, dev):
    """A tensor the binding allocates for a call on `stream`: allocated with that stream
    current, so torch's caching allocator orders any reuse of its memory after the work
    enqueued on `stream`, whichever stream was current when the binding was called."""
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=dev)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _expect(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _prefill_args(q, k, v, block_table, num_blocks, k_scale, q_len, kv_len, out, stream,
                  q_dtype=torch.bfloat16):
    """Checks dtypes, shapes, contiguity and device; returns the C arguments and out
    (allocated for `stream` when the caller passes none)."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gqa_attn_prefill runs on the GPU; q is on " + str(dev))
    q_len = q.shape[0] if q_len is None else q_len
    paged = block_table is not None
    if paged:
        if kv_len is None:
            raise ValueError("kv_len is required with a block table")
        nb = k.shape[0] if num_blocks is None else num_blocks
        _expect(block_table, "block_table", torch.int32, (math.ceil(kv_len / BLOCK_SIZE),), dev)
        v_shape = (nb, NUM_KV_HEADS, BLOCK_SIZE, HEAD_DIM)
        # INT8 keys use the split-d page layout [block, kv_head, 256 / 16, 16, 16]
        k_shape = ((nb, NUM_KV_HEADS, HEAD_DIM // 16, BLOCK_SIZE, 16) if k_scale is not None
                   else v_shape)
    else:
        kv_len = k.shape[0] if kv_len is None else kv_len
        nb = 0
        k_shape = v_shape = (kv_len, NUM_KV_HEADS, HEAD_DIM)
    _expect(q, "q", q_dtype, (q_len, NUM_Q_HEADS, HEAD_DIM), dev)
    _expect(k, "k", torch.int8 if k_scale is not None else torch.bfloat16, k_shape, dev)
    _expect(v, "v", torch.bfloat16, v_shape, dev)
    if k_scale is not None:
        ks_shape = (nb, NUM_KV_HEADS, BLOCK_SIZE) if paged else (kv_len, NUM_KV_HEADS)
        _expect(k_scale, "k_scale", torch.float32, ks_shape, dev)
    if out is None:
        out = _alloc_on(stream, (q_len, NUM_Q_HEADS, HEAD_DIM), torch.bfloat16, dev)
    else:
        _expect(out, "out", torch.bfloat16, (q_len, NUM_Q_HEADS, HEAD_DIM), dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(block_table), nb, _ptr(k_scale), q_len, kv_len,
            _ptr(out))
    return args, out, (q_len, kv_len, paged, k_scale is not None)


def gqa_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     block_table: torch.Tensor | None = None, num_blocks: int | None = None,
                     k_scale: torch.Tensor | None = None, q_len: int | None = None,
                     kv_len: int | None = None, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Causal GQA prefill attention; see gqa_attn_prefill in include/gqa_prefill.h.

    q: bf16 [q_len, 24, 256]. Contiguous: k, v [kv_len, 4, 256]. Paged (block_table
    given): k, v caches [num_blocks, 4, 16, 256] and block_table int32
    [ceil(kv_len / 16)] (kv_len must then be given). INT8 keys: k int8 and
    k_scale float32 [kv_len, 4]; paged, k is the split-d cache int8
    [num_blocks, 4, 16, 16, 16] and k_scale float32 [num_blocks, 4, 16].
    Returns out (bf16 [q_len, 24, 256]).
    """
    s = _launch_stream(q.device, stream)
    args, out, _ = _prefill_args(q, k, v, block_table, num_blocks, k_scale, q_len, kv_len, out, s)
    st = library().gqa_attn_prefill(*args, _stream_handle(s))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill")
    return out


def gqa_attn_prefill_ws(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        block_table: torch.Tensor | None = None, num_blocks: int | None = None,
                        k_scale: torch.Tensor | None = None, q_len: int | None = None,
                        kv_len: int | None = None, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """gqa_attn_prefill that may split the history into KV segments (see
    gqa_attn_prefill_ws in include/gqa_prefill.h). `workspace` is a device tensor of
    at least gqa_attn_prefill_workspace_size() bytes; when it is None and the call
    splits, one is allocated through torch for this call."""
    s = _launch_stream(q.device, stream)
    args, out, lens = _prefill_args(q, k, v, block_table, num_blocks, k_scale, q_len, kv_len,
                                    out, s)
    ws, ws_ptr, ws_bytes = _workspace_args(workspace, lens, q.device, s)
    st = library().gqa_attn_prefill_ws(*args, ws_ptr, ws_bytes, _stream_handle(s))
    del ws   # held until the launch is enqueued
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_ws")
    return out


def gqa_attn_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             block_table: torch.Tensor | None = None,
                             num_blocks: int | None = None, k_scale: torch.Tensor | None = None,
                             q_len: int | None = None, kv_len: int | None = None,
                             out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """gqa_attn_prefill_ws with the KV-segment partials in the library's own scratch
    memory (see gqa_attn_prefill_noalloc in include/gqa_prefill.h). `out` is required:
    this call allocates nothing. Calls that may overlap on one GPU race."""
    if out is None:
        raise ValueError("gqa_attn_prefill_noalloc allocates nothing: pass out")
    s = _launch_stream(q.device, stream)
    args, out, _ = _prefill_args(q, k, v, block_table, num_blocks, k_scale, q_len, kv_len, out, s)
    st = library().gqa_attn_prefill_noalloc(*args, _stream_handle(s))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_noalloc")
    return out


def _workspace_args(workspace, lens, dev, stream):
    """(tensor, pointer, bytes) of the caller's workspace, or of one allocated through
    torch for this call on `stream` when it is None and the call splits. The caller
    keeps the tensor referenced until the launch is enqueued."""
    if workspace is None:
        need = gqa_attn_prefill_workspace_size(*lens)
        if need > 0:
            workspace = _alloc_on(stream, (need,), torch.uint8, dev)
    if workspace is None:
        return None, None, 0
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on " + str(dev))
    return workspace, _ptr(workspace), workspace.numel() * workspace.element_size()


def gqa_attn_prefill_qint8(q_codes: torch.Tensor, q_scale: torch.Tensor, k: torch.Tensor,
                           v: torch.Tensor, block_table: torch.Tensor | None = None,
                           num_blocks: int | None = None, k_scale: torch.Tensor | None = None,
                           q_len: int | None = None, kv_len: int | None = None,
                           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """INT8-key attention with Q quantised beforehand (see gqa_attn_prefill_qint8 in
    include/gqa_prefill.h): q_codes int8 [q_len, 24, 256] and q_scale float32
    [q_len, 24], as gqa_quantize_rows_int8 returns them; k_scale is required; the
    other arguments are those of gqa_attn_prefill_ws."""
    if k_scale is None:
        raise ValueError("gqa_attn_prefill_qint8 takes INT8 keys: k_scale is required")
    s = _launch_stream(q_codes.device, stream)
    args, out, lens = _prefill_args(q_codes, k, v, block_table, num_blocks, k_scale, q_len,
                                    kv_len, out, s, q_dtype=torch.int8)
    _expect(q_scale, "q_scale", torch.float32, (lens[0], NUM_Q_HEADS), q_codes.device)
    ws, ws_ptr, ws_bytes = _workspace_args(workspace, lens, q_codes.device, s)
    st = library().gqa_attn_prefill_qint8(args[0], _ptr(q_scale), *args[1:], ws_ptr, ws_bytes,
                                          _stream_handle(s))
    del ws   # held until the launch is enqueued
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_qint8")
    return out


def gqa_quantize_rows_int8(x: torch.Tensor, xq: torch.Tensor | None = None,
                           scale: torch.Tensor | None = None, stream=None):
    """Per-row INT8 quantisation of bf16 rows of 256; returns (xq int8, scale float32).

    x may have any leading shape [..., 256]; xq has x's shape and scale its
    leading shape.
    """
    if x.device.type != "cuda":
        raise ValueError("gqa_quantize_rows_int8 runs on the GPU")
    if x.dtype != torch.bfloat16 or x.shape[-1] != HEAD_DIM or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 tensor [..., 256]")
    rows = x.numel() // HEAD_DIM
    s = _launch_stream(x.device, stream)
    if xq is None:
        xq = _alloc_on(s, x.shape, torch.int8, x.device)
    if scale is None:
        scale = _alloc_on(s, x.shape[:-1], torch.float32, x.device)
    _expect(xq, "xq", torch.int8, x.shape, x.device)
    _expect(scale, "scale", torch.float32, x.shape[:-1], x.device)
    st = library().gqa_quantize_rows_int8(_ptr(x), rows, _ptr(xq), _ptr(scale),
                                          _stream_handle(s))
    if st != GQA_OK:
        raise GqaError(st, "gqa_quantize_rows_int8")
    return xq, scale


def gqa_quantize_v_int8(v: torch.Tensor, v_ld: int | None = None, v_codes: torch.Tensor | None = None,
                        v_scale: torch.Tensor | None = None, stream=None):
    """INT8 codes of V per (KV head, feature) column for gqa_attn_prefill_int8kv (see
    gqa_quantize_v_int8 in include/gqa_prefill.h). v: bf16 [kv_len, 4, 256]. Returns
    (v_codes int8 [4, 256, v_ld], v_scale float32 [4, 256]); v_ld defaults to kv_len
    rounded up to a multiple of 16."""
    if v.device.type != "cuda":
        raise ValueError("gqa_quantize_v_int8 runs on the GPU")
    kv_len = v.shape[0]
    _expect(v, "v", torch.bfloat16, (kv_len, NUM_KV_HEADS, HEAD_DIM), v.device)
    v_ld = (kv_len + 15) // 16 * 16 if v_ld is None else v_ld
    s = _launch_stream(v.device, stream)
    if v_codes is None:
        v_codes = _alloc_on(s, (NUM_KV_HEADS, HEAD_DIM, v_ld), torch.int8, v.device)
    if v_scale is None:
        v_scale = _alloc_on(s, (NUM_KV_HEADS, HEAD_DIM), torch.float32, v.device)
    _expect(v_codes, "v_codes", torch.int8, (NUM_KV_HEADS, HEAD_DIM, v_ld), v.device)
    _expect(v_scale, "v_scale", torch.float32, (NUM_KV_HEADS, HEAD_DIM), v.device)
    st = library().gqa_quantize_v_int8(_ptr(v), kv_len, v_ld, _ptr(v_codes), _ptr(v_scale),
                                       _stream_handle(s))
    if st != GQA_OK:
        raise GqaError(st, "gqa_quantize_v_int8")
    return v_codes, v_scale


def gqa_attn_prefill_int8kv(q: torch.Tensor, k: torch.Tensor, k_scale: torch.Tensor,
                            v_codes: torch.Tensor, v_scale: torch.Tensor,
                            q_scale: torch.Tensor | None = None, kv_len: int | None = None,
                            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Attention with INT8 keys, INT8 values and an INT8 P·V product (see
    gqa_attn_prefill_int8kv in include/gqa_prefill.h). q: bf16 [q_len, 24, 256], or int8
    codes with q_scale float32 [q_len, 24]; k int8 [kv_len, 4, 256] with k_scale float32
    [kv_len, 4]; v_codes int8 [4, 256, v_ld] and v_scale float32 [4, 256] as
    gqa_quantize_v_int8 returns them. Returns out (bf16 [q_len, 24, 256])."""
    dev = q.device
    s = _launch_stream(dev, stream)
    q_len = q.shape[0]
    kv_len = k.shape[0] if kv_len is None else kv_len
    _expect(q, "q", torch.int8 if q_scale is not None else torch.bfloat16,
            (q_len, NUM_Q_HEADS, HEAD_DIM), dev)
    if q_scale is not None:
        _expect(q_scale, "q_scale", torch.float32, (q_len, NUM_Q_HEADS), dev)
    _expect(k, "k", torch.int8, (kv_len, NUM_KV_HEADS, HEAD_DIM), dev)
    _expect(k_scale, "k_scale", torch.float32, (kv_len, NUM_KV_HEADS), dev)
    if v_codes.dim() != 3:
        raise ValueError("v_codes must be [4, 256, v_ld]")
    v_ld = v_codes.shape[2]
    _expect(v_codes, "v_codes", torch.int8, (NUM_KV_HEADS, HEAD_DIM, v_ld), dev)
    _expect(v_scale, "v_scale", torch.float32, (NUM_KV_HEADS, HEAD_DIM), dev)
    if out is None:
        out = _alloc_on(s, (q_len, NUM_Q_HEADS, HEAD_DIM), torch.bfloat16, dev)
    else:
        _expect(out, "out", torch.bfloat16, (q_len, NUM_Q_HEADS, HEAD_DIM), dev)
    st = library().gqa_attn_prefill_int8kv(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale),
                                           _ptr(v_codes), _ptr(v_scale), v_ld, q_len, kv_len,
                                           _ptr(out), _stream_handle(s))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_int8kv")
    return out
