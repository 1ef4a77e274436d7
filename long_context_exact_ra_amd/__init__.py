"""Blockwise exact attention of Ring Attention on MI355X (gfx950): the
forward of one device's ring share and its backward (contiguous or striped
placement of the sequence), and the blockwise feedforward of the Blockwise
Transformer.

A thin ctypes binding over the C ABI in ``include/ra_attn.h`` (library
``libra_attn.so`` next to this file).  It only marshals arguments: every
step of the computation runs in the library's own HIP kernels.  PyTorch provides device memory and the
stream.  There is no fallback: if the library is missing every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = ["RaError", "blockwise_attn_fwd", "blockwise_attn_bwd", "blockwise_ffn",
           "attn_decode", "decode_workspace_bytes", "decode_key_splits",
           "ffn_workspace_bytes", "fwd_split_workspace_bytes", "fwd_key_splits",
           "bwd_split_workspace_bytes",
           "blockwise_plan", "last_error", "lib_path",
           "load_library", "version", "RA_OK", "RA_E_INVALID", "RA_E_UNSUPPORTED",
           "RA_E_HIP", "RA_BF16", "RA_F32", "RA_PLACE_CONTIGUOUS", "RA_PLACE_STRIPED"]

RA_OK, RA_E_INVALID, RA_E_UNSUPPORTED, RA_E_HIP = 0, 1, 2, 3
RA_BF16, RA_F32 = 0, 1
RA_PLACE_CONTIGUOUS, RA_PLACE_STRIPED = 0, 1
_PLACEMENTS = {"contiguous": RA_PLACE_CONTIGUOUS, "striped": RA_PLACE_STRIPED}


def _placement(name: str) -> int:
    if name not in _PLACEMENTS:
        raise ValueError(f"placement must be one of {sorted(_PLACEMENTS)}")
    return _PLACEMENTS[name]


_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, "libra_attn.so")


class RaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ra_attn status {status}: {message}")
        self.status = status


def load_library():
    """Load ``libra_attn.so`` (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run __graft_entry__.build() or "
            "python -m long_context_exact_ra_amd.build")
    lib = ctypes.CDLL(path)
    c_i64, c_i32, c_vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    fwd_args = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32,
                c_i64, c_i64, c_i64, c_i64, ctypes.c_int, c_vp, c_vp]
    lib.ra_blockwise_attn_fwd.argtypes = fwd_args + [c_vp]
    lib.ra_blockwise_attn_fwd.restype = ctypes.c_int
    lib.ra_blockwise_attn_fwd_ex.argtypes = fwd_args + [c_vp, c_vp]
    lib.ra_blockwise_attn_fwd_ex.restype = ctypes.c_int
    lib.ra_blockwise_attn_fwd_placed.argtypes = (fwd_args[:9] + [ctypes.c_int] + fwd_args[9:]
                                                 + [c_vp, c_vp])
    lib.ra_blockwise_attn_fwd_placed.restype = ctypes.c_int
    lib.ra_blockwise_attn_fwd_split.argtypes = (fwd_args[:9] + [ctypes.c_int] + fwd_args[9:]
                                                + [c_vp, c_i32, c_vp, c_i64, c_vp])
    lib.ra_blockwise_attn_fwd_split.restype = ctypes.c_int
    lib.ra_blockwise_attn_fwd_split_noalloc.argtypes = (fwd_args[:9] + [ctypes.c_int]
                                                        + fwd_args[9:] + [c_vp, c_i32, c_vp])
    lib.ra_blockwise_attn_fwd_split_noalloc.restype = ctypes.c_int
    lib.ra_blockwise_attn_fwd_split_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64,
                                                                c_i32]
    lib.ra_blockwise_attn_fwd_split_workspace_bytes.restype = c_i64
    lib.ra_blockwise_attn_fwd_key_splits.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, c_i64,
                                                     c_i32, c_i32, ctypes.c_int, c_i32]
    lib.ra_blockwise_attn_fwd_key_splits.restype = c_i32
    lib.ra_blockwise_attn_bwd.argtypes = fwd_args[:14] + [c_vp] * 8
    lib.ra_blockwise_attn_bwd.restype = ctypes.c_int
    lib.ra_blockwise_attn_bwd_placed.argtypes = (fwd_args[:9] + [ctypes.c_int] + fwd_args[9:14]
                                                 + [c_vp] * 8)
    lib.ra_blockwise_attn_bwd_placed.restype = ctypes.c_int
    lib.ra_blockwise_attn_bwd_split.argtypes = (fwd_args[:9] + [ctypes.c_int] + fwd_args[9:14]
                                                + [c_vp] * 7 + [c_i32, c_vp, c_i64, c_vp])
    lib.ra_blockwise_attn_bwd_split.restype = ctypes.c_int
    lib.ra_blockwise_attn_bwd_split_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64,
                                                                c_i32]
    lib.ra_blockwise_attn_bwd_split_workspace_bytes.restype = c_i64
    lib.ra_blockwise_ffn_workspace_bytes.argtypes = [c_i64, c_i64]
    lib.ra_blockwise_ffn_workspace_bytes.restype = c_i64
    lib.ra_blockwise_ffn.argtypes = [c_vp] * 5 + [c_i64] * 5 + [ctypes.c_int, c_vp, c_vp,
                                                                c_i64, c_vp]
    lib.ra_blockwise_ffn.restype = ctypes.c_int
    lib.ra_attn_decode_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i32]
    lib.ra_attn_decode_workspace_bytes.restype = c_i64
    lib.ra_attn_decode_key_splits.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i32]
    lib.ra_attn_decode_key_splits.restype = c_i32
    lib.ra_attn_decode.argtypes = ([c_vp] * 3 + [c_i64] * 6 + [ctypes.c_int, c_i32, c_vp, c_i64,
                                   c_vp, c_vp, c_vp])
    lib.ra_attn_decode.restype = ctypes.c_int
    lib.ra_blockwise_plan.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i32, c_i32,
                                      c_vp, c_vp, c_vp]
    lib.ra_blockwise_plan.restype = ctypes.c_int
    lib.ra_blockwise_plan_placed.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i32, c_i32,
                                             ctypes.c_int, c_vp, c_vp, c_vp]
    lib.ra_blockwise_plan_placed.restype = ctypes.c_int
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_version.argtypes = []
    lib.ra_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().ra_last_error().decode()


def version() -> str:
    return load_library().ra_version().decode()


def _check(status: int):
    if status != RA_OK:
        raise RaError(status, last_error())


def _one_device(**tensors):
    """The one GPU that every given tensor (None skipped) lives on.  The
    library takes raw device pointers and launches on the current device, so
    a tensor on another GPU is refused here; the callers make that GPU
    current around the call."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def blockwise_plan(causal_block_size: Optional[int], q_chunk: int, k_chunk: int,
                   seq_q: int, ring_size: int, ring_index: int,
                   placement: str = "contiguous"):
    """Host-only ring order and chunk-pair skip decisions.

    Returns (kv_block_of_step int32 [N], run_bits uint8 [N, Lq/qc, Lq/kc],
    n_run_chunk_pairs).  placement: "contiguous" or "striped".
    """
    import numpy as np
    lib = load_library()
    order = np.zeros(max(ring_size, 1), dtype=np.int32)
    nq = seq_q // q_chunk if q_chunk > 0 else 0
    nk = seq_q // k_chunk if k_chunk > 0 else 0
    run = np.zeros((max(ring_size, 1), nq, nk), dtype=np.uint8)
    n = ctypes.c_int64(0)
    _check(lib.ra_blockwise_plan_placed(int(causal_block_size or 0), q_chunk, k_chunk, seq_q,
                                        ring_size, ring_index, _placement(placement),
                                        order.ctypes.data, run.ctypes.data,
                                        ctypes.addressof(n)))
    return order, run, n.value


def fwd_split_workspace_bytes(batch: int, seq_q: int, heads: int, head_dim: int,
                              key_splits: int) -> int:
    """Device bytes ``ra_blockwise_attn_fwd_split`` needs as workspace."""
    return int(load_library().ra_blockwise_attn_fwd_split_workspace_bytes(
        batch, seq_q, heads, head_dim, key_splits))


def bwd_split_workspace_bytes(batch: int, seq_q: int, heads: int, head_dim: int,
                              key_splits: int) -> int:
    """Device bytes ``ra_blockwise_attn_bwd_split`` needs as workspace."""
    return int(load_library().ra_blockwise_attn_bwd_split_workspace_bytes(
        batch, seq_q, heads, head_dim, key_splits))


def fwd_key_splits(batch: int, seq_q: int, heads: int, dtype: int,
                   causal_block_size: Optional[int], ring_size: int, ring_index: int,
                   compute_units: int, placement: str = "contiguous") -> int:
    """The library's key split count for a share on a GPU with
    ``compute_units`` compute units (1 = no split)."""
    return int(load_library().ra_blockwise_attn_fwd_key_splits(
        batch, seq_q, heads, dtype, int(causal_block_size or 0), ring_size, ring_index,
        _placement(placement), compute_units))


def blockwise_attn_fwd(q, k, v, segment_ids=None, causal_block_size: Optional[int] = None,
                       q_chunk: int = 512, k_chunk: int = 512, ring_size: int = 1,
                       ring_index: int = 0, *, out=None, lse=None, run_map=None,
                       stream=None, placement: str = "contiguous", key_splits=1,
                       workspace=None) -> Tuple[object, object]:
    """Forward of ring position ``ring_index``: returns (out, lse).

    q: [B, Lq, H, D] and k, v: [B, ring_size * Lq, H, D], contiguous CUDA
    (HIP) tensors of one dtype (bfloat16 or float32); segment_ids: int32
    [B, ring_size * Lq] or None; causal_block_size None/0 = non-causal.
    out ([B, Lq, H, D], q's dtype) and lse ([B, H, Lq], float32) are
    allocated when not given.  run_map: optional uint8 device tensor
    [ring_size, Lq / q_chunk, Lq / k_chunk] that receives the kernel's
    chunk-pair decisions.  The work is enqueued on ``stream`` (default: the
    current torch stream).  placement: "contiguous" (block r holds positions
    r*Lq ..) or "striped" (block r holds positions r, r + N, ..; k, v and
    segment_ids in that storage order; token causal or non-causal only).
    key_splits: 1 (the walk of each query tile runs in one workgroup), an
    integer up to 64 (``ra_blockwise_attn_fwd_split``: the walk is cut into
    that many runs whose partial results a second kernel folds), or "auto"
    (the library's count for this GPU's compute units).  workspace: a device
    tensor of at least ``fwd_split_workspace_bytes`` bytes, allocated when
    not given and the call splits; or the string "scratch"
    (``ra_blockwise_attn_fwd_split_noalloc``: the partials go to the
    library's own 64 MiB scratch and the library allocates nothing; pass out
    and lse to allocate nothing here either).
    """
    import torch
    lib = load_library()
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D device tensor")
    B, Lq, H, D = q.shape
    if tuple(k.shape) != (B, ring_size * Lq, H, D) or k.shape != v.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)} != {(B, ring_size * Lq, H, D)}")
    seg_ptr = None
    if segment_ids is not None:
        if (segment_ids.dtype != torch.int32 or not segment_ids.is_cuda
                or not segment_ids.is_contiguous()
                or tuple(segment_ids.shape) != (B, ring_size * Lq)):
            raise ValueError("segment_ids must be a contiguous int32 device tensor [B, S]")
        seg_ptr = segment_ids.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous with q's shape and dtype")
    if tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, Lq]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    dt = RA_BF16 if q.dtype == torch.bfloat16 else RA_F32
    place = _placement(placement)
    if key_splits == "auto":
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        key_splits = fwd_key_splits(B, Lq, H, dt, causal_block_size, ring_size, ring_index, cus,
                                    placement)
    key_splits = int(key_splits)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), seg_ptr, int(causal_block_size or 0),
            q_chunk, k_chunk, ring_size, ring_index, B, Lq, H, D, dt,
            out.data_ptr(), lse.data_ptr()]
    map_ptr = None
    if run_map is not None:
        nq = Lq // q_chunk if q_chunk else 0
        nk = Lq // k_chunk if k_chunk else 0
        if (run_map.dtype != torch.uint8 or not run_map.is_cuda
                or not run_map.is_contiguous()
                or tuple(run_map.shape) != (ring_size, nq, nk)):
            raise ValueError("run_map must be a contiguous uint8 device tensor [N, nq, nk]")
        map_ptr = run_map.data_ptr()
    dev = _one_device(q=q, k=k, v=v, segment_ids=segment_ids, out=out, lse=lse, run_map=run_map,
                      workspace=workspace if key_splits != 1 and not isinstance(workspace, str)
                      else None)
    with torch.cuda.device(dev):
        if isinstance(workspace, str):
            if workspace != "scratch":
                raise ValueError('workspace must be a device tensor, None or "scratch"')
            _check(lib.ra_blockwise_attn_fwd_split_noalloc(*args[:9], place, *args[9:], map_ptr,
                                                           key_splits, sptr))
        elif key_splits != 1:
            need = fwd_split_workspace_bytes(B, Lq, H, D, key_splits)
            if workspace is None:
                workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
            if not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous device tensor")
            ws_bytes = workspace.numel() * workspace.element_size()
            _check(lib.ra_blockwise_attn_fwd_split(*args[:9], place, *args[9:], map_ptr, key_splits,
                                                   workspace.data_ptr(), ws_bytes, sptr))
        elif place != RA_PLACE_CONTIGUOUS:
            _check(lib.ra_blockwise_attn_fwd_placed(*args[:9], place, *args[9:], map_ptr, sptr))
        elif map_ptr is not None:
            _check(lib.ra_blockwise_attn_fwd_ex(*args, map_ptr, sptr))
        else:
            _check(lib.ra_blockwise_attn_fwd(*args, sptr))
    return out, lse


def blockwise_attn_bwd(q, k, v, out, lse, dout, segment_ids=None,
                       causal_block_size: Optional[int] = None, q_chunk: int = 512,
                       k_chunk: int = 512, ring_size: int = 1, ring_index: int = 0, *,
                       dq=None, dk=None, dv=None, delta=None, stream=None,
                       placement: str = "contiguous", key_splits=1, workspace=None):
    """Backward of ring position ``ring_index``: returns (dq, dk, dv, delta).

    q, k, v, segment_ids and the mask arguments as for blockwise_attn_fwd
    (bfloat16 or float32); out and lse are that forward's outputs and dout
    the upstream gradient of out ([B, Lq, H, D], q's dtype).  dq [B, Lq, H, D],
    dk, dv [B, ring_size * Lq, H, D] and delta [B, H, Lq] are float32 and
    allocated when not given; dk and dv hold this share's contribution.
    placement: as for blockwise_attn_fwd (dk, dv and segment_ids in storage
    order).  key_splits / workspace: as for blockwise_attn_fwd
    (``ra_blockwise_attn_bwd_split``; the split applies to the dq kernel,
    whose addends a last kernel sums).
    """
    import torch
    lib = load_library()
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("the backward takes bfloat16 or float32 inputs")
    dt = RA_BF16 if q.dtype == torch.bfloat16 else RA_F32
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D device tensor of q's dtype")
    B, Lq, H, D = q.shape
    S = ring_size * Lq
    if tuple(k.shape) != (B, S, H, D) or k.shape != v.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)} != {(B, S, H, D)}")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    if (tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32 or not lse.is_cuda
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 device tensor [B, H, Lq]")
    seg_ptr = None
    if segment_ids is not None:
        if (segment_ids.dtype != torch.int32 or not segment_ids.is_cuda
                or not segment_ids.is_contiguous() or tuple(segment_ids.shape) != (B, S)):
            raise ValueError("segment_ids must be a contiguous int32 device tensor [B, S]")
        seg_ptr = segment_ids.data_ptr()
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, Lq, H, D), **f32) if dq is None else dq
    dk = torch.empty((B, S, H, D), **f32) if dk is None else dk
    dv = torch.empty((B, S, H, D), **f32) if dv is None else dv
    delta = torch.empty((B, H, Lq), **f32) if delta is None else delta
    for name, t, shape in (("dq", dq, (B, Lq, H, D)), ("dk", dk, (B, S, H, D)),
                           ("dv", dv, (B, S, H, D)), ("delta", delta, (B, H, Lq))):
        if (tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 device tensor {shape}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if key_splits == "auto":
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        key_splits = fwd_key_splits(B, Lq, H, dt, causal_block_size, ring_size,
                                    ring_index, cus, placement)
    key_splits = int(key_splits)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), seg_ptr, int(causal_block_size or 0),
            q_chunk, k_chunk, ring_size, ring_index, _placement(placement), B, Lq, H, D, dt,
            out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
            dv.data_ptr(), delta.data_ptr()]
    dev = _one_device(q=q, k=k, v=v, out=out, lse=lse, dout=dout, segment_ids=segment_ids, dq=dq,
                      dk=dk, dv=dv, delta=delta,
                      workspace=workspace if key_splits != 1 else None)
    with torch.cuda.device(dev):
        if key_splits != 1:
            need = bwd_split_workspace_bytes(B, Lq, H, D, key_splits)
            if workspace is None:
                workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
            if not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous device tensor")
            ws_bytes = workspace.numel() * workspace.element_size()
            _check(lib.ra_blockwise_attn_bwd_split(*args, key_splits, workspace.data_ptr(),
                                                   ws_bytes, sptr))
        else:
            _check(lib.ra_blockwise_attn_bwd_placed(*args, sptr))
    return dq, dk, dv, delta


def ffn_workspace_bytes(chunk_size: int, ffn_hidden: int) -> int:
    """Bytes of workspace ``blockwise_ffn`` needs (one chunk's bf16 hidden
    activations)."""
    return int(load_library().ra_blockwise_ffn_workspace_bytes(chunk_size, ffn_hidden))


def blockwise_ffn(x, w1, b1, w2, b2, chunk_size: int, *, y=None, workspace=None,
                  stream=None):
    """y = max(0, x W1 + b1) W2 + b2 computed one sequence chunk at a time.

    x [B, L, hidden], w1 [hidden, ffn], b1 [ffn], w2 [ffn, hidden], b2
    [hidden]: contiguous bfloat16 device tensors; chunk_size divides L.  y
    and the workspace (uint8, at least ffn_workspace_bytes(chunk_size, ffn)
    bytes) are allocated when not given.  Returns y.
    """
    import torch
    lib = load_library()
    for name, t in (("x", x), ("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    if x.dim() != 3:
        raise ValueError("x must be [batch, seq, hidden]")
    B, L, H = x.shape
    Fh = w1.shape[1] if w1.dim() == 2 else -1
    if (tuple(w1.shape) != (H, Fh) or tuple(b1.shape) != (Fh,) or tuple(w2.shape) != (Fh, H)
            or tuple(b2.shape) != (H,)):
        raise ValueError("weights must be w1 [hidden, ffn], b1 [ffn], w2 [ffn, hidden], b2 [hidden]")
    if y is None:
        y = torch.empty_like(x)
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("y must be contiguous with x's shape and dtype")
    need = ffn_workspace_bytes(chunk_size, Fh) if chunk_size > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    dev = _one_device(x=x, w1=w1, b1=b1, w2=w2, b2=b2, y=y, workspace=workspace)
    with torch.cuda.device(dev):
        _check(lib.ra_blockwise_ffn(x.data_ptr(), w1.data_ptr(), b1.data_ptr(), w2.data_ptr(),
                                    b2.data_ptr(), B, L, H, Fh, chunk_size, RA_BF16, y.data_ptr(),
                                    workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), sptr))
    return y


def decode_workspace_bytes(batch: int, n_new: int, heads: int, head_dim: int,
                           key_splits: int) -> int:
    """Bytes of workspace ``attn_decode`` needs for ``key_splits`` splits (0
    for one split)."""
    return int(load_library().ra_attn_decode_workspace_bytes(batch, n_new, heads, head_dim,
                                                             key_splits))


def decode_key_splits(batch: int, n_new: int, heads: int, cache_idx: int,
                      compute_units: int) -> int:
    """The library's key-split count for a decoding step."""
    return int(load_library().ra_attn_decode_key_splits(batch, n_new, heads, cache_idx,
                                                        compute_units))


def attn_decode(q, k_cache, v_cache, cache_idx: int, *, key_splits="auto", workspace=None,
                out=None, lse=None, stream=None) -> Tuple[object, object]:
    """One incremental-decoding step: returns (out, lse).

    q: [B, n_new, H, D], the step's new tokens at positions cache_idx ..
    cache_idx + n_new - 1; k_cache, v_cache: [B, R, H, D] with their rows
    up to cache_idx + n_new - 1 filled (the new tokens' keys and values
    included).  Contiguous device tensors of one dtype (bfloat16 or float32).
    Query t attends to cache rows 0 .. cache_idx + t.  out ([B, n_new, H, D],
    q's dtype) and lse ([B, H, n_new], float32) are allocated when not given.
    key_splits: an integer in [1, 1024] or "auto" (the library's count for
    this GPU); workspace: a device tensor of at least
    ``decode_workspace_bytes`` bytes, allocated when not given and needed.
    """
    import torch
    lib = load_library()
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {q.dtype}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D device tensor")
    B, T, H, D = q.shape
    R = k_cache.shape[1]
    if (k_cache.shape[0], k_cache.shape[2], k_cache.shape[3]) != (B, H, D) or \
            v_cache.shape != k_cache.shape:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous with q's shape and dtype")
    if tuple(lse.shape) != (B, H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, n_new]")
    if key_splits == "auto":
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        key_splits = decode_key_splits(B, T, H, cache_idx, cus)
    key_splits = int(key_splits)
    ws_ptr, ws_bytes = None, 0
    if key_splits > 1:
        need = decode_workspace_bytes(B, T, H, D, key_splits)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    dt = RA_BF16 if q.dtype == torch.bfloat16 else RA_F32
    dev = _one_device(q=q, k_cache=k_cache, v_cache=v_cache, out=out, lse=lse,
                      workspace=workspace if key_splits > 1 else None)
    with torch.cuda.device(dev):
        _check(lib.ra_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                  int(cache_idx), R, B, T, H, D, dt, key_splits, ws_ptr, ws_bytes,
                                  out.data_ptr(), lse.data_ptr(), sptr))
    return out, lse
