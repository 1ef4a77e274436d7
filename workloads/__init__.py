"""Seeded synthetic workloads for the blockwise ring-attention forward.

This module only *generates inputs*: shapes, seeds, Gaussian draws and
document-length segment ids.  It holds none of the attention arithmetic, so
both the GPU library's tests/benchmark and the CPU oracle can be fed from it
without sharing any of the method's code.

The workloads stand in for the pages' training runs (7B- and 65B-parameter
models at up to 4M-token context on TPUv4-1024, "Ring Attention with
Blockwise Transformers for Near-Infinite Context", section 五 "实验结果"):
one device's share of the ring at the real per-device shape, with Gaussian
Q/K/V.  No dataset or trained weight is involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "block_seed", "document_segments",
           "make_block", "make_dout", "make_q", "make_qkv", "make_segments", "to_storage_order",
           "FfnWorkload", "FFN_WORKLOADS", "make_ffn_inputs",
           "DecodeWorkload", "DECODE_WORKLOADS", "make_decode_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_q: int                 # local query block length Lq (= KV block length)
    ring_size: int             # N
    ring_indices: Tuple[int, ...]
    heads: int
    head_dim: int
    dtype: str                 # "bf16" | "f32"
    causal_block_size: Optional[int]   # None = non-causal
    q_chunk: int
    k_chunk: int
    segments: bool = False
    std: float = 1.0           # Q, K, V ~ std * N(0, 1)
    seed: int = 0
    poison_unused: bool = False  # fill KV blocks that no chunk pair reads with NaN
    placement: str = "contiguous"  # or "striped": block r holds positions r, r + N, ...
    notes: str = field(default="", compare=False)

    @property
    def seq_k(self) -> int:
        return self.ring_size * self.seq_q


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_plumbing", 1, 64, 4, (0, 1, 2, 3), 2, 64, "f32", None,
                 32, 32, seed=20261201,
                 notes="seq 256 = 4 ring blocks of 64; non-causal; fp32"),
        Workload("small_causal", 1, 1024, 8, tuple(range(8)), 8, 128, "bf16", 1,
                 512, 512, seed=20261202,
                 notes="seq 8192 = 8 ring blocks of 1024; token causal"),
        Workload("share_7b_512k", 1, 32768, 16, (15,), 32, 128, "bf16", 1,
                 2048, 2048, seed=20261203,
                 notes="7B-shaped share: ring position 15 of 16, 512K context"),
        Workload("packed_documents", 4, 2048, 8, tuple(range(8)), 32, 128, "bf16", 1,
                 512, 512, segments=True, seed=20261204,
                 notes="seq 16384 = 8 blocks of 2048; causal + document segments"),
        Workload("share_65b_4m", 1, 16384, 256, (128,), 64, 128, "bf16", 16384,
                 512, 512, std=0.5, seed=20261205, poison_unused=True,
                 notes="65B-shaped share: ring position 128 of 256, 4M context, "
                       "block-causal with causal_block_size 16384"),
        # striped placement (block r holds positions r, r + N, r + 2N, ...)
        Workload("small_causal_striped", 1, 1024, 8, tuple(range(8)), 8, 128, "bf16", 1,
                 512, 512, seed=20261208, placement="striped",
                 notes="small_causal's shape under striped placement"),
        Workload("share_7b_512k_striped", 1, 32768, 16, (15,), 32, 128, "bf16", 1,
                 2048, 2048, seed=20261209, placement="striped",
                 notes="the 7B-shaped share under striped placement, ring position 15 of 16"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def block_seed(base: int, tensor: str, block: int) -> int:
    """Seed of one ring block of one tensor, so that any block can be
    regenerated on its own (q: 0, k: 1, v: 2)."""
    return base * 4099 + {"q": 0, "k": 1, "v": 2}[tensor] * 1_000_003 + block


def document_segments(batch: int, seq: int, seed: int, mean: int = 2048,
                      lo: int = 64, hi: int = 16384) -> np.ndarray:
    """Segment ids of packed documents: lengths ~ Geometric(1/mean) clipped to
    [lo, hi], drawn until the row is full; the last document is truncated to
    fit.  The id of a token is the ordinal of its document in the row."""
    rng = np.random.default_rng(seed)
    out = np.empty((batch, seq), dtype=np.int32)
    for b in range(batch):
        pos = 0
        doc = 0
        while pos < seq:
            n = int(np.clip(rng.geometric(1.0 / mean), lo, hi))
            n = min(n, seq - pos)
            out[b, pos:pos + n] = doc
            pos += n
            doc += 1
    return out


def _torch():
    import torch
    return torch


def _dtype(name: str):
    torch = _torch()
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_block(shape: Sequence[int], seed: int, std: float, dtype: str,
               device) -> "object":
    """One Gaussian block: N(0,1) drawn in fp32 with a seeded generator on
    ``device``, scaled by ``std`` and rounded (RNE) to ``dtype``."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(_dtype(dtype))


def make_q(w: Workload, ring_index: int, device="cpu"):
    """Q for ring position ``ring_index`` alone (the same draw as make_qkv)."""
    return make_block((w.batch, w.seq_q, w.heads, w.head_dim),
                      block_seed(w.seed, "q", ring_index), w.std, w.dtype, device)


def make_dout(w: Workload, ring_index: int, device="cpu"):
    """An upstream gradient of the output for ring position ``ring_index``:
    N(0,1) drawn in fp32 with its own seed, rounded to the workload dtype."""
    return make_block((w.batch, w.seq_q, w.heads, w.head_dim),
                      w.seed * 7919 + 5 * 1_000_003 + ring_index, 1.0, w.dtype, device)


def make_qkv(w: Workload, ring_index: int, device="cpu",
             kv_blocks: Optional[Sequence[int]] = None):
    """Q for ring position ``ring_index`` and K, V for the whole ring.

    Each ring block is drawn with its own seed.  Blocks not listed in
    ``kv_blocks`` (default: all) are filled with NaN: a poisoned block must
    never influence the result.
    """
    torch = _torch()
    B, Lq, H, D = w.batch, w.seq_q, w.heads, w.head_dim
    q = make_q(w, ring_index, device)
    k = torch.empty((B, w.seq_k, H, D), dtype=_dtype(w.dtype), device=device)
    v = torch.empty_like(k)
    blocks = set(range(w.ring_size) if kv_blocks is None else kv_blocks)
    for kb in range(w.ring_size):
        sl = slice(kb * Lq, (kb + 1) * Lq)
        if kb in blocks:
            k[:, sl] = make_block((B, Lq, H, D), block_seed(w.seed, "k", kb),
                                  w.std, w.dtype, device)
            v[:, sl] = make_block((B, Lq, H, D), block_seed(w.seed, "v", kb),
                                  w.std, w.dtype, device)
        else:
            k[:, sl] = float("nan")
            v[:, sl] = float("nan")
    return q, k, v


def to_storage_order(x: np.ndarray, ring_size: int, placement: str) -> np.ndarray:
    """Reorder a natural-order [B, S, ...] array into the storage order of a
    placement: unchanged for contiguous; for striped, block kb (rows kb * Lq
    .. kb * Lq + Lq - 1) takes positions kb, kb + N, kb + 2N, ..."""
    if placement == "contiguous":
        return x
    B, S = x.shape[:2]
    y = x.reshape((B, S // ring_size, ring_size) + x.shape[2:])
    return np.ascontiguousarray(np.swapaxes(y, 1, 2)).reshape(x.shape)


def make_segments(w: Workload, device="cpu"):
    """Segment ids [B, S] (int32) for workloads with packed documents, else
    None; documents are laid out along the global positions and the ids are
    returned in the workload's storage order."""
    if not w.segments:
        return None
    torch = _torch()
    seg = document_segments(w.batch, w.seq_k, w.seed + 3)
    seg = to_storage_order(seg, w.ring_size, w.placement)
    return torch.from_numpy(seg).to(device)


# ---------------------------------------------------------------------------
# Blockwise feedforward
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class FfnWorkload:
    """Shapes of one blockwise-feedforward call: x [batch, seq, hidden],
    w1 [hidden, ffn], w2 [ffn, hidden], processed in chunks of ``chunk``."""
    name: str
    batch: int
    seq: int
    hidden: int
    ffn: int
    chunk: int
    seed: int = 0


FFN_WORKLOADS = {w.name: w for w in [
    # the 7B model's width (4096) with a 4x feedforward, over the 7B share's
    # local block of 32768 tokens, chunks of 2048
    FfnWorkload("ffn_7b_share", 1, 32768, 4096, 16384, 2048, seed=20261206),
    FfnWorkload("ffn_small", 2, 256, 256, 1024, 64, seed=20261207),
]}


def make_ffn_inputs(w: FfnWorkload, device="cpu"):
    """x ~ N(0, 1); w1 ~ N(0, 1/hidden); w2 ~ N(0, 1/ffn); b1, b2 ~ N(0, 0.1^2);
    each drawn in fp32 with its own seed and rounded (RNE) to bf16."""
    H, Fh = w.hidden, w.ffn
    x = make_block((w.batch, w.seq, H), w.seed * 31 + 1, 1.0, "bf16", device)
    w1 = make_block((H, Fh), w.seed * 31 + 2, H ** -0.5, "bf16", device)
    b1 = make_block((Fh,), w.seed * 31 + 3, 0.1, "bf16", device)
    w2 = make_block((Fh, H), w.seed * 31 + 4, Fh ** -0.5, "bf16", device)
    b2 = make_block((H,), w.seed * 31 + 5, 0.1, "bf16", device)
    return x, w1, b1, w2, b2


@dataclass(frozen=True)
class DecodeWorkload:
    """One decoding step over a KV cache: q [batch, n_new, heads, head_dim]
    at positions cache_idx .. cache_idx + n_new - 1, cache [batch,
    cache_rows, heads, head_dim] with rows up to cache_idx + n_new - 1
    filled; rows past them hold NaN (they must never be read)."""
    name: str
    batch: int
    heads: int
    head_dim: int
    cache_rows: int
    cache_idx: int
    n_new: int
    dtype: str = "bf16"
    std: float = 1.0
    seed: int = 0

    @property
    def n_keys(self) -> int:
        return self.cache_idx + self.n_new


DECODE_WORKLOADS = {w.name: w for w in [
    # the 7B-shaped model (32 heads of 128) generating the last token of
    # its 512K context: the whole cache is read once
    DecodeWorkload("decode_7b_512k", 1, 32, 128, 524288, 524287, 1, seed=20261208),
    # a small batched step with several new tokens (a ragged cache length)
    DecodeWorkload("decode_small", 2, 8, 128, 8192, 5000, 4, seed=20261209),
]}


def make_decode_inputs(w: DecodeWorkload, device="cpu"):
    """q, k_cache, v_cache ~ std * N(0, 1), each drawn in fp32 with its own
    seed and rounded (RNE) to the dtype; cache rows past the step's last
    token are NaN."""
    q = make_block((w.batch, w.n_new, w.heads, w.head_dim), w.seed * 31 + 1, w.std, w.dtype,
                   device)
    k = make_block((w.batch, w.cache_rows, w.heads, w.head_dim), w.seed * 31 + 2, w.std,
                   w.dtype, device)
    v = make_block((w.batch, w.cache_rows, w.heads, w.head_dim), w.seed * 31 + 3, w.std,
                   w.dtype, device)
    if w.n_keys < w.cache_rows:
        k[:, w.n_keys:] = float("nan")
        v[:, w.n_keys:] = float("nan")
    return q, k, v
