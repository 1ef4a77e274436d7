"""CPU fp64 oracle for one incremental-decoding step over a KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the library
in ``long_context_exact_ra_amd`` never does, and this module imports nothing
from it.

Sources (web pages; cited by title and section):

* "RingAttention与传统注意力机制对比为什么它是大语言模型的终极解决方案",
  section "3. 推理成本显著降低" (at inference the blockwise structure makes
  incremental decoding and KV-cache handling efficient; the module tree
  lists an inference variant of the ring code) and section "关键参数配置"
  (``cache_idx`` is the index into the inference cache).
* "从论文到代码：深入理解RingAttention的块注意力计算逻辑", section
  "RingAttention的算法原理" (``cache_idx`` is an argument of the ring
  forward beside the segment ids) and section "3. 因果注意力掩码支持"
  (causal masking: a query sees only keys at or before its position).
* "Ring Attention with Blockwise Transformers for Near-Infinite Context",
  section 三, the self-attention equation softmax(Q K^T / sqrt(d)) V.

Readings (the pages print no decoding code; each reading is also listed in
the design notes of the repository):

* ``cache_idx`` is the number of tokens already in the cache: the step's
  n_new query tokens have global positions cache_idx .. cache_idx + n_new
  - 1, and their keys and values already sit in cache rows cache_idx ..
  cache_idx + n_new - 1 (the caller writes them, as a cache update does);
* the mask is token causal on those positions: query t sees cache rows
  0 .. cache_idx + t; cache rows past cache_idx + n_new - 1 are never read;
* the outputs follow the forward's conventions: out [B, n_new, H, D] and the
  natural-log lse [B, H, n_new].

Everything is float64; matmul and exp are library primitives used as single
steps, nothing is tiled or reordered.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly on the CPU
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _scale(head_dim: int) -> float:
    """1 / sqrt(D), the self-attention equation's scale."""
    return 1.0 / np.sqrt(head_dim)


def _query_positions(cache_idx: int, n_new: int) -> np.ndarray:
    """Global positions of the step's new tokens: cache_idx .. + n_new - 1."""
    return cache_idx + np.arange(n_new)


def _rows_read(cache_idx: int, n_new: int) -> int:
    """Cache rows the step reads: every token up to the last new one."""
    return cache_idx + n_new


def _visible(pos_q: np.ndarray, pos_k: np.ndarray) -> np.ndarray:
    """Token-causal visibility [Tq, Tk]: a key at or before the query."""
    return pos_k[None, :] <= pos_q[:, None]


def decode_attention(q, k_cache, v_cache, cache_idx: int,
                     heads: Optional[Sequence[int]] = None):
    """Masked softmax(q K^T / sqrt(D)) V of one decoding step.

    q: [B, T, H, D], the step's T new query tokens (positions cache_idx ..
    cache_idx + T - 1); k_cache, v_cache: [B, R, H, D] with R >= cache_idx +
    T, rows 0 .. cache_idx + T - 1 valid (later rows are ignored).  heads:
    optional subset of heads.

    Returns (out [B, T, Hs, D], lse [B, Hs, T]) in float64.
    """
    qf = _as_f64(q)
    B, T, H, D = qf.shape
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != B or \
            tuple(k_cache.shape[2:]) != (H, D):
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match q {qf.shape}")
    cache_idx = int(cache_idx)
    if cache_idx < 0 or cache_idx + T > k_cache.shape[1]:
        raise ValueError(f"cache_idx {cache_idx} + {T} new tokens outside the "
                         f"{k_cache.shape[1]} cache rows")
    n = _rows_read(cache_idx, T)
    heads = list(range(H)) if heads is None else list(heads)
    scale = _scale(D)
    allow = _visible(_query_positions(cache_idx, T), np.arange(n))  # cache row j = position j
    out = np.zeros((B, T, len(heads), D), dtype=np.float64)
    lse = np.zeros((B, len(heads), T), dtype=np.float64)
    for b in range(B):
        for hi, h in enumerate(heads):
            # Only the rows read are upcast, one head at a time.
            kf = _as_f64(k_cache[b, :n, h, :])
            vf = _as_f64(v_cache[b, :n, h, :])
            s = (qf[b, :, h, :] @ kf.T) * scale
            s = np.where(allow, s, -np.inf)
            m = s.max(axis=1)
            has = np.isfinite(m)              # (every query sees key 0 under the readings)
            p = np.where(allow, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
            den = p.sum(axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                out[b, :, hi, :] = np.where(has[:, None],
                                            (p @ vf) / np.where(has, den, 1.0)[:, None],
                                            0.0)
                lse[b, hi, :] = np.where(has, m + np.log(np.where(has, den, 1.0)), -np.inf)
    return out, lse
