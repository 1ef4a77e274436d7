"""CPU fp64 oracle for the backward of the blockwise exact attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the library
in ``long_context_exact_ra_amd`` never does, and this module imports nothing
from it.

What it computes.  The pages state that the ring-attention implementation
holds a forward and a backward pass (the carry-based forward of
"从论文到代码：深入理解RingAttention的块注意力计算逻辑" is paired with a
backward function there) and that the method is exact ("Ring Attention with
Blockwise Transformers for Near-Infinite Context", section 四), but they
print no backward equations.  The backward is therefore taken as the exact
derivative of the forward's plain definition (the self-attention equation of
section 三, with the visibility mask of ``attention.visible``): for one query
row i with visible keys j,

    s_ij = scale * <q_i, k_j>,   p_ij = exp(s_ij - lse_i),   out_i = sum_j p_ij v_j

and, for an upstream gradient dout, by the chain rule:

    dv_j  = sum_i p_ij dout_i
    dp_ij = <dout_i, v_j>
    ds_ij = p_ij * (dp_ij - delta_i),  delta_i = sum_j p_ij dp_ij = <dout_i, out_i>
    dq_i  = scale * sum_j ds_ij k_j
    dk_j  = scale * sum_i ds_ij q_i

(the middle line is the Jacobian of a softmax row applied to dp).  A row
with no visible key has a constant output and contributes nothing.

Everything is float64; inputs are upcast exactly.  Matrix products and exp
are library primitives used as single steps; nothing is tiled or fused.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import (_as_f64, _check_kv_tail_masked, _scale, key_positions,
                        query_positions, visible)

__all__ = ["attention_bwd"]


def _softmax_rows(s: np.ndarray, allow: np.ndarray):
    """p = softmax over the visible entries of each row, and the row lse.
    Rows without a visible entry give p = 0 and lse = -inf."""
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    has = np.isfinite(m)
    e = np.where(allow, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
    den = e.sum(axis=1)
    p = np.where(has[:, None], e / np.where(has, den, 1.0)[:, None], 0.0)
    return p, has


def _row_delta(dout_rows: np.ndarray, out_rows: np.ndarray) -> np.ndarray:
    """delta_i = <dout_i, out_i> = sum_j p_ij dp_ij (the softmax-Jacobian term)."""
    return np.einsum("id,id->i", dout_rows, out_rows)


def _ds_from_dp(p: np.ndarray, dp: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """Gradient of the scores: the Jacobian of each softmax row applied to dp."""
    return p * (dp - delta[:, None])


def attention_bwd(q, k, v, dout, segment_ids=None, causal_block_size=None,
                  ring_size: int = 1, ring_index: int = 0,
                  rows: Optional[Sequence[int]] = None,
                  heads: Optional[Sequence[int]] = None,
                  kv_len: Optional[int] = None,
                  max_scores: int = 1 << 24,
                  placement: str = "contiguous",
                  keys: Optional[Sequence[int]] = None):
    """Gradients of sum(dout * out) for one device's query block.

    q, dout: [B, Lq, H, D] (ring position ``ring_index``); k, v: [B, S, H, D]
    with S = ring_size * Lq (or the first ``kv_len`` keys when the rest are
    causally invisible from every requested row); segment_ids [B, S] in
    storage order (the order of the rows of k) or None.
    rows / heads: optional subsets of local query rows / heads.
    placement: "contiguous" or "striped", as in ``attention.attention_fwd``.
    keys: optional subset of key storage rows (indices into the first
    ``kv_len`` rows of k); dk and dv are then returned for those keys only,
    in the given order.  The scores, probabilities and row terms are still
    taken over every key of each row: a key's gradient is a sum over all
    rows that see it, and each row's softmax runs over all its keys.

    Returns (dq [B, R, Hs, D], dk [B, K, Hs, D], dv [B, K, Hs, D]) in
    float64, K = kv_len or len(keys).  dq is exact for the selected rows; dk
    and dv hold the contributions of the selected rows only (the full
    gradient of this device's share when ``rows`` is None).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    dout = _as_f64(dout)
    B, Lq, H, D = q.shape
    S = ring_size * Lq
    kv_len = S if kv_len is None else int(kv_len)
    if k.shape != (B, kv_len, H, D) or v.shape != (B, kv_len, H, D):
        raise ValueError(f"k/v shape {k.shape} != {(B, kv_len, H, D)}")
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    if not 0 <= ring_index < ring_size:
        raise ValueError("ring_index out of range")
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(H)) if heads is None else list(heads)
    seg = None if segment_ids is None else np.asarray(
        segment_ids.cpu().numpy() if hasattr(segment_ids, "cpu") else segment_ids,
        dtype=np.int64)

    pq_all = query_positions(Lq, ring_index, ring_size, placement)[rows]
    sq_all = ring_index * Lq + rows          # storage rows of the queries
    if placement == "striped" and kv_len < S:
        raise ValueError("kv_len < seq_k is only supported for contiguous placement")
    _check_kv_tail_masked(pq_all, kv_len, S, causal_block_size)
    pk = key_positions(S, ring_size, placement)[:kv_len]
    scale = _scale(D)
    ksel = np.arange(kv_len) if keys is None else np.asarray(keys, dtype=np.int64)
    if ksel.size and (ksel.min() < 0 or ksel.max() >= kv_len):
        raise ValueError("keys must index the first kv_len key rows")

    dq = np.zeros((B, rows.shape[0], len(heads), D), dtype=np.float64)
    dk = np.zeros((B, ksel.shape[0], len(heads), D), dtype=np.float64)
    dv = np.zeros((B, ksel.shape[0], len(heads), D), dtype=np.float64)
    step = max(1, max_scores // max(kv_len, 1))
    for b in range(B):
        for hi, h in enumerate(heads):
            K = k[b, :, h, :]
            V = v[b, :, h, :]
            for r0 in range(0, rows.shape[0], step):
                sel = rows[r0:r0 + step]
                pq = pq_all[r0:r0 + step]
                Q = q[b, sel, h, :]
                dO = dout[b, sel, h, :]
                allow = visible(pq, pk, causal_block_size,
                                None if seg is None else seg[b, sq_all[r0:r0 + step]],
                                None if seg is None else seg[b, :kv_len])
                s = np.where(allow, (Q @ K.T) * scale, -np.inf)
                p, _ = _softmax_rows(s, allow)
                out_rows = p @ V
                dp = dO @ V.T
                ds = _ds_from_dp(p, dp, _row_delta(dO, out_rows))
                dq[b, r0:r0 + step, hi, :] = (ds @ K) * scale
                if keys is not None:
                    ds = ds[:, ksel]
                    p = p[:, ksel]
                dk[b, :, hi, :] += (ds.T @ Q) * scale
                dv[b, :, hi, :] += p.T @ dO
    return dq, dk, dv
