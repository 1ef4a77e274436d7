"""Helpers shared by the GPU parity tests: slicing device tensors into the
CPU oracle and the acceptance bounds."""

from __future__ import annotations

import numpy as np
import torch

import oracle

# Acceptance bounds.  bf16 inputs: max |err| <= 2e-2 and mean |err| <= 2e-3
# on out and lse; fp32 inputs: max |err| <= 1e-5.  The relative L2 guard
# keeps the absolute bounds from passing vacuously on long rows, where |out|
# itself is ~1e-3.
BOUNDS = {
    torch.bfloat16: dict(max=2e-2, mean=2e-3, rel_l2=1e-2),
    torch.float32: dict(max=1e-5, mean=1e-5, rel_l2=1e-5),
}


def log(*a):
    print(*a, flush=True)


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(out, lse, ref, ref_lse, dtype, what=""):
    """Compare kernel outputs (numpy fp64) against the oracle; returns the
    error metrics and asserts the bounds."""
    b = BOUNDS[dtype]
    err = np.abs(out - ref)
    lerr = np.abs(lse - ref_lse)
    rel = float(np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-300))
    m = dict(out_max=float(err.max(initial=0)), out_mean=float(err.mean()) if err.size else 0.0,
             rel_l2=rel, lse_max=float(lerr.max(initial=0)),
             lse_mean=float(lerr.mean()) if lerr.size else 0.0)
    log(f"  parity {what}: " + " ".join(f"{k}={v:.3e}" for k, v in m.items()))
    assert np.isfinite(out).all() and np.isfinite(lse).all(), what
    assert m["out_max"] <= b["max"] and m["out_mean"] <= b["mean"], (what, m)
    assert m["lse_max"] <= b["max"] and m["lse_mean"] <= b["mean"], (what, m)
    if err.size:
        assert m["rel_l2"] <= b["rel_l2"], (what, m)
    return m


def oracle_sample(q, k, v, seg, causal, ring_size, ring_index, head, rows, kv_len=None,
                  placement="contiguous"):
    """Oracle for one head and a subset of local query rows, slicing the
    device tensors so that only that head (and only the first kv_len keys)
    crosses to the host."""
    kv_len = k.shape[1] if kv_len is None else kv_len
    qh = q[:, :, head:head + 1].contiguous().cpu()
    kh = k[:, :kv_len, head:head + 1].contiguous().cpu()
    vh = v[:, :kv_len, head:head + 1].contiguous().cpu()
    sg = None if seg is None else seg.cpu().numpy()
    out, lse = oracle.attention_fwd(qh, kh, vh, sg, causal, ring_size, ring_index,
                                    rows=rows, kv_len=kv_len, placement=placement)
    return out[:, :, 0, :], lse[:, 0, :]


def visible_kv_len(w, ring_index) -> int:
    """Keys a causal share can see at most: up to the end of the causal block
    of its last query (all keys when non-causal)."""
    if not w.causal_block_size:
        return w.seq_k
    last = ring_index * w.seq_q + w.seq_q - 1
    c = w.causal_block_size
    return int(min(w.seq_k, (last // c + 1) * c))


def sample_rows(w, seed, n):
    """Seeded rows plus the first and last row of every query chunk."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(w.seq_q, size=min(n, w.seq_q), replace=False).tolist())
    for a in range(w.seq_q // w.q_chunk):
        rows.add(a * w.q_chunk)
        rows.add((a + 1) * w.q_chunk - 1)
    return np.array(sorted(rows), dtype=np.int64)
