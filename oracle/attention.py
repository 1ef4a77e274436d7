"""CPU fp64 oracle for the blockwise exact-attention forward of Ring Attention.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the GPU path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it; the library in ``long_context_exact_ra_amd`` never does,
and this module imports nothing from it.

Sources (web pages; cited by title and section):

* [RA-review] "Ring Attention with Blockwise Transformers for Near-Infinite
  Context" (paper review of arXiv:2310.01889), section 三 "技术架构":
  the self-attention equation softmax(Q K^T / sqrt(d)) V, the split of the
  sequence into N blocks held one per device, the ring algorithm (at outer
  step i device j uses block (j - i) mod N), and the permutation-invariance
  property (the blocks may be folded in any order with the lazy-softmax
  accumulation).  Section 四 states the method is exact.
* [RA-code] "从论文到代码：深入理解RingAttention的块注意力计算逻辑"
  ("From paper to code: RingAttention's block-attention logic"), section
  "1. 分块处理机制" (chunking by query_chunk_size / key_chunk_size with
  integer division), section "2. 数值稳定的注意力计算" (the running-max,
  numerator, denominator carry and its exp(prev_max - max) correction) and
  section "3. 因果注意力掩码支持" (chunk pairs are skipped unless the
  below-or-on-diagonal test passes; causal_block_size selects the causal
  granularity).

* [RA-review] section 六 "相关工作" and section 七 "局限性": causal
  attention leaves the ring unbalanced (later devices hold more visible
  pairs), which Striped Attention's striped partition of the sequence
  removes; it applies to causal attention only.

Readings taken where the pages are silent (each is also listed in the
design notes of the repository):

* scale is 1/sqrt(D) (the LaTeX of the self-attention equation; its
  plain-text rendering lost the square root);
* causal masking is inclusive: key position pk is visible from query
  position pq iff floor(pq / c) >= floor(pk / c) (c = causal_block_size;
  c = 1 is token-level, None is non-causal);
* segment ids: a key is visible only from a query with the same id;
* the chunk-pair skip test passes iff the chunk pair holds at least one
  causally visible pair; segment ids never affect skipping;
* the carry starts at max = -inf, numerator = 0, denominator = 0, and a
  correction whose old max is -inf is 0 (the old numerator and denominator
  are 0, so any finite factor gives the same result);
* striped placement: global position p is held by device p mod N at local
  index p div N (device r's block holds positions r, r + N, r + 2N, ...);
  k, v and segment ids are stored block by block in that order (storage
  row kb * Lq + j holds position j * N + kb), and every mask is taken on
  global positions;
* outputs: out = numerator / denominator and the natural-log log-sum-exp
  lse = max + ln(denominator), laid out [B, H, Lq]; a query row with no
  visible key gets out = 0 and lse = -inf.

Everything here computes in float64.  Inputs are upcast exactly.  Nothing is
tiled, fused or reordered beyond what the definitions state: matmul and exp
are library primitives used as single steps.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "query_positions",
    "key_positions",
    "visible",
    "attention_fwd",
    "lazy_blockwise_fwd",
    "ring_order",
    "below_or_on_diag",
    "skip_map_closed",
    "skip_map_bruteforce",
    "count_visible_pairs",
    "striped_pair_runs",
    "PLACEMENTS",
]


# ---------------------------------------------------------------------------
# Positions and the visibility mask
# ---------------------------------------------------------------------------

PLACEMENTS = ("contiguous", "striped")


def _check_placement(placement: str) -> None:
    if placement not in PLACEMENTS:
        raise ValueError(f"placement must be one of {PLACEMENTS}")


def query_positions(seq_q: int, ring_index: int, ring_size: int = 1,
                    placement: str = "contiguous") -> np.ndarray:
    """Global positions of the local query block.

    Contiguous ([RA-review] 三 "分块注意力"): the sequence Q = [Q_0 ..
    Q_{N-1}] is split into N equal blocks and device i holds Q_i, so local
    row t of device i sits at global position i * Lq + t.
    Striped (reading of [RA-review] 六/七): local row t of device i sits at
    global position t * N + i.
    """
    _check_placement(placement)
    t = np.arange(seq_q, dtype=np.int64)
    if placement == "striped":
        return t * ring_size + ring_index
    return ring_index * seq_q + t


def key_positions(seq_k: int, ring_size: int = 1,
                  placement: str = "contiguous") -> np.ndarray:
    """Global positions of the stored keys, in storage order.

    Storage row s = kb * Lq + j holds key j of block kb: global position s
    (contiguous: K = [K_0 .. K_{N-1}] in global order) or j * N + kb
    (striped).
    """
    _check_placement(placement)
    s = np.arange(seq_k, dtype=np.int64)
    if placement == "striped":
        seq_q = seq_k // ring_size
        return (s % seq_q) * ring_size + s // seq_q
    return s


def _scale(head_dim: int) -> float:
    """Softmax scale 1/sqrt(d) of the self-attention equation ([RA-review] 三)."""
    return 1.0 / math.sqrt(head_dim)


def _causal_visible(pq: np.ndarray, pk: np.ndarray,
                    causal_block_size: Optional[int]) -> np.ndarray:
    """Inclusive block-causal visibility floor(pq/c) >= floor(pk/c).

    [RA-code] "3. 因果注意力掩码支持": attention only to the past, with the
    granularity given by causal_block_size (1 = token level; None = off).
    Returns a [len(pq), len(pk)] bool array.
    """
    if causal_block_size is None:
        return np.ones((pq.shape[0], pk.shape[0]), dtype=bool)
    c = int(causal_block_size)
    return (pq // c)[:, None] >= (pk // c)[None, :]


def _segment_visible(seg_q: Optional[np.ndarray],
                     seg_k: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Same-segment visibility (reading: equal ids attend to each other)."""
    if seg_q is None:
        return None
    return seg_q[:, None] == seg_k[None, :]


def visible(pq: np.ndarray, pk: np.ndarray, causal_block_size: Optional[int],
            seg_q: Optional[np.ndarray] = None,
            seg_k: Optional[np.ndarray] = None) -> np.ndarray:
    """The full visibility mask for query positions pq and key positions pk."""
    m = _causal_visible(pq, pk, causal_block_size)
    s = _segment_visible(seg_q, seg_k)
    if s is not None:
        m = m & s
    return m


# ---------------------------------------------------------------------------
# C1: the plain definition
# ---------------------------------------------------------------------------

def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly on the CPU
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _check_kv_tail_masked(pq: np.ndarray, kv_len: int, seq_k: int,
                          causal_block_size: Optional[int]) -> None:
    """When only the first kv_len keys are supplied, every omitted key must be
    causally invisible from every requested row, otherwise the result would
    silently change."""
    if kv_len >= seq_k:
        return
    if causal_block_size is None:
        raise ValueError("kv_len < seq_k is only meaningful for causal masks")
    c = int(causal_block_size)
    # The first omitted key has the smallest block index of all omitted keys.
    if int(pq.max()) // c >= kv_len // c:
        raise ValueError("an omitted key would be visible to a requested row")


def attention_fwd(q, k, v, segment_ids=None, causal_block_size=None,
                  ring_size: int = 1, ring_index: int = 0,
                  rows: Optional[Sequence[int]] = None,
                  heads: Optional[Sequence[int]] = None,
                  kv_len: Optional[int] = None,
                  max_scores: int = 1 << 25,
                  placement: str = "contiguous"):
    """Masked softmax(Q K^T / sqrt(D)) V for one device's query block.

    [RA-review] 三 "核心公式" (self-attention), with the query block and
    key/value layout of "分块注意力" and "环形通信".

    q: [B, Lq, H, D] (this device's block, ring position ``ring_index``)
    k, v: [B, S, H, D] with S = ring_size * Lq, all blocks in global order;
          or only the first ``kv_len`` keys when the rest are provably
          causally invisible from every requested row.
    segment_ids: [B, S] ints over the whole sequence in storage order (the
          order of the rows of k), or None.
    rows / heads: optional subsets of local query rows / heads.
    placement: "contiguous" (the pages' blocks) or "striped" (position p on
          device p mod N); it sets the global positions that the causal
          mask compares.

    Returns (out [B, R, Hs, D], lse [B, Hs, R]) in float64 where R and Hs are
    the numbers of selected rows and heads.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Lq, H, D = q.shape
    S = ring_size * Lq
    kv_len = S if kv_len is None else int(kv_len)
    if k.shape != (B, kv_len, H, D) or v.shape != (B, kv_len, H, D):
        raise ValueError(f"k/v shape {k.shape} != {(B, kv_len, H, D)}")
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

    out = np.zeros((B, rows.shape[0], len(heads), D), dtype=np.float64)
    lse = np.full((B, len(heads), rows.shape[0]), -np.inf, dtype=np.float64)
    step = max(1, max_scores // max(kv_len, 1))
    for b in range(B):
        for hi, h in enumerate(heads):
            K = k[b, :, h, :]
            V = v[b, :, h, :]
            for r0 in range(0, rows.shape[0], step):
                sel = rows[r0:r0 + step]
                pq = pq_all[r0:r0 + step]
                s = (q[b, sel, h, :] @ K.T) * scale
                allow = visible(pq, pk, causal_block_size,
                                None if seg is None else seg[b, sq_all[r0:r0 + step]],
                                None if seg is None else seg[b, :kv_len])
                s = np.where(allow, s, -np.inf)
                m = s.max(axis=1) if kv_len > 0 else np.full(len(sel), -np.inf)
                has = np.isfinite(m)
                p = np.where(allow, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
                den = p.sum(axis=1)
                num = p @ V
                with np.errstate(divide="ignore", invalid="ignore"):
                    out[b, r0:r0 + step, hi, :] = np.where(
                        has[:, None], num / np.where(has, den, 1.0)[:, None], 0.0)
                    lse[b, hi, r0:r0 + step] = np.where(
                        has, m + np.log(np.where(has, den, 1.0)), -np.inf)
    return out, lse


# ---------------------------------------------------------------------------
# Ring order and the chunk-pair skip test
# ---------------------------------------------------------------------------

def ring_order(ring_size: int, ring_index: int) -> list:
    """KV block used at each outer step: block (j - i) mod N on device j at
    step i ([RA-review] 三 "环形注意力算法")."""
    return [(ring_index - t) % ring_size for t in range(ring_size)]


def below_or_on_diag(q_chunk_global: int, q_chunk: int, k_chunk_global: int,
                     k_chunk: int, causal_block_size: int) -> bool:
    """Chunk-pair run test of [RA-code] "3. 因果注意力掩码支持".

    The pages name the test and its arguments (global chunk indices, chunk
    sizes, causal_block_size) but do not print its body.  Reading: the pair
    runs iff it holds at least one causally visible (query, key) pair, i.e.
    the causal block of the pair's last query is not before the causal block
    of its first key.
    """
    last_q = (q_chunk_global + 1) * q_chunk - 1
    first_k = k_chunk_global * k_chunk
    c = causal_block_size
    return last_q // c >= first_k // c


def _chunk_counts(seq_q: int, q_chunk: int, k_chunk: int):
    # [RA-code] "1. 分块处理机制": the block is cut into seq_q / q_chunk query
    # chunks and seq_q / k_chunk key chunks by exact integer division.
    if seq_q % q_chunk or seq_q % k_chunk:
        raise ValueError("chunk sizes must divide the block length")
    return seq_q // q_chunk, seq_q // k_chunk


def striped_pair_runs(a: int, q_chunk: int, kb: int, bb: int, k_chunk: int,
                      ring_size: int, ring_index: int, causal_block_size: int) -> bool:
    """The same run test under striped placement: positions grow with the
    local index inside every block, so the pair holds a visible pair iff its
    last query (local row (a+1)*qc - 1, position ((a+1)*qc - 1) * N + r) sees
    its first key (local row bb*kc of block kb, position bb*kc*N + kb)."""
    last_q = ((a + 1) * q_chunk - 1) * ring_size + ring_index
    first_k = bb * k_chunk * ring_size + kb
    c = causal_block_size
    return last_q // c >= first_k // c


def skip_map_closed(causal_block_size, q_chunk: int, k_chunk: int, seq_q: int,
                    ring_size: int, ring_index: int, placement: str = "contiguous"):
    """The skip decisions by the closed-form test, in ring-step order.

    Returns (kv_block_of_step int32 [N], run uint8 [N, Lq/qc, Lq/kc]) where
    run[t, a, b] = 1 iff query chunk a of this device runs against key chunk
    b of the block used at step t.
    """
    _check_placement(placement)
    nq, nk = _chunk_counts(seq_q, q_chunk, k_chunk)
    order = ring_order(ring_size, ring_index)
    run = np.zeros((ring_size, nq, nk), dtype=np.uint8)
    for t, kb in enumerate(order):
        for a in range(nq):
            for bb in range(nk):
                if causal_block_size is None or causal_block_size == 0:
                    run[t, a, bb] = 1
                elif placement == "striped":
                    run[t, a, bb] = striped_pair_runs(a, q_chunk, kb, bb, k_chunk, ring_size,
                                                      ring_index, int(causal_block_size))
                else:
                    run[t, a, bb] = below_or_on_diag(
                        ring_index * nq + a, q_chunk, kb * nk + bb, k_chunk,
                        int(causal_block_size))
    return np.asarray(order, dtype=np.int32), run


def skip_map_bruteforce(causal_block_size, q_chunk: int, k_chunk: int,
                        seq_q: int, ring_size: int, ring_index: int,
                        placement: str = "contiguous"):
    """The same decisions by brute force: a chunk pair runs iff any of its
    (query, key) pairs is causally visible."""
    nq, nk = _chunk_counts(seq_q, q_chunk, k_chunk)
    order = ring_order(ring_size, ring_index)
    c = None if not causal_block_size else int(causal_block_size)
    pq = query_positions(seq_q, ring_index, ring_size, placement)
    pk_all = key_positions(ring_size * seq_q, ring_size, placement)
    run = np.zeros((ring_size, nq, nk), dtype=np.uint8)
    for t, kb in enumerate(order):
        pk = pk_all[kb * seq_q:(kb + 1) * seq_q]
        allow = _causal_visible(pq, pk, c)
        for a in range(nq):
            for bb in range(nk):
                run[t, a, bb] = bool(allow[a * q_chunk:(a + 1) * q_chunk,
                                           bb * k_chunk:(bb + 1) * k_chunk].any())
    return np.asarray(order, dtype=np.int32), run


def count_visible_pairs(seq_q: int, ring_size: int, ring_index: int,
                        causal_block_size, segment_ids=None, batch: int = 1,
                        rows: Optional[Iterable[int]] = None,
                        placement: str = "contiguous") -> int:
    """Number of visible (query, key) pairs for one head, summed over the
    batch, by explicit enumeration (used to check work counts).  Segment ids
    are in storage order."""
    c = None if not causal_block_size else int(causal_block_size)
    S = ring_size * seq_q
    sel = np.arange(seq_q, dtype=np.int64) if rows is None else np.asarray(list(rows),
                                                                           dtype=np.int64)
    pq = query_positions(seq_q, ring_index, ring_size, placement)[sel]
    sq = ring_index * seq_q + sel
    pk = key_positions(S, ring_size, placement)
    total = 0
    for b in range(batch):
        seg = None if segment_ids is None else np.asarray(segment_ids)[b]
        for r0 in range(0, pq.shape[0], 256):
            p = pq[r0:r0 + 256]
            total += int(visible(p, pk, c, None if seg is None else seg[sq[r0:r0 + 256]],
                                 seg).sum())
    return total


# ---------------------------------------------------------------------------
# C2: the lazy (online) softmax carry, block by block, chunk by chunk
# ---------------------------------------------------------------------------

def lazy_blockwise_fwd(q, k, v, segment_ids=None, causal_block_size=None,
                       ring_size: int = 1, ring_index: int = 0,
                       q_chunk: Optional[int] = None,
                       k_chunk: Optional[int] = None,
                       order: Optional[Sequence[int]] = None,
                       use_skip: bool = True,
                       placement: str = "contiguous"):
    """The blockwise formulation: fold KV blocks into a running carry.

    [RA-review] 三 "排列不变性": attention of Q_i over all blocks equals the
    lazy-softmax accumulation of the per-block attentions, in any block
    order.  [RA-code] "2. 数值稳定的注意力计算" gives the per-chunk update:

        new_max   = max(prev_max, rowmax(w))
        exp_w     = exp(w - new_max)
        corr      = exp(prev_max - new_max)
        numerator = numerator * corr + exp_w @ V_chunk
        denom     = denom * corr + rowsum(exp_w)

    where w are the (masked) scaled logits of the chunk pair.  Blocks are
    visited in ``order`` (default: the ring order), key chunks of a block in
    order, and a chunk pair is skipped when the below-or-on-diagonal test
    fails ([RA-code] "3. 因果注意力掩码支持"; under striped placement the
    same test on the pair's positions).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Lq, H, D = q.shape
    S = ring_size * Lq
    if k.shape != (B, S, H, D) or v.shape != (B, S, H, D):
        raise ValueError("k/v must hold all ring blocks")
    qc = Lq if q_chunk is None else q_chunk
    kc = Lq if k_chunk is None else k_chunk
    nq, nk = _chunk_counts(Lq, qc, kc)
    order = ring_order(ring_size, ring_index) if order is None else list(order)
    if sorted(order) != list(range(ring_size)):
        raise ValueError("order must be a permutation of the blocks")
    c = None if not causal_block_size else int(causal_block_size)
    seg = None if segment_ids is None else np.asarray(segment_ids, dtype=np.int64)
    scale = _scale(D)
    pq_all = query_positions(Lq, ring_index, ring_size, placement)
    pk_all = key_positions(S, ring_size, placement)

    out = np.zeros((B, Lq, H, D), dtype=np.float64)
    lse = np.full((B, H, Lq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for a in range(nq):
                rs = slice(a * qc, (a + 1) * qc)
                Qa = q[b, rs, h, :]
                pq = pq_all[rs]
                sq = np.arange(ring_index * Lq + a * qc, ring_index * Lq + (a + 1) * qc)
                prev_max = np.full(qc, -np.inf)
                numer = np.zeros((qc, D))
                denom = np.zeros(qc)
                for kb in order:
                    for bb in range(nk):
                        if use_skip and c is not None:
                            runs = (striped_pair_runs(a, qc, kb, bb, kc, ring_size,
                                                      ring_index, c)
                                    if placement == "striped" else
                                    below_or_on_diag(ring_index * nq + a, qc, kb * nk + bb,
                                                     kc, c))
                            if not runs:
                                continue
                        ks = slice(kb * Lq + bb * kc, kb * Lq + (bb + 1) * kc)
                        pk = pk_all[ks]
                        w = (Qa @ k[b, ks, h, :].T) * scale
                        allow = visible(pq, pk, c,
                                        None if seg is None else seg[b, sq],
                                        None if seg is None else seg[b, ks])
                        w = np.where(allow, w, -np.inf)
                        new_max = np.maximum(prev_max, w.max(axis=1))
                        fin = np.isfinite(new_max)
                        base = np.where(fin, new_max, 0.0)
                        exp_w = np.where(allow, np.exp(w - base[:, None]), 0.0)
                        corr = np.where(np.isfinite(prev_max),
                                        np.exp(prev_max - base), 0.0)
                        numer = numer * corr[:, None] + exp_w @ v[b, ks, h, :]
                        denom = denom * corr + exp_w.sum(axis=1)
                        prev_max = new_max
                has = denom > 0
                with np.errstate(divide="ignore", invalid="ignore"):
                    out[b, rs, h, :] = np.where(
                        has[:, None], numer / np.where(has, denom, 1.0)[:, None], 0.0)
                    lse[b, h, rs] = np.where(
                        has, prev_max + np.log(np.where(has, denom, 1.0)), -np.inf)
    return out, lse
