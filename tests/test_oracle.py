"""Pins of the CPU oracle to facts outside itself (no GPU).

Every pin below checks the oracle against something it does not contain: a
library routine that reduces to the textbook formula (torch's
scaled_dot_product_attention, matmul and logsumexp on the CPU in float64), a
closed form (Q = 0, V = 1), an invariant (permutation invariance of the block
order, rows of probabilities summing to 1), or an independent construction
(per-document attention stitched together, full-sequence attention stitched
from ring positions, skip maps by brute force).  ``test_planted_mistakes``
then plants plausible mistakes in the oracle and checks that each one makes
at least one pin fail.
"""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as oa


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask=None, is_causal=False):
    """torch SDPA on [B, L, H, D] float64 CPU arrays -> [B, L, H, D]."""
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                       is_causal=is_causal)
    return o.permute(0, 2, 1, 3).numpy()


def _torch_lse(q, k, mask=None):
    """logsumexp of the scaled logits by torch matmul + logsumexp, [B, H, L]."""
    tq, tk = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) / math.sqrt(q.shape[-1])
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()


def _block_causal_mask(S, c):
    """Block-lower-triangular mask built as a Kronecker product of a lower
    triangle of blocks with all-ones c x c tiles (no floor division)."""
    nb = -(-S // c)
    m = torch.kron(torch.tril(torch.ones(nb, nb)), torch.ones(c, c))
    return m[:S, :S].bool()


# ---------------------------------------------------------------------------
# pins (plain functions so the planted-mistake test can rerun them)
# ---------------------------------------------------------------------------

def pin_sdpa_noncausal():
    B, L, H, D = 2, 40, 3, 16
    q, k, v = (_rand((B, L, H, D), s) for s in (1, 2, 3))
    out, _ = oracle.attention_fwd(q, k, v, None, None, 1, 0)
    np.testing.assert_allclose(out, _sdpa(q, k, v), rtol=0, atol=1e-12)


def pin_sdpa_causal():
    B, L, H, D = 1, 48, 2, 32
    q, k, v = (_rand((B, L, H, D), s) for s in (4, 5, 6))
    out, _ = oracle.attention_fwd(q, k, v, None, 1, 1, 0)
    np.testing.assert_allclose(out, _sdpa(q, k, v, is_causal=True), rtol=0, atol=1e-12)


def pin_sdpa_block_causal():
    B, L, H, D = 1, 45, 2, 8
    q, k, v = (_rand((B, L, H, D), s) for s in (7, 8, 9))
    for c in (2, 4, 7, 45, 64):
        mask = _block_causal_mask(L, c)
        out, _ = oracle.attention_fwd(q, k, v, None, c, 1, 0)
        np.testing.assert_allclose(out, _sdpa(q, k, v, mask=mask), rtol=0, atol=1e-12)


def pin_lse_logsumexp():
    B, L, H, D = 2, 33, 2, 16
    q, k, v = (_rand((B, L, H, D), s) for s in (10, 11, 12))
    for c in (None, 1, 5):
        mask = None if c is None else _block_causal_mask(L, c)
        _, lse = oracle.attention_fwd(q, k, v, None, c, 1, 0)
        np.testing.assert_allclose(lse, _torch_lse(q, k, mask), rtol=0, atol=1e-12)


def pin_ring_stitching():
    """Concatenating the outputs of all ring positions = full-sequence
    attention with the same mask (N = 1)."""
    B, Lq, H, D, N = 1, 16, 2, 8, 4
    S = N * Lq
    k, v = (_rand((B, S, H, D), s) for s in (13, 14))
    qfull = _rand((B, S, H, D), 15)
    for c in (None, 1, 3, Lq, 2 * Lq):
        ref, ref_lse = oracle.attention_fwd(qfull, k, v, None, c, 1, 0)
        outs, lses = [], []
        for r in range(N):
            o, l = oracle.attention_fwd(qfull[:, r * Lq:(r + 1) * Lq], k, v, None, c, N, r)
            outs.append(o)
            lses.append(l)
        np.testing.assert_allclose(np.concatenate(outs, 1), ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.concatenate(lses, 2), ref_lse, rtol=0, atol=1e-12)


def pin_ring_stitching_vs_sdpa():
    """Ring positions stitched together equal torch's causal SDPA over the
    whole sequence: pins the global query offset of every ring position."""
    B, Lq, H, D, N = 1, 12, 2, 8, 3
    S = N * Lq
    q, k, v = (_rand((B, S, H, D), s) for s in (16, 17, 18))
    ref = _sdpa(q, k, v, is_causal=True)
    for r in range(N):
        o, _ = oracle.attention_fwd(q[:, r * Lq:(r + 1) * Lq], k, v, None, 1, N, r)
        np.testing.assert_allclose(o, ref[:, r * Lq:(r + 1) * Lq], rtol=0, atol=1e-12)


def pin_q_zero_closed_form():
    """Q = 0: every logit is 0, so out_i is the mean of the visible V rows and
    lse_i = ln(number of visible keys).  The expected values come from prefix
    sums over each document (no mask matrix)."""
    B, Lq, H, D, N = 2, 24, 2, 4, 3
    S = N * Lq
    v = _rand((B, S, H, D), 19)
    k = _rand((B, S, H, D), 20)
    seg = np.zeros((B, S), dtype=np.int32)
    seg[0, 10:30] = 1
    seg[0, 30:] = 2
    seg[1, 5:] = 1
    for r in range(N):
        q = np.zeros((B, Lq, H, D))
        out, lse = oracle.attention_fwd(q, k, v, seg, 1, N, r)
        for b in range(B):
            for i in range(Lq):
                p = r * Lq + i
                start = p
                while start > 0 and seg[b, start - 1] == seg[b, p]:
                    start -= 1
                n = p - start + 1
                np.testing.assert_allclose(out[b, i], v[b, start:p + 1].mean(0),
                                           rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[b, :, i], math.log(n), rtol=0, atol=1e-12)


def pin_v_ones():
    B, Lq, H, D, N = 1, 16, 2, 8, 2
    q, k = _rand((B, Lq, H, D), 21), _rand((B, N * Lq, H, D), 22)
    v = np.ones((B, N * Lq, H, D))
    for c in (None, 1, 5):
        for r in range(N):
            out, _ = oracle.attention_fwd(q, k, v, None, c, N, r)
            np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)


def pin_probability_rows():
    """V = identity (D = S): out reproduces the probability rows, which sum to
    1, vanish on masked keys and equal torch.softmax of torch's logits."""
    B, Lq, H, N = 1, 8, 2, 4
    S = N * Lq
    D = S
    q, k = _rand((B, Lq, H, D), 23), _rand((B, S, H, D), 24)
    v = np.broadcast_to(np.eye(S)[None, :, None, :], (B, S, H, S)).copy()
    r = 2
    out, _ = oracle.attention_fwd(q, k, v, None, 1, N, r)
    np.testing.assert_allclose(out.sum(-1), 1.0, rtol=0, atol=1e-13)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) / math.sqrt(D)
    mask = _block_causal_mask(S, 1)[r * Lq:(r + 1) * Lq]
    p = torch.softmax(s.masked_fill(~mask, float("-inf")), -1).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(out, p, rtol=0, atol=1e-13)


def pin_lazy_all_permutations():
    """Permutation invariance: folding the N blocks into the lazy-softmax
    carry in any order gives the plain definition."""
    B, Lq, H, D, N = 1, 16, 2, 8, 4
    S = N * Lq
    q = _rand((B, Lq, H, D), 25)
    k, v = _rand((B, S, H, D), 26), _rand((B, S, H, D), 27)
    seg = np.repeat(np.arange(S // 11 + 1), 11)[:S][None].astype(np.int32)
    for c, sg, r in ((None, None, 1), (1, None, 3), (5, None, 2), (1, seg, 3)):
        ref, ref_lse = oracle.attention_fwd(q, k, v, sg, c, N, r)
        for order in itertools.permutations(range(N)):
            out, lse = oracle.lazy_blockwise_fwd(q, k, v, sg, c, N, r, 8, 4, order)
            np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def pin_lazy_ring_order_chunks():
    """The ring order with every divisor chunking equals the definition."""
    B, Lq, H, D, N = 2, 12, 1, 4, 3
    S = N * Lq
    q = _rand((B, Lq, H, D), 28)
    k, v = _rand((B, S, H, D), 29), _rand((B, S, H, D), 30)
    for c in (None, 1, 4, 12, 36):
        for r in range(N):
            ref, ref_lse = oracle.attention_fwd(q, k, v, None, c, N, r)
            for qc in (1, 3, 4, 12):
                for kc in (2, 6, 12):
                    out, lse = oracle.lazy_blockwise_fwd(q, k, v, None, c, N, r, qc, kc)
                    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
                    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def pin_segments_per_document():
    """Segment masking equals running each document alone (token causal is
    shift-invariant, so a document is an independent N = 1 sequence)."""
    B, Lq, H, D, N = 1, 20, 2, 8, 2
    S = N * Lq
    bounds = [0, 7, 8, 19, 33, S]
    seg = np.zeros((B, S), dtype=np.int32)
    for i in range(len(bounds) - 1):
        seg[0, bounds[i]:bounds[i + 1]] = i
    qfull = _rand((B, S, H, D), 31)
    k, v = _rand((B, S, H, D), 32), _rand((B, S, H, D), 33)
    got = np.concatenate([oracle.attention_fwd(qfull[:, r * Lq:(r + 1) * Lq], k, v,
                                               seg, 1, N, r)[0] for r in range(N)], 1)
    for i in range(len(bounds) - 1):
        s = slice(bounds[i], bounds[i + 1])
        ref, _ = oracle.attention_fwd(qfull[:, s], k[:, s], v[:, s], None, 1, 1, 0)
        np.testing.assert_allclose(got[:, s], ref, rtol=0, atol=1e-12)


def pin_one_segment_is_no_segment():
    B, Lq, H, D, N = 2, 8, 2, 8, 2
    q = _rand((B, Lq, H, D), 34)
    k, v = _rand((B, N * Lq, H, D), 35), _rand((B, N * Lq, H, D), 36)
    seg = np.full((B, N * Lq), 7, dtype=np.int32)
    for c in (None, 1):
        a = oracle.attention_fwd(q, k, v, seg, c, N, 1)
        b = oracle.attention_fwd(q, k, v, None, c, N, 1)
        np.testing.assert_allclose(a[0], b[0], rtol=0, atol=0)
        np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)


def pin_zero_length():
    """With inclusive causal masks and per-position segment ids every query
    sees at least itself, so an empty row only arises with no rows at all;
    the oracle returns empty outputs of the right shapes."""
    B, H, D = 1, 1, 4
    q = np.zeros((B, 0, H, D))
    out, lse = oracle.attention_fwd(q, q, q, None, 1, 1, 0)
    assert out.shape == (1, 0, 1, 4) and lse.shape == (1, 1, 0)


def pin_skip_map_closed_vs_bruteforce():
    """The closed-form chunk-pair test equals 'any visible pair in the chunk
    pair', exhaustively over small grids."""
    for Lq in (4, 6, 8, 12, 16):
        divs = [d for d in range(1, Lq + 1) if Lq % d == 0]
        for N in (1, 2, 3, 5):
            for c in (None, 1, 2, 3, 5, 8, Lq, 2 * Lq):
                for qc in divs:
                    for kc in divs:
                        for r in range(N):
                            a = oracle.skip_map_closed(c, qc, kc, Lq, N, r)
                            b = oracle.skip_map_bruteforce(c, qc, kc, Lq, N, r)
                            assert (a[0] == b[0]).all()
                            assert (a[1] == b[1]).all(), (Lq, N, c, qc, kc, r)


def pin_skip_map_known_counts():
    """Counts derived by hand from the definitions.

    * 7B-shaped share (Lq 32768, chunks 2048, ring position 15 of 16, token
      causal): the 15 earlier blocks run fully (15 * 16 * 16 chunk pairs) and
      the own block runs its lower triangle with the diagonal (16 * 17 / 2).
    * 65B-shaped share (Lq 16384, chunks 512, ring position 128 of 256,
      causal_block_size 16384 = Lq): blocks 0..128 run fully, 129..255 never.
    """
    order, run = oracle.skip_map_closed(1, 2048, 2048, 32768, 16, 15)
    assert list(order) == [15 - t for t in range(16)]
    assert int(run.sum()) == 15 * 256 + 136
    assert run[0].tolist() == np.tril(np.ones((16, 16), dtype=np.uint8)).tolist()
    order, run = oracle.skip_map_closed(16384, 512, 512, 16384, 256, 128)
    assert list(order[:3]) == [128, 127, 126] and order[129] == 255
    per_step = run.reshape(256, -1).sum(1)
    assert (per_step[:129] == 32 * 32).all() and (per_step[129:] == 0).all()


def pin_ring_order():
    """At outer step i device j uses block (j - i) mod N: the own block first,
    then the block that arrived from the previous device."""
    assert oracle.ring_order(4, 0) == [0, 3, 2, 1]
    assert oracle.ring_order(4, 2) == [2, 1, 0, 3]
    assert oracle.ring_order(1, 0) == [0]


def pin_visible_pair_count():
    """Visible pairs at ring position r with token causal: r*Lq*Lq from the
    earlier blocks plus Lq*(Lq+1)/2 from the own block."""
    for Lq, N, r in ((8, 4, 0), (8, 4, 3), (16, 2, 1)):
        assert oracle.count_visible_pairs(Lq, N, r, 1) == r * Lq * Lq + Lq * (Lq + 1) // 2
        assert oracle.count_visible_pairs(Lq, N, r, None) == N * Lq * Lq


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_kv_len_guard():
    B, Lq, H, D, N = 1, 8, 1, 4, 4
    q = _rand((B, Lq, H, D), 40)
    k, v = _rand((B, N * Lq, H, D), 41), _rand((B, N * Lq, H, D), 42)
    full = oracle.attention_fwd(q, k, v, None, Lq, N, 1)
    part = oracle.attention_fwd(q, k[:, :2 * Lq], v[:, :2 * Lq], None, Lq, N, 1,
                                kv_len=2 * Lq)
    np.testing.assert_allclose(part[0], full[0], rtol=0, atol=0)
    with pytest.raises(ValueError):
        oracle.attention_fwd(q, k[:, :Lq], v[:, :Lq], None, Lq, N, 1, kv_len=Lq)


def test_rows_heads_subset():
    B, Lq, H, D, N = 2, 16, 3, 8, 2
    q = _rand((B, Lq, H, D), 43)
    k, v = _rand((B, N * Lq, H, D), 44), _rand((B, N * Lq, H, D), 45)
    full, full_lse = oracle.attention_fwd(q, k, v, None, 1, N, 1)
    rows, heads = [0, 5, 15], [2, 0]
    sub, sub_lse = oracle.attention_fwd(q, k, v, None, 1, N, 1, rows=rows, heads=heads)
    np.testing.assert_allclose(sub, full[:, rows][:, :, heads], rtol=0, atol=0)
    np.testing.assert_allclose(sub_lse, full_lse[:, heads][:, :, rows], rtol=0, atol=0)


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _mut_scale_no_sqrt(monkeypatch):
    monkeypatch.setattr(oa, "_scale", lambda d: 1.0 / d)


def _mut_scale_dropped(monkeypatch):
    monkeypatch.setattr(oa, "_scale", lambda d: 1.0)


def _mut_causal_strict(monkeypatch):
    def strict(pq, pk, c):
        if c is None:
            return np.ones((pq.shape[0], pk.shape[0]), dtype=bool)
        return (pq // c)[:, None] > (pk // c)[None, :]
    monkeypatch.setattr(oa, "_causal_visible", strict)


def _mut_causal_reversed(monkeypatch):
    def rev(pq, pk, c):
        if c is None:
            return np.ones((pq.shape[0], pk.shape[0]), dtype=bool)
        return (pq // c)[:, None] <= (pk // c)[None, :]
    monkeypatch.setattr(oa, "_causal_visible", rev)


def _mut_causal_token_level(monkeypatch):
    def tok(pq, pk, c):
        if c is None:
            return np.ones((pq.shape[0], pk.shape[0]), dtype=bool)
        return pq[:, None] >= pk[None, :]
    monkeypatch.setattr(oa, "_causal_visible", tok)


def _mut_no_ring_offset(monkeypatch):
    monkeypatch.setattr(oa, "query_positions",
                        lambda seq_q, r, *rest: np.arange(seq_q, dtype=np.int64))


def _mut_segments_ignored(monkeypatch):
    monkeypatch.setattr(oa, "_segment_visible", lambda a, b: None)


def _mut_ring_order_reversed(monkeypatch):
    monkeypatch.setattr(oa, "ring_order",
                        lambda n, r: [(r + t) % n for t in range(n)])


def _mut_diag_test_first_query(monkeypatch):
    def bad(qg, qc, kg, kc, c):
        return (qg * qc) // c >= (kg * kc) // c
    monkeypatch.setattr(oa, "below_or_on_diag", bad)


def _mut_diag_test_last_key(monkeypatch):
    def bad(qg, qc, kg, kc, c):
        return ((qg + 1) * qc - 1) // c >= ((kg + 1) * kc - 1) // c
    monkeypatch.setattr(oa, "below_or_on_diag", bad)


MUTATIONS = [_mut_scale_no_sqrt, _mut_scale_dropped, _mut_causal_strict,
             _mut_causal_reversed, _mut_causal_token_level, _mut_no_ring_offset,
             _mut_segments_ignored, _mut_ring_order_reversed,
             _mut_diag_test_first_query, _mut_diag_test_last_key]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m.__name__ for m in MUTATIONS])
def test_planted_mistakes(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutation.__name__}"
