"""Pins of the oracle's striped placement (no GPU).

Striped placement (the reading of the load-balancing placement that
"Ring Attention with Blockwise Transformers for Near-Infinite Context"
names in sections 六 and 七): global position p lives on device p mod N at
local index p div N, and k, v and segment ids are stored block by block.
The pins build that layout by reshaping natural-order tensors (no call into
the oracle's position code) and compare against torch SDPA over the natural
order with masks built by torch (a lower triangle, a Kronecker block
triangle, an equality of document ids); the work count per device against a
hand-derived closed form; the skip maps against brute force; the lazy
blockwise carry against the plain definition in every block order.  The
planted mistakes at the end must each fail a pin.
"""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as oa
import oracle.backward as ob


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _to_striped(x, N):
    """Natural order [B, S, ...] -> storage order: block kb holds positions
    kb, kb + N, kb + 2N, ... (row kb * Lq + j is position j * N + kb)."""
    B, S = x.shape[:2]
    Lq = S // N
    y = x.reshape((B, Lq, N) + x.shape[2:])
    return np.ascontiguousarray(np.swapaxes(y, 1, 2)).reshape(x.shape)


def _sdpa(q, k, v, mask):
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    return o.permute(0, 2, 1, 3).numpy()


def _torch_lse(q, k, mask):
    tq, tk = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) / math.sqrt(q.shape[-1])
    s = s.masked_fill(~mask, float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()


def _block_causal_mask(S, c):
    nb = -(-S // c)
    m = torch.kron(torch.tril(torch.ones(nb, nb)), torch.ones(c, c))
    return m[:S, :S].bool()


def _documents(B, S, seed):
    rng = np.random.default_rng(seed)
    seg = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        pos, doc = 0, 0
        while pos < S:
            n = int(rng.integers(1, 9))
            seg[b, pos:pos + n] = doc
            pos += n
            doc += 1
    return seg


def _stitch_case(N, Lq, c, with_seg, seed):
    """Every device's striped share against full-sequence SDPA rows."""
    B, H, D = 2, 2, 16
    S = N * Lq
    q, k, v = (_rand((B, S, H, D), seed + i) for i in range(3))
    mask = torch.ones(S, S, dtype=torch.bool) if c is None else _block_causal_mask(S, c)
    seg = None
    if with_seg:
        seg = _documents(B, S, seed + 7)
        ts = torch.from_numpy(seg)
        mask = mask[None, None] & (ts[:, None, :, None] == ts[:, None, None, :])
    ref = _sdpa(q, k, v, mask)
    ref_lse = _torch_lse(q, k, mask)
    qs, ks, vs = (_to_striped(x, N) for x in (q, k, v))
    segs = None if seg is None else _to_striped(seg, N)
    for r in range(N):
        out, lse = oracle.attention_fwd(qs[:, r * Lq:(r + 1) * Lq], ks, vs, segs, c, N, r,
                                        placement="striped")
        np.testing.assert_allclose(out, ref[:, r::N], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse[:, :, r::N], rtol=0, atol=1e-12)


def pin_striped_token_causal_stitching():
    _stitch_case(4, 12, 1, False, 100)


def pin_striped_block_causal_stitching():
    for c in (2, 3, 8):
        _stitch_case(3, 10, c, False, 200 + c)


def pin_striped_segments_stitching():
    _stitch_case(4, 10, 1, True, 300)


def pin_striped_noncausal_stitching():
    _stitch_case(3, 8, None, False, 400)


def pin_striped_work_balance():
    """Token-causal visible pairs per device.  Row i of device r (position
    iN + r) sees, in block kb, the keys j with jN + kb <= iN + r: i + 1 of
    them when kb <= r, i when kb > r.  Summed over N blocks and Lq rows:
    N Lq (Lq + 1) / 2 - Lq (N - 1 - r).  Contiguous placement instead gives
    device r r Lq^2 + Lq (Lq + 1) / 2."""
    N, Lq = 5, 24
    for r in range(N):
        striped = oracle.count_visible_pairs(Lq, N, r, 1, placement="striped")
        assert striped == N * Lq * (Lq + 1) // 2 - Lq * (N - 1 - r), r
        contiguous = oracle.count_visible_pairs(Lq, N, r, 1)
        assert contiguous == r * Lq * Lq + Lq * (Lq + 1) // 2, r
    # the striped counts of all devices add up to the whole causal triangle
    S = N * Lq
    total = sum(oracle.count_visible_pairs(Lq, N, r, 1, placement="striped") for r in range(N))
    assert total == S * (S + 1) // 2


def pin_striped_skip_maps():
    for N, Lq, qc, kc in ((4, 16, 4, 8), (3, 12, 6, 4), (2, 8, 8, 2)):
        for c in (1, 2, 3, 5, 64):
            for r in range(N):
                o1, m1 = oracle.skip_map_closed(c, qc, kc, Lq, N, r, placement="striped")
                o2, m2 = oracle.skip_map_bruteforce(c, qc, kc, Lq, N, r, placement="striped")
                assert (o1 == o2).all() and (m1 == m2).all(), (N, Lq, qc, kc, c, r)


def pin_striped_lazy_any_order():
    B, N, Lq, H, D = 1, 3, 8, 2, 8
    S = N * Lq
    q = _rand((B, Lq, H, D), 500)
    k, v = (_rand((B, S, H, D), s) for s in (501, 502))
    seg = _to_striped(_documents(B, S, 503), N)
    r = 1
    ref, ref_lse = oracle.attention_fwd(q, k, v, seg, 1, N, r, placement="striped")
    for order in itertools.permutations(range(N)):
        out, lse = oracle.lazy_blockwise_fwd(q, k, v, seg, 1, N, r, 4, 2, order=order,
                                             placement="striped")
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def _striped_backward_case(N, Lq, c, seed):
    B, H, D = 1, 2, 8
    S = N * Lq
    q, k, v, g = (_rand((B, S, H, D), seed + i) for i in range(4))
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    mask = _block_causal_mask(S, c)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    o.backward(torch.from_numpy(g).permute(0, 2, 1, 3))
    rq, rk, rv = (t.grad.permute(0, 2, 1, 3).numpy() for t in (tq, tk, tv))
    qs, ks, vs, gs = (_to_striped(x, N) for x in (q, k, v, g))
    dk_sum = np.zeros_like(ks)
    dv_sum = np.zeros_like(vs)
    for r in range(N):
        sl = slice(r * Lq, (r + 1) * Lq)
        dq, dk, dv = ob.attention_bwd(qs[:, sl], ks, vs, gs[:, sl], None, c, N, r,
                                      placement="striped")
        np.testing.assert_allclose(dq, rq[:, r::N], rtol=0, atol=1e-12)
        dk_sum += dk
        dv_sum += dv
    np.testing.assert_allclose(dk_sum, _to_striped(rk, N), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_sum, _to_striped(rv, N), rtol=0, atol=1e-12)


def pin_striped_backward_stitching():
    """Striped backward: each device's dq rows and its dk/dv addends, summed
    over devices and put back in natural order, equal torch float64
    autograd through SDPA on the whole sequence: token causal, a causal
    block dividing N, one that is a multiple of N, and one that is neither."""
    _striped_backward_case(3, 8, 1, 600)
    _striped_backward_case(4, 8, 2, 610)
    _striped_backward_case(3, 8, 6, 620)
    _striped_backward_case(4, 6, 3, 630)


STRIPED_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", STRIPED_PINS, ids=[p.__name__ for p in STRIPED_PINS])
def test_pin_striped(pin):
    pin()


def test_to_striped_layout():
    """The test's own layout helper: storage row kb * Lq + j holds position
    j * N + kb."""
    N, Lq = 3, 4
    x = np.arange(N * Lq)[None, :, None]
    y = _to_striped(x, N)[0, :, 0]
    assert list(y) == [j * N + kb for kb in range(N) for j in range(Lq)]


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _mut_query_positions_transposed(mp):
    orig = oa.query_positions

    def bad(seq_q, r, n=1, placement="contiguous"):
        if placement == "striped":
            return r * seq_q + np.arange(seq_q, dtype=np.int64)
        return orig(seq_q, r, n, placement)
    mp.setattr(oa, "query_positions", bad)


def _mut_key_positions_contiguous(mp):
    mp.setattr(oa, "key_positions",
               lambda seq_k, n=1, placement="contiguous": np.arange(seq_k, dtype=np.int64))


def _mut_key_stripes_reversed(mp):
    """Block kb taken to hold the stripe of device N - 1 - kb."""
    def bad(seq_k, n=1, placement="contiguous"):
        s = np.arange(seq_k, dtype=np.int64)
        if placement == "striped":
            lq = seq_k // n
            return (s % lq) * n + (n - 1 - s // lq)
        return s
    mp.setattr(oa, "key_positions", bad)


def _mut_segments_by_position(mp):
    """Query segment ids looked up at the global position instead of the
    storage row."""
    orig = oa.visible

    def bad(pq, pk, c, seg_q=None, seg_k=None):
        if seg_q is not None and seg_k is not None and seg_k.shape[0] > pq.max():
            seg_q = seg_k[pq]
        return orig(pq, pk, c, seg_q, seg_k)
    mp.setattr(oa, "visible", bad)


def _mut_striped_strict(mp):
    orig = oa._causal_visible

    def bad(pq, pk, c):
        if c is None:
            return orig(pq, pk, c)
        return (pq // c)[:, None] > (pk // c)[None, :]
    mp.setattr(oa, "_causal_visible", bad)


def _mut_striped_pair_runs_first_query(mp):
    def bad(a, qc, kb, bb, kc, n, r, c):
        first_q = (a * qc) * n + r
        return first_q // c >= (bb * kc * n + kb) // c
    mp.setattr(oa, "striped_pair_runs", bad)


STRIPED_MUTATIONS = [_mut_query_positions_transposed, _mut_key_positions_contiguous,
                     _mut_key_stripes_reversed, _mut_segments_by_position,
                     _mut_striped_strict, _mut_striped_pair_runs_first_query]


@pytest.mark.parametrize("mutation", STRIPED_MUTATIONS, ids=[m.__name__ for m in STRIPED_MUTATIONS])
def test_planted_mistakes_striped(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = []
    for pin in STRIPED_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutation.__name__}"
