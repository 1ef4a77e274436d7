"""Pins of the backward oracle to facts outside itself (no GPU).

The backward oracle writes the derivative of the attention definition out by
hand.  Each pin checks it against something it does not contain: torch
autograd through ``scaled_dot_product_attention`` on the CPU in float64 with
masks built here from positions (a library routine reducing to the textbook
formula, differentiated by the library), central finite differences of the
*forward* oracle, and invariants of the exact gradient (the gradient of the
scores sums to zero over each row, so sum_j dk_j = 0; each probability row
sums to one, so sum_j dv_j = sum_i dout_i; shifting every value row by the
same vector leaves dq and dk unchanged).  ``test_planted_mistakes_bwd`` plants
plausible mistakes and checks that each makes at least one pin fail.
"""


import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as oa
import oracle.backward as ob


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _autograd(q, k, v, dout, mask):
    """dq, dk, dv of sum(dout * SDPA(q, k, v, mask)) by torch autograd, float64
    CPU; arrays are [B, L, H, D], mask [B or 1, Lq, S] bool (True = attend)."""
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).clone().requires_grad_(True)
                  for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask[:, None])
    o.backward(torch.from_numpy(dout).permute(0, 2, 1, 3))
    return tuple(t.grad.permute(0, 2, 1, 3).numpy() for t in (tq, tk, tv))


def _causal_mask_torch(Lq, S, r, c):
    """Mask [1, Lq, S] of a query block at ring position r, built with torch
    from a Kronecker block-lower-triangle (no floor division)."""
    nb = -(-S // c)
    full = torch.kron(torch.tril(torch.ones(nb, nb)), torch.ones(c, c))[:S, :S].bool()
    return full[r * Lq:(r + 1) * Lq][None]


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * max(1.0, np.max(np.abs(b)) if b.size else 1.0), err


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_bwd_autograd_token_causal():
    B, Lq, N, H, D, r = 2, 8, 3, 2, 16, 1
    S = N * Lq
    q, k, v, do = (_rand(s, i) for i, s in enumerate(
        [(B, Lq, H, D), (B, S, H, D), (B, S, H, D), (B, Lq, H, D)]))
    ref = _autograd(q, k, v, do, _causal_mask_torch(Lq, S, r, 1))
    got = oracle.attention_bwd(q, k, v, do, None, 1, N, r)
    for g, e in zip(got, ref):
        _close(g, e)


def pin_bwd_autograd_block_causal():
    B, Lq, N, H, D, r, c = 1, 12, 3, 2, 8, 2, 5
    S = N * Lq
    q, k, v, do = (_rand(s, 10 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, S, H, D), (B, S, H, D), (B, Lq, H, D)]))
    ref = _autograd(q, k, v, do, _causal_mask_torch(Lq, S, r, c))
    got = oracle.attention_bwd(q, k, v, do, None, c, N, r)
    for g, e in zip(got, ref):
        _close(g, e)


def pin_bwd_autograd_segments_noncausal():
    B, Lq, N, H, D, r = 2, 10, 2, 2, 8, 1
    S = N * Lq
    q, k, v, do = (_rand(s, 20 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, S, H, D), (B, S, H, D), (B, Lq, H, D)]))
    seg = np.array([[0] * 7 + [1] * 9 + [2] * 4, [5] * 12 + [6] * 8], dtype=np.int64)
    ts = torch.from_numpy(seg)
    mask = ts[:, r * Lq:(r + 1) * Lq, None] == ts[:, None, :]
    ref = _autograd(q, k, v, do, mask)
    got = oracle.attention_bwd(q, k, v, do, seg, None, N, r)
    for g, e in zip(got, ref):
        _close(g, e)


def pin_bwd_finite_differences():
    """Central differences of L = sum(dout * out) through the forward oracle."""
    B, Lq, N, H, D, r = 1, 6, 2, 1, 4, 1
    S = N * Lq
    q, k, v, do = (_rand(s, 30 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, S, H, D), (B, S, H, D), (B, Lq, H, D)]))
    seg = np.array([[0] * 5 + [1] * 7])
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, seg, 1, N, r)

    def loss(qq, kk, vv):
        out, _ = oracle.attention_fwd(qq, kk, vv, seg, 1, N, r)
        return float(np.sum(out * do))

    eps = 1e-6
    rng = np.random.default_rng(7)
    for x, g, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        for _ in range(6):
            idx = tuple(rng.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def pin_bwd_invariants():
    B, Lq, N, H, D, r = 2, 16, 4, 2, 8, 2
    S = N * Lq
    q, k, v, do = (_rand(s, 40 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, S, H, D), (B, S, H, D), (B, Lq, H, D)]))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, None, 3, N, r)
    # every row sees at least its own key: rows of p sum to one
    _close(dv.sum(axis=1), do.sum(axis=1))
    _close(dk.sum(axis=1), np.zeros_like(dk.sum(axis=1)))
    # a common shift of all value rows moves out by the shift only
    shift = _rand((1, 1, H, D), 49)
    dq2, dk2, dv2 = oracle.attention_bwd(q, k, v + shift, do, None, 3, N, r)
    _close(dq2, dq)
    _close(dk2, dk)
    _close(dv2, dv)


def pin_bwd_zero_upstream():
    B, Lq, N, H, D = 1, 8, 2, 1, 8
    q, k, v = _rand((B, Lq, H, D), 50), _rand((B, N * Lq, H, D), 51), _rand((B, N * Lq, H, D), 52)
    for g in oracle.attention_bwd(q, k, v, np.zeros((B, Lq, H, D)), None, 1, N, 1):
        assert not np.any(g)


def pin_bwd_ring_stitching():
    """The shares of all ring positions add up to the full-sequence gradient."""
    B, Lq, N, H, D = 1, 6, 3, 2, 8
    S = N * Lq
    Q, k, v, dO = (_rand(s, 60 + i) for i, s in enumerate(
        [(B, S, H, D), (B, S, H, D), (B, S, H, D), (B, S, H, D)]))
    full = torch.tril(torch.ones(S, S)).bool()[None]
    rdq, rdk, rdv = _autograd(Q, k, v, dO, full)
    dk = np.zeros_like(rdk)
    dv = np.zeros_like(rdv)
    for r in range(N):
        sl = slice(r * Lq, (r + 1) * Lq)
        gq, gk, gv = oracle.attention_bwd(Q[:, sl], k, v, dO[:, sl], None, 1, N, r)
        _close(gq, rdq[:, sl])
        dk += gk
        dv += gv
    _close(dk, rdk)
    _close(dv, rdv)


def pin_bwd_row_subsets_add_up():
    B, Lq, N, H, D, r = 1, 12, 2, 2, 8, 1
    q, k, v, do = (_rand(s, 70 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, N * Lq, H, D), (B, N * Lq, H, D), (B, Lq, H, D)]))
    full = oracle.attention_bwd(q, k, v, do, None, 1, N, r)
    a = np.arange(0, Lq, 2)
    b = np.arange(1, Lq, 2)
    ga = oracle.attention_bwd(q, k, v, do, None, 1, N, r, rows=a)
    gb = oracle.attention_bwd(q, k, v, do, None, 1, N, r, rows=b)
    _close(ga[0], full[0][:, a])
    _close(gb[0], full[0][:, b])
    _close(ga[1] + gb[1], full[1])
    _close(ga[2] + gb[2], full[2])


def pin_bwd_key_subset_matches_autograd():
    """keys=J returns the gradient of exactly those keys: autograd's full dk
    and dv sliced at J, for keys from every block, out of order, one key
    listed twice (block-causal ring share with segment ids)."""
    B, Lq, N, H, D, r, c = 2, 8, 4, 2, 8, 2, 3
    S = N * Lq
    q, k, v, do = (_rand(s, 90 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, S, H, D), (B, S, H, D), (B, Lq, H, D)]))
    seg = np.array([[0] * 13 + [1] * 11 + [2] * 8, [4] * 20 + [7] * 12], dtype=np.int64)
    ts = torch.from_numpy(seg)
    mask = _causal_mask_torch(Lq, S, r, c) & (ts[:, r * Lq:(r + 1) * Lq, None] == ts[:, None, :])
    rdq, rdk, rdv = _autograd(q, k, v, do, mask)
    keys = [31, 0, 9, 17, 17, 24, 5, 22]
    gq, gk, gv = oracle.attention_bwd(q, k, v, do, seg, c, N, r, keys=keys)
    _close(gq, rdq)
    _close(gk, rdk[:, keys])
    _close(gv, rdv[:, keys])


def pin_bwd_sparse_upstream():
    """With dout zero outside a set of rows R, the share's whole gradient
    (autograd over every row) equals the contributions of the rows in R:
    dk and dv are those of rows=R, dq vanishes outside R."""
    B, Lq, N, H, D, r = 1, 16, 3, 2, 8, 2
    S = N * Lq
    q, k, v, do = (_rand(s, 100 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, S, H, D), (B, S, H, D), (B, Lq, H, D)]))
    R = np.array([0, 3, 4, 11, 15])
    sparse = np.zeros_like(do)
    sparse[:, R] = do[:, R]
    rdq, rdk, rdv = _autograd(q, k, v, sparse, _causal_mask_torch(Lq, S, r, 1))
    gq, gk, gv = oracle.attention_bwd(q, k, v, sparse, None, 1, N, r, rows=R)
    _close(gq, rdq[:, R])
    others = np.setdiff1d(np.arange(Lq), R)
    assert not np.any(rdq[:, others])
    _close(gk, rdk)
    _close(gv, rdv)


BWD_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_bwd_")]


@pytest.mark.parametrize("pin", BWD_PINS, ids=[p.__name__ for p in BWD_PINS])
def test_pin_bwd(pin):
    pin()


def test_bwd_kv_len_truncation():
    B, Lq, N, H, D, r = 1, 8, 4, 1, 8, 1
    q, k, v, do = (_rand(s, 80 + i) for i, s in enumerate(
        [(B, Lq, H, D), (B, N * Lq, H, D), (B, N * Lq, H, D), (B, Lq, H, D)]))
    full = oracle.attention_bwd(q, k, v, do, None, 1, N, r)
    kv = (r + 1) * Lq
    part = oracle.attention_bwd(q, k[:, :kv], v[:, :kv], do, None, 1, N, r, kv_len=kv)
    _close(part[0], full[0])
    _close(part[1], full[1][:, :kv])
    _close(part[2], full[2][:, :kv])
    assert not np.any(full[1][:, kv:]) and not np.any(full[2][:, kv:])


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _mut_delta_dropped(mp):
    mp.setattr(ob, "_row_delta", lambda do, out: np.zeros(do.shape[0]))


def _mut_ds_sign(mp):
    mp.setattr(ob, "_ds_from_dp", lambda p, dp, delta: p * (delta[:, None] - dp))


def _mut_ds_no_p(mp):
    mp.setattr(ob, "_ds_from_dp", lambda p, dp, delta: dp - delta[:, None])


def _mut_scale_dropped(mp):
    mp.setattr(ob, "_scale", lambda d: 1.0)


def _mut_scale_no_sqrt(mp):
    mp.setattr(ob, "_scale", lambda d: 1.0 / d)


def _mut_softmax_unnormalised(mp):
    def bad(s, allow):
        e = np.where(allow, np.exp(s), 0.0)
        return e, np.ones(s.shape[0], dtype=bool)
    mp.setattr(ob, "_softmax_rows", bad)


def _mut_causal_strict(mp):
    def strict(pq, pk, c, sq=None, sk=None):
        m = oa.visible(pq, pk, c, sq, sk)
        return m & (pq[:, None] != pk[None, :])
    mp.setattr(ob, "visible", strict)


def _mut_segments_ignored(mp):
    mp.setattr(ob, "visible", lambda pq, pk, c, sq=None, sk=None: oa.visible(pq, pk, c))


def _mut_no_ring_offset(mp):
    mp.setattr(ob, "query_positions", lambda lq, r, *rest: np.arange(lq, dtype=np.int64))


BWD_MUTATIONS = [_mut_delta_dropped, _mut_ds_sign, _mut_ds_no_p, _mut_scale_dropped,
                 _mut_scale_no_sqrt, _mut_softmax_unnormalised, _mut_causal_strict,
                 _mut_segments_ignored, _mut_no_ring_offset]


@pytest.mark.parametrize("mutation", BWD_MUTATIONS, ids=[m.__name__ for m in BWD_MUTATIONS])
def test_planted_mistakes_bwd(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = []
    for pin in BWD_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutation.__name__}"
