"""Pins of the decoding oracle to facts outside itself (no GPU).

``oracle.decode_attention`` is one decoding step: the n_new tokens at
positions cache_idx .. cache_idx + n_new - 1 attend to the cache rows up to
their own position.  Each pin checks it against something it does not
contain:

* torch's ``scaled_dot_product_attention`` (a library routine for the
  textbook formula) in float64 with a mask built here from a lower triangle;
* the forward oracle (pinned on its own in ``test_oracle.py``): the decode of
  the last n_new tokens of a sequence equals the last rows of the causal
  forward over that sequence;
* closed forms: q = 0 gives the mean of the visible value rows and lse =
  ln(number of visible keys); a first token (cache_idx 0, n_new 1) returns
  v_0 and lse = q.k_0 / sqrt(D);
* the rows past the step's last token are never read (NaN there changes
  nothing).

``test_planted_mistakes_decode`` plants plausible mistakes in the oracle and
checks that each makes at least one pin fail.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.decode as od


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, err


def _sdpa(q, k, v, cache_idx):
    """torch SDPA in float64 on the CPU: queries [B, T, H, D] against the
    first cache_idx + T rows; the mask is the last T rows of a lower
    triangle of side cache_idx + T."""
    B, T, H, D = q.shape
    n = cache_idx + T
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool))[n - T:]
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).permute(0, 2, 1, 3)
                  for x in (q, k[:, :n], v[:, :n]))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask[None, None])
    s = (tq @ tk.transpose(-1, -2)) / np.sqrt(D)
    s = s.masked_fill(~mask[None, None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)                      # [B, H, T]
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


CASES = [  # (B, T, H, D, cache_idx, rows)
    (1, 1, 1, 4, 0, 1),
    (1, 1, 2, 8, 9, 12),
    (2, 3, 2, 16, 5, 8),
    (1, 8, 3, 8, 0, 8),
    (2, 5, 1, 32, 40, 64),
]


@pytest.mark.parametrize("B,T,H,D,ci,R", CASES)
def test_decode_matches_sdpa(B, T, H, D, ci, R):
    q, k, v = _rand((B, T, H, D), 1), _rand((B, R, H, D), 2), _rand((B, R, H, D), 3)
    out, lse = oracle.decode_attention(q, k, v, ci)
    ro, rl = _sdpa(q, k, v, ci)
    _close(out, ro)
    _close(lse, rl)


@pytest.mark.parametrize("T,L", [(1, 7), (4, 12), (12, 12)])
def test_decode_is_last_rows_of_causal_forward(T, L):
    """The decode of tokens L - T .. L - 1 equals those rows of the causal
    forward over the whole sequence (ring of one block)."""
    B, H, D = 2, 2, 8
    qf, k, v = _rand((B, L, H, D), 4), _rand((B, L, H, D), 5), _rand((B, L, H, D), 6)
    out, lse = oracle.decode_attention(qf[:, L - T:], k, v, L - T)
    fo, fl = oracle.attention_fwd(qf, k, v, causal_block_size=1, rows=range(L - T, L))
    _close(out, fo)
    _close(lse, fl)


def test_decode_zero_query_is_mean_of_visible_values():
    B, T, H, D, ci = 1, 4, 2, 8, 6
    k, v = _rand((B, ci + T + 3, H, D), 7), _rand((B, ci + T + 3, H, D), 8)
    out, lse = oracle.decode_attention(np.zeros((B, T, H, D)), k, v, ci)
    for t in range(T):
        n_vis = ci + t + 1
        _close(out[:, t], v[:, :n_vis].mean(axis=1))
        _close(lse[:, :, t], np.full((B, H), np.log(n_vis)))


def test_decode_first_token():
    D = 16
    q, k, v = _rand((1, 1, 2, D), 9), _rand((1, 3, 2, D), 10), _rand((1, 3, 2, D), 11)
    out, lse = oracle.decode_attention(q, k, v, 0)
    _close(out[0, 0], v[0, 0])
    _close(lse[0, :, 0], (q[0, 0] * k[0, 0]).sum(axis=-1) / np.sqrt(D))


def test_decode_ignores_rows_past_the_step():
    B, T, H, D, ci, R = 1, 3, 2, 8, 10, 20
    q, k, v = _rand((B, T, H, D), 12), _rand((B, R, H, D), 13), _rand((B, R, H, D), 14)
    ref = oracle.decode_attention(q, k, v, ci)
    k2, v2 = k.copy(), v.copy()
    k2[:, ci + T:] = np.nan
    v2[:, ci + T:] = np.nan
    got = oracle.decode_attention(q, k2, v2, ci)
    _close(got[0], ref[0], 0.0)
    _close(got[1], ref[1], 0.0)


def test_decode_rejects_overrun():
    q, k = np.zeros((1, 2, 1, 4)), np.zeros((1, 5, 1, 4))
    with pytest.raises(ValueError):
        oracle.decode_attention(q, k, k, 4)


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _mut_mask_strict(mp):
    mp.setattr(od, "_visible", lambda pq, pk: pk[None, :] < pq[:, None])


def _mut_mask_all(mp):
    mp.setattr(od, "_visible", lambda pq, pk: np.ones((pq.size, pk.size), dtype=bool))


def _mut_positions_shifted(mp):
    mp.setattr(od, "_query_positions", lambda ci, n: ci + 1 + np.arange(n))


def _mut_positions_reversed(mp):
    mp.setattr(od, "_query_positions", lambda ci, n: ci + np.arange(n)[::-1])


def _mut_scale_no_sqrt(mp):
    mp.setattr(od, "_scale", lambda d: 1.0 / d)


def _mut_rows_one_short(mp):
    mp.setattr(od, "_rows_read", lambda ci, n: ci + n - 1)


def _mut_rows_cache_only(mp):
    mp.setattr(od, "_rows_read", lambda ci, n: max(ci, 1))


MUTATIONS = [_mut_mask_strict, _mut_mask_all, _mut_positions_shifted, _mut_positions_reversed,
             _mut_scale_no_sqrt, _mut_rows_one_short, _mut_rows_cache_only]

PINS = [
    lambda: test_decode_matches_sdpa(*CASES[2]),
    lambda: test_decode_matches_sdpa(*CASES[4]),
    lambda: test_decode_is_last_rows_of_causal_forward(4, 12),
    test_decode_zero_query_is_mean_of_visible_values,
    test_decode_first_token,
    test_decode_ignores_rows_past_the_step,
]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_mistakes_decode(mutate, monkeypatch):
    mutate(monkeypatch)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin caught {mutate.__name__}"
