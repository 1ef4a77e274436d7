"""The pair counts behind bench.py's flop figures (no GPU).

The headline rate is 4 D H times the number of causally visible (query,
key) pairs.  These tests pin bench.py's closed-form counts to the pair
count of the 7B-shaped share written out by hand (15 full blocks plus the
diagonal triangle), and to the oracle's explicit enumeration on small
shapes for every placement and mask; the per-segment count is pinned to
brute force.
"""

import numpy as np
import pytest

import bench
import oracle
import workloads


def test_share_7b_pairs_closed_form():
    w = workloads.get("share_7b_512k")
    Lq = w.seq_q
    n = int(bench.visible_keys_per_row(Lq, w.ring_size, 15, 1).sum())
    # ring position 15 of 16: blocks 0..14 fully visible, block 15 a triangle
    assert n == 15 * Lq * Lq + Lq * (Lq + 1) // 2 == 16_643_014_656
    assert bench.causal_flops(w, 15) == 4.0 * 128 * 32 * n == 2.72679152123904e14


@pytest.mark.parametrize("placement,causal", [("contiguous", 1), ("contiguous", 3),
                                              ("contiguous", 16), ("contiguous", None),
                                              ("striped", 1), ("striped", None)])
def test_visible_keys_match_oracle_enumeration(placement, causal):
    Lq, N = 24, 4
    for r in range(N):
        rows = bench.visible_keys_per_row(Lq, N, r, causal, placement)
        for i in (0, 5, Lq - 1):
            assert rows[i] == oracle.count_visible_pairs(Lq, N, r, causal, rows=[i],
                                                         placement=placement), (r, i)
        assert int(rows.sum()) == oracle.count_visible_pairs(Lq, N, r, causal,
                                                             placement=placement)


def test_segment_visible_keys_brute_force():
    rng = np.random.default_rng(5)
    Lq, N = 16, 4
    S = Lq * N
    for trial in range(5):
        # arbitrary labels, documents and repeated ids included
        seg = rng.integers(0, 4, S) if trial % 2 else np.repeat(np.arange(S // 8), 8)
        for r in range(N):
            got = bench.segment_visible_keys_per_row(seg, Lq, r)
            want = [sum(1 for j in range(r * Lq + i + 1) if seg[j] == seg[r * Lq + i])
                    for i in range(Lq)]
            assert list(got) == want, (trial, r)
            assert int(got.sum()) == oracle.count_visible_pairs(Lq, N, r, 1, seg[None, :])


def test_segment_counts_never_exceed_causal():
    w = workloads.get("packed_documents")
    seg = np.repeat(np.arange(w.seq_k // 512), 512)
    for r in (0, 3, 7):
        causal = bench.visible_keys_per_row(w.seq_q, w.ring_size, r, 1)
        within = bench.segment_visible_keys_per_row(seg, w.seq_q, r)
        assert (within <= causal).all() and (within >= 1).all()


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus N > 1 exits with a message before touching a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_timed_call_parity_accepts_and_rejects():
    """The bench's check of the timed call: an output equal to the oracle's
    (up to bf16 rounding) passes; a dropped row, a zero output (which the
    absolute bounds alone would accept at long shapes) and a shifted lse
    fail.  CPU tensors stand in for the device buffers."""
    import torch
    rng = np.random.default_rng(11)
    R, D, L = 16, 128, 64
    rows = np.sort(rng.choice(L, R, replace=False))
    ro = rng.standard_normal((1, R, 1, D)) * 1e-3
    rl = 13.0 + rng.standard_normal((1, 1, R))
    out = torch.zeros((1, L, 2, D), dtype=torch.bfloat16)
    lse = torch.zeros((1, 2, L), dtype=torch.float32)
    out[0, rows, 0] = torch.from_numpy(ro[0, :, 0]).to(torch.bfloat16)
    lse[0, 0, rows] = torch.from_numpy(rl[0, 0]).float()
    ok = bench.timed_call_parity((out, lse), (ro, rl), 15, rows)
    assert ok["pass"] and ok["out_rel_l2"] < 1e-2
    bad = out.clone()
    bad[0, rows[3], 0] = 0
    assert not bench.timed_call_parity((bad, lse), (ro, rl), 15, rows)["pass"]
    assert not bench.timed_call_parity((torch.zeros_like(out), lse), (ro, rl), 15,
                                       rows)["pass"]
    assert not bench.timed_call_parity((out, lse + 0.05), (ro, rl), 15, rows)["pass"]
    # backward: dq
    rq = rng.standard_normal((1, R, 1, D))
    dq = torch.zeros((1, L, 2, D), dtype=torch.float32)
    dq[0, rows, 0] = torch.from_numpy(rq[0, :, 0]).float()
    assert bench.timed_call_parity((dq,), (rq,), 15, rows)["pass"]
    dq[0, rows[0], 0] *= -1
    assert not bench.timed_call_parity((dq,), (rq,), 15, rows)["pass"]
