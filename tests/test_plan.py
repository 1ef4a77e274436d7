"""The library's host planner (ra_blockwise_plan) against the oracle's skip
maps, bit-exact (CPU only)."""

import numpy as np
import pytest

import long_context_exact_ra_amd as ra
import oracle
import workloads


def test_planner_matches_oracle_exhaustive():
    n = 0
    for Lq in (4, 6, 12, 16):
        divs = [d for d in range(1, Lq + 1) if Lq % d == 0]
        for N in (1, 2, 3, 5):
            for c in (None, 1, 2, 3, 5, 8, Lq, 2 * Lq, 10 ** 9):
                for qc in divs:
                    for kc in divs:
                        for r in range(N):
                            o_ref, run_ref = oracle.skip_map_bruteforce(c, qc, kc, Lq, N, r)
                            o, run, cnt = ra.blockwise_plan(c, qc, kc, Lq, N, r)
                            assert (o == o_ref).all()
                            assert (run == run_ref).all(), (Lq, N, c, qc, kc, r)
                            assert cnt == int(run_ref.sum())
                            n += 1
    assert n > 5000


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_planner_matches_oracle_on_workloads(name):
    w = workloads.get(name)
    for r in w.ring_indices:
        o_ref, run_ref = oracle.skip_map_closed(w.causal_block_size, w.q_chunk, w.k_chunk,
                                                w.seq_q, w.ring_size, r)
        o, run, cnt = ra.blockwise_plan(w.causal_block_size, w.q_chunk, w.k_chunk, w.seq_q,
                                        w.ring_size, r)
        assert (o == o_ref).all()
        assert np.array_equal(run, run_ref)
        assert cnt == int(run_ref.sum())
