"""GPU parity of the forward under striped placement against the fp64 oracle.

Striped placement: block r of q, k, v and segment ids holds the global
positions r, r + N, r + 2N, ... (the load-balancing placement that "Ring
Attention with Blockwise Transformers for Near-Infinite Context" names in
sections 六 and 七).  The same acceptance bounds as the contiguous forward
(bf16: max 2e-2, mean 2e-3, relative L2 1e-2; fp32: max 1e-5), and the
kernel's chunk-pair decisions must equal the oracle's striped skip map byte
for byte.
"""

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import check, log, oracle_sample, sample_rows, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
STRIPED = "striped"


def _run(q, k, v, seg, w, r, run_map=True):
    rm = None
    if run_map:
        rm = torch.full((w.ring_size, w.seq_q // w.q_chunk, w.seq_q // w.k_chunk), 7,
                        dtype=torch.uint8, device=q.device)
    out, lse = ra.blockwise_attn_fwd(q, k, v, seg, w.causal_block_size, w.q_chunk, w.k_chunk,
                                     w.ring_size, r, run_map=rm, placement=STRIPED)
    torch.cuda.synchronize()
    return out, lse, rm


def _check_map(rm, w, r):
    _, ref = oracle.skip_map_closed(w.causal_block_size, w.q_chunk, w.k_chunk, w.seq_q,
                                    w.ring_size, r, placement=STRIPED)
    assert np.array_equal(rm.cpu().numpy(), ref), f"striped run map differs at r={r}"


def test_small_causal_striped_all_positions():
    w = workloads.get("small_causal_striped")
    for r in w.ring_indices:
        log(f"small_causal_striped r={r}")
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        out, lse, rm = _run(q, k, v, None, w, r)
        ref, ref_lse = oracle.attention_fwd(q, k, v, None, 1, w.ring_size, r,
                                            placement=STRIPED)
        check(to_np(out), to_np(lse), ref, ref_lse, torch.bfloat16, f"striped small r={r}")
        _check_map(rm, w, r)


EDGE = [
    # B, Lq, N, H, D, dtype, causal, qc, kc, segments, r
    (1, 96, 3, 2, 64, "bf16", 1, 32, 32, False, 1),
    (2, 128, 4, 2, 128, "bf16", 1, 64, 32, True, 3),
    (1, 256, 2, 2, 128, "bf16", 1, 128, 64, True, 0),
    (1, 32, 5, 1, 128, "bf16", 1, 32, 32, False, 4),
    (1, 64, 4, 2, 64, "f32", 1, 32, 32, False, 2),
    (1, 96, 3, 2, 128, "f32", 1, 32, 32, True, 0),
    (1, 160, 2, 2, 128, "bf16", 100000, 32, 32, False, 1),
    # block causal: c divides N (token causal on shifted coordinates) ...
    (1, 128, 4, 2, 128, "bf16", 2, 32, 32, False, 1),
    (1, 128, 4, 2, 128, "bf16", 2, 64, 32, True, 3),
    (1, 96, 8, 2, 64, "bf16", 4, 32, 32, False, 5),
    (1, 64, 4, 2, 64, "f32", 4, 32, 32, False, 2),
    # ... or is a multiple of N (block causal on the local rows)
    (2, 128, 4, 2, 128, "bf16", 8, 64, 32, True, 2),
    (1, 160, 2, 2, 128, "bf16", 6, 32, 32, False, 1),
    (1, 96, 3, 2, 64, "bf16", 96, 32, 32, False, 1),
    (1, 96, 3, 2, 128, "f32", 12, 32, 32, False, 0),
]


@pytest.mark.parametrize("case", EDGE, ids=[str(c) for c in EDGE])
def test_striped_edge(case):
    B, Lq, N, H, D, dt, c, qc, kc, segs, r = case
    w = workloads.Workload(f"striped_edge{case}", B, Lq, N, (r,), H, D, dt, c, qc, kc,
                           segments=segs, seed=777 + Lq + N + D, placement=STRIPED)
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    seg = None
    if segs:
        # short documents along the global positions, in storage order
        rng = np.random.default_rng(w.seed)
        nat = np.cumsum(rng.random((B, w.seq_k)) < 0.05, axis=1).astype(np.int32)
        seg = torch.from_numpy(workloads.to_storage_order(nat, N, STRIPED)).to(DEV)
    out, lse, rm = _run(q, k, v, seg, w, r)
    ref, ref_lse = oracle.attention_fwd(q, k, v, None if seg is None else seg.cpu().numpy(),
                                        c, N, r, placement=STRIPED)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    check(to_np(out), to_np(lse), ref, ref_lse, dtype, f"striped edge {case}")
    _check_map(rm, w, r)


def test_striped_noncausal_equals_contiguous():
    """Without a causal mask the placement only renames positions: both
    calls see every key, so both match the oracle, and each other within
    the bf16 bounds (not bit for bit: the striped walk folds the key tiles
    in another order)."""
    w = workloads.Workload("nc", 1, 256, 4, (2,), 4, 128, "bf16", None, 64, 64, seed=4321)
    q, k, v = workloads.make_qkv(w, 2, device=DEV)
    a, la = ra.blockwise_attn_fwd(q, k, v, None, None, 64, 64, 4, 2, placement=STRIPED)
    b, lb = ra.blockwise_attn_fwd(q, k, v, None, None, 64, 64, 4, 2)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_fwd(q, k, v, None, None, 4, 2)
    check(to_np(a), to_np(la), ref, ref_lse, torch.bfloat16, "striped non-causal")
    check(to_np(a), to_np(la), to_np(b), to_np(lb), torch.bfloat16, "striped vs contiguous")


@pytest.mark.timeout(600)
def test_share_7b_striped_sampled():
    w = workloads.get("share_7b_512k_striped")
    for r in (15, 0):
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        log(f"share_7b_512k_striped r={r}: inputs ready")
        out, lse, rm = _run(q, k, v, None, w, r)
        log(f"share_7b_512k_striped r={r}: forward done")
        _check_map(rm, w, r)
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        for head in (0, 31):
            rows = sample_rows(w, 300 + head + r, 16)
            log(f"share_7b_512k_striped r={r} head={head} rows={len(rows)}")
            ref, ref_lse = oracle_sample(q, k, v, None, 1, w.ring_size, r, head, rows,
                                         placement=STRIPED)
            check(to_np(out[:, rows, head]), to_np(lse[:, head, rows]), ref, ref_lse,
                  torch.bfloat16, f"7b striped r={r} h={head}")
        del q, k, v, out, lse, rm
        torch.cuda.empty_cache()


def test_striped_rejects_block_causal_without_coordinates():
    """A causal block that neither divides the ring size nor is a multiple
    of it has no form on key coordinates: refused before any launch."""
    q = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, 256, 1, 128), dtype=torch.bfloat16, device=DEV)
    for c in (3, 6, 10):
        with pytest.raises(ra.RaError) as e:
            ra.blockwise_attn_fwd(q, k, k, None, c, 32, 32, 4, 1, placement=STRIPED)
        assert e.value.status == ra.RA_E_UNSUPPORTED
