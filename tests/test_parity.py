"""GPU parity: the HIP forward (through the C ABI) against the CPU fp64
oracle on the same seeded inputs, element by element.

Small workloads are checked on every row; the large ones at their real
shapes on sampled rows and heads that the oracle computes one by one, plus
closed forms that hold at any size.  Every launch uses the configuration the
benchmark times (the same entry point and chunk sizes).
"""

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import (check, log, oracle_sample, sample_rows, to_np, visible_kv_len)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (deselect them with -m 'not gpu')")
    ra.load_library()
    yield
    torch.cuda.synchronize()


def run(q, k, v, seg, w, r, run_map=False):
    rm = None
    if run_map:
        rm = torch.full((w.ring_size, w.seq_q // w.q_chunk, w.seq_q // w.k_chunk), 7,
                        dtype=torch.uint8, device=q.device)
    out, lse = ra.blockwise_attn_fwd(q, k, v, seg, w.causal_block_size, w.q_chunk,
                                     w.k_chunk, w.ring_size, r, run_map=rm)
    torch.cuda.synchronize()
    return out, lse, rm


def check_run_map(rm, w, r):
    _, ref = oracle.skip_map_closed(w.causal_block_size, w.q_chunk, w.k_chunk, w.seq_q,
                                    w.ring_size, r)
    got = rm.cpu().numpy()
    assert np.array_equal(got, ref), f"run map differs at ring position {r}"


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_tiny_plumbing_all_positions():
    w = workloads.get("tiny_plumbing")
    outs = []
    for r in w.ring_indices:
        log(f"tiny_plumbing r={r}")
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        out, lse, rm = run(q, k, v, None, w, r, run_map=True)
        ref, ref_lse = oracle.attention_fwd(q, k, v, None, w.causal_block_size,
                                            w.ring_size, r)
        check(to_np(out), to_np(lse), ref, ref_lse, torch.float32, f"tiny r={r}")
        check_run_map(rm, w, r)
        outs.append((q, k, v, out))
    # Non-causal: the same query block at another ring position only changes
    # the order in which blocks are folded, not the result.
    q, k, v, out0 = outs[0]
    for r in (1, 2, 3):
        out_r, _, _ = run(q, k, v, None, w, r)
        np.testing.assert_allclose(to_np(out_r), to_np(out0), rtol=0, atol=1e-5)


def test_small_causal_all_positions():
    w = workloads.get("small_causal")
    for r in w.ring_indices:
        log(f"small_causal r={r}")
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        out, lse, rm = run(q, k, v, None, w, r, run_map=True)
        ref, ref_lse = oracle.attention_fwd(q, k, v, None, 1, w.ring_size, r)
        check(to_np(out), to_np(lse), ref, ref_lse, torch.bfloat16, f"small_causal r={r}")
        check_run_map(rm, w, r)


def test_packed_documents_all_positions():
    w = workloads.get("packed_documents")
    seg = workloads.make_segments(w, device=DEV)
    for r in w.ring_indices:
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        out, lse, rm = run(q, k, v, seg, w, r, run_map=True)
        check_run_map(rm, w, r)
        kv_len = visible_kv_len(w, r)
        for head, nrows in ((0, w.seq_q), (13, 192), (31, 192)):
            rows = np.arange(w.seq_q) if nrows == w.seq_q else sample_rows(w, 100 + r, nrows)
            log(f"packed_documents r={r} head={head} rows={len(rows)}")
            ref, ref_lse = oracle_sample(q, k, v, seg, 1, w.ring_size, r, head, rows, kv_len)
            check(to_np(out[:, rows, head]), to_np(lse[:, head, rows]), ref, ref_lse,
                  torch.bfloat16, f"packed r={r} h={head}")


@pytest.mark.timeout(600)
def test_share_7b_512k_sampled():
    """The 7B-shaped share at its real shape: sampled rows of EVERY head
    (each XCD group of the grid holds four consecutive heads), the run map,
    and a second launch that must agree bit for bit."""
    w = workloads.get("share_7b_512k")
    r = w.ring_indices[0]
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    log("share_7b_512k: inputs ready")
    out, lse, rm = run(q, k, v, None, w, r, run_map=True)
    log("share_7b_512k: forward done")
    check_run_map(rm, w, r)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    out2, lse2, _ = run(q, k, v, None, w, r)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "7B share not bitwise repeatable"
    # one host copy of the inputs, sliced per head
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for head in range(w.heads):
        rows = sample_rows(w, 200 + head, 8)
        ref, ref_lse = oracle.attention_fwd(qc[:, :, head:head + 1], kc[:, :, head:head + 1],
                                            vc[:, :, head:head + 1], None, 1, w.ring_size, r,
                                            rows=rows)
        check(to_np(out[:, rows, head]), to_np(lse[:, head, rows]), ref[:, :, 0, :],
              ref_lse[:, 0, :], torch.bfloat16, f"7b h={head} ({len(rows)} rows)")


@pytest.mark.timeout(900)
def test_share_65b_4m_sampled_and_poisoned():
    """The 65B-shaped share at its real shape, with the never-read blocks
    NaN: sampled rows of one head per XCD group of the grid (heads 8x ..
    8x + 7 run on XCD x)."""
    w = workloads.get("share_65b_4m")
    r = w.ring_indices[0]
    order, run_bits = oracle.skip_map_closed(w.causal_block_size, w.q_chunk, w.k_chunk,
                                             w.seq_q, w.ring_size, r)
    used = sorted({int(order[t]) for t in range(w.ring_size) if run_bits[t].any()})
    assert used == list(range(129))
    # Blocks no chunk pair reads are NaN: they must never reach the result.
    q, k, v = workloads.make_qkv(w, r, device=DEV, kv_blocks=used)
    log("share_65b_4m: inputs ready")
    out, lse, rm = run(q, k, v, None, w, r, run_map=True)
    log("share_65b_4m: forward done")
    check_run_map(rm, w, r)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    kv_len = visible_kv_len(w, r)
    assert kv_len == 129 * w.seq_q
    for head in (0, 9, 18, 27, 36, 45, 54, 63):
        rows = sample_rows(w, 300 + head, 8)
        log(f"share_65b_4m head={head} rows={len(rows)}")
        ref, ref_lse = oracle_sample(q, k, v, None, w.causal_block_size, w.ring_size, r,
                                     head, rows, kv_len)
        check(to_np(out[:, rows, head]), to_np(lse[:, head, rows]), ref, ref_lse,
              torch.bfloat16, f"65b h={head}")


# ---------------------------------------------------------------------------
# closed forms at full size, determinism
# ---------------------------------------------------------------------------

@pytest.mark.timeout(600)
def test_share_7b_q_zero_closed_form():
    """Q = 0: every logit is 0, so out_i = mean of the visible V rows and
    lse_i = ln(number of visible keys), at the 7B share's real shape."""
    w = workloads.get("share_7b_512k")
    r = w.ring_indices[0]
    _, k, v = workloads.make_qkv(w, r, device=DEV)
    q = torch.zeros((w.batch, w.seq_q, w.heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    out, lse, _ = run(q, k, v, None, w, r)
    rows = sample_rows(w, 400, 64)
    for head in (0, 31):
        vh = v[0, :, head].double().cpu().numpy()
        csum = np.cumsum(vh, axis=0)
        npos = r * w.seq_q + rows + 1                  # visible keys of each row
        ref = csum[npos - 1] / npos[:, None]
        ref_lse = np.log(npos.astype(np.float64))
        log(f"q_zero head={head}")
        check(to_np(out[0, rows, head]), to_np(lse[0, head, rows]), ref, ref_lse,
              torch.bfloat16, f"q0 h={head}")


def test_bitwise_repeat():
    """No atomics and a fixed reduction order: repeated calls agree bitwise."""
    for name in ("small_causal", "packed_documents"):
        w = workloads.get(name)
        r = w.ring_indices[-1]
        seg = workloads.make_segments(w, device=DEV)
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        o1, l1, _ = run(q, k, v, seg, w, r)
        o2, l2, _ = run(q, k, v, seg, w, r)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), name


# ---------------------------------------------------------------------------
# edge cases: ragged lengths, odd causal blocks, head dims, dtypes, segments
# ---------------------------------------------------------------------------

EDGE = [
    # B, Lq, N, H, D, dtype, c, qc, kc, segments
    (1, 96, 3, 2, 128, "bf16", 1, 32, 96, False),      # ragged: 96 rows, 3 sub-tiles
    (3, 160, 2, 3, 64, "bf16", 1, 32, 32, False),      # D = 64, batch 3
    (2, 224, 3, 2, 128, "bf16", 37, 32, 224, False),   # odd causal block
    (1, 128, 4, 2, 128, "bf16", 96, 64, 32, False),    # causal block not a tile multiple
    (1, 64, 5, 2, 128, "bf16", 10 ** 9, 32, 64, False),  # block longer than the sequence
    (1, 192, 2, 2, 128, "bf16", None, 64, 96, False),  # non-causal, ragged tiles
    (2, 256, 2, 2, 128, "bf16", 1, 128, 64, True),     # segments
    (1, 96, 2, 2, 128, "f32", 1, 32, 32, False),       # fp32, D = 128
    (2, 64, 3, 3, 64, "f32", 5, 32, 32, True),         # fp32, segments, block causal
    (1, 32, 1, 1, 128, "bf16", 1, 32, 32, False),      # one sub-tile, one block
]


@pytest.mark.parametrize("case", EDGE, ids=[f"e{i}" for i in range(len(EDGE))])
def test_edge_cases(case):
    B, Lq, N, H, D, dt, c, qc, kc, segs = case
    w = workloads.Workload("edge", B, Lq, N, tuple(range(N)), H, D, dt, c, qc, kc,
                           segments=False, seed=1000 + Lq + N)
    seg = None
    if segs:
        rng = np.random.default_rng(5)
        cuts = np.sort(rng.choice(np.arange(1, N * Lq), size=N * 3, replace=False))
        row = np.zeros(N * Lq, dtype=np.int32)
        for i, cpos in enumerate(cuts):
            row[cpos:] = i + 1
        seg = torch.from_numpy(np.stack([np.roll(row, 17 * b) for b in range(B)])).to(DEV)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    for r in range(N):
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        out, lse, rm = run(q, k, v, seg, w, r, run_map=True)
        ref, ref_lse = oracle.attention_fwd(q, k, v, None if seg is None else seg.cpu().numpy(),
                                            c, N, r)
        check(to_np(out), to_np(lse), ref, ref_lse, dtype, f"edge {case} r={r}")
        check_run_map(rm, w, r)


def test_empty_call():
    q = torch.empty((0, 64, 2, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((0, 128, 2, 128), dtype=torch.bfloat16, device=DEV)
    out, lse = ra.blockwise_attn_fwd(q, k, k, None, 1, 32, 32, 2, 1)
    assert out.shape == q.shape and lse.shape == (0, 2, 64)


def test_invalid_call_raises():
    q = torch.zeros((1, 64, 2, 96), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, 128, 2, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ra.RaError) as e:
        ra.blockwise_attn_fwd(q, k, k, None, 1, 32, 32, 2, 1)
    assert e.value.status == ra.RA_E_UNSUPPORTED
