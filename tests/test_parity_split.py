"""GPU parity of the key-split forward (ra_blockwise_attn_fwd_split): every
query tile's key walk cut into runs that fold into partial results, then
combined.  Checked against the CPU fp64 oracle on every row of the small
workloads, all ring positions, both placements and both dtypes, on edge
shapes (segments, ragged tiles, block-causal, D = 64, more splits than key
tiles), and with a workspace full of NaN (its contents on entry must not
matter).  The chunk-pair map of a split call must equal the oracle's."""

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import check, log, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (deselect them with -m 'not gpu')")
    ra.load_library()
    yield
    torch.cuda.synchronize()


def run_split(q, k, v, seg, w, r, splits, workspace=None):
    rm = torch.full((w.ring_size, w.seq_q // w.q_chunk, w.seq_q // w.k_chunk), 7,
                    dtype=torch.uint8, device=q.device)
    out, lse = ra.blockwise_attn_fwd(q, k, v, seg, w.causal_block_size, w.q_chunk, w.k_chunk,
                                     w.ring_size, r, run_map=rm, placement=w.placement,
                                     key_splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    _, ref_map = oracle.skip_map_closed(w.causal_block_size, w.q_chunk, w.k_chunk, w.seq_q,
                                        w.ring_size, r, placement=w.placement)
    assert np.array_equal(rm.cpu().numpy(), ref_map), f"run map differs at r={r}"
    return out, lse


def dtype_of(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


@pytest.mark.parametrize("name,splits", [("small_causal", "auto"), ("small_causal", 3),
                                         ("small_causal_striped", "auto"),
                                         ("tiny_plumbing", 2), ("tiny_plumbing", 3)])
def test_split_workloads_all_positions(name, splits):
    w = workloads.get(name)
    for r in w.ring_indices:
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        if splits == "auto":
            n = ra.fwd_key_splits(w.batch, w.seq_q, w.heads, ra.RA_BF16, w.causal_block_size,
                                  w.ring_size, r,
                                  torch.cuda.get_device_properties(DEV).multi_processor_count,
                                  w.placement)
            log(f"{name} r={r}: {n} key splits")
            assert n > 1 or r == 0
        out, lse = run_split(q, k, v, None, w, r, splits)
        ref, ref_lse = oracle.attention_fwd(q, k, v, None, w.causal_block_size, w.ring_size, r,
                                            placement=w.placement)
        check(to_np(out), to_np(lse), ref, ref_lse, dtype_of(w), f"{name} split={splits} r={r}")


def test_split_matches_unsplit():
    """The split result equals the one-workgroup walk up to the rounding of
    the fold (bf16 bounds)."""
    w = workloads.get("small_causal")
    r = w.ring_indices[-1]
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    o1, l1 = ra.blockwise_attn_fwd(q, k, v, None, 1, w.q_chunk, w.k_chunk, w.ring_size, r)
    for splits in (2, 8, 16):
        o2, l2 = ra.blockwise_attn_fwd(q, k, v, None, 1, w.q_chunk, w.k_chunk, w.ring_size, r,
                                       key_splits=splits)
        torch.cuda.synchronize()
        check(to_np(o2), to_np(l2), to_np(o1), to_np(l1), torch.bfloat16, f"vs unsplit {splits}")


def test_split_workspace_contents_do_not_matter():
    w = workloads.get("small_causal")
    r = 5
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    splits = 8
    nbytes = ra.fwd_split_workspace_bytes(w.batch, w.seq_q, w.heads, w.head_dim, splits)
    assert nbytes == splits * w.batch * w.heads * w.seq_q * (w.head_dim + 2) * 4
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    out, lse = run_split(q, k, v, None, w, r, splits, workspace=ws)
    ref, ref_lse = oracle.attention_fwd(q, k, v, None, 1, w.ring_size, r)
    check(to_np(out), to_np(lse), ref, ref_lse, torch.bfloat16, "NaN workspace")
    # the same workspace again, now holding the previous call's partials
    q2, k2, v2 = workloads.make_qkv(w, 2, device=DEV)
    out2, lse2 = run_split(q2, k2, v2, None, w, 2, splits, workspace=ws)
    ref2, ref_lse2 = oracle.attention_fwd(q2, k2, v2, None, 1, w.ring_size, 2)
    check(to_np(out2), to_np(lse2), ref2, ref_lse2, torch.bfloat16, "reused workspace")


SPLIT_EDGE = [
    # B, Lq, N, H, D, dtype, c, qc, kc, segments, placement, splits
    (1, 96, 3, 2, 128, "bf16", 1, 32, 96, False, "contiguous", 4),
    (3, 160, 2, 3, 64, "bf16", 1, 32, 32, False, "contiguous", 5),
    (2, 224, 3, 2, 128, "bf16", 37, 32, 224, False, "contiguous", 3),
    (1, 192, 2, 2, 128, "bf16", None, 64, 96, False, "contiguous", 7),
    (2, 256, 2, 2, 128, "bf16", 1, 128, 64, True, "contiguous", 6),
    (2, 256, 2, 2, 128, "bf16", 1, 128, 64, True, "striped", 6),
    (1, 96, 2, 2, 128, "f32", 1, 32, 32, False, "contiguous", 4),
    (2, 64, 3, 3, 64, "f32", 5, 32, 32, True, "contiguous", 3),
    (1, 32, 1, 1, 128, "bf16", 1, 32, 32, False, "contiguous", 64),   # splits >> tiles
    (1, 64, 4, 2, 64, "f32", None, 32, 32, False, "striped", 64),
    (1, 256, 4, 2, 128, "bf16", 2, 64, 64, False, "striped", 5),
    (2, 128, 2, 2, 128, "bf16", 8, 64, 64, True, "striped", 4),
]


@pytest.mark.parametrize("case", SPLIT_EDGE, ids=[f"s{i}" for i in range(len(SPLIT_EDGE))])
def test_split_edge_cases(case):
    B, Lq, N, H, D, dt, c, qc, kc, segs, place, splits = case
    w = workloads.Workload("split_edge", B, Lq, N, tuple(range(N)), H, D, dt, c, qc, kc,
                           seed=2000 + Lq + N, placement=place)
    seg = None
    if segs:
        rng = np.random.default_rng(6)
        cuts = np.sort(rng.choice(np.arange(1, N * Lq), size=N * 3, replace=False))
        row = np.zeros(N * Lq, dtype=np.int32)
        for i, cpos in enumerate(cuts):
            row[cpos:] = i + 1
        seg = torch.from_numpy(np.stack([np.roll(row, 11 * b) for b in range(B)])).to(DEV)
    for r in range(N):
        q, k, v = workloads.make_qkv(w, r, device=DEV)
        out, lse = run_split(q, k, v, seg, w, r, splits)
        ref, ref_lse = oracle.attention_fwd(q, k, v, None if seg is None else seg.cpu().numpy(),
                                            c, N, r, placement=place)
        check(to_np(out), to_np(lse), ref, ref_lse, dtype_of(w), f"split edge {case} r={r}")


def test_split_rejects_bad_workspace():
    w = workloads.get("small_causal")
    q, k, v = workloads.make_qkv(w, 1, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ra.RaError) as e:
        ra.blockwise_attn_fwd(q, k, v, None, 1, 512, 512, 8, 1, key_splits=4, workspace=small)
    assert e.value.status == ra.RA_E_INVALID
    with pytest.raises(ra.RaError) as e:
        ra.blockwise_attn_fwd(q, k, v, None, 1, 512, 512, 8, 1, key_splits=65)
    assert e.value.status == ra.RA_E_INVALID


def test_split_packed_documents_sampled():
    """Packed documents (segment ids, 1024 query tiles) with the walk forced
    into 3 runs: every row of one head and sampled rows of another against
    the oracle, and the chunk map."""
    from parity import oracle_sample, sample_rows, visible_kv_len
    w = workloads.get("packed_documents")
    seg = workloads.make_segments(w, device=DEV)
    r = 5
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    out, lse = run_split(q, k, v, seg, w, r, 3)
    kv_len = visible_kv_len(w, r)
    for head, nrows in ((0, w.seq_q), (21, 192)):
        rows = np.arange(w.seq_q) if nrows == w.seq_q else sample_rows(w, 700, nrows)
        log(f"packed_documents split=3 r={r} head={head} rows={len(rows)}")
        ref, ref_lse = oracle_sample(q, k, v, seg, 1, w.ring_size, r, head, rows, kv_len)
        check(to_np(out[:, rows, head]), to_np(lse[:, head, rows]), ref, ref_lse,
              torch.bfloat16, f"packed split h={head}")


@pytest.mark.timeout(600)
def test_split_share_7b_sampled():
    """The 7B-shaped share (16 blocks of 32768 keys) with each query tile's
    walk cut into 2 runs, so that the second run seeks into the middle of
    the ring walk: sampled rows of two heads against the oracle."""
    from parity import oracle_sample, sample_rows
    w = workloads.get("share_7b_512k")
    r = w.ring_indices[0]
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    log("share_7b_512k split=2: inputs ready")
    out, lse = ra.blockwise_attn_fwd(q, k, v, None, 1, w.q_chunk, w.k_chunk, w.ring_size, r,
                                     key_splits=2)
    torch.cuda.synchronize()
    log("share_7b_512k split=2: forward done")
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    for head in (3, 30):
        rows = sample_rows(w, 800 + head, 24)
        log(f"share_7b_512k split=2 head={head} rows={len(rows)}")
        ref, ref_lse = oracle_sample(q, k, v, None, 1, w.ring_size, r, head, rows)
        check(to_np(out[:, rows, head]), to_np(lse[:, head, rows]), ref, ref_lse,
              torch.bfloat16, f"7b split h={head}")
