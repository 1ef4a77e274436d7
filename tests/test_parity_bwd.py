"""GPU parity of the backward (dq, dk, dv, delta) against the fp64 oracle.

Each case runs the library forward, then the library backward on the same
seeded inputs and a seeded upstream gradient, and compares with
``oracle.attention_bwd`` computed from the same (bf16-rounded) inputs.

Bounds (no tolerance is given for the backward; derived from the
arithmetic): the kernels round p and ds to bf16 (relative error <= 2^-9,
round to nearest even) as operands of fp32-accumulating matrix products, so
each gradient is a sum of terms with independent relative errors of that
size; its relative L2 error is expected around 2^-9 ~ 2e-3.  The test
requires relative L2 <= 1e-2 and max |err| <= 2e-2 * max |ref| per tensor.
float32 inputs: every operand stays float32 (products on float32 MFMA, the
exponential v_exp_f32 to about 1 ulp), so the errors are float32 rounding
over sums of up to S terms: relative L2 <= 1e-5 and max |err| <= 1e-4 *
max |ref|.  delta is a plain fp32 reduction of the kernel's own out:
relative L2 <= 1e-5 against the same sum in fp64.
"""

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import log, to_np

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_REL = 2e-2
REL_L2_F32 = 1e-5
MAX_REL_F32 = 1e-4


def _cmp(name, got, ref, what, f32=False):
    err = np.abs(got - ref)
    scale = max(float(np.abs(ref).max(initial=0)), 1e-30)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"  bwd {what} {name}: rel_l2={rel:.3e} max_err/max_ref={float(err.max(initial=0)) / scale:.3e}")
    assert np.isfinite(got).all(), (what, name)
    assert rel <= (REL_L2_F32 if f32 else REL_L2), (what, name, rel)
    assert float(err.max(initial=0)) <= (MAX_REL_F32 if f32 else MAX_REL) * scale, (what, name)


def _short_documents(B, S, seed):
    """Segment ids of documents 1..80 tokens long (many per sequence)."""
    rng = np.random.default_rng(seed)
    seg = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        pos, doc = 0, 0
        while pos < S:
            n = int(rng.integers(1, 81))
            seg[b, pos:pos + n] = doc
            pos += n
            doc += 1
    return seg


def _run(w, r, dev, key_splits=1, workspace=None):
    q, k, v = workloads.make_qkv(w, r, device=dev)
    dout = workloads.make_dout(w, r, device=dev)
    seg = workloads.make_segments(w, device=dev)
    if seg is not None and "edge" in w.name:
        nat = _short_documents(w.batch, w.seq_k, w.seed + 1)
        seg = torch.from_numpy(workloads.to_storage_order(nat, w.ring_size, w.placement)).to(dev)
    out, lse = ra.blockwise_attn_fwd(q, k, v, seg, w.causal_block_size, w.q_chunk, w.k_chunk,
                                     w.ring_size, r, placement=w.placement)
    dq, dk, dv, delta = ra.blockwise_attn_bwd(q, k, v, out, lse, dout, seg, w.causal_block_size,
                                              w.q_chunk, w.k_chunk, w.ring_size, r,
                                              placement=w.placement, key_splits=key_splits,
                                              workspace=workspace)
    torch.cuda.synchronize()
    return q, k, v, dout, seg, out, (dq, dk, dv, delta)


def _check_delta(dout, out, delta, what):
    ref = np.einsum("bihd,bihd->bhi", to_np(dout), to_np(out))
    got = to_np(delta)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"  bwd {what} delta: rel_l2={rel:.3e}")
    assert rel <= 1e-5, (what, rel)


def _full_case(w, r, heads=None, key_splits=1):
    dev = torch.device("cuda:0")
    q, k, v, dout, seg, out, (dq, dk, dv, delta) = _run(w, r, dev, key_splits)
    what = f"{w.name} r={r} splits={key_splits}"
    _check_delta(dout, out, delta, what)
    hs = list(range(w.heads)) if heads is None else list(heads)
    sl = lambda t: t[:, :, hs].contiguous().cpu()
    rdq, rdk, rdv = oracle.attention_bwd(sl(q), sl(k), sl(v), sl(dout),
                                         None if seg is None else seg.cpu().numpy(),
                                         w.causal_block_size, w.ring_size, r,
                                         placement=w.placement)
    f32 = q.dtype == torch.float32
    _cmp("dq", to_np(dq[:, :, hs]), rdq, what, f32)
    _cmp("dk", to_np(dk[:, :, hs]), rdk, what, f32)
    _cmp("dv", to_np(dv[:, :, hs]), rdv, what, f32)


@pytest.mark.parametrize("r", [0, 3, 7])
def test_bwd_small_causal(r):
    _full_case(workloads.get("small_causal"), r)


def test_bwd_packed_documents():
    _full_case(workloads.get("packed_documents"), 5, heads=[0, 17])


EDGE = [
    # B, Lq, N, H, D, causal, qc, kc, segments, r
    (1, 64, 2, 2, 128, 1, 64, 64, False, 1),
    (2, 96, 3, 2, 64, 1, 32, 32, False, 2),
    (1, 128, 1, 4, 128, None, 128, 128, False, 0),
    (1, 160, 2, 2, 128, 5, 32, 32, False, 1),
    (2, 128, 2, 2, 128, 1, 64, 64, True, 1),
    (1, 32, 4, 1, 128, 1, 32, 32, False, 3),
    (1, 256, 2, 2, 128, 100000, 64, 64, False, 1),
    (1, 512, 3, 1, 128, 64, 128, 128, True, 2),
]


@pytest.mark.parametrize("case", EDGE, ids=[str(c) for c in EDGE])
def test_bwd_edge(case):
    B, Lq, N, H, D, c, qc, kc, segs, r = case
    w = workloads.Workload(f"edge{case}", B, Lq, N, (r,), H, D, "bf16", c, qc, kc,
                           segments=segs, seed=4242 + Lq + D + N)
    _full_case(w, r)


def test_bwd_share_7b_sampled_and_invariants():
    """The 7B-shaped share at full size: dq on sampled rows of two heads
    against the oracle; dk and dv through invariants of the exact gradient
    (sum_j dk_j = 0; sum_j dv_j = sum_i dout_i, each probability row summing
    to one) on every head."""
    w = workloads.get("share_7b_512k")
    r = w.ring_indices[0]
    dev = torch.device("cuda:0")
    q, k, v, dout, seg, out, (dq, dk, dv, delta) = _run(w, r, dev)
    what = f"{w.name} r={r}"
    ref = torch.einsum("bihd,bihd->bhi", dout.double(), out.double())
    rel = float((delta.double() - ref).norm() / ref.norm())
    log(f"  bwd {what} delta: rel_l2={rel:.3e}")
    assert rel <= 1e-5
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(w.seq_q, size=48, replace=False))
    for h in (0, 21):
        sl = lambda t: t[:, :, h:h + 1].contiguous().cpu()
        rdq, _, _ = oracle.attention_bwd(sl(q), sl(k), sl(v), sl(dout), None,
                                         w.causal_block_size, w.ring_size, r, rows=rows)
        _cmp(f"dq[h{h}, 48 rows]", to_np(dq[:, rows, h:h + 1]), rdq, what)
    # invariants, per head, in fp64 on the device
    sk = dk.double().sum(dim=1)                     # [B, H, D], should be 0
    scale_k = dk.double().abs().sum(dim=1)
    ratio = float((sk.abs() / scale_k.clamp_min(1e-30)).max())
    log(f"  bwd {what} |sum_j dk_j| / sum_j |dk_j| max={ratio:.3e}")
    assert ratio <= 1e-3
    sv = dv.double().sum(dim=1)
    so = dout.double().sum(dim=1)
    relv = float((sv - so).norm() / so.norm())
    log(f"  bwd {what} sum_j dv_j vs sum_i dout_i: rel_l2={relv:.3e}")
    assert relv <= REL_L2
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def _sparse_rows(w, seed, per_tile=64, n_per_tile=2):
    """n_per_tile seeded rows in every per_tile-row query tile of the share,
    so that every query tile the dK/dV kernel streams holds rows of R."""
    rng = np.random.default_rng(seed)
    rows = []
    for t0 in range(0, w.seq_q, per_tile):
        n = min(per_tile, w.seq_q - t0)
        rows.extend((t0 + rng.choice(n, size=min(n_per_tile, n), replace=False)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _sparse_upstream_case(w, r, heads, seed, n_per_tile):
    """The share at full size with dout zero outside a row set R (every
    query tile holds rows of R).  The exact gradient is then the sum of the
    contributions of the rows in R alone (the oracle's rows=R), so dk and dv
    can be compared element by element on EVERY key of the sampled heads --
    every ring block, up to the last keys, whose float32 dk/dv addresses lie
    past 2^31 bytes -- while the kernels run their full grids.  dq must
    vanish exactly outside R on every head."""
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_qkv(w, r, device=dev)
    R = _sparse_rows(w, seed, n_per_tile=n_per_tile)
    keep = torch.zeros((1, w.seq_q, 1, 1), dtype=torch.bfloat16, device=dev)
    keep[:, torch.from_numpy(R).to(dev)] = 1
    dout = workloads.make_dout(w, r, device=dev) * keep
    out, lse = ra.blockwise_attn_fwd(q, k, v, None, w.causal_block_size, w.q_chunk, w.k_chunk,
                                     w.ring_size, r, placement=w.placement)
    dq, dk, dv, delta = ra.blockwise_attn_bwd(q, k, v, out, lse, dout, None,
                                              w.causal_block_size, w.q_chunk, w.k_chunk,
                                              w.ring_size, r, placement=w.placement)
    torch.cuda.synchronize()
    what = f"{w.name} r={r} sparse upstream ({len(R)} rows)"
    log(f"{what}: backward done")
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    others = torch.ones(w.seq_q, dtype=torch.bool, device=dev)
    others[torch.from_numpy(R).to(dev)] = False
    assert int(torch.count_nonzero(dq[:, others])) == 0, "dq nonzero outside the rows of R"
    # invariants on every head: sum_j dk_j = 0, sum_j dv_j = sum_{i in R} dout_i
    sk = dk.double().sum(dim=1)
    ratio = float((sk.abs() / dk.double().abs().sum(dim=1).clamp_min(1e-30)).max())
    assert ratio <= 1e-3, ratio
    so = dout.double().sum(dim=1)
    relv = float((dv.double().sum(dim=1) - so).norm() / so.norm())
    log(f"  bwd {what}: |sum dk|/sum|dk| max={ratio:.3e}, sum dv rel_l2={relv:.3e}")
    assert relv <= REL_L2
    for h in heads:
        sl = lambda t: t[:, :, h:h + 1].contiguous().cpu()
        rdq, rdk, rdv = oracle.attention_bwd(sl(q), sl(k), sl(v), sl(dout), None,
                                             w.causal_block_size, w.ring_size, r, rows=R,
                                             max_scores=1 << 26, placement=w.placement)
        _cmp(f"dq[h{h}, R]", to_np(dq[:, R, h:h + 1]), rdq, what)
        gk, gv = to_np(dk[:, :, h:h + 1]), to_np(dv[:, :, h:h + 1])
        _cmp(f"dk[h{h}, all {w.seq_k} keys]", gk, rdk, what)
        _cmp(f"dv[h{h}, all {w.seq_k} keys]", gv, rdv, what)
        # per ring block, so that a block written to the wrong place or not
        # at all shows by name
        for kb in range(w.ring_size):
            ks = slice(kb * w.seq_q, (kb + 1) * w.seq_q)
            for name, g, e in (("dk", gk, rdk), ("dv", gv, rdv)):
                rel = float(np.linalg.norm(g[:, ks] - e[:, ks])
                            / max(np.linalg.norm(e[:, ks]), 1e-300))
                assert rel <= REL_L2, (what, h, name, kb, rel)


@pytest.mark.timeout(600)
def test_bwd_share_7b_sparse_upstream_elementwise():
    """dk and dv of the 7B-shaped share compared element by element on all
    524288 keys of two heads (on different XCD groups of the dK/dV grid)."""
    w = workloads.get("share_7b_512k")
    _sparse_upstream_case(w, w.ring_indices[0], heads=(0, 21), seed=79, n_per_tile=2)


@pytest.mark.timeout(600)
def test_bwd_share_7b_striped_sparse_upstream_elementwise():
    """The same under striped placement (ring position 15), one head."""
    w = workloads.get("share_7b_512k_striped")
    _sparse_upstream_case(w, 15, heads=(13,), seed=80, n_per_tile=1)


@pytest.mark.parametrize("r", [0, 5])
def test_bwd_small_causal_striped(r):
    _full_case(workloads.get("small_causal_striped"), r)


STRIPED_EDGE = [
    # B, Lq, N, H, D, qc, kc, segments, r
    (1, 96, 3, 2, 128, 32, 32, False, 1),   # 256-key workgroups span three blocks
    (2, 128, 4, 2, 64, 64, 32, True, 2),
    (1, 256, 2, 2, 128, 64, 64, True, 0),
    (1, 32, 5, 1, 128, 32, 32, False, 4),
]


@pytest.mark.parametrize("case", STRIPED_EDGE, ids=[str(c) for c in STRIPED_EDGE])
def test_bwd_striped_edge(case):
    B, Lq, N, H, D, qc, kc, segs, r = case
    w = workloads.Workload(f"striped_edge{case}", B, Lq, N, (r,), H, D, "bf16", 1, qc, kc,
                           segments=segs, seed=5151 + Lq + D + N, placement="striped")
    _full_case(w, r)


STRIPED_BLOCK_EDGE = [
    # B, Lq, N, H, D, causal, qc, kc, segments, r: the causal block divides
    # N (token causal on shifted coordinates) or is a multiple of it (block
    # causal on the local rows)
    (1, 128, 4, 2, 128, 2, 32, 32, False, 1),
    (1, 96, 8, 2, 64, 4, 32, 32, False, 5),
    (2, 128, 4, 2, 128, 8, 64, 32, True, 2),
    (1, 160, 2, 2, 128, 6, 32, 32, False, 1),
    (1, 288, 3, 2, 128, 96, 32, 32, False, 2),  # 256-key workgroups span blocks
]


@pytest.mark.parametrize("case", STRIPED_BLOCK_EDGE, ids=[str(c) for c in STRIPED_BLOCK_EDGE])
def test_bwd_striped_block_causal(case):
    B, Lq, N, H, D, c, qc, kc, segs, r = case
    w = workloads.Workload(f"striped_block{case}", B, Lq, N, (r,), H, D, "bf16", c, qc, kc,
                           segments=segs, seed=5252 + Lq + D + N + c, placement="striped")
    _full_case(w, r)


def test_bwd_share_7b_striped_sampled():
    """The 7B-shaped striped share at ring position 15: dq on sampled rows
    of one head against the oracle, dk and dv through the invariants."""
    w = workloads.get("share_7b_512k_striped")
    r = 15
    dev = torch.device("cuda:0")
    q, k, v, dout, seg, out, (dq, dk, dv, delta) = _run(w, r, dev)
    what = f"{w.name} r={r}"
    rows = np.sort(np.random.default_rng(78).choice(w.seq_q, size=24, replace=False))
    sl = lambda t: t[:, :, 7:8].contiguous().cpu()
    rdq, _, _ = oracle.attention_bwd(sl(q), sl(k), sl(v), sl(dout), None, 1, w.ring_size, r,
                                     rows=rows, placement="striped")
    _cmp("dq[h7, 24 rows]", to_np(dq[:, rows, 7:8]), rdq, what)
    sk = dk.double().sum(dim=1)
    ratio = float((sk.abs() / dk.double().abs().sum(dim=1).clamp_min(1e-30)).max())
    log(f"  bwd {what} |sum_j dk_j| / sum_j |dk_j| max={ratio:.3e}")
    assert ratio <= 1e-3
    relv = float((dv.double().sum(dim=1) - dout.double().sum(dim=1)).norm()
                 / dout.double().sum(dim=1).norm())
    log(f"  bwd {what} sum_j dv_j vs sum_i dout_i: rel_l2={relv:.3e}")
    assert relv <= REL_L2


F32_CASES = [
    # B, Lq, N, H, D, causal, qc, kc, segments, r, placement, splits
    (1, 64, 4, 2, 64, None, 32, 32, False, 0, "contiguous", 1),   # the tiny workload's shape
    (1, 64, 4, 2, 64, None, 32, 32, False, 3, "contiguous", 1),
    (2, 96, 3, 2, 128, 1, 32, 32, False, 2, "contiguous", 1),
    (1, 160, 2, 2, 128, 5, 32, 32, False, 1, "contiguous", 1),
    (2, 128, 2, 2, 64, 1, 64, 64, True, 1, "contiguous", 1),
    (1, 288, 3, 1, 128, 1, 32, 32, False, 2, "contiguous", 1),   # key workgroups span blocks
    (1, 128, 4, 2, 128, 1, 32, 32, False, 1, "striped", 1),
    (1, 128, 4, 2, 64, 8, 32, 32, True, 2, "striped", 1),
    (1, 256, 2, 2, 128, 1, 64, 64, False, 1, "contiguous", 4),   # dq key splits
    (1, 128, 4, 1, 64, 2, 32, 32, False, 3, "striped", 3),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[str(c) for c in F32_CASES])
def test_bwd_f32(case):
    B, Lq, N, H, D, c, qc, kc, segs, r, place, splits = case
    w = workloads.Workload(f"f32_edge{case}", B, Lq, N, (r,), H, D, "f32", c, qc, kc,
                           segments=segs, seed=7171 + Lq + D + N, placement=place)
    _full_case(w, r, key_splits=splits)


def test_bwd_tiny_plumbing_all_positions():
    w = workloads.get("tiny_plumbing")
    for r in w.ring_indices:
        _full_case(w, r)


def test_bwd_rejects_bad_dtypes_and_nulls():
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 32, 1, 128), dtype=torch.float16, device=dev)
    with pytest.raises(TypeError):
        ra.blockwise_attn_bwd(q, q, q, q, torch.zeros((1, 1, 32), device=dev), q)
    lib = ra.load_library()
    st = lib.ra_blockwise_attn_bwd(None, None, None, None, 0, 32, 32, 1, 0, 1, 32, 1, 128,
                                   ra.RA_BF16, None, None, None, None, None, None, None, None)
    assert st == ra.RA_E_INVALID, ra.last_error()


# ---------------------------------------------------------------------------
# key splits of the dq kernel (ra_blockwise_attn_bwd_split)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("r", [0, 7])
def test_bwd_small_causal_split(r):
    _full_case(workloads.get("small_causal"), r, key_splits="auto")


def test_bwd_small_causal_striped_split():
    _full_case(workloads.get("small_causal_striped"), 6, key_splits=5)


@pytest.mark.parametrize("r", [0, 7])
def test_bwd_small_causal_striped_auto_split(r):
    """The count the helper picks for this share (12: the four query tiles
    take 3, 6, 9 and 12 runs of the dq kernel's exact grid), as bench.py
    times it."""
    _full_case(workloads.get("small_causal_striped"), r, key_splits="auto")


SPLIT_EDGE = [
    # B, Lq, N, H, D, causal, qc, kc, segments, r, placement, splits
    (2, 96, 3, 2, 64, 1, 32, 32, False, 2, "contiguous", 3),
    (1, 128, 1, 4, 128, None, 128, 128, False, 0, "contiguous", 2),
    (2, 128, 2, 2, 128, 1, 64, 64, True, 1, "contiguous", 4),
    (1, 512, 3, 1, 128, 64, 128, 128, True, 2, "contiguous", 7),
    (2, 128, 4, 2, 64, 1, 64, 32, True, 2, "striped", 6),
    (1, 256, 4, 2, 128, 2, 64, 64, False, 1, "striped", 5),
    (2, 128, 2, 2, 128, 8, 64, 32, True, 1, "striped", 3),
    (1, 32, 4, 1, 128, 1, 32, 32, False, 3, "contiguous", 64),   # splits >> tiles
]


@pytest.mark.parametrize("case", SPLIT_EDGE, ids=[str(c) for c in SPLIT_EDGE])
def test_bwd_split_edge(case):
    B, Lq, N, H, D, c, qc, kc, segs, r, place, splits = case
    w = workloads.Workload(f"split_edge{case}", B, Lq, N, (r,), H, D, "bf16", c, qc, kc,
                           segments=segs, seed=6161 + Lq + D + N, placement=place)
    _full_case(w, r, key_splits=splits)


def test_bwd_split_workspace_and_unsplit_agree():
    """A workspace full of NaN on entry does not matter; dk, dv and delta do
    not depend on the split (bitwise), dq only through the order of its
    float32 sum."""
    w = workloads.get("small_causal")
    r = 4
    dev = torch.device("cuda:0")
    splits = 8
    nbytes = ra.bwd_split_workspace_bytes(w.batch, w.seq_q, w.heads, w.head_dim, splits)
    assert nbytes == splits * w.batch * w.seq_q * w.heads * w.head_dim * 4
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=dev)
    _, _, _, _, _, _, g1 = _run(w, r, dev)
    _, _, _, _, _, _, g2 = _run(w, r, dev, key_splits=splits, workspace=ws)
    for name, a, b in zip(("dk", "dv", "delta"), g1[1:], g2[1:]):
        assert torch.equal(a, b), name
    _cmp("dq split vs unsplit", to_np(g2[0]), to_np(g1[0]), "small_causal r=4")
    rel = float((g2[0].double() - g1[0].double()).norm() / g1[0].double().norm())
    assert rel <= 1e-5, rel
