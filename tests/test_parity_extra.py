"""GPU parity on inputs chosen to reach particular kernel paths.

* Large logits whose row maxima jump from block to block: the forward keeps
  a row's running max until a weight would exceed 2^8 and rescales only
  then, so these inputs take both the kept-max and the rescale paths (some
  jumps are far above 2^8, some below).
* Segment ids that repeat and are not monotone along the sequence: the
  kernels skip a 32-key half only when its key ids miss the id range of the
  queries, which must hold for any labelling.

Bounds as in the other parity tests (bf16: out and lse max 2e-2, mean 2e-3,
relative L2 1e-2; gradients relative L2 1e-2 and max 2e-2 of the largest).
"""

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import check, log, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _scaled_inputs(w, r, block_scale):
    """Q, K, V of the workload with K's block kb scaled by block_scale[kb]
    and V brought back to unit scale (in fp32, then rounded to bf16 again),
    so that the outputs stay in the range the absolute bounds assume."""
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    sc = torch.tensor(np.repeat(block_scale, w.seq_q), dtype=torch.float32, device=DEV)
    k = (k.float() * sc[None, :, None, None]).to(torch.bfloat16)
    v = (v.float() / w.std).to(torch.bfloat16)
    return q, k, v


def _repeating_segments(B, S, period, n_ids, seed):
    """Ids that cycle through n_ids labels in runs of random length around
    `period`, so equal ids reappear far apart."""
    rng = np.random.default_rng(seed)
    seg = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        pos, i = 0, 0
        while pos < S:
            n = int(rng.integers(period // 2, 2 * period))
            seg[b, pos:pos + n] = (i * 7 + b) % n_ids
            pos += n
            i += 1
    return seg


@pytest.mark.parametrize("r", [3, 7])
def test_fwd_jumping_row_maxima(r):
    w = workloads.Workload("jump", 1, 256, 8, (r,), 4, 128, "bf16", 1, 64, 64, std=2.0,
                           seed=31337 + r)
    scale = np.array([1.0, 3.0, 0.5, 2.5, 1.5, 0.25, 3.5, 2.0])
    q, k, v = _scaled_inputs(w, r, scale)
    out, lse = ra.blockwise_attn_fwd(q, k, v, None, 1, 64, 64, 8, r)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_fwd(q, k, v, None, 1, 8, r)
    log(f"  jump r={r}: lse range {ref_lse.min():.1f} .. {ref_lse.max():.1f}")
    check(to_np(out), to_np(lse), ref, ref_lse, torch.bfloat16, f"jumping maxima r={r}")


def _grad_cmp(name, got, ref, what):
    err = np.abs(got - ref)
    scale = max(float(np.abs(ref).max(initial=0)), 1e-30)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"  bwd {what} {name}: rel_l2={rel:.3e} max_err/max_ref={float(err.max(initial=0)) / scale:.3e}")
    assert np.isfinite(got).all()
    assert rel <= 1e-2 and float(err.max(initial=0)) <= 2e-2 * scale, (what, name, rel)


def test_bwd_jumping_row_maxima():
    r = 5
    w = workloads.Workload("jumpb", 1, 256, 8, (r,), 2, 128, "bf16", 1, 64, 64, std=1.5,
                           seed=4711)
    scale = np.array([1.0, 2.5, 0.5, 2.0, 1.5, 0.25, 3.0, 2.0])
    q, k, v = _scaled_inputs(w, r, scale)
    dout = workloads.make_dout(w, r, device=DEV)
    out, lse = ra.blockwise_attn_fwd(q, k, v, None, 1, 64, 64, 8, r)
    dq, dk, dv, _ = ra.blockwise_attn_bwd(q, k, v, out, lse, dout, None, 1, 64, 64, 8, r)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(q, k, v, dout, None, 1, 8, r)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        _grad_cmp(name, to_np(got), ref, "jumping maxima")


@pytest.mark.parametrize("placement", ["contiguous", "striped"])
def test_repeating_segments_fwd_bwd(placement):
    B, Lq, N, H, D, r = 2, 256, 4, 2, 128, 2
    w = workloads.Workload("rep", B, Lq, N, (r,), H, D, "bf16", 1, 64, 64, seed=2024,
                           placement=placement)
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    dout = workloads.make_dout(w, r, device=DEV)
    nat = _repeating_segments(B, w.seq_k, 100, 5, 99)
    seg_np = workloads.to_storage_order(nat, N, placement)
    seg = torch.from_numpy(seg_np).to(DEV)
    out, lse = ra.blockwise_attn_fwd(q, k, v, seg, 1, 64, 64, N, r, placement=placement)
    dq, dk, dv, _ = ra.blockwise_attn_bwd(q, k, v, out, lse, dout, seg, 1, 64, 64, N, r,
                                          placement=placement)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_fwd(q, k, v, seg_np, 1, N, r, placement=placement)
    check(to_np(out), to_np(lse), ref, ref_lse, torch.bfloat16, f"repeating ids {placement}")
    refs = oracle.attention_bwd(q, k, v, dout, seg_np, 1, N, r, placement=placement)
    for name, got, rf in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        _grad_cmp(name, to_np(got), rf, f"repeating ids {placement}")
