"""GPU parity of the blockwise feedforward against the fp64 oracle.

Bounds, derived from the arithmetic: bf16 inputs multiply exactly into fp32
accumulators; the hidden activation is rounded to bf16 (relative <= 2^-9)
before the second product and y is rounded to bf16 (relative <= 2^-9), so
y's relative L2 error is expected near 2^-9 ~ 2e-3.  Required: relative L2
<= 1e-2 and max |err| <= 2e-2 * max |ref|.
"""

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import log, to_np

pytestmark = pytest.mark.gpu


def _cmp(got, ref, what):
    err = np.abs(got - ref)
    scale = max(float(np.abs(ref).max(initial=0)), 1e-30)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"  ffn {what}: rel_l2={rel:.3e} max_err/max_ref={float(err.max(initial=0)) / scale:.3e}")
    assert np.isfinite(got).all(), what
    assert rel <= 1e-2, (what, rel)
    assert float(err.max(initial=0)) <= 2e-2 * scale, what


CASES = [
    # batch, seq, hidden, ffn, chunk
    (2, 256, 256, 1024, 64),
    (1, 96, 192, 768, 32),
    (3, 64, 128, 512, 64),
    (1, 128, 64, 256, 1),
    (2, 512, 512, 1536, 512),
    # K walked in 32-deep stages and X in 64-deep pairs: an odd number of
    # stages (the last pair half past K), partial last stages, ragged M and N
    (1, 80, 96, 200, 40),
    (2, 64, 40, 72, 64),
    # the same tails in the 256 x 256 kernel (first product: 8 x 32 tiles)
    (1, 2048, 96, 8192, 2048),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_ffn_parity(case):
    B, L, H, Fh, C = case
    w = workloads.FfnWorkload(f"ffn{case}", B, L, H, Fh, C, seed=900 + L + H)
    dev = torch.device("cuda:0")
    x, w1, b1, w2, b2 = workloads.make_ffn_inputs(w, device=dev)
    y = ra.blockwise_ffn(x, w1, b1, w2, b2, C)
    torch.cuda.synchronize()
    ref = oracle.blockwise_ffn(x, w1, b1, w2, b2, C)
    _cmp(to_np(y), ref, str(case))


def test_ffn_7b_share_sampled_rows_and_chunk_sizes():
    w = workloads.FFN_WORKLOADS["ffn_7b_share"]
    dev = torch.device("cuda:0")
    x, w1, b1, w2, b2 = workloads.make_ffn_inputs(w, device=dev)
    y = ra.blockwise_ffn(x, w1, b1, w2, b2, w.chunk)
    y512 = ra.blockwise_ffn(x, w1, b1, w2, b2, 512)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(w.seq, size=64, replace=False))
    ref = oracle.ffn(x[0, rows].cpu(), w1.cpu(), b1.cpu(), w2.cpu(), b2.cpu())
    _cmp(to_np(y[0, rows]), ref, "ffn_7b_share 64 rows")
    _cmp(to_np(y512[0, rows]), ref, "ffn_7b_share chunk 512, 64 rows")
    # the chunk size only bounds memory: both runs agree everywhere
    d = (y.float() - y512.float()).abs().max().item()
    log(f"  ffn_7b_share chunk 2048 vs 512: max |diff| = {d:.3e}")
    assert d <= 2e-2 * y.float().abs().max().item()


def test_ffn_rejects_small_workspace_and_bad_chunk():
    dev = torch.device("cuda:0")
    w = workloads.FfnWorkload("t", 1, 64, 64, 128, 32, seed=3)
    x, w1, b1, w2, b2 = workloads.make_ffn_inputs(w, device=dev)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(ra.RaError) as e:
        ra.blockwise_ffn(x, w1, b1, w2, b2, 32, workspace=small)
    assert e.value.status == ra.RA_E_INVALID
    with pytest.raises(ra.RaError) as e:
        ra.blockwise_ffn(x, w1, b1, w2, b2, 48)
    assert e.value.status == ra.RA_E_INVALID
