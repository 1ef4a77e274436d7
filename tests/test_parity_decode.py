"""GPU parity of the decoding step (``ra_attn_decode``) against the fp64
oracle (``oracle.decode_attention``).

bf16 steps run on the matrix cores (one tile of 32 queries per workgroup
up to 32 new tokens, four tiles sharing each key tile beyond), float32
steps on the vector ALUs; the cases cover each.  Bounds
as for the forward (``parity.BOUNDS``): bf16 inputs max |err| <=
2e-2, mean |err| <= 2e-3 and relative L2 <= 1e-2 on out and lse; float32
inputs 1e-5.  Cache rows past the step's last token hold NaN in every case,
so a kernel that read them would fail.
"""

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import check, log, to_np

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _inputs(B, T, H, D, R, ci, dtype, seed):
    w = workloads.DecodeWorkload("case", B, H, D, R, ci, T, dtype=dtype, seed=seed)
    return workloads.make_decode_inputs(w, device=torch.device("cuda:0"))


def _check_all(q, k, v, ci, out, lse, dtype, what, heads=None):
    ref, ref_lse = oracle.decode_attention(q.cpu(), k, v, ci, heads=heads)
    o = to_np(out if heads is None else out[:, :, heads])
    l = to_np(lse if heads is None else lse[:, heads])
    return check(o, l, ref, ref_lse, DT[dtype], what)


CASES = [  # B, T, H, D, cache rows, cache_idx, dtype, key splits
    (1, 1, 4, 128, 1100, 1000, "bf16", 1),         # one split: normalised in the kernel
    (1, 1, 4, 128, 1100, 1000, "bf16", "auto"),
    (2, 3, 2, 64, 700, 613, "bf16", 5),            # 4 queries per workgroup, D 64
    (1, 8, 2, 128, 300, 200, "bf16", 7),           # 8 queries per workgroup
    (1, 13, 3, 128, 400, 250, "bf16", 3),          # two query groups, the second partial
    (2, 2, 2, 128, 1000, 998, "bf16", 2),          # cache full to its last row
    (1, 1, 2, 128, 64, 0, "bf16", 1),              # the first token: one key
    (1, 8, 2, 128, 8, 0, "bf16", 1),               # every key new: causal among them
    (1, 1, 2, 128, 2000, 100, "bf16", 64),         # most splits empty
    (1, 64, 2, 64, 2000, 1500, "bf16", 3),
    (1, 256, 1, 128, 600, 300, "bf16", 2),         # the largest step
    (1, 9, 2, 128, 100, 50, "bf16", 1),           # matrix cores: one partial group, one split
    (1, 32, 2, 128, 40, 0, "bf16", 1),             # matrix cores: every key new
    (2, 40, 3, 128, 2500, 1777, "bf16", "auto"),   # matrix cores: 2 groups, ragged rows
    (1, 33, 2, 64, 33, 0, "bf16", 1),              # query tiles sharing key tiles: every key new
    (1, 100, 2, 128, 700, 500, "bf16", 3),         # four query tiles, the last partial
    (1, 129, 1, 128, 300, 100, "bf16", 1),         # two groups of four tiles, one split
    (2, 200, 2, 64, 1000, 800, "bf16", 2),         # shared key tiles, batch 2, D 64, two groups
    (1, 256, 2, 128, 3000, 2744, "bf16", "auto"),  # the largest step, the library's split count
    (1, 1, 4, 128, 1100, 1000, "f32", "auto"),
    (1, 100, 1, 64, 400, 300, "f32", 3),           # float32: 13 groups of 8 queries
    (2, 5, 2, 64, 300, 217, "f32", 1),
    (1, 16, 2, 128, 500, 400, "f32", 4),
]


@pytest.mark.parametrize("B,T,H,D,R,ci,dtype,P", CASES)
def test_decode_parity(B, T, H, D, R, ci, dtype, P):
    log(f"decode B={B} T={T} H={H} D={D} rows={R} cache_idx={ci} {dtype} P={P}")
    q, k, v = _inputs(B, T, H, D, R, ci, dtype, seed=B * 1000 + T * 10 + ci)
    out, lse = ra.attn_decode(q, k, v, ci, key_splits=P)
    torch.cuda.synchronize()
    _check_all(q, k, v, ci, out, lse, dtype, f"T={T} P={P}")


def test_decode_first_token_returns_its_value():
    q, k, v = _inputs(1, 1, 3, 128, 16, 0, "f32", seed=5)
    out, lse = ra.attn_decode(q, k, v, 0, key_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out[0, 0], v[0, 0])
    ref = (q[0, 0].double() * k[0, 0].double()).sum(-1) / np.sqrt(128)
    assert float((lse[0, :, 0].double() - ref).abs().max()) <= 1e-5


def test_decode_workspace_contents_do_not_matter():
    """Every split writes its whole partial before the fold reads it: a
    NaN-filled workspace gives the same result, twice in a row."""
    B, T, H, D, R, ci = 2, 4, 2, 128, 3000, 2500
    q, k, v = _inputs(B, T, H, D, R, ci, "bf16", seed=11)
    P = 6
    ws = torch.full((ra.decode_workspace_bytes(B, T, H, D, P) // 4,), float("nan"),
                    dtype=torch.float32, device=q.device)
    o1, l1 = ra.attn_decode(q, k, v, ci, key_splits=P, workspace=ws)
    ws.fill_(float("nan"))
    o2, l2 = ra.attn_decode(q, k, v, ci, key_splits=P, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _check_all(q, k, v, ci, o1, l1, "bf16", "NaN workspace")


def test_decode_split_counts_agree():
    """1, 3 and 17 splits fold the same rows: equal within the bf16 bounds
    (the fold order changes only rounding)."""
    q, k, v = _inputs(1, 2, 4, 128, 5000, 4321, "bf16", seed=12)
    res = [ra.attn_decode(q, k, v, 4321, key_splits=P) for P in (1, 3, 17)]
    torch.cuda.synchronize()
    for P, (o, l) in zip((1, 3, 17), res):
        _check_all(q, k, v, 4321, o, l, "bf16", f"P={P}")


def test_decode_small_workload():
    w = workloads.DECODE_WORKLOADS["decode_small"]
    q, k, v = workloads.make_decode_inputs(w, device=torch.device("cuda:0"))
    out, lse = ra.attn_decode(q, k, v, w.cache_idx)
    torch.cuda.synchronize()
    _check_all(q, k, v, w.cache_idx, out, lse, w.dtype, w.name)


def test_decode_7b_512k_sampled_heads():
    """The 7B-shaped step at full size (the whole 512K-row cache of 32 heads,
    the launch configuration the benchmark times): eight heads, one from
    each group of four, against the oracle over all 524288 keys."""
    w = workloads.DECODE_WORKLOADS["decode_7b_512k"]
    q, k, v = workloads.make_decode_inputs(w, device=torch.device("cuda:0"))
    out, lse = ra.attn_decode(q, k, v, w.cache_idx)
    torch.cuda.synchronize()
    heads = [0, 5, 10, 15, 16, 21, 26, 31]
    _check_all(q, k, v, w.cache_idx, out, lse, w.dtype, w.name, heads=heads)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())


def test_decode_step_on_the_forward_ring_layout():
    """A step of n_new = 64 tokens ending at row 20 * 64 of a one-batch cache
    is the forward's ring share (block length 64, ring position 19 of 20):
    both entry points match the oracle."""
    T, N, H, D = 64, 20, 2, 128
    ci = (N - 1) * T
    q, k, v = _inputs(1, T, H, D, N * T, ci, "bf16", seed=21)
    out_d, lse_d = ra.attn_decode(q, k, v, ci, key_splits=4)
    out_f, lse_f = ra.blockwise_attn_fwd(q, k, v, None, 1, 32, 32, N, N - 1, key_splits=4)
    torch.cuda.synchronize()
    _check_all(q, k, v, ci, out_d, lse_d, "bf16", "decode")
    _check_all(q, k, v, ci, out_f, lse_f, "bf16", "forward ring share")
