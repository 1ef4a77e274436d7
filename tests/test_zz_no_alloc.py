"""GPU: the no-allocation forward (ra_blockwise_attn_fwd_split_noalloc,
partials in the library's own scratch) against the split forward with a
caller-owned workspace (ra_blockwise_attn_fwd_split), both called through
the C ABI: two calls in a row, the second on a smaller share, each equal bit
for bit to the workspace call (same kernels, same order of arithmetic) and
within the bf16 bounds of the fp64 oracle."""

import ctypes

import numpy as np
import pytest
import torch

import long_context_exact_ra_amd as ra
import oracle
import workloads
from parity import check, log, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _args(w, r, q, k, v, out, lse):
    return [q.data_ptr(), k.data_ptr(), v.data_ptr(), None, int(w.causal_block_size or 0),
            w.q_chunk, w.k_chunk, w.ring_size, r, ra.RA_PLACE_CONTIGUOUS, w.batch, w.seq_q,
            w.heads, w.head_dim, ra.RA_BF16, out.data_ptr(), lse.data_ptr(), None]


def _both(w, r, splits):
    lib = ra.load_library()
    q, k, v = workloads.make_qkv(w, r, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    outs = []
    for noalloc in (False, True):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((w.batch, w.heads, w.seq_q), float("nan"), dtype=torch.float32,
                         device=DEV)
        a = _args(w, r, q, k, v, out, lse)
        if noalloc:
            st = lib.ra_blockwise_attn_fwd_split_noalloc(*a, splits, stream)
        else:
            nbytes = ra.fwd_split_workspace_bytes(w.batch, w.seq_q, w.heads, w.head_dim, splits)
            ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
            st = lib.ra_blockwise_attn_fwd_split(*a, splits, ws.data_ptr(), nbytes, stream)
        assert st == ra.RA_OK, ra.last_error()
        torch.cuda.synchronize()
        outs.append((out, lse))
    return q, k, v, outs


@pytest.mark.parametrize("case", ["small_causal r=7, 8 splits then a 4-head share, 3 splits"])
def test_noalloc_matches_workspace_call_twice(case):
    first = workloads.get("small_causal")
    smaller = workloads.Workload("noalloc_small", 1, 512, 4, (2,), 4, 128, "bf16", 1, 64, 64,
                                 seed=31337)
    for w, r, splits in ((first, 7, 8), (smaller, 2, 3)):
        need = ra.fwd_split_workspace_bytes(w.batch, w.seq_q, w.heads, w.head_dim, splits)
        log(f"noalloc: {w.name} r={r} splits={splits} partials={need} bytes")
        assert 0 < need <= (64 << 20)
        q, k, v, ((o_ws, l_ws), (o_na, l_na)) = _both(w, r, splits)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), (case, w.name)
        ref, ref_lse = oracle.attention_fwd(q, k, v, None, w.causal_block_size, w.ring_size, r)
        check(to_np(o_na), to_np(l_na), ref, ref_lse, torch.bfloat16,
              f"noalloc {w.name} r={r} splits={splits}")
