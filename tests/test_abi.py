"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects malformed arguments on the host before any device work."""

import ctypes
import os
import re

import pytest

import long_context_exact_ra_amd as ra

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "ra_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ra_blockwise_attn_fwd", "ra_blockwise_attn_fwd_ex", "ra_blockwise_plan",
              "ra_last_error", "ra_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ra.load_library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_error_string():
    assert re.fullmatch(r"\d+\.\d+\.\d+\+[0-9a-f]{16}", ra.version())
    assert isinstance(ra.last_error(), str)


# A forward call with fake (never dereferenced) pointers: every case below
# must fail validation on the host, so no pointer is touched and no HIP call
# is made.
FAKE = 0x1000


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, seg=None, c=1, qc=64, kc=64, N=4, r=0, B=1, Lq=128,
             H=2, D=128, dt=ra.RA_BF16, out=FAKE, lse=FAKE)
    a.update(kw)
    lib = ra.load_library()
    return lib.ra_blockwise_attn_fwd(a["q"], a["k"], a["v"], a["seg"], a["c"], a["qc"],
                                     a["kc"], a["N"], a["r"], a["B"], a["Lq"], a["H"],
                                     a["D"], a["dt"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(N=0), ra.RA_E_INVALID, "ring_size"),
    (dict(r=4), ra.RA_E_INVALID, "ring_index"),
    (dict(r=-1), ra.RA_E_INVALID, "ring_index"),
    (dict(c=-1), ra.RA_E_INVALID, "causal_block_size"),
    (dict(qc=0), ra.RA_E_INVALID, "positive"),
    (dict(kc=-64), ra.RA_E_INVALID, "positive"),
    (dict(qc=96), ra.RA_E_INVALID, "divide"),
    (dict(qc=48, kc=48, Lq=96), ra.RA_E_UNSUPPORTED, "multiples of 32"),
    (dict(B=-1), ra.RA_E_INVALID, "batch"),
    (dict(H=-2), ra.RA_E_INVALID, "batch and heads"),
    (dict(Lq=-128), ra.RA_E_INVALID, "seq_q"),
    (dict(D=0), ra.RA_E_INVALID, "head_dim"),
    (dict(D=96), ra.RA_E_UNSUPPORTED, "head_dim"),
    (dict(dt=7), ra.RA_E_UNSUPPORTED, "dtype"),
    (dict(q=None), ra.RA_E_INVALID, "non-NULL"),
    (dict(v=None), ra.RA_E_INVALID, "non-NULL"),
    (dict(lse=None), ra.RA_E_INVALID, "non-NULL"),
    (dict(N=1 << 20, Lq=1 << 12, qc=64, kc=64), ra.RA_E_UNSUPPORTED, "2^31"),
    (dict(H=1 << 20, D=128), ra.RA_E_UNSUPPORTED, "2^24"),
])
def test_invalid_arguments(kw, status, needle):
    assert fwd(**kw) == status
    assert needle in ra.last_error()


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Lq=0),
                                dict(B=0, q=None, k=None, v=None, out=None, lse=None)])
def test_empty_call_is_a_noop(kw):
    assert fwd(**kw) == ra.RA_OK
    assert ra.last_error() == ""


def test_plan_rejects_bad_arguments():
    lib = ra.load_library()
    order = (ctypes.c_int32 * 4)()
    assert lib.ra_blockwise_plan(1, 64, 64, 128, 4, 4, order, None, None) == ra.RA_E_INVALID
    assert lib.ra_blockwise_plan(1, 64, 48, 128, 4, 0, order, None, None) == ra.RA_E_INVALID
    assert lib.ra_blockwise_plan(1, 64, 64, 128, 4, 0, None, None, None) == ra.RA_E_INVALID
    # The planner itself has no 32-multiple restriction.
    assert lib.ra_blockwise_plan(1, 3, 5, 15, 4, 0, order, None, None) == ra.RA_OK


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError):
        ra.blockwise_attn_fwd(q, q, q, None, 1, 32, 32)


def test_ffn_validation_without_gpu():
    """Argument errors of the feedforward are caught on the host."""
    lib = ra.load_library()
    assert lib.ra_blockwise_ffn_workspace_bytes(2048, 16384) == 2048 * 16384 * 2
    assert lib.ra_blockwise_ffn_workspace_bytes(0, 16384) == 0
    p = 1  # a non-null dummy pointer, never dereferenced on these paths
    call = lambda **kw: lib.ra_blockwise_ffn(
        *(kw.get(n, p) for n in ("x", "w1", "b1", "w2", "b2")),
        kw.get("batch", 1), kw.get("seq", 64), kw.get("hidden", 64), kw.get("ffn", 128),
        kw.get("chunk", 32), kw.get("dtype", ra.RA_BF16), kw.get("y", p), kw.get("ws", p),
        kw.get("wsb", 1 << 20), None)
    assert call(chunk=48) == ra.RA_E_INVALID
    assert call(chunk=0) == ra.RA_E_INVALID
    assert call(hidden=0) == ra.RA_E_INVALID
    assert call(dtype=ra.RA_F32) == ra.RA_E_UNSUPPORTED
    assert call(wsb=100) == ra.RA_E_INVALID
    assert call(x=None) == ra.RA_E_INVALID
    assert call(batch=0) == ra.RA_OK  # empty call: no device work
    assert call(seq=0) == ra.RA_OK


def test_striped_plan_matches_oracle():
    """The host planner's striped chunk-pair decisions equal the oracle's
    closed form (itself pinned to brute force)."""
    import oracle
    for c in (1, 2, 3, None):
        for N, Lq, qc, kc in ((4, 64, 32, 32), (3, 96, 32, 96), (16, 128, 64, 32)):
            for r in range(N):
                o, run, n = ra.blockwise_plan(c, qc, kc, Lq, N, r, placement="striped")
                o2, run2 = oracle.skip_map_closed(c, qc, kc, Lq, N, r, placement="striped")
                assert (o == o2).all() and (run == run2).all(), (c, N, Lq, r)
                assert n == int(run2.sum())


def test_placed_validation_without_gpu():
    lib = ra.load_library()
    call = lambda c, place, batch=1: lib.ra_blockwise_attn_fwd_placed(
        None, None, None, None, c, 32, 32, 4, 1, place, batch, 32, 1, 128, ra.RA_BF16,
        None, None, None, None)
    # N = 4: causal blocks that divide 4 or are multiples of it are served,
    # others have no form on key coordinates and are refused, even when
    # empty; accepted masks get as far as the null tensors.
    for c in (3, 6, 10):
        assert call(c, ra.RA_PLACE_STRIPED) == ra.RA_E_UNSUPPORTED
        assert "divides ring_size" in ra.last_error()
        assert call(c, ra.RA_PLACE_STRIPED, batch=0) == ra.RA_E_UNSUPPORTED
    for c in (2, 4, 8, 12):
        assert call(c, ra.RA_PLACE_STRIPED) == ra.RA_E_INVALID
    assert call(1, 7) == ra.RA_E_INVALID
    assert call(1, ra.RA_PLACE_STRIPED, batch=0) == ra.RA_OK      # empty call
    assert call(128, ra.RA_PLACE_STRIPED, batch=0) == ra.RA_OK    # block >= sequence: non-causal
    assert call(1, ra.RA_PLACE_STRIPED) == ra.RA_E_INVALID        # null q, k, v
    order = (ctypes.c_int32 * 4)()
    assert lib.ra_blockwise_plan_placed(1, 32, 32, 32, 4, 1, 9, order, None, None) == ra.RA_E_INVALID


def test_bwd_placed_validation_without_gpu():
    lib = ra.load_library()
    call = lambda c, place, batch=1: lib.ra_blockwise_attn_bwd_placed(
        None, None, None, None, c, 32, 32, 4, 1, place, batch, 32, 1, 128, ra.RA_BF16,
        None, None, None, None, None, None, None, None)
    assert call(3, ra.RA_PLACE_STRIPED) == ra.RA_E_UNSUPPORTED
    assert call(2, ra.RA_PLACE_STRIPED) == ra.RA_E_INVALID  # served; null tensors
    assert call(8, ra.RA_PLACE_STRIPED) == ra.RA_E_INVALID
    assert call(1, 5) == ra.RA_E_INVALID
    assert call(1, ra.RA_PLACE_STRIPED, batch=0) == ra.RA_OK
    assert call(1, ra.RA_PLACE_STRIPED) == ra.RA_E_INVALID  # null tensors


def test_split_validation_without_gpu():
    """Key-split arguments are checked on the host before any device work."""
    lib = ra.load_library()
    P = 0x1000  # fake device pointers: every call below fails validation first
    call = lambda splits, ws=P, wsb=1 << 40, batch=1: lib.ra_blockwise_attn_fwd_split(
        P, P, P, None, 1, 32, 32, 4, 1, ra.RA_PLACE_CONTIGUOUS, batch, 64, 2, 128, ra.RA_BF16,
        P, P, None, splits, ws, wsb, None)
    assert call(0) == ra.RA_E_INVALID
    assert call(65) == ra.RA_E_INVALID
    assert call(4, ws=None) == ra.RA_E_INVALID
    need = ra.fwd_split_workspace_bytes(1, 64, 2, 128, 4)
    assert need == 4 * 1 * 2 * 64 * 130 * 4
    assert call(4, wsb=need - 1) == ra.RA_E_INVALID
    assert "workspace" in ra.last_error()
    assert call(4, batch=0) == ra.RA_OK          # empty call: nothing to do
    assert ra.fwd_split_workspace_bytes(1, 64, 2, 128, 1) == 0


def test_key_split_recommendation():
    """Splits only when the grid leaves compute units idle, the split grid at
    one workgroup per compute unit at most and at least 4 key tiles per run
    of the longest walk."""
    ks = lambda B, Lq, H, dt, c, N, r, cu=256, pl="contiguous": ra.fwd_key_splits(
        B, Lq, H, dt, c, N, r, cu, pl)
    # 7B share: 4096 workgroups of 256 rows already fill 256 compute units
    assert ks(1, 32768, 32, ra.RA_BF16, 1, 16, 15) == 1
    # small causal share: 32 workgroups; r = 7 walks 8192 keys = 128 tiles
    assert ks(1, 1024, 8, ra.RA_BF16, 1, 8, 7) == 8
    # r = 0 walks 1024 keys = 16 tiles: at most 4 splits of 4 tiles
    assert ks(1, 1024, 8, ra.RA_BF16, 1, 8, 0) == 4
    assert ks(1, 1024, 8, ra.RA_BF16, 1, 8, 1) == 8
    # fp32 workgroups hold 128 rows; non-causal walks every key
    assert ks(1, 64, 2, ra.RA_F32, None, 4, 0) == 1     # 4 tiles: too short to split
    assert ks(1, 32, 2, ra.RA_BF16, 1, 4, 3) == 1       # 128 visible keys = 2 tiles

    assert ks(1, 1024, 2, ra.RA_F32, None, 8, 3, cu=64) == 4
    assert ks(0, 1024, 8, ra.RA_BF16, 1, 8, 0) == 1
    assert ks(1, 1024, 8, ra.RA_BF16, 1, 8, 8) == 1     # invalid ring index
    # striped: every ring position's longest walk touches every block (128
    # tiles), so r = 0 splits as much as r = 7.  Runs are weighted by walk
    # length: at 12 splits the four query tiles take 3, 6, 9 and 12 runs, 240
    # workgroups for the 8 heads; 13 would need more than 256.
    assert ks(1, 1024, 8, ra.RA_BF16, 1, 8, 0, pl="striped") == 12
    assert ks(1, 1024, 8, ra.RA_BF16, 1, 8, 7, pl="striped") == 12
    # striped with a causal block of 2 positions on 8 devices: token causal
    # on coordinates, ring position 0 shifts blocks 2..7 (stripe_hi 2), the
    # same walk lengths as c = 1 at position 1; a block of 3 is refused
    assert ks(1, 1024, 8, ra.RA_BF16, 2, 8, 0, pl="striped") == \
        ks(1, 1024, 8, ra.RA_BF16, 1, 8, 1, pl="striped")
    assert ks(1, 1024, 8, ra.RA_BF16, 3, 8, 0, pl="striped") == 1


def test_bwd_split_validation_without_gpu():
    lib = ra.load_library()
    P = 0x1000
    call = lambda splits, ws=P, wsb=1 << 40, batch=1: lib.ra_blockwise_attn_bwd_split(
        P, P, P, None, 1, 32, 32, 4, 1, ra.RA_PLACE_CONTIGUOUS, batch, 64, 2, 128, ra.RA_BF16,
        P, P, P, P, P, P, P, splits, ws, wsb, None)
    assert call(0) == ra.RA_E_INVALID
    assert call(65) == ra.RA_E_INVALID
    assert call(3, ws=None) == ra.RA_E_INVALID
    need = ra.bwd_split_workspace_bytes(1, 64, 2, 128, 3)
    assert need == 3 * 64 * 2 * 128 * 4
    assert call(3, wsb=need - 1) == ra.RA_E_INVALID
    assert call(3, batch=0) == ra.RA_OK
    assert ra.bwd_split_workspace_bytes(1, 64, 2, 128, 1) == 0


@pytest.mark.parametrize("which", ["q", "k", "v", "out", "lse", "seg"])
def test_misaligned_pointers_rejected(which):
    """Every tensor is moved in 16-byte (ids and lse: 4-byte) units, so the
    host rejects misaligned pointers before any device work."""
    kw = {which: FAKE + 2}
    if which == "seg":
        kw["seg"] = FAKE + 2
    st = fwd(**kw)
    assert st == ra.RA_E_INVALID, ra.last_error()
    assert "aligned" in ra.last_error()


def test_misaligned_workspace_and_bwd_rejected():
    lib = ra.load_library()
    P = 0x1000
    st = lib.ra_blockwise_attn_fwd_split(P, P, P, None, 1, 32, 32, 4, 1, ra.RA_PLACE_CONTIGUOUS,
                                         1, 64, 2, 128, ra.RA_BF16, P, P, None, 4, P + 8,
                                         1 << 40, None)
    assert st == ra.RA_E_INVALID and "aligned" in ra.last_error()
    for bad in range(7):   # out, lse, dout, dq, dk, dv, delta
        ptrs = [P] * 7
        ptrs[bad] += 2
        st = lib.ra_blockwise_attn_bwd_split(P, P, P, None, 1, 32, 32, 4, 1,
                                             ra.RA_PLACE_CONTIGUOUS, 1, 64, 2, 128, ra.RA_BF16,
                                             *ptrs, 1, None, 0, None)
        assert st == ra.RA_E_INVALID and "aligned" in ra.last_error(), bad


def test_noalloc_refuses_partials_beyond_its_scratch():
    """ra_blockwise_attn_fwd_split_noalloc refuses, before any HIP call, a
    call whose split partials exceed its 64 MiB scratch (the 7B-shaped share
    with 2 key splits needs 1.09 GB), and says how much it would need."""
    lib = ra.load_library()
    P = 0x1000
    st = lib.ra_blockwise_attn_fwd_split_noalloc(P, P, P, None, 1, 2048, 2048, 16, 15,
                                                 ra.RA_PLACE_CONTIGUOUS, 1, 32768, 32, 128,
                                                 ra.RA_BF16, P, P, None, 2, None)
    assert st == ra.RA_E_UNSUPPORTED
    msg = ra.last_error()
    assert "1090519040 bytes" in msg and "67108864" in msg, msg
    # just past the limit: 2 splits x 64528 rows x (128 + 2) x 4 bytes
    assert ra.fwd_split_workspace_bytes(1, 64528, 1, 128, 2) == 67109120 > (64 << 20)
    assert ra.fwd_split_workspace_bytes(1, 64527, 1, 128, 2) <= (64 << 20)
    st = lib.ra_blockwise_attn_fwd_split_noalloc(P, P, P, None, 1, 32, 32, 1, 0,
                                                 ra.RA_PLACE_CONTIGUOUS, 1, 64528, 1, 128,
                                                 ra.RA_BF16, P, P, None, 2, None)
    assert st == ra.RA_E_UNSUPPORTED


def test_ffn_host_validation():
    """The feedforward's own GEMM needs hidden and ffn_hidden multiples of 8
    and aligned operands; both are refused on the host, before any HIP call."""
    lib = ra.load_library()
    P = 0x1000
    ws = ra.ffn_workspace_bytes(64, 256)
    st = lib.ra_blockwise_ffn(P, P, P, P, P, 1, 64, 60, 256, 64, ra.RA_BF16, P, P, ws, None)
    assert st == ra.RA_E_UNSUPPORTED and "multiples of 8" in ra.last_error()
    st = lib.ra_blockwise_ffn(P, P, P, P, P, 1, 64, 64, 252, 64, ra.RA_BF16, P, P,
                              ra.ffn_workspace_bytes(64, 252), None)
    assert st == ra.RA_E_UNSUPPORTED
    st = lib.ra_blockwise_ffn(P + 8, P, P, P, P, 1, 64, 64, 256, 64, ra.RA_BF16, P, P, ws, None)
    assert st == ra.RA_E_INVALID and "aligned" in ra.last_error()
    st = lib.ra_blockwise_ffn(P, P, P + 2, P, P, 1, 64, 64, 256, 64, ra.RA_BF16, P, P, ws, None)
    assert st == ra.RA_E_INVALID
    st = lib.ra_blockwise_ffn(P, P, P, P, P, 1, 64, 64, 256, 64, ra.RA_F32, P, P, ws, None)
    assert st == ra.RA_E_UNSUPPORTED


def test_decode_validation_without_gpu():
    """Argument errors of the decoding step are caught on the host, and the
    key-split and workspace helpers follow their stated rules."""
    lib = ra.load_library()
    p = 4096  # an aligned non-null dummy pointer, never dereferenced on these paths
    call = lambda **kw: lib.ra_attn_decode(
        kw.get("q", p), kw.get("k", p), kw.get("v", p), kw.get("ci", 100), kw.get("rows", 128),
        kw.get("batch", 1), kw.get("n_new", 1), kw.get("heads", 2), kw.get("d", 128),
        kw.get("dtype", ra.RA_BF16), kw.get("P", 2), kw.get("ws", p), kw.get("wsb", 1 << 20),
        kw.get("out", p), kw.get("lse", p), None)
    assert call(ci=-1) == ra.RA_E_INVALID
    assert call(ci=128) == ra.RA_E_INVALID          # the new token past the cache rows
    assert call(n_new=30) == ra.RA_E_INVALID        # 100 + 30 > 128
    assert call(ci=2 ** 63 - 1) == ra.RA_E_INVALID  # cache_idx + n_new would wrap
    assert call(rows=-5, ci=0) == ra.RA_E_INVALID
    assert call(batch=-1) == ra.RA_E_INVALID
    assert call(d=0) == ra.RA_E_INVALID
    assert call(P=0) == ra.RA_E_INVALID
    assert call(P=1025) == ra.RA_E_INVALID
    assert call(d=96) == ra.RA_E_UNSUPPORTED
    assert call(dtype=7) == ra.RA_E_UNSUPPORTED
    assert call(n_new=257, rows=1024) == ra.RA_E_UNSUPPORTED
    assert call(q=None) == ra.RA_E_INVALID
    assert call(lse=p + 2) == ra.RA_E_INVALID      # misaligned
    assert call(out=p + 8) == ra.RA_E_INVALID
    assert call(ws=None) == ra.RA_E_INVALID         # two splits need a workspace
    assert call(wsb=100) == ra.RA_E_INVALID
    assert call(ws=p + 4) == ra.RA_E_INVALID
    assert call(batch=0) == ra.RA_OK                # empty calls: no device work
    assert call(n_new=0) == ra.RA_OK
    assert call(heads=0) == ra.RA_OK
    assert "cache" in ra.last_error() or ra.last_error() == ""
    # workspace: P * B * H * n_new * (D + 2) float32, none for one split
    assert lib.ra_attn_decode_workspace_bytes(1, 3, 2, 128, 4) == 4 * 1 * 2 * 3 * 130 * 4
    assert lib.ra_attn_decode_workspace_bytes(1, 3, 2, 128, 1) == 0
    # split count: about 8 workgroups per compute unit, >= 1024 keys per split,
    # >= 512 while the grid would leave compute units idle
    assert lib.ra_attn_decode_key_splits(1, 1, 32, 524287, 256) == 64
    assert lib.ra_attn_decode_key_splits(1, 1, 32, 8191, 256) == 8     # 256 workgroups: 1024 keys
    assert lib.ra_attn_decode_key_splits(1, 1, 32, 5000, 256) == 8     # 160 at 1024: 8 x 626 keys
    assert lib.ra_attn_decode_key_splits(2, 4, 8, 5000, 256) == 10     # 80 at 1024: 10 x 501 keys
    assert lib.ra_attn_decode_key_splits(1, 1, 1, 300, 256) == 1       # never below 512 keys
    assert lib.ra_attn_decode_key_splits(64, 1, 32, 524287, 256) == 1
    assert lib.ra_attn_decode_key_splits(1, 1, 1, 10 ** 9, 256) == 1024
    assert lib.ra_attn_decode_key_splits(0, 1, 32, 100, 256) == 1


def test_bindings_refuse_tensors_on_two_devices():
    """The library takes raw pointers and launches on the current device:
    the bindings find the one GPU every tensor lives on, and refuse a host
    tensor or a tensor on a second GPU before any call."""
    from types import SimpleNamespace as T
    g0a, g0b = T(is_cuda=True, device="cuda:0"), T(is_cuda=True, device="cuda:0")
    g1, host = T(is_cuda=True, device="cuda:1"), T(is_cuda=False, device="cpu")
    assert ra._one_device(q=g0a, k=g0b, segment_ids=None, out=g0a) == "cuda:0"
    with pytest.raises(ValueError, match="workspace is on cuda:1"):
        ra._one_device(q=g0a, k=g0b, workspace=g1)
    with pytest.raises(ValueError, match="lse must be a device tensor"):
        ra._one_device(q=g0a, lse=host)
