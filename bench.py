"""Benchmark of the blockwise ring-attention forward on one MI355X.

One step = one forward of a device's whole ring share (every KV block in
ring order, skipping, softmax carry, normalisation, lse) through the C ABI,
by default on the 7B-shaped share: batch 1, 32 heads, head_dim 128, bf16,
local query block 32768 at ring position 15 of 16 (512K context), token
causal, chunks 2048.  ``--workload`` times another bf16 workload instead (a
step is then one call per ring position the workload lists); ``--pass bwd``
times the backward (dq, dk, dv of the same share, from the forward's out and
lse and a seeded upstream gradient) instead of the forward; ``--pass ffn``
times the blockwise feedforward of the 7B-shaped share (batch 1, 32768
tokens, hidden 4096, feedforward width 16384, chunks of 2048 rows);
``--pass decode`` times one incremental-decoding step over a KV cache (by
default the 7B-shaped model's last token of a 512K-token cache: 32 heads of
128, bf16), an HBM-bound step reported in GB/s of cache read.  Inputs are
seeded Gaussian tensors already resident in HBM.

Prints one JSON line with the causal-adjusted TFLOP/s, the roofline of the
kernel (MFMA bound, bf16 dense peak) and the CPU oracle timed on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOAD = "share_7b_512k"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3            # MI355X dense fp32 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "blockwise_fwd_share_7b_512k_traffic.json")


def visible_keys_per_row(seq_q: int, ring_size: int, ring_index: int, causal,
                         placement: str = "contiguous") -> np.ndarray:
    """Causally visible keys of each local query row (segments ignored).
    Striped placement (token causal): row i sees i + 1 keys of each block
    kb <= r and i of each block kb > r."""
    S = ring_size * seq_q
    i = np.arange(seq_q, dtype=np.int64)
    if not causal:
        return np.full(seq_q, S, dtype=np.int64)
    if placement == "striped":
        if int(causal) != 1:
            raise ValueError("striped placement is token causal")
        return ring_size * (i + 1) - (ring_size - 1 - ring_index)
    c = int(causal)
    pq = ring_index * seq_q + i
    return np.minimum((pq // c + 1) * c, S)


def segment_visible_keys_per_row(seg_b: np.ndarray, seq_q: int, ring_index: int) -> np.ndarray:
    """Keys each local query row sees under token-causal masking and segment
    ids (contiguous placement): the keys at or before the row's position with
    the row's id, i.e. the row's rank among the positions carrying its id,
    plus one."""
    S = seg_b.shape[0]
    order = np.argsort(seg_b, kind="stable")
    ids = seg_b[order]
    starts = np.r_[0, np.flatnonzero(np.diff(ids)) + 1]
    first = np.repeat(starts, np.diff(np.r_[starts, S]))
    rank = np.empty(S, dtype=np.int64)
    rank[order] = np.arange(S) - first
    return rank[ring_index * seq_q + np.arange(seq_q)] + 1


def causal_flops(w, ring_index: int, seg=None) -> float:
    """F = 4 * D * H * sum over rows of visible keys: two GEMMs, two flops
    per multiply-add, per visible (query, key) pair.  Without segment ids
    the pairs are the causally visible ones; with them (token causal,
    contiguous placement) only pairs inside one segment count."""
    if seg is not None:
        if w.causal_block_size != 1 or w.placement != "contiguous":
            raise ValueError("segment pair counts cover token-causal contiguous shares")
        s_np = seg.cpu().numpy()
        n = sum(int(segment_visible_keys_per_row(s_np[b], w.seq_q, ring_index).sum())
                for b in range(w.batch))
        return 4.0 * w.head_dim * w.heads * n
    n = int(visible_keys_per_row(w.seq_q, w.ring_size, ring_index, w.causal_block_size,
                                 w.placement).sum())
    return 4.0 * w.head_dim * w.heads * w.batch * n


def measured_traffic(build_id: str):
    """HBM bytes per launch of the forward kernel measured with rocprofv3
    counters, reported only when the loaded library was built from the
    current sources (its build id, a hash of the device sources) and the
    forward kernel's sources are those the counters were taken on."""
    from long_context_exact_ra_amd import build as _b
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if build_id != _b.device_sources_sha16():
        return None  # a stale library
    if t.get("fwd_sources_sha16") != _b.fwd_sources_sha16():
        return None
    return t.get("hbm_bytes_per_launch")


def record_traffic(fetch_dir: str, write_dir: str, calib_mib: int) -> dict:
    """Write the traffic record from two rocprofv3 --pmc runs of
    ``bench.py --steps 1 --warmup 0 --cpu-rows 0 --calib-copy-mib M`` (one
    with FETCH_SIZE, one with WRITE_SIZE; their output directories).  Each
    counter of the forward dispatch is scaled by true bytes / counted bytes
    of the plain copy of M MiB that runs first (it reads and writes M MiB).
    Host only; the record is keyed to the build of the library in the tree."""
    import csv
    import glob

    from long_context_exact_ra_amd import build as _b

    def read(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        fwd, copy = [], []
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                if "fwd_bf16_kernel" in name:
                    fwd.append(float(r["Counter_Value"]))
                elif "MulFunctor<unsigned char>" in name:
                    copy.append(float(r["Counter_Value"]))
        if len(fwd) != 1 or len(copy) != 1:
            raise SystemExit(f"{d}: expected one forward and one copy dispatch, "
                             f"found {len(fwd)} and {len(copy)}")
        return fwd[0], copy[0]

    if calib_mib <= 0:
        raise SystemExit("--record-traffic needs the --calib-copy-mib of the counter runs")
    calib = calib_mib << 20
    fk, fc = read(fetch_dir, "FETCH_SIZE")
    wk, wc = read(write_dir, "WRITE_SIZE")
    ff = round(calib / (fc * 1024), 5)
    wf = round(calib / (wc * 1024), 5)
    rec = {"kernel_sha256_16": _b.device_sources_sha16(), "workload": WORKLOAD,
           "fetch_size_kib": fk, "write_size_kib": wk, "calib_copy_bytes": calib,
           "calib_fetch_size_kib": fc, "calib_write_size_kib": wc,
           "fetch_factor": ff, "write_factor": wf,
           "hbm_bytes_per_launch": int(round(fk * 1024 * ff + wk * 1024 * wf)),
           "fwd_sources_sha16": _b.fwd_sources_sha16()}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(w, q, k, v, seg, ring_index: int, rows: int, flops_total: float,
                 dout=None):
    """The CPU oracle, as it stands, on a bounded sample: one head and
    ``rows`` query rows of the same workload (each row over all its visible
    keys).  Rate in the metric's unit (causal-adjusted TFLOP/s); the sample
    text also gives the oracle's time for the whole step, extrapolated
    linearly (rows are independent).  Returns the record, the sampled rows
    and the oracle's results on them (out and lse, or dq for the backward)."""
    import oracle
    import torch
    head = 0
    sel = np.unique(np.linspace(0, w.seq_q - 1, min(rows, w.seq_q)).astype(np.int64))
    kv_len = w.seq_k if (not w.causal_block_size or w.placement != "contiguous") else int(
        min(w.seq_k, ((ring_index * w.seq_q + w.seq_q - 1) // w.causal_block_size + 1)
            * w.causal_block_size))
    qh = q[:1, :, head:head + 1].contiguous().cpu()
    kh = k[:1, :kv_len, head:head + 1].contiguous().cpu()
    vh = v[:1, :kv_len, head:head + 1].contiguous().cpu()
    segh = None if seg is None else seg[:1].cpu().numpy()
    gh = None if dout is None else dout[:1, :, head:head + 1].contiguous().cpu()
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - informational only
        cores = torch.get_num_threads()
    t0 = time.perf_counter()
    if gh is None:
        ref = oracle.attention_fwd(qh, kh, vh, segh, w.causal_block_size, w.ring_size,
                                   ring_index, rows=sel, kv_len=kv_len, placement=w.placement)
    else:
        ref = oracle.attention_bwd(qh, kh, vh, gh, segh, w.causal_block_size, w.ring_size,
                                   ring_index, rows=sel, kv_len=kv_len,
                                   placement=w.placement)[:1]
    dt = time.perf_counter() - t0
    # the same pair count as the headline: the causally visible pairs
    pairs = int(visible_keys_per_row(w.seq_q, w.ring_size, ring_index,
                                     w.causal_block_size, w.placement)[sel].sum())
    flops = (4.0 if gh is None else 10.0) * w.head_dim * pairs
    rate = flops / dt
    return sel, ref, {"value": rate / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{w.name}{'' if gh is None else ' backward'}: batch entry 0, head 0, "
                      f"{len(sel)} query rows spread over the block of ring "
                      f"position {ring_index}, each over its {kv_len}-key visible range; numpy "
                      f"fp64 on {cpu_model()}; {dt:.1f} s for {flops / 1e9:.1f} GFLOP; the whole "
                      f"step would take {flops_total / rate / 3600:.1f} h at this rate "
                      f"(linear extrapolation)"}


# Parity bounds of the timed call against the oracle sample: bf16 out and
# lse max |err| <= 2e-2, mean |err| <= 2e-3, relative L2 of out <= 1e-2 (it
# keeps the absolute bounds from passing on long rows, where |out| ~ 1e-3);
# backward dq: relative L2 <= 1e-2 and max |err| <= 2e-2 max |ref| (fp32
# inputs, no operand rounded below fp32: 1e-5 and 1e-4).
FWD_BOUNDS = {"max": 2e-2, "mean": 2e-3, "rel_l2": 1e-2}
FWD_BOUNDS_F32 = {"max": 1e-5, "mean": 1e-5, "rel_l2": 1e-5}   # fp32 inputs
BWD_BOUNDS = {"rel_l2": 1e-2, "max_rel": 2e-2}
BWD_BOUNDS_F32 = {"rel_l2": 1e-5, "max_rel": 1e-4}


def timed_call_parity(got, ref, ring_index: int, rows, f32: bool = False) -> dict:
    """Errors of the timed call's own outputs (head 0 of batch entry 0, the
    oracle sample's rows) against the oracle; ``got`` is (out, lse) or (dq,)."""
    def f64(t):
        return t.detach().float().cpu().numpy().astype(np.float64)

    rec = {"ring_index": ring_index, "head": 0, "rows": int(len(rows))}
    if len(got) == 2:
        out, lse = f64(got[0][:1, rows, 0]), f64(got[1][:1, 0, rows])
        ro, rl = ref[0][:, :, 0, :], ref[1][:, 0, :]
        e, le = np.abs(out - ro), np.abs(lse - rl)
        bd = FWD_BOUNDS_F32 if f32 else FWD_BOUNDS
        rec.update(out_max=float(e.max()), out_mean=float(e.mean()),
                   out_rel_l2=float(np.linalg.norm(out - ro) / np.linalg.norm(ro)),
                   lse_max=float(le.max()), lse_mean=float(le.mean()), bounds=bd)
        ok = (rec["out_max"] <= bd["max"] and rec["out_mean"] <= bd["mean"]
              and rec["out_rel_l2"] <= bd["rel_l2"]
              and rec["lse_max"] <= bd["max"] and rec["lse_mean"] <= bd["mean"])
    else:
        dq, rq = f64(got[0][:1, rows, 0]), ref[0][:, :, 0, :]
        e = np.abs(dq - rq)
        bd = BWD_BOUNDS_F32 if f32 else BWD_BOUNDS
        rec.update(dq_max_rel=float(e.max() / np.abs(rq).max()),
                   dq_rel_l2=float(np.linalg.norm(dq - rq) / np.linalg.norm(rq)),
                   bounds=bd)
        ok = rec["dq_rel_l2"] <= bd["rel_l2"] and rec["dq_max_rel"] <= bd["max_rel"]
    rec["pass"] = bool(ok and all(np.isfinite(v) for v in rec.values()
                                  if isinstance(v, float)))
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows of the CPU oracle sample (0 = skip)")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=["tiny_plumbing", "small_causal", "share_7b_512k", "packed_documents",
                             "share_65b_4m", "small_causal_striped", "share_7b_512k_striped",
                             "decode_7b_512k", "decode_small"],
                    help="workload to time (default: the 7B-shaped share; tiny_plumbing is "
                         "fp32, forward only)")
    ap.add_argument("--ring-index", type=int, default=None,
                    help="time this ring position instead of the workload's own list")
    ap.add_argument("--pass", dest="pass_", choices=["fwd", "bwd", "ffn", "decode"],
                    default="fwd",
                    help="time the attention forward (default), its backward, the "
                         "blockwise feedforward, or a decoding step (workloads decode_*)")
    ap.add_argument("--key-splits", default="auto",
                    help="key splits per query tile of the forward (and of the backward's "
                         "dq kernel): 'auto' = the library's count for this GPU, 1 for "
                         "shares that fill it; an integer forces it")
    ap.add_argument("--n-new", type=int, default=None,
                    help="decoding: new tokens per step instead of the workload's (the cache "
                         "index moves back so the step still ends at the cache's last row)")
    ap.add_argument("--batch", type=int, default=None,
                    help="decoding: batch size instead of the workload's")
    ap.add_argument("--dtype", choices=["bf16", "f32"], default=None,
                    help="decoding: input dtype instead of the workload's")
    ap.add_argument("--cache-rows", type=int, default=None,
                    help="decoding: cache rows instead of the workload's (the step still ends "
                         "at the last row)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first; its "
                         "FETCH_SIZE/WRITE_SIZE counters calibrate HBM byte counts")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: write the traffic record from two rocprofv3 --pmc "
                         "output directories (FETCH_SIZE, WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic, args.calib_copy_mib)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the ring exchange between GPUs is not part of this library)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_exact_ra_amd as ra
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ra.load_library()
    dev = torch.device("cuda:0")
    if args.pass_ == "ffn":
        bench_ffn(args, dev)
        return
    if args.pass_ == "decode" or args.workload.startswith("decode_"):
        bench_decode(args, dev)
        return
    w = workloads.get(args.workload)
    if args.ring_index is not None:
        import dataclasses
        if not 0 <= args.ring_index < w.ring_size:
            print(f"--ring-index must be in [0, {w.ring_size})", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, ring_indices=(args.ring_index,))
    r = w.ring_indices[0]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    q, k, v = workloads.make_qkv(w, r, device=dev)
    qs = [q] + [workloads.make_q(w, ri, device=dev) for ri in w.ring_indices[1:]]
    seg = workloads.make_segments(w, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1, out=dst)  # one elementwise kernel: reads n bytes, writes n
        torch.cuda.synchronize()
        del src, dst

    bwd = args.pass_ == "bwd"
    if bwd:
        # the forward's outputs of every listed ring position, and the gradients
        douts = [workloads.make_dout(w, ri, device=dev) for ri in w.ring_indices]
        fw = [ra.blockwise_attn_fwd(qi, k, v, seg, w.causal_block_size, w.q_chunk, w.k_chunk,
                                    w.ring_size, ri, placement=w.placement)
              for ri, qi in zip(w.ring_indices, qs)]
        f32 = dict(dtype=torch.float32, device=dev)
        dq = torch.empty(q.shape, **f32)
        dk = torch.empty(k.shape, **f32)
        dv = torch.empty(k.shape, **f32)
        delta = torch.empty((w.batch, w.heads, w.seq_q), **f32)
        torch.cuda.synchronize()

    # Key splits of each ring position, and one workspace for the largest
    # (allocated here, outside the timed region).
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    splits = [ra.fwd_key_splits(w.batch, w.seq_q, w.heads,
                                ra.RA_F32 if w.dtype == "f32" else ra.RA_BF16, w.causal_block_size,
                                w.ring_size, ri, cus, w.placement) if args.key_splits == "auto"
              else int(args.key_splits) for ri in w.ring_indices]
    ws_fn = ra.bwd_split_workspace_bytes if args.pass_ == "bwd" else ra.fwd_split_workspace_bytes
    ws_bytes = max(ws_fn(w.batch, w.seq_q, w.heads, w.head_dim, n) for n in splits)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        for i, (ri, qi) in enumerate(zip(w.ring_indices, qs)):
            if bwd:
                ra.blockwise_attn_bwd(qi, k, v, fw[i][0], fw[i][1], douts[i], seg,
                                      w.causal_block_size, w.q_chunk, w.k_chunk, w.ring_size,
                                      ri, dq=dq, dk=dk, dv=dv, delta=delta,
                                      placement=w.placement, key_splits=splits[i],
                                      workspace=workspace)
            else:
                ra.blockwise_attn_fwd(qi, k, v, seg, w.causal_block_size, w.q_chunk,
                                      w.k_chunk, w.ring_size, ri, out=out, lse=lse,
                                      placement=w.placement, key_splits=splits[i],
                                      workspace=workspace)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = float(np.mean(per))
    checked = (dq, dk, dv) if bwd else (out, lse)
    if not all(bool(torch.isfinite(t).all()) for t in checked):
        raise RuntimeError("non-finite output")

    # backward: the 5 matrix products of the algorithm (S, dP, dV, dK, dQ)
    # per visible pair against the forward's 2
    # With segment ids the headline still counts the causally visible pairs;
    # the pairs inside one segment (the work that is not masked away) are
    # reported beside it.
    mult = 2.5 if bwd else 1.0
    flops = sum(causal_flops(w, ri) for ri in w.ring_indices) * mult
    tflops = flops / (ms * 1e-3) / 1e12
    f32 = w.dtype == "f32"
    peak = PEAK_F32_TFLOPS if f32 else PEAK_BF16_TFLOPS
    seg_adjusted = None
    if seg is not None:
        seg_flops = sum(causal_flops(w, ri, seg) for ri in w.ring_indices) * mult
        seg_adjusted = {"value": round(seg_flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                        "flops_per_step": seg_flops,
                        "pairs": "visible under the causal and the segment mask"}
    build_id = ra.version().split("+", 1)[-1]
    traffic = measured_traffic(build_id) if (w.name == WORKLOAD and not bwd) else None
    rec = {
        "metric": ("causal-adjusted attention backward TFLOP/s per MI355X (5 matrix products "
                   "per visible pair; % of bf16 MFMA peak in roofline.frac)") if bwd else
                  "causal-adjusted attention TFLOP/s per MI355X (% of bf16 MFMA peak in roofline.frac)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if f32 else "bf16",
        "data": f"synthetic: seeded Gaussian Q/K/V (std {w.std:g}), {'fp32' if f32 else 'bf16'}"
                + (", Geometric document lengths as segment ids" if w.segments else ""),
        "config": {"workload": w.name, "batch": w.batch, "seq_q": w.seq_q,
                   "ring_size": w.ring_size,
                   "ring_index": r if len(w.ring_indices) == 1 else list(w.ring_indices),
                   "context": w.seq_k, "segments": bool(w.segments),
                   "heads": w.heads, "head_dim": w.head_dim,
                   "causal_block_size": w.causal_block_size,
                   "q_chunk": w.q_chunk, "k_chunk": w.k_chunk, "pass": args.pass_,
                   "placement": w.placement,
                   "key_splits": splits[0] if len(splits) == 1 else splits,
                   "flops_per_step": flops, "ms_min": round(min(per), 3),
                   "ms_median": round(float(np.median(per)), 3),
                   "wall_s": round(wall, 3)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4),
                     "traffic": traffic},
        "library_build": build_id,
    }
    if seg_adjusted is not None:
        rec["segment_adjusted"] = seg_adjusted
    parity_ok = True
    if args.cpu_rows > 0:
        # The buffers hold the last listed ring position's results: time the
        # oracle on that position and compare it with the timed call.
        r_last = w.ring_indices[-1]
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        sel, ref, rec["cpu_baseline"] = cpu_baseline(w, qs[-1], k, v, seg, r_last,
                                                     args.cpu_rows, flops,
                                                     douts[-1] if bwd else None)
        rec["parity"] = timed_call_parity((dq,) if bwd else (out, lse), ref, r_last, sel, f32)
        parity_ok = rec["parity"]["pass"]
    else:
        rec["cpu_baseline"] = None
        rec["parity"] = None
    print(json.dumps(rec), flush=True)
    if not parity_ok:
        print("bench.py: the timed call's output is outside the parity bounds", file=sys.stderr)
        sys.exit(3)


def bench_ffn(args, dev):
    """Time the blockwise feedforward of the 7B-shaped share: one step is
    the whole sequence, chunk by chunk, two bias-fused GEMMs per chunk."""
    import torch

    import long_context_exact_ra_amd as ra
    import oracle
    import workloads

    w = workloads.FFN_WORKLOADS["ffn_7b_share"]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    x, w1, b1, w2, b2 = workloads.make_ffn_inputs(w, device=dev)
    y = torch.empty_like(x)
    ws = torch.empty(ra.ffn_workspace_bytes(w.chunk, w.ffn), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        ra.blockwise_ffn(x, w1, b1, w2, b2, w.chunk, y=y, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = float(np.mean(per))
    if not bool(torch.isfinite(y).all()):
        raise RuntimeError("non-finite output")
    # two products of 2 * hidden * ffn flops per token
    flops = 4.0 * w.batch * w.seq * w.hidden * w.ffn
    tflops = flops / (ms * 1e-3) / 1e12

    # Context only: the same chunked feedforward through torch's addmm
    # (hipBLASLt GEMMs with a bias epilogue, the ReLU a separate kernel),
    # timed the same way.  Not the library's number.
    xs = x.view(w.batch * w.seq, w.hidden)
    hbuf = torch.empty((w.chunk, w.ffn), dtype=x.dtype, device=dev)
    ybuf = torch.empty_like(xs)

    def torch_step():
        for r0 in range(0, w.batch * w.seq, w.chunk):
            torch.addmm(b1, xs[r0:r0 + w.chunk], w1, out=hbuf)
            torch.relu_(hbuf)
            torch.addmm(b2, hbuf, w2, out=ybuf[r0:r0 + w.chunk])

    for _ in range(args.warmup):
        torch_step()
    torch.cuda.synchronize()
    tev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    tev[0].record(stream)
    for i in range(args.steps):
        torch_step()
        tev[i + 1].record(stream)
    torch.cuda.synchronize()
    t_ms = float(np.mean([tev[i].elapsed_time(tev[i + 1]) for i in range(args.steps)]))
    d_vs_torch = float((ybuf.view_as(y).float() - y.float()).abs().max())
    rec = {
        "metric": "blockwise feedforward TFLOP/s per MI355X (% of bf16 MFMA peak in roofline.frac)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Gaussian x (std 1), weights with std fan_in^-1/2, "
                "biases std 0.1, bf16",
        "config": {"workload": w.name, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "ffn": w.ffn, "chunk": w.chunk, "pass": "ffn", "flops_per_step": flops,
                   "ms_min": round(min(per), 3), "wall_s": round(wall, 3)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "hipblaslt_context": {"ms_per_step": round(t_ms, 3),
                              "value": round(flops / (t_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                              "what": "torch addmm (hipBLASLt, bias epilogue) + relu_ per chunk",
                              "max_abs_diff_vs_library": d_vs_torch},
        "library_build": ra.version().split("+", 1)[-1],
    }
    if args.cpu_rows > 0:
        # the oracle's blockwise feedforward over the whole step (every
        # token, chunk by chunk): about ten seconds of fp64 BLAS work
        print("[bench] timing the CPU oracle on the whole step", file=sys.stderr, flush=True)
        xs = x.cpu()
        ps = [t.cpu() for t in (w1, b1, w2, b2)]
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # pragma: no cover - informational only
            cores = torch.get_num_threads()
        t0 = time.perf_counter()
        oracle.blockwise_ffn(xs, *ps, w.chunk)
        dt = time.perf_counter() - t0
        rate = flops / dt
        rec["cpu_baseline"] = {
            "value": rate / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{w.name}: the whole step ({w.seq} tokens in chunks of {w.chunk}) "
                      f"through the fp64 blockwise feedforward (numpy on {cpu_model()}); "
                      f"{dt:.1f} s for {flops / 1e12:.2f} TFLOP"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


PEAK_HBM_GBS = 8000.0              # MI355X HBM3E


def bench_decode(args, dev):
    """Time one decoding step over a KV cache: every valid cache row of
    every head is read once (the whole step, its key splits' fold included,
    between the events)."""
    import torch

    import long_context_exact_ra_amd as ra
    import oracle
    import workloads

    name = args.workload if args.workload.startswith("decode_") else "decode_7b_512k"
    w = workloads.DECODE_WORKLOADS[name]
    if (args.n_new is not None or args.batch is not None or args.dtype is not None
            or args.cache_rows is not None):
        import dataclasses
        n_new = w.n_new if args.n_new is None else args.n_new
        rows = w.cache_rows if args.cache_rows is None else args.cache_rows
        w = dataclasses.replace(w, n_new=n_new, cache_rows=rows,
                                cache_idx=w.cache_idx + w.n_new - n_new + rows - w.cache_rows,
                                batch=w.batch if args.batch is None else args.batch,
                                dtype=w.dtype if args.dtype is None else args.dtype)
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    q, k, v = workloads.make_decode_inputs(w, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads, w.n_new), dtype=torch.float32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    P = (ra.decode_key_splits(w.batch, w.n_new, w.heads, w.cache_idx, cus)
         if args.key_splits == "auto" else int(args.key_splits))
    ws = torch.empty(max(ra.decode_workspace_bytes(w.batch, w.n_new, w.heads, w.head_dim, P), 1),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1, out=dst)  # one elementwise kernel: reads n bytes, writes n
        torch.cuda.synchronize()
        del src, dst

    def step():
        ra.attn_decode(q, k, v, w.cache_idx, key_splits=P, workspace=ws, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = float(np.mean(per))
    if not (bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())):
        raise RuntimeError("non-finite output")
    elt = 2 if w.dtype == "bf16" else 4
    # algorithmic bytes: K and V of every valid cache row of every head once,
    # plus q, out and lse
    row_bytes = 2 * w.head_dim * elt                  # per (cache row, head)
    kv_bytes = float(w.batch * w.heads * w.n_keys * row_bytes)
    io_bytes = float(2 * w.batch * w.n_new * w.heads * w.head_dim * elt
                     + 4 * w.batch * w.heads * w.n_new)
    gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    pairs = w.batch * w.heads * sum(w.cache_idx + t + 1 for t in range(w.n_new))
    flops = 4.0 * w.head_dim * pairs
    # parity of the timed call and the CPU oracle on a bounded sample: the
    # step's rows of a few heads over the whole cache
    n_heads = max(1, min(w.heads, 4))
    heads = sorted(set(int(h) for h in np.linspace(0, w.heads - 1, n_heads).round()))
    parity, cpu = None, None
    if args.cpu_rows > 0:
        print("[bench] timing the CPU oracle on sampled heads", file=sys.stderr, flush=True)
        qc = q.cpu()
        kc = k[:, :w.n_keys, heads].cpu()
        vc = v[:, :w.n_keys, heads].cpu()
        qs = qc[:, :, heads].contiguous()
        t1 = time.perf_counter()
        ref, ref_lse = oracle.decode_attention(qs, kc, vc, w.cache_idx)
        dt = time.perf_counter() - t1
        got = out[:, :, heads].float().cpu().numpy().astype(np.float64)
        got_l = lse[:, heads].cpu().numpy().astype(np.float64)
        err, lerr = np.abs(got - ref), np.abs(got_l - ref_lse)
        rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
        b = ({"max": 2e-2, "mean": 2e-3, "rel_l2": 1e-2} if w.dtype == "bf16"
             else {"max": 1e-5, "mean": 1e-5, "rel_l2": 1e-5})
        parity = {"heads": heads, "out_max": float(err.max()), "out_mean": float(err.mean()),
                  "out_rel_l2": rel, "lse_max": float(lerr.max()),
                  "lse_mean": float(lerr.mean()), "bounds": b,
                  "pass": bool(err.max() <= b["max"] and err.mean() <= b["mean"]
                               and lerr.max() <= b["max"] and rel <= b["rel_l2"])}
        sample_bytes = float(w.batch * len(heads) * w.n_keys * row_bytes)
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # pragma: no cover - informational only
            cores = torch.get_num_threads()
        cpu = {"value": sample_bytes / dt / 1e9, "unit": "GB/s", "cores": int(cores),
               "kind": "oracle",
               "sample": f"{w.name}: heads {heads} of batch entry 0..{w.batch - 1}, the step's "
                         f"{w.n_new} new tokens over all {w.n_keys} cache rows; numpy fp64 on "
                         f"{cpu_model()}; {dt:.1f} s for {sample_bytes / 1e9:.2f} GB of cache"}
    rec = {
        "metric": "decoding step: KV-cache read GB/s per MI355X (% of HBM bandwidth in "
                  "roofline.frac)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": f"synthetic: seeded Gaussian q, K and V caches (std {w.std}), {w.dtype}",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads,
                   "head_dim": w.head_dim, "cache_rows": w.cache_rows, "cache_idx": w.cache_idx,
                   "n_new": w.n_new, "pass": "decode", "key_splits": P,
                   "bytes_per_step": kv_bytes + io_bytes, "flops_per_step": flops,
                   "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
                   "tokens_per_s": round(w.batch * w.n_new / (ms * 1e-3), 1),
                   "ms_min": round(min(per), 4), "ms_median": round(float(np.median(per)), 4),
                   "wall_s": round(wall, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "library_build": ra.version().split("+", 1)[-1],
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)
    if parity is not None and not parity["pass"]:
        sys.exit(3)


if __name__ == "__main__":
    main()
