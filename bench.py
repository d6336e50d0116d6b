"""PBSA benchmark on one MI355X: ms per chunk of the persistent-mode hot path.

One step = one chunk of one attention layer (one denoising pass) on the Wan2.1-1.3B-shaped
5-second workload: 12 heads, head_dim 128, 1560-token frames, 3-frame chunks (4680
queries), 21-frame history, 64-token blocks, capacity 64 (1 sink), window 6 frames,
top-32:
    pool(q) + score_topk + attn_fwd + memory_update (which pools k)
on seeded synthetic bf16 inputs already resident in HBM.  The cache is bootstrapped by
replaying the 7 history chunks; each timed step then feeds the measured chunk's tensors
again, so the rollout keeps sliding with steady shapes.  The K timed steps run with no
event between their launches.

Prints one JSON line.  `roofline` is for the dominant kernel (attention forward, bf16 MFMA):
achieved = algorithmic FLOP per launch (4 * head_dim per attended (query, key) pair)
divided by that kernel's mean duration: K back-to-back launches on the state the timed
steps left, between two HIP events on the stream they run on.
`cpu_baseline` times the fp64 oracle's chunk step on this host for one head and scales it
to the 12 heads of a chunk.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--train]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PBSA ms/chunk + effective TFLOP/s & % MFMA/HBM roofline, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--train", action="store_true",
                    help="also time the trainable two-level fwd+bwd clip (extra field)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "attn_fwd_wan_5s_traffic.json"),
                    help="HBM traffic per attention launch from rocprofv3 counters (if present)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured ceilings (MFMA, copy, gather, full-history pool)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-probe run into the traffic file, then exit")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy a 512 MiB buffer 3 times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    return ap.parse_args()


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.traffic)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU (no sharding across GPUs); --gpus must be 1"}))
        sys.exit(2)
    import torch
    from block_sparse_attention_pbsa_amd import ops, runtime, synth

    wl = synth.WORKLOADS["wan_5s"]
    seed = synth.SEEDS["wan_5s"]
    shape = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                      wl.capacity, wl.sinks, wl.topk, wl.scale)
    torch.cuda.set_device(0)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)

    layer = runtime.PersistentLayer(shape)
    layer.reset()
    for c in range(wl.measured_chunk):
        q, k, v = synth.chunk_qkv(wl, seed, c)
        layer.step(dev(q), dev(k), dev(v), attend=False)
    qn, kn, vn = synth.chunk_qkv(wl, seed, wl.measured_chunk)
    q, k, v = dev(qn), dev(kn), dev(vn)
    torch.cuda.synchronize()
    print(f"bootstrapped {wl.measured_chunk} chunks", file=sys.stderr, flush=True)

    def attended_flop():
        """4*d * sum over (head, query token) of attended keys, from the current state."""
        bid = layer.cache.block_id.cpu().numpy()
        ln = layer.cache.len.cpu().numpy()
        C, nb, n = wl.capacity, wl.nb, wl.frame_tokens
        total = 0
        layer.route(q)  # routing for the current state (outside any timed region)
        sels = layer.sel.cpu().numpy()
        for h in range(wl.heads):
            p_keys = int(ln[h, :C][bid[h, :C] >= 0].sum())
            ring = {int(g): int(l) for g, l in zip(bid[h, C:], ln[h, C:]) if g >= 0}
            sel = sels[h]
            for r in range(shape.nq):
                keys = p_keys + wl.chunk_frames * n + sum(ring[int(g)] for g in sel[r] if g >= 0)
                qlen = min(64, n - 64 * (r % nb))
                total += qlen * keys
        return 4 * wl.head_dim * total

    stream = torch.cuda.current_stream()

    def step():
        layer.step(q, k, v)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps

    def timed(fn, reps):
        """Mean duration (ms) of `reps` back-to-back launches of fn, HIP events on the
        stream the kernels run on (no event between launches, so no gap is counted)."""
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # The attention of the state the timed steps left (its routing refreshed first):
    # `steps` back-to-back launches; the attended FLOP are counted for the same state.
    flop = attended_flop()
    torch.cuda.synchronize()
    attn_avg = timed(lambda: layer.attend(q, k, v), args.steps)
    achieved = flop / (attn_avg * 1e-3) / 1e12

    # the memory update, timed on a copy of the cache (each call appends the chunk again)
    import copy
    cache2 = copy.copy(layer.cache)
    for name_ in ("k", "v", "rep", "block_id", "len"):
        setattr(cache2, name_, getattr(layer.cache, name_).clone())
    upd_ms = timed(lambda: ops.pbsa_memory_update(shape, layer.scores, cache2, k, v, None,
                                                  layer.workspace), 20)
    del cache2

    ops_ms = {
        "route": timed(lambda: ops.pbsa_route(shape, q, layer.cache, layer.q_rep, layer.scores,
                                              layer.sel), 20),
        "pool_q": timed(lambda: ops.pbsa_pool(shape, q, wl.chunk_frames, layer.q_rep), 20),
        "score_topk": timed(lambda: ops.pbsa_score_topk(shape, layer.q_rep, layer.cache,
                                                        layer.scores, layer.sel), 20),
        "attn_fwd": attn_avg,
        "memory_update": upd_ms,
    }
    pool_bytes = shape.chunk_tokens * wl.heads * wl.head_dim * 2 + shape.nq * wl.heads * wl.head_dim * 4

    # counters taken on another version of the kernel's sources do not count
    traffic = None
    if os.path.exists(args.traffic):
        try:
            rec = json.load(open(args.traffic))
            if rec.get("source_sha256") == kernel_source_hash():
                traffic = rec.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    result = {
        "metric": METRIC,
        "value": round(ms_step, 4),
        "unit": "ms/chunk",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "wan_5s: Wan2.1-1.3B-shaped 5 s rollout, one layer, one chunk",
                   "heads": wl.heads, "head_dim": wl.head_dim, "frame_tokens": wl.frame_tokens,
                   "chunk_frames": wl.chunk_frames, "query_tokens": shape.chunk_tokens,
                   "history_frames": wl.history_frames, "block": wl.block,
                   "capacity": wl.capacity, "sinks": wl.sinks,
                   "window_frames": wl.window_frames, "topk": wl.topk},
        "tflops_effective": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "attn_fwd_flop": int(flop),
        "attn_fwd_ms": round(attn_avg, 4),
        "ops_ms_mean": {k_: round(v_, 4) for k_, v_ in ops_ms.items()},
        # derived, not measured as one run: T = 4 denoising passes per chunk (route + attention
        # each) sharing the memory, then one update
        "derived_ms_per_chunk_T4": round(4 * (ops_ms["route"] + attn_avg) + upd_ms, 4),
        "pool_q_gbs": round(pool_bytes / (ops_ms["pool_q"] * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": TRAFFIC_KERNEL},
    }

    if not args.no_probes:
        result["probes"] = bench_probes(torch, ops, synth, shape, layer, q, k, v, stream)

    if args.train:
        result["train"] = bench_train(torch, ops, runtime, synth, dev, stream)

    if args.copy_probe:
        src = torch.ones(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = src.numel() * 2

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, seed)
    print(json.dumps(result), flush=True)


TRAFFIC_KERNEL = "attn_fwd_kernel<128, true, false>"
KERNEL_SOURCES = ("attn_fwd.hip", "attn_common.h", "common.h", "launch.h")


def kernel_source_hash():
    """sha256 (first 16 hex digits) of the sources the timed attention kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_pbsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def write_traffic(fetch_dir, write_dir, out_path):
    """HBM bytes per attention launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the counter reads for the 512 MiB copy of the same run."""
    def read(d, counter):
        rows = [r for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv")))
                if r["Counter_Name"] == counter]
        kern = [float(r["Counter_Value"]) for r in rows if TRAFFIC_KERNEL in r["Kernel_Name"]]
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        if not kern:
            raise SystemExit(f"no {TRAFFIC_KERNEL} dispatch in {d}")
        return float(np.mean(kern)), copy, len(kern)
    f_k, f_c, n = read(fetch_dir, "FETCH_SIZE")
    w_k, w_c, _ = read(write_dir, "WRITE_SIZE")
    copy_kib = 512 * 1024  # the copy reads and writes 512 MiB
    ff, wf = copy_kib / f_c, copy_kib / w_c
    rd, wr = int(f_k * ff * 1024), int(w_k * wf * 1024)
    rec = {"kernel": f"pbsa::{TRAFFIC_KERNEL}",
           "workload": "wan_5s measured chunk (12 heads, d=128, 4680 queries, C=64, W=6, K=32)",
           "source_sha256": kernel_source_hash(),
           "fetch_size_kib_per_dispatch": round(f_k, 1), "write_size_kib_per_dispatch": round(w_k, 1),
           "calibration": {"copy": "__amd_rocclr_copyBuffer of 512 MiB (bench.py --copy-probe)",
                           "fetch_size_kib": f_c, "write_size_kib": w_c,
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "bytes_per_launch": rd + wr, "dispatches": n}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def _timed_reps(torch, stream, fn, reps, flush=None):
    """Median and p10/p90 of `reps` runs of fn (ms), HIP events on `stream`; flush() runs
    before each rep outside the timed region (cold runs)."""
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def bench_probes(torch, ops, synth, shape, layer, q, k, v, stream):
    """Measured ceilings next to the published peaks (extra field):
      mfma   - independent v_mfma_f32_32x32x16_bf16 chains on every SIMD (pbsa_probe_mfma);
      copy   - a 512 MiB device copy (read + write bytes / time);
      gather - the attention's gathers without its math (pbsa_probe_gather) on the measured
               chunk: bytes moved into LDS per launch (one 1 KB instruction per piece; a
               step moves 32 KB per workgroup) / time, warm and cold;
      pool_full_history - pbsa_pool over the 1-minute workload's whole history
               (240 frames x 1560 tokens x 12 heads x 128, 1.15 GB read), warm and cold.
    Cold runs first read a 512 MiB buffer (larger than the 256 MB last-level cache)."""
    out = {}
    flush_buf = torch.ones(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda")
    flush_sink = torch.empty((), dtype=torch.bfloat16, device="cuda")

    def flush():
        # a 512 MiB read (not a write: dirty lines would be written back during the timed
        # launch and charged to it)
        flush_sink.copy_(flush_buf.sum())

    # MFMA ceiling
    mf = torch.empty(131072, dtype=torch.float32, device="cuda")
    iters = 20000
    flop = ops.pbsa_probe_mfma(iters, mf)
    torch.cuda.synchronize()
    med, _, _ = _timed_reps(torch, stream, lambda: ops.pbsa_probe_mfma(iters, mf), 5)
    out["mfma"] = {"tflops": round(flop / (med * 1e-3) / 1e12, 1), "ms": round(med, 3),
                   "frac_of_peak": round(flop / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    # copy ceiling
    src = torch.ones(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    med, _, _ = _timed_reps(torch, stream, lambda: dst.copy_(src), 5)
    cb = 2 * src.numel() * 2
    out["copy"] = {"gbs": round(cb / (med * 1e-3) / 1e9, 1), "ms": round(med, 3),
                   "frac_of_peak": round(cb / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del src, dst
    # gather of the measured chunk (routing already current)
    layer.route(q)
    bid = layer.cache.block_id.cpu().numpy()
    sel = layer.sel.cpu().numpy()
    C, nq = shape.capacity, shape.nq
    steps = 0
    unique_slots = 0  # distinct cache slots the launch reads (P, and routed window blocks)
    for h in range(shape.heads):
        routed = {int(g) for g in sel[h].ravel() if g >= 0}
        unique_slots += int((bid[h, :C] >= 0).sum()) + len(routed)
        for pr in range((nq + 1) // 2):
            # blocks routed by both query blocks of the pair join the shared steps
            sa = {int(g) for g in sel[h, 2 * pr] if g >= 0}
            sb = {int(g) for g in sel[h, 2 * pr + 1] if g >= 0} if 2 * pr + 1 < nq else set()
            nshared = int((bid[h, :C] >= 0).sum()) + nq + len(sa & sb)
            nsh2 = nshared + (nshared & 1)
            # + the two steps gathered ahead past the end
            steps += nsh2 + 2 * max(len(sa - sb), len(sb - sa)) + 2
    gbytes = steps * 32 * 1024
    g = lambda: ops.pbsa_probe_gather(shape, q, layer.cache, k, v, layer.sel)
    g()
    torch.cuda.synchronize()
    warm, _, _ = _timed_reps(torch, stream, g, 10)
    cold, c10, c90 = _timed_reps(torch, stream, g, 10, flush)
    # unique KV bytes: each distinct slot's K and V (64 rows) plus the chunk's own K and V
    ubytes = unique_slots * 2 * 64 * shape.head_dim * 2 + \
        2 * shape.chunk_tokens * shape.heads * shape.head_dim * 2
    out["gather"] = {"bytes_moved_to_lds": gbytes, "unique_kv_bytes": ubytes,
                     "ms_warm": round(warm, 4),
                     "ms_cold": round(cold, 4), "ms_cold_p10_p90": [round(c10, 4), round(c90, 4)],
                     "gbs_warm": round(gbytes / (warm * 1e-3) / 1e9, 1),
                     "gbs_cold": round(gbytes / (cold * 1e-3) / 1e9, 1),
                     "unique_gbs_cold": round(ubytes / (cold * 1e-3) / 1e9, 1)}
    # full-history pooling at the 1-minute workload's size (seeded synthetic tokens)
    wl = synth.WORKLOADS["wan_1min"]
    frames = wl.history_frames
    T = frames * wl.frame_tokens
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.SEEDS["wan_1min"])
    x = torch.randn((T, wl.heads, wl.head_dim), generator=gen, device="cuda",
                    dtype=torch.float32).to(torch.bfloat16)
    pshape = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, frames, scale=wl.scale)
    brep = torch.empty((wl.heads, frames * wl.nb, wl.head_dim), dtype=torch.float32, device="cuda")
    frep = torch.empty((wl.heads, frames, wl.head_dim), dtype=torch.float32, device="cuda")
    p = lambda: ops.pbsa_pool(pshape, x, frames, brep, frep)
    p()
    torch.cuda.synchronize()
    warm, _, _ = _timed_reps(torch, stream, p, 10)
    cold, c10, c90 = _timed_reps(torch, stream, p, 10, flush)
    pb = x.numel() * 2 + brep.numel() * 4 + frep.numel() * 4
    out["pool_full_history"] = {
        "workload": "wan_1min history: 240 frames x 1560 tokens, 12 heads, d=128",
        "bytes": pb, "ms_warm": round(warm, 4), "ms_cold": round(cold, 4),
        "ms_cold_p10_p90": [round(c10, 4), round(c90, 4)],
        "gbs_warm": round(pb / (warm * 1e-3) / 1e9, 1), "gbs_cold": round(pb / (cold * 1e-3) / 1e9, 1),
        "frac_hbm_cold": round(pb / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del x, brep, frep
    # the training clip's queries and keys (block and frame representatives of each)
    wl = synth.WORKLOADS["wan_train"]
    frames = wl.clip_chunks * wl.chunk_frames
    T = frames * wl.frame_tokens
    gen.manual_seed(synth.SEEDS["wan_train"])
    xs = [torch.randn((T, wl.heads, wl.head_dim), generator=gen, device="cuda",
                      dtype=torch.float32).to(torch.bfloat16) for _ in range(2)]
    pshape = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, frames, scale=wl.scale)
    reps = [(torch.empty((wl.heads, frames * wl.nb, wl.head_dim), dtype=torch.float32,
                         device="cuda"),
             torch.empty((wl.heads, frames, wl.head_dim), dtype=torch.float32, device="cuda"))
            for _ in range(2)]

    def pc():
        for x_, (b_, f_) in zip(xs, reps):
            ops.pbsa_pool(pshape, x_, frames, b_, f_)
    pc()
    torch.cuda.synchronize()
    warm, _, _ = _timed_reps(torch, stream, pc, 10)
    cold, c10, c90 = _timed_reps(torch, stream, pc, 10, flush)
    pb = sum(x_.numel() * 2 for x_ in xs) + sum(b_.numel() * 4 + f_.numel() * 4 for b_, f_ in reps)
    out["pool_train_clip"] = {
        "workload": "wan_train clip q and k: 24 frames x 1560 tokens, 12 heads, d=128 (2 launches)",
        "bytes": pb, "ms_warm": round(warm, 4), "ms_cold": round(cold, 4),
        "ms_cold_p10_p90": [round(c10, 4), round(c90, 4)],
        "gbs_cold": round(pb / (cold * 1e-3) / 1e9, 1),
        "frac_hbm_cold": round(pb / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del xs, reps, flush_buf
    torch.cuda.empty_cache()
    return out


def bench_train(torch, ops, runtime, synth, dev, stream):
    """Trainable two-level path on the 24-frame clip: fwd+bwd ms per clip (extra field)."""
    wl = synth.WORKLOADS["wan_train"]
    seed = synth.SEEDS["wan_train"]
    shape = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, scale=wl.scale)
    qn, kn, vn = synth.clip_qkv(wl, seed)
    q, k, v = dev(qn), dev(kn), dev(vn)
    dout = dev(synth.clip_dout(wl, seed, qn.shape[0]))
    ks = runtime.cag_budgets(synth.clip_alphas(wl, seed), wl.topk, wl.clip_chunks)
    clip = runtime.TwoLevelClip(shape, wl.clip_chunks, wl.top_frames,
                                max(max(ks), wl.chunk_frames * wl.nb))
    clip.select(q, k, ks)
    torch.cuda.synchronize()
    sel, nsel = clip.sel.cpu().numpy(), clip.nsel.cpu().numpy()
    n, nb = wl.frame_tokens, wl.nb
    keys = 0
    for h in range(wl.heads):
        for r in range(nsel.shape[1]):
            qlen = min(64, n - 64 * (r % nb))
            keys += qlen * sum(min(64, n - 64 * (int(g) % nb)) for g in sel[h, r, :nsel[h, r]])
    fwd_flop = 4 * wl.head_dim * keys
    bwd_flop = 8 * wl.head_dim * keys

    def run(fn, reps=10):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    sel_ms = run(lambda: clip.select(q, k, ks))
    fwd_ms = run(lambda: clip.forward(q, k, v))
    bwd_ms = run(lambda: clip.backward(q, k, v, dout))
    return {"workload": "wan_train: 24-frame clip, 8 chunks, two-level top-8 frames",
            "select_ms": round(sel_ms, 4), "fwd_ms": round(fwd_ms, 4),
            "bwd_ms": round(bwd_ms, 4),
            "fwd_tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
            "bwd_tflops": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 2),
            "fwd_flop": int(fwd_flop), "bwd_flop": int(bwd_flop)}


def cpu_baseline(wl, seed):
    """The fp64 oracle's chunk step (select, gathered attention, update) for every head of
    the measured chunk, on this host: each head's state is built untimed, then its chunk
    step is timed; the value is the sum over heads in ms per chunk."""
    import oracle as orc
    from block_sparse_attention_pbsa_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - reporting only
        threads = os.cpu_count() or 1
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    history = [synth.chunk_qkv(wl, seed, c) for c in range(wl.measured_chunk)]
    q, k, v = synth.chunk_qkv(wl, seed, wl.measured_chunk)
    sec = 0.0
    for h in range(wl.heads):
        ro = orc.PersistentRollout(sch, wl.head_dim)
        for qc, kc, vc in history:
            ro.update(ro.select(qc[:, h]), kc[:, h], vc[:, h])
        qh, kh, vh = q[:, h].copy(), k[:, h].copy(), v[:, h].copy()
        t = time.perf_counter()
        rt = ro.select(qh)
        ro.attend(qh, kh, vh, rt["sel"])
        ro.update(rt, kh, vh)
        sec += time.perf_counter() - t
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    return {"value": round(sec * 1e3, 1), "unit": "ms/chunk", "cores": threads,
            "kind": "oracle",
            "sample": f"all {wl.heads} heads of the wan_5s measured chunk (pool, score, route, "
                      "gathered fp64 attention over all 4680 queries, Top-C update), each "
                      "head's chunk step timed after its rollout state was built untimed; "
                      f"{os.cpu_count()} logical CPUs ({model})"}


if __name__ == "__main__":
    main()
