"""PBSA benchmark on one MI355X: ms per chunk of the persistent-mode hot path.

One step = one chunk of one attention layer (one denoising pass) of an autoregressive
rollout:
    route(q)  [pool of q, coarse scores against P_t and the window, top-K]
    attn_fwd  [attention over P_t, the routed window blocks and the chunk]
    memory_update  [Top-C update, sinks pinned; pools k into the appended blocks]
on seeded synthetic bf16 inputs already resident in HBM.  The default workload is the
1-minute rollout (12 heads, d=128, 1560-token frames, 3-frame chunks = 4680 queries,
240-frame history, 64-token blocks, capacity 256 with 1 sink, window 6 frames, top-64).
The cache is built by replaying the history chunks (route + update); then K successive
chunks -- the measured chunk (the one right after the history) and the ones after it,
drawn beforehand and resident in HBM -- are timed back to back.  The W warm-up chunks run
from the same state, which is restored afterwards, so the timed chunks, their routing and
their attended FLOP depend on neither K nor W.

Prints one JSON line.  `roofline` is for the dominant kernel (attention forward, bf16
MFMA): achieved = algorithmic FLOP of the timed chunks (4 * head_dim per attended
(query, key) pair, counted from each chunk's cache state and routing) divided by the sum
of that kernel's durations, each measured with HIP events around its launch inside the
timed region, on the stream it runs on.  `cpu_baseline` times the fp64 oracle's chunk
step on this host for a sample of heads of the measured chunk, scaled to all heads.
Extra fields: the other persistent workloads (5 s line; 20 s per-chunk times over the
whole rollout), the trainable path's forward + backward, the dense-vs-persistent KV
footprint, the T-pass chunk step, and measured device ceilings (probes).

  python bench.py [--config NAME] [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
                  [--no-extras] [--no-probes]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PBSA ms/chunk + effective TFLOP/s & % MFMA/HBM roofline, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0      # dense E4M3 MFMA, published
PEAK_HBM_GBS = 8000.0
PERSISTENT = ("tiny", "wan_5s", "wan_20s", "wan_1min")
DESCR = {
    "tiny": "tiny: 1 head, d=64, 256-token frames, 1-frame chunks, 4-frame history, C=4, W=2, K=4",
    "wan_5s": "wan_5s: Wan2.1-1.3B-shaped 5 s rollout, one layer, one chunk after a 21-frame history",
    "wan_20s": "wan_20s: Wan2.1-1.3B-shaped 20 s rollout, one layer, one chunk after an 81-frame history",
    "wan_1min": "wan_1min: Wan2.1-1.3B-shaped 1 min rollout, one layer, one chunk after a 240-frame history",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="wan_1min", choices=PERSISTENT,
                    help="persistent-mode workload of the headline line")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of the measured chunk the oracle times (0: by workload)")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline line only (no other workloads, training path, T passes)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured ceilings (MFMA, copy, gather, full-history pool)")
    ap.add_argument("--passes", type=int, default=4,
                    help="denoising passes per chunk of the multi-pass extra field")
    ap.add_argument("--traffic", default=None,
                    help="HBM traffic per attention launch from rocprofv3 counters "
                         "(default profiles/attn_fwd_<config>_traffic.json, if present)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-probe run into the traffic file, then exit")
    ap.add_argument("--train-only", action="store_true",
                    help="only the trainable path's extra field (for profiling its kernels)")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only the FP8-cache fields at --config: the bf16-arithmetic attention "
                         "over the decoded cache and the FP8-arithmetic attention")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy a 512 MiB buffer 3 times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    a = ap.parse_args()
    if a.traffic is None:
        a.traffic = os.path.join(ROOT, "profiles", f"attn_fwd_{a.config}_traffic.json")
    a.steps = max(1, a.steps)
    a.warmup = max(0, a.warmup)
    return a


# ------------------------------------------------------------------------------ helpers
class Ctx:
    """torch, the package modules, the stream and host->device helpers."""

    def __init__(self):
        import torch
        from block_sparse_attention_pbsa_amd import ops, runtime, synth
        self.torch, self.ops, self.runtime, self.synth = torch, ops, runtime, synth
        torch.cuda.set_device(0)
        self.stream = torch.cuda.current_stream()

    def dev(self, x):
        return self.torch.from_numpy(np.ascontiguousarray(x)).cuda().to(self.torch.bfloat16)

    def sync(self):
        self.torch.cuda.synchronize()

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def timed(self, fn, reps):
        """Mean duration (ms) of `reps` back-to-back runs of fn between two HIP events on
        the stream the kernels run on (no event between runs)."""
        fn()
        self.sync()
        a, b = self.event(), self.event()
        a.record(self.stream)
        for _ in range(reps):
            fn()
        b.record(self.stream)
        self.sync()
        return a.elapsed_time(b) / reps


def shape_of(ops, wl, kv_format=0, route_mode=0):
    return ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                     wl.capacity, wl.sinks, wl.topk, wl.scale, route_mode=route_mode,
                     kv_format=kv_format)


def gen_chunks(synth, wl, seed, idxs, passes=1):
    """Host Q, K, V of the given chunks (all `passes` denoising passes of each, the last one
    the chunk's own), drawn on worker threads, yielded in order."""
    idxs = list(idxs)

    def one(c):
        if passes == 1:
            return synth.chunk_qkv(wl, seed, c)
        return [synth.pass_qkv(wl, seed, c, p, passes) for p in range(passes)]
    with ThreadPoolExecutor(8) as ex:
        yield from ex.map(one, idxs)


def _cache_tensors(cache):
    ts = [cache.k, cache.v, cache.rep, cache.block_id, cache.len]
    return ts + ([cache.chunk_dev] if cache.chunk_dev is not None else [])


def snapshot(cache):
    return [t.clone() for t in _cache_tensors(cache)], cache.chunk_index


def restore(cache, snap):
    ts, idx = snap
    for t, s in zip(_cache_tensors(cache), ts):
        t.copy_(s)
    cache.chunk_index = idx


def attended(wl, shape, bid, ln, sel):
    """(attended (query, key) pairs summed over heads and query tokens, distinct cache
    slots read) for one chunk, from the cache state (block ids and lengths per slot) and
    the routing the attention sees."""
    H, C, nb, n, W, F = wl.heads, wl.capacity, wl.nb, wl.frame_tokens, wl.window_frames, \
        wl.chunk_frames
    whole = wl.sinks if shape.route_mode == 1 else C   # slots attended whole
    occ = bid[:, :whole] >= 0
    pkeys = (ln[:, :whole] * occ).sum(1)
    g = sel.astype(np.int64)
    valid = g >= 0
    gs = np.where(valid, g, 0)
    slot = C + ((gs // nb) % W) * nb + gs % nb
    if shape.route_mode == 1:
        # routed ids may be persistent blocks: their slot from the table
        ring_ok = np.take_along_axis(bid, slot.reshape(H, -1), axis=1).reshape(sel.shape) == gs
        for h in range(H):
            where = {int(x): i for i, x in enumerate(bid[h, :C]) if x >= 0}
            bad = valid[h] & ~ring_ok[h]
            slot[h][bad] = [where.get(int(x), 0) for x in gs[h][bad]]
    rl = np.take_along_axis(ln.astype(np.int64), slot.reshape(H, -1), axis=1).reshape(sel.shape)
    keys = pkeys[:, None] + F * n + (rl * valid).sum(2)
    r = np.arange(shape.nq)
    qlen = np.minimum(64, n - 64 * (r % nb))
    slots_read = int(occ.sum()) + sum(len(set(gs[h][valid[h]].tolist())) for h in range(H))
    if shape.route_mode == 1:
        # routed persistent blocks are read in their slots (counted once per head)
        slots_read = int(occ.sum()) + sum(len(set(slot[h][valid[h]].tolist())) for h in range(H))
    return int((keys * qlen[None, :]).sum()), slots_read


def attn_bytes(wl, shape, slots_read):
    """Algorithmic HBM bytes of one attention launch: the distinct KV blocks it reads (64
    padded rows of K and V each), the chunk's K and V, Q, O and LSE."""
    d, H, T = wl.head_dim, wl.heads, shape.chunk_tokens
    return slots_read * 2 * 64 * d * 2 + 2 * T * H * d * 2 + 2 * T * H * d * 2 + T * H * 4


# ------------------------------------------------------------------------------ headline
def persistent_line(cx, name, steps, warmup, oracle_heads=(), kv_format=0, route_mode=0,
                    fp8_arithmetic=False):
    """Bootstrap `name`'s rollout to its measured chunk, then time `steps` successive
    chunks.  Returns (result dict, layer, device chunks, oracle rollouts, host measured chunk)."""
    ops, runtime, synth = cx.ops, cx.runtime, cx.synth
    wl, seed = synth.WORKLOADS[name], synth.SEEDS[name]
    shape = shape_of(ops, wl, kv_format, route_mode)
    layer = runtime.PersistentLayer(shape, fp8_arithmetic=fp8_arithmetic)
    layer.reset()
    m = wl.measured_chunk
    ros = {}
    if oracle_heads:
        import oracle as orc
        sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                           wl.capacity, wl.sinks, wl.topk, wl.scale)
        ros = {h: orc.PersistentRollout(sch, wl.head_dim) for h in oracle_heads}
    t_boot = time.perf_counter()
    for q, k, v in gen_chunks(synth, wl, seed, range(m)):
        layer.step(cx.dev(q), cx.dev(k), cx.dev(v), attend=False)
        for h, ro in ros.items():
            ro.update(ro.select(q[:, h]), k[:, h], v[:, h])
    n_dev = max(steps, warmup)
    chunks, measured_host = [], None
    for i, (q, k, v) in enumerate(gen_chunks(synth, wl, seed, range(m, m + n_dev))):
        chunks.append((cx.dev(q), cx.dev(k), cx.dev(v)))
        if i == 0:
            measured_host = (q, k, v)
    cx.sync()
    print(f"{name}: bootstrapped {m} chunks in {time.perf_counter() - t_boot:.1f} s",
          file=sys.stderr, flush=True)
    snap = snapshot(layer.cache)

    # counting pass: each timed chunk's attended pairs from its cache state and routing
    pairs, slots = [], []
    for i in range(steps):
        q, k, v = chunks[i]
        layer.route(q)
        cx.sync()
        p_, s_ = attended(wl, shape, layer.cache.block_id.cpu().numpy(),
                          layer.cache.len.cpu().numpy(), layer.sel.cpu().numpy())
        pairs.append(p_)
        slots.append(s_)
        layer.attend(q, k, v)
        layer.update(k, v)
    restore(layer.cache, snap)
    for i in range(warmup):
        layer.step(*chunks[i])
    restore(layer.cache, snap)
    cx.sync()

    # timed region: `steps` successive chunks back to back; events around each attention
    ev = [(cx.event(), cx.event()) for _ in range(steps)]
    t0, t1 = cx.event(), cx.event()
    t0.record(cx.stream)
    for i in range(steps):
        q, k, v = chunks[i]
        layer.route(q)
        ev[i][0].record(cx.stream)
        layer.attend(q, k, v)
        ev[i][1].record(cx.stream)
        layer.update(k, v)
    t1.record(cx.stream)
    cx.sync()
    ms_step = t0.elapsed_time(t1) / steps
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    flop = [4 * wl.head_dim * p_ for p_ in pairs]
    achieved = sum(flop) / (sum(attn_ms) * 1e-3) / 1e12
    abytes = [attn_bytes(wl, shape, s_) for s_ in slots]

    # each op alone at the measured chunk's state (diagnostic)
    restore(layer.cache, snap)
    q, k, v = chunks[0]
    layer.route(q)
    cx.sync()
    cache2 = cx.ops.Cache(shape)
    for nm in ("k", "v", "rep", "block_id", "len"):
        getattr(cache2, nm).copy_(getattr(layer.cache, nm))
    cache2.chunk_index = layer.cache.chunk_index
    ops_ms = {
        "route": cx.timed(lambda: ops.pbsa_route(shape, q, layer.cache, layer.q_rep, layer.scores,
                                                 layer.sel), 20),
        "pool_q": cx.timed(lambda: ops.pbsa_pool(shape, q, wl.chunk_frames, layer.q_rep), 20),
        "score_topk": cx.timed(lambda: ops.pbsa_score_topk(shape, layer.q_rep, layer.cache,
                                                           layer.scores, layer.sel), 20),
        "attn_fwd": cx.timed(lambda: layer.attend(q, k, v), 20),
        # repeated on a copy of the cache (each call appends the chunk again)
        "memory_update": cx.timed(lambda: ops.pbsa_memory_update(
            shape, layer.scores, cache2, k, v, None, layer.workspace), 20),
    }
    del cache2
    res = {
        "workload": DESCR[name],
        "ms_per_chunk": round(ms_step, 4),
        "chunks_timed": [m, m + steps - 1],
        "attn_fwd_ms_mean": round(float(np.mean(attn_ms)), 4),
        "attn_fwd_ms_min_max": [round(min(attn_ms), 4), round(max(attn_ms), 4)],
        "attn_fwd_flop_mean": int(np.mean(flop)),
        "attn_fwd_tflops": round(achieved, 2),
        "attn_fwd_frac_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "attn_fwd_algorithmic_bytes_mean": int(np.mean(abytes)),
        "tflops_effective_step": round(sum(flop) / (ms_step * steps * 1e-3) / 1e12, 2),
        "ops_ms_alone": {k_: round(v_, 4) for k_, v_ in ops_ms.items()},
        "cache_bytes": ops.pbsa_cache_bytes(shape),
    }
    restore(layer.cache, snap)
    cx.sync()
    return res, layer, chunks, ros, measured_host, (sum(flop), sum(attn_ms), ms_step, abytes)


def copy_probe(cx):
    """Three copies of a 512 MiB buffer: known bytes for calibrating FETCH_SIZE and
    WRITE_SIZE in a profiled run."""
    src = cx.torch.ones(256 * 1024 * 1024, dtype=cx.torch.bfloat16, device="cuda")
    dst = cx.torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    cx.sync()


def fp8_lines(cx, name, steps, warmup):
    """The FP8 cache at `name`: the attention over the decoded codes (bf16 arithmetic) and
    pbsa_attn_fwd_fp8 (FP8 arithmetic, also reported against the FP8 peak)."""
    out = {}
    for tag, f8 in (("fp8_cache", False), ("fp8_arithmetic", True)):
        r, lay, ch, _, _, _ = persistent_line(cx, name, steps, warmup, kv_format=1,
                                              fp8_arithmetic=f8)
        r["workload"] += f"; {tag.replace('_', ' ')}"
        if f8:
            r["attn_fwd_frac_fp8_peak"] = round(r["attn_fwd_tflops"] / PEAK_FP8_TFLOPS, 4)
        out[f"{name}_{tag}"] = r
        del lay, ch
        cx.torch.cuda.empty_cache()
    return out


def rollout_per_chunk(cx, name):
    """Every chunk of `name`'s rollout with attention (route, attention, update), each
    chunk timed with events around its step; the rollout runs twice and the second run is
    reported (the first warms up).  Returns per-chunk ms."""
    ops, runtime, synth = cx.ops, cx.runtime, cx.synth
    wl, seed = synth.WORKLOADS[name], synth.SEEDS[name]
    shape = shape_of(ops, wl)
    layer = runtime.PersistentLayer(shape)
    m = wl.measured_chunk
    chunks = [(cx.dev(q), cx.dev(k), cx.dev(v)) for q, k, v in gen_chunks(synth, wl, seed,
                                                                         range(m + 1))]
    ms = []
    for rep in range(2):
        layer.reset()
        ev = [(cx.event(), cx.event()) for _ in chunks]
        for (q, k, v), (a, b) in zip(chunks, ev):
            a.record(cx.stream)
            layer.step(q, k, v)
            b.record(cx.stream)
        cx.sync()
        ms = [a.elapsed_time(b) for a, b in ev]
    del chunks
    full = -(-wl.window_frames // wl.chunk_frames)   # first chunk with a full window
    return {"workload": DESCR[name] + "; every chunk of the rollout",
            "last_chunk_ms": round(ms[m], 4),
            "mean_ms_window_full": round(float(np.mean(ms[full:])), 4),
            "chunks_in_mean": [full, m],
            "first_chunks_ms": [round(x, 4) for x in ms[:full]]}


def multi_pass(cx, name, passes, chunks_n):
    """T denoising passes per chunk sharing the persistent memory: T x (route, attention)
    on each pass's own Q, K, V, then one memory update with the last pass's scores and
    K/V; `chunks_n` successive chunks from the measured one, timed back to back, through
    the plain call sequence and through the captured chunk step."""
    ops, runtime, synth = cx.ops, cx.runtime, cx.synth
    wl, seed = synth.WORKLOADS[name], synth.SEEDS[name]
    shape = shape_of(ops, wl)
    layer = runtime.PersistentLayer(shape, passes=passes, device_counter=True)
    layer.reset()
    m = wl.measured_chunk
    for q, k, v in gen_chunks(synth, wl, seed, range(m)):
        layer.step(cx.dev(q), cx.dev(k), cx.dev(v), attend=False)
    chunks = [[tuple(cx.dev(x) for x in qkv) for qkv in ps]
              for ps in gen_chunks(synth, wl, seed, range(m, m + chunks_n), passes)]
    cx.sync()
    snap = snapshot(layer.cache)
    out = {"workload": DESCR[name], "passes": passes, "chunks_timed": [m, m + chunks_n - 1]}
    for mode in ("sequence", "fused_call", "graph"):
        run = {"sequence": layer.step_passes, "fused_call": layer.step_fused,
               "graph": layer.step_graph}[mode]
        for ps in chunks:        # warm (and, for the graph, capture) every chunk first
            run(ps)
        restore(layer.cache, snap)
        cx.sync()
        a, b = cx.event(), cx.event()
        a.record(cx.stream)
        for ps in chunks:
            run(ps)
        b.record(cx.stream)
        cx.sync()
        out[f"ms_per_chunk_{mode}"] = round(a.elapsed_time(b) / chunks_n, 4)
        restore(layer.cache, snap)
        cx.sync()
    layer.close_graphs()
    del chunks
    return out


def persistent_backward(cx, name):
    """Sparse Forcing's own trainable layout: forward and backward of the persistent-mode
    attention (P_t, the routed window blocks and the chunk) at `name`'s measured chunk, with
    the gradient of every cache slot (extra field)."""
    ops, runtime, synth = cx.ops, cx.runtime, cx.synth
    wl, seed = synth.WORKLOADS[name], synth.SEEDS[name]
    shape = shape_of(ops, wl)
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    m = wl.measured_chunk
    for q, k, v in gen_chunks(synth, wl, seed, range(m)):
        layer.step(cx.dev(q), cx.dev(k), cx.dev(v), attend=False)
    q, k, v = (cx.dev(x) for x in synth.chunk_qkv(wl, seed, m))
    dout = cx.dev(synth.clip_dout(wl, seed, shape.chunk_tokens))
    layer.route(q)
    cx.sync()
    pairs, _ = attended(wl, shape, layer.cache.block_id.cpu().numpy(),
                        layer.cache.len.cpu().numpy(), layer.sel.cpu().numpy())
    T, H, d = shape.chunk_tokens, wl.heads, wl.head_dim
    dq, dk, dv = (cx.torch.empty(T, H, d, dtype=cx.torch.bfloat16, device="cuda")
                  for _ in range(3))
    dkc, dvc = cx.torch.empty_like(layer.cache.k), cx.torch.empty_like(layer.cache.v)
    ws = cx.torch.empty(ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_BWD_PERSISTENT),
                        dtype=cx.torch.uint8, device="cuda")
    fwd_ms = cx.timed(lambda: layer.attend(q, k, v), 10)
    bwd_ms = cx.timed(lambda: ops.pbsa_attn_bwd_persistent(
        shape, q, layer.cache, k, v, layer.sel, layer.o, layer.lse, dout, dq, dk, dv, dkc, dvc,
        ws), 10)
    bwd_flop = 8 * d * pairs
    return {"workload": DESCR[name] + "; gradient of the persistent-mode attention",
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_bwd_ms_per_chunk": round(fwd_ms + bwd_ms, 4),
            "bwd_flop": int(bwd_flop),
            "bwd_tflops": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 2),
            "bwd_frac_bf16_peak": round(bwd_flop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def footprint(synth, ops):
    """Per layer: a dense KV cache of the whole history plus the chunk, against the
    persistent cache (P_t and the window in 64-row slots, plus representatives, ids and
    lengths) plus the chunk."""
    out = {}
    for name in ("wan_5s", "wan_20s", "wan_1min"):
        wl = synth.WORKLOADS[name]
        shape = shape_of(ops, wl)
        kv_tok = wl.heads * wl.head_dim * 2 * 2   # K and V bytes per token
        dense = (wl.history_frames + wl.chunk_frames) * wl.frame_tokens * kv_tok
        cache = wl.heads * shape.slots * (2 * 64 * wl.head_dim * 2 + wl.head_dim * 4 + 8)
        chunk = shape.chunk_tokens * kv_tok
        out[name] = {"dense_bytes": dense, "persistent_bytes": cache + chunk,
                     "persistent_cache_bytes": cache,
                     "persistent_over_dense": round((cache + chunk) / dense, 4)}
    return out


# ------------------------------------------------------------------------------ main
def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.traffic, args.config)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "PBSA runs on one GPU here: the path is sharded by head "
                                   "across GPUs only by design (no collectives are built); "
                                   "--gpus must be 1"}))
        sys.exit(2)
    cx = Ctx()
    if args.train_only:
        out = {"wan_train": bench_train(cx)}
        if args.copy_probe:
            copy_probe(cx)
        print(json.dumps(out), flush=True)
        return
    name = args.config
    wl = cx.synth.WORKLOADS[name]
    if args.fp8_only:
        out = fp8_lines(cx, name, args.steps, args.warmup)
        if args.copy_probe:
            copy_probe(cx)
        print(json.dumps(out), flush=True)
        return
    cpu_heads = ()
    if not args.no_cpu:
        n_h = args.cpu_heads or {"tiny": 1, "wan_5s": 12, "wan_20s": 8, "wan_1min": 8}[name]
        cpu_heads = tuple(range(min(n_h, wl.heads)))
    res, layer, chunks, ros, measured_host, (flop_sum, attn_ms_sum, ms_step, abytes) = \
        persistent_line(cx, name, args.steps, args.warmup, cpu_heads)
    achieved = flop_sum / (attn_ms_sum * 1e-3) / 1e12

    traffic = None
    if os.path.exists(args.traffic):
        try:
            rec = json.load(open(args.traffic))
            if rec.get("source_sha256") == kernel_source_hash():
                traffic = rec.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    shape = shape_of(cx.ops, wl)
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
        "config": {"workload": DESCR[name], "heads": wl.heads, "head_dim": wl.head_dim,
                   "frame_tokens": wl.frame_tokens, "chunk_frames": wl.chunk_frames,
                   "query_tokens": shape.chunk_tokens, "history_frames": wl.history_frames,
                   "block": wl.block, "capacity": wl.capacity, "sinks": wl.sinks,
                   "window_frames": wl.window_frames, "topk": wl.topk},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": TRAFFIC_KERNEL,
                     "algorithmic_bytes": int(np.mean(abytes))},
    }
    result.update({k_: v_ for k_, v_ in res.items() if k_ != "workload"})

    if not args.no_probes:
        q, k, v = chunks[0]
        result["probes"] = bench_probes(cx, shape, layer, q, k, v)
    del chunks, layer
    cx.torch.cuda.empty_cache()

    if not args.no_extras:
        extras = {}
        for other in ("wan_5s", "wan_20s", "wan_1min"):
            if other == name:
                continue
            r, lay, ch, _, _, _ = persistent_line(cx, other, 10, 3)
            extras[other] = r
            del lay, ch
            cx.torch.cuda.empty_cache()
        # FP8 cache (E4M3 codes, power-of-two scale per block; the attention in bf16 over
        # the decoded codes, and in FP8 arithmetic) and routing over P and the window
        # together, on the headline workload
        extras.update(fp8_lines(cx, name, 10, 3))
        r, lay, ch, _, _, _ = persistent_line(cx, name, 10, 3, route_mode=1)
        r["workload"] += "; union routing"
        extras[f"{name}_union_routing"] = r
        del lay, ch
        cx.torch.cuda.empty_cache()
        extras["wan_20s_rollout"] = rollout_per_chunk(cx, "wan_20s")
        cx.torch.cuda.empty_cache()
        extras[f"{name}_T{args.passes}"] = multi_pass(cx, name, args.passes, 6)
        cx.torch.cuda.empty_cache()
        extras["wan_train"] = bench_train(cx)
        cx.torch.cuda.empty_cache()
        for nm in ("wan_5s", name):
            extras[f"{nm}_persistent_fwd_bwd"] = persistent_backward(cx, nm)
            cx.torch.cuda.empty_cache()
        result["extras"] = extras
        result["footprint"] = footprint(cx.synth, cx.ops)

    if args.copy_probe:
        src = cx.torch.ones(256 * 1024 * 1024, dtype=cx.torch.bfloat16, device="cuda")
        dst = cx.torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        cx.sync()
        result["copy_probe_bytes"] = src.numel() * 2

    if cpu_heads:
        result["cpu_baseline"] = cpu_baseline(wl, cx.synth.SEEDS[name], ros, measured_host)
    print(json.dumps(result), flush=True)


TRAFFIC_KERNEL = "attn_fwd_kernel<128, true, false, false>"
KERNEL_SOURCES = ("attn_fwd.hip", "attn_lists.h", "attn_common.h", "common.h")


def kernel_source_hash():
    """sha256 (first 16 hex digits) of the sources the timed attention kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_pbsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def write_traffic(fetch_dir, write_dir, out_path, config):
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
           "workload": DESCR[config] + " (every attention launch of the run)",
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


def _timed_reps(cx, fn, reps, flush=None):
    """Median and p10/p90 of `reps` runs of fn (ms), HIP events on the stream; flush() runs
    before each rep outside the timed region (cold runs)."""
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = cx.event(), cx.event()
        a.record(cx.stream)
        fn()
        b.record(cx.stream)
        cx.sync()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def bench_probes(cx, shape, layer, q, k, v):
    """Measured ceilings next to the published peaks (extra field):
      mfma   - independent v_mfma_f32_32x32x16_bf16 chains on every SIMD (pbsa_probe_mfma);
      copy   - a 512 MiB device copy (read + write bytes / time);
      gather - the attention's gathers without its math (pbsa_probe_gather) on the measured
               chunk: bytes moved into LDS per launch (one 1 KB instruction per piece; a
               step moves 32 KB per workgroup) / time, warm and cold;
      pool_full_history - pbsa_pool over the 1-minute workload's whole history
               (240 frames x 1560 tokens x 12 heads x 128, 1.15 GB read), warm and cold;
      pool_train_clip - the training clip's q and k (block and frame representatives).
    Cold runs first read a 512 MiB buffer (larger than the 256 MB last-level cache)."""
    torch, ops, synth = cx.torch, cx.ops, cx.synth
    out = {}
    flush_buf = torch.ones(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda")
    flush_sink = torch.empty((), dtype=torch.bfloat16, device="cuda")

    def flush():
        # a 512 MiB read (not a write: dirty lines would be written back during the timed
        # launch and charged to it)
        flush_sink.copy_(flush_buf.sum())

    mf = torch.empty(131072, dtype=torch.float32, device="cuda")
    iters = 20000
    flop = ops.pbsa_probe_mfma(iters, mf)
    cx.sync()
    med, _, _ = _timed_reps(cx, lambda: ops.pbsa_probe_mfma(iters, mf), 5)
    out["mfma"] = {"tflops": round(flop / (med * 1e-3) / 1e12, 1), "ms": round(med, 3),
                   "frac_of_peak": round(flop / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    src = torch.ones(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    med, _, _ = _timed_reps(cx, lambda: dst.copy_(src), 5)
    cb = 2 * src.numel() * 2
    out["copy"] = {"gbs": round(cb / (med * 1e-3) / 1e9, 1), "ms": round(med, 3),
                   "frac_of_peak": round(cb / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del src, dst
    # gather of the measured chunk (its routing made current)
    layer.route(q)
    bid = layer.cache.block_id.cpu().numpy()
    sel = layer.sel.cpu().numpy()
    C, nq = shape.capacity, shape.nq
    steps = 0
    unique_slots = 0
    for h in range(shape.heads):
        routed = {int(g) for g in sel[h].ravel() if g >= 0}
        unique_slots += int((bid[h, :C] >= 0).sum()) + len(routed)
        for pr in range((nq + 1) // 2):
            sa = {int(g) for g in sel[h, 2 * pr] if g >= 0}
            sb = {int(g) for g in sel[h, 2 * pr + 1] if g >= 0} if 2 * pr + 1 < nq else set()
            nshared = int((bid[h, :C] >= 0).sum()) + nq + len(sa & sb)
            nsh2 = nshared + (nshared & 1)
            steps += nsh2 + 2 * max(len(sa - sb), len(sb - sa)) + 2
    gbytes = steps * 32 * 1024
    g = lambda: ops.pbsa_probe_gather(shape, q, layer.cache, k, v, layer.sel)
    g()
    cx.sync()
    warm, _, _ = _timed_reps(cx, g, 10)
    cold, c10, c90 = _timed_reps(cx, g, 10, flush)
    ubytes = unique_slots * 2 * 64 * shape.head_dim * 2 + \
        2 * shape.chunk_tokens * shape.heads * shape.head_dim * 2
    out["gather"] = {"bytes_moved_to_lds": gbytes, "unique_kv_bytes": ubytes,
                     "ms_warm": round(warm, 4),
                     "ms_cold": round(cold, 4), "ms_cold_p10_p90": [round(c10, 4), round(c90, 4)],
                     "gbs_warm": round(gbytes / (warm * 1e-3) / 1e9, 1),
                     "gbs_cold": round(gbytes / (cold * 1e-3) / 1e9, 1),
                     "unique_gbs_cold": round(ubytes / (cold * 1e-3) / 1e9, 1)}
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
    cx.sync()
    warm, _, _ = _timed_reps(cx, p, 10)
    cold, c10, c90 = _timed_reps(cx, p, 10, flush)
    pb = x.numel() * 2 + brep.numel() * 4 + frep.numel() * 4
    out["pool_full_history"] = {
        "workload": "wan_1min history: 240 frames x 1560 tokens, 12 heads, d=128",
        "bytes": pb, "ms_warm": round(warm, 4), "ms_cold": round(cold, 4),
        "ms_cold_p10_p90": [round(c10, 4), round(c90, 4)],
        "gbs_warm": round(pb / (warm * 1e-3) / 1e9, 1), "gbs_cold": round(pb / (cold * 1e-3) / 1e9, 1),
        "frac_hbm_cold": round(pb / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del x, brep, frep
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
    cx.sync()
    warm, _, _ = _timed_reps(cx, pc, 10)
    cold, c10, c90 = _timed_reps(cx, pc, 10, flush)
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


def bench_train(cx):
    """Trainable two-level path on the 24-frame clip: selection, forward and backward, ms
    per clip and per chunk (extra field)."""
    ops, runtime, synth = cx.ops, cx.runtime, cx.synth
    wl = synth.WORKLOADS["wan_train"]
    seed = synth.SEEDS["wan_train"]
    shape = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, scale=wl.scale)
    qn, kn, vn = synth.clip_qkv(wl, seed)
    q, k, v = cx.dev(qn), cx.dev(kn), cx.dev(vn)
    dout = cx.dev(synth.clip_dout(wl, seed, qn.shape[0]))
    ks = runtime.cag_budgets(synth.clip_alphas(wl, seed), wl.topk, wl.clip_chunks)
    clip = runtime.TwoLevelClip(shape, wl.clip_chunks, wl.top_frames,
                                max(max(ks), wl.chunk_frames * wl.nb))
    clip.select(q, k, ks)
    cx.sync()
    sel, nsel = clip.sel.cpu().numpy(), clip.nsel.cpu().numpy()
    n, nb = wl.frame_tokens, wl.nb
    blen = np.minimum(64, n - 64 * (np.arange(sel.shape[1]) % nb))
    keys = 0
    for h in range(wl.heads):
        for r in range(nsel.shape[1]):
            keys += int(blen[r]) * int(blen[sel[h, r, :nsel[h, r]]].sum())
    fwd_flop = 4 * wl.head_dim * keys
    bwd_flop = 8 * wl.head_dim * keys
    sel_ms = cx.timed(lambda: clip.select(q, k, ks), 10)
    fwd_ms = cx.timed(lambda: clip.forward(q, k, v), 10)
    bwd_ms = cx.timed(lambda: clip.backward(q, k, v, dout), 10)
    C = wl.clip_chunks
    return {"workload": "wan_train: 24-frame clip (8 chunks of 3 frames, 37,440 tokens), "
                        "two-level top-8 frames, per-chunk budgets",
            "select_ms": round(sel_ms, 4), "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_bwd_ms_per_clip": round(sel_ms + fwd_ms + bwd_ms, 4),
            "fwd_bwd_ms_per_chunk": round((sel_ms + fwd_ms + bwd_ms) / C, 4),
            "fwd_tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
            "bwd_tflops": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 2),
            "bwd_frac_bf16_peak": round(bwd_flop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "fwd_flop": int(fwd_flop), "bwd_flop": int(bwd_flop)}


def cpu_baseline(wl, seed, ros, measured_host):
    """The fp64 oracle's chunk step (pool, score, route, gathered attention over all the
    chunk's queries, Top-C update) on this host, for the heads whose rollout state was
    built (untimed) during the bootstrap; scaled to all heads, in ms per chunk."""
    import oracle  # noqa: F401  (test infrastructure: the CPU-baseline leg only)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - reporting only
        threads = os.cpu_count() or 1
    q, k, v = measured_host
    sec = 0.0
    for h, ro in ros.items():
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
    n = len(ros)
    return {"value": round(sec * 1e3 * wl.heads / n, 1), "unit": "ms/chunk", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {wl.heads} heads of the {wl.name} measured chunk (pool, score, "
                      "route, gathered fp64 attention over all the chunk's queries, Top-C update), "
                      f"timed {sec:.1f} s after each head's rollout state was built untimed, "
                      f"scaled to {wl.heads} heads; {os.cpu_count()} logical CPUs ({model})"}


if __name__ == "__main__":
    main()
