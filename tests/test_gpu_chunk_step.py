"""The fused chunk step (pbsa_chunk_step) and its captured HIP graph (pbsa_chunk_graph_*)
against the plain call sequence and the fp64 oracle.

A chunk of T denoising passes routes and attends every pass against the same persistent
memory and window, then updates the memory once with the last pass (Sparse Forcing,
gist.science, 2.B; the Chinese page's 2.1).  Three layers run the same rollout: the call
sequence from Python, the one-call step and the graph (captured once for a set of staging
buffers into which every chunk's inputs are copied, so the graph is replayed for every
chunk with eager work in between).  Their outputs and caches must be bit-identical after
every chunk; at the measured chunk every pass's routing and attention are checked against
the oracle, and after every update the persistent set is checked against the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from block_sparse_attention_pbsa_amd import ops, runtime, synth
from parity import assert_close_attn, check_topk, say

pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)


def shape_of(wl, fp8=False):
    return ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                     wl.capacity, wl.sinks, wl.topk, wl.scale,
                     kv_format=ops.PBSA_KV_FP8 if fp8 else ops.PBSA_KV_BF16)


def caches_equal(a, b):
    names = ("k", "v", "rep", "block_id", "len") + (("kv_scale",) if a.kv_scale is not None
                                                    else ())
    return all(torch.equal(getattr(a, nm), getattr(b, nm)) for nm in names)


@pytest.mark.parametrize("name,passes,heads,rows,fp8,arith8", [
    ("tiny", 3, (0,), None, False, False),
    ("wan_5s", 4, (0, 7), "sampled", False, False),
    ("wan_5s", 2, (3,), "sampled", True, False),
    ("wan_5s", 2, (5,), "sampled", True, True),
])
def test_chunk_step_fused_and_graph(name, passes, heads, rows, fp8, arith8):
    wl, seed = synth.WORKLOADS[name], synth.SEEDS[name]
    shape = shape_of(wl, fp8)
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    # (arith8: the attentions in FP8 arithmetic, pbsa_attn_fwd_fp8)
    seq = runtime.PersistentLayer(shape, passes=passes, fp8_arithmetic=arith8)
    fus = runtime.PersistentLayer(shape, passes=passes, fp8_arithmetic=arith8)
    gra = runtime.PersistentLayer(shape, passes=passes, device_counter=True, fp8_arithmetic=arith8)
    for lay in (seq, fus, gra):
        lay.reset()
    T = shape.chunk_tokens
    staging = [tuple(torch.empty(T, wl.heads, wl.head_dim, dtype=torch.bfloat16, device="cuda")
                     for _ in range(3)) for _ in range(passes)]
    ros = {h: orc.PersistentRollout(sch, wl.head_dim, kv_fp8=fp8) for h in heads}
    last = wl.measured_chunk
    resync = 0
    for c in range(last + 1):
        say(f"[chunk step {name}{' fp8' if fp8 else ''}{' arith8' if arith8 else ''}, "
            f"{passes} passes] chunk {c}")
        host = [synth.pass_qkv(wl, seed, c, p, passes) for p in range(passes)]
        ps = [tuple(dev(x) for x in qkv) for qkv in host]
        for buf, src in zip(staging, ps):
            for b_, s_ in zip(buf, src):
                b_.copy_(s_)
        sels = None
        if c == last:
            # the selection each pass will use (routing reads the cache only)
            sels = []
            for q, _, _ in ps:
                seq.route(q)
                sels.append(seq.sel.cpu().numpy())
        routed = {h: ros[h].select(host[-1][0][:, h]) for h in heads}
        seq.step_passes(ps)
        fus.step_fused(ps)
        gra.step_graph(staging)
        torch.cuda.synchronize()
        for p in range(passes):
            assert torch.equal(seq.os[p], fus.os[p]) and torch.equal(seq.os[p], gra.os[p]), p
            assert torch.equal(seq.lses[p], fus.lses[p]) and torch.equal(seq.lses[p], gra.lses[p])
        assert caches_equal(seq.cache, fus.cache) and caches_equal(seq.cache, gra.cache)
        assert seq.cache.chunk_index == fus.cache.chunk_index == gra.cache.chunk_index == c + 1
        assert int(gra.cache.chunk_dev.item()) == c + 1
        if c == last:
            for p, (q, k, v) in enumerate(host):
                for h in heads:
                    rt = ros[h].select(q[:, h])
                    for r in range(shape.nq):
                        got = [int(g) for g in sels[p][h, r] if g >= 0]
                        check_topk(got, rt["cand"], rt["scores_cand"][r], wl.topk)
                    gsel = [[int(g) for g in sels[p][h, r] if g >= 0] for r in range(shape.nq)]
                    idx = np.arange(T) if rows is None else np.unique(np.r_[
                        0:64, 1536:1560, T - 24:T,
                        np.random.default_rng(p + 10 * h).choice(T, 48, replace=False)])
                    o = seq.os[p][:, h].float().cpu().numpy()
                    if arith8:
                        # within the oracle's bound on the rounding of the probabilities
                        o_ref, l_ref, bnd = ros[h].attend_fp8(q[:, h], k[:, h], v[:, h], gsel,
                                                              rows=idx)
                        err = np.abs(o[idx] - o_ref[idx])
                        tol = bnd[idx] + 2.0 ** -8 * np.abs(o_ref[idx]) + 1e-4
                        say(f"  pass {p} head {h}: max err/tol {(err / tol).max():.3f}")
                        assert np.all(err <= tol)
                    else:
                        o_ref, l_ref = ros[h].attend(q[:, h], k[:, h], v[:, h], gsel, rows=idx)
                        assert_close_attn(o[idx], o_ref[idx], f"pass {p} head {h}")
                    assert np.abs(seq.lses[p][h].cpu().numpy()[idx] - l_ref[idx]).max() < 1e-3
        # the update against the oracle's (last pass)
        q, k, v = host[-1]
        for h in heads:
            ro = ros[h]
            cand, m = ro.update_candidates(routed[h])
            gp = sorted(int(g) for g in seq.cache.block_id[h, :wl.capacity].cpu() if g >= 0)
            exact, _ = check_topk([g for g in gp if g >= wl.sinks], cand, m,
                                  wl.capacity - wl.sinks)
            ro.update(routed[h], k[:, h], v[:, h], P_override=None if exact else gp)
            resync += not exact
            assert gp == ro.P
    say(f"  resyncs: {resync}")
    gra.close_graphs()


def test_chunk_graph_rejects_another_cache():
    wl = synth.WORKLOADS["tiny"]
    shape = shape_of(wl)
    a = runtime.PersistentLayer(shape, passes=1, device_counter=True)
    a.reset()
    q, k, v = (dev(x) for x in synth.chunk_qkv(wl, 3, 0))
    g = ops.ChunkGraph(shape, ops.chunk_args(shape, [(q, k, v)], a.q_rep, a.scores, a.sel, a.os,
                                             a.lses, a.workspace), a.cache, keep=(q, k, v))
    other = ops.Cache(shape, device_counter=True)
    with pytest.raises(ops.PbsaError) as e:
        g.launch(other)
    assert e.value.status == 6
    g.launch(a.cache)
    torch.cuda.synchronize()
    assert a.cache.chunk_index == 1 and int(a.cache.chunk_dev.item()) == 1
    g.close()
    plain = runtime.PersistentLayer(shape)
    with pytest.raises(ValueError):
        ops.ChunkGraph(shape, ops.chunk_args(shape, [(q, k, v)], plain.q_rep, plain.scores,
                                             plain.sel, plain.os, plain.lses, plain.workspace),
                       plain.cache)
