"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on seeded inputs.

Selections and persistent-memory contents must match exactly wherever the exact score gap
at the selection boundary exceeds 1e-5; inside such near-ties any correct set is accepted
and the oracle continues from the GPU's choice.  Attention outputs and gradients are
checked against the oracle evaluated on the GPU's (validated) selection: max-abs <= 2e-2,
mean-abs <= 2e-3 and relative L2 <= 1e-2 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from block_sparse_attention_pbsa_amd import ops, runtime, synth
from parity import assert_close_attn, check_topk, err_stats, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


def dev(x):
    """float32 array of bf16 values -> device bf16 tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)


def host(t):
    return t.float().cpu().numpy()


def shape_of(wl, **over):
    kw = dict(heads=wl.heads, head_dim=wl.head_dim, frame_tokens=wl.frame_tokens,
              chunk_frames=wl.chunk_frames, window_frames=wl.window_frames,
              capacity=wl.capacity, sinks=wl.sinks, topk=wl.topk, scale=wl.scale)
    kw.update(over)
    return ops.Shape(**kw)


def schedule_of(wl, union=False):
    return orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                        wl.capacity, wl.sinks, wl.topk, wl.scale, union)


# --------------------------------------------------------------------------- pooling
@pytest.mark.parametrize("name", ["tiny", "wan_5s"])
@pytest.mark.parametrize("layout", ["thd", "htd"])
def test_pool_parity(name, layout):
    wl = synth.WORKLOADS[name]
    say(f"[pool] {name} {layout}")
    _, k, _ = synth.chunk_qkv(wl, synth.SEEDS[name], 1)
    shape = shape_of(wl)
    F, H, d, nb = wl.chunk_frames, wl.heads, wl.head_dim, wl.nb
    x = dev(k)
    if layout == "htd":
        x = x.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    br = torch.empty(H, F * nb, d, device="cuda")
    fr = torch.empty(H, F, d, device="cuda")
    ops.pbsa_pool(shape, x, F, br, fr)
    torch.cuda.synchronize()
    for h in range(H):
        rb, rf = orc.mean_pool(k[:, h], wl.frame_tokens, wl.block)
        assert np.abs(br[h].cpu().numpy() - rb).max() < 2e-6
        assert np.abs(fr[h].cpu().numpy() - rf).max() < 2e-6


def test_pool_ragged_frames_and_d64():
    # 100-token frames: blocks of 64 and 36 tokens; 5 frames; head_dim 64
    shape = ops.Shape(heads=3, head_dim=64, frame_tokens=100, chunk_frames=5)
    say("[pool] ragged d64")
    x = synth.round_bf16(synth.tiny_tokens(5, (500, 3, 64)) * 3 + 1)
    br = torch.empty(3, 10, 64, device="cuda")
    fr = torch.empty(3, 5, 64, device="cuda")
    ops.pbsa_pool(shape, dev(x), 5, br, fr)
    torch.cuda.synchronize()
    for h in range(3):
        rb, rf = orc.mean_pool(x[:, h], 100, 64)
        assert np.abs(br[h].cpu().numpy() - rb).max() < 4e-6
        assert np.abs(fr[h].cpu().numpy() - rf).max() < 4e-6


# --------------------------------------------------------------------------- rollout
def gpu_P(layer, h, C):
    bid = layer.cache.block_id[h, :C].cpu().numpy()
    return sorted(int(g) for g in bid if g >= 0)


def check_slots(layer, ro, h, wl):
    """Every occupied slot holds exactly its block: tokens bit-exact, rows past len zero,
    representative within fp32 rounding of the block mean."""
    bid = layer.cache.block_id[h].cpu().numpy()
    ln = layer.cache.len[h].cpu().numpy()
    kk = layer.cache.k[h].view(torch.int16).cpu().numpy()
    vv = layer.cache.v[h].view(torch.int16).cpu().numpy()
    rep = layer.cache.rep[h].cpu().numpy()
    for s, g in enumerate(bid):
        if g < 0:
            continue
        a, b = orc.block_token_range(int(g), wl.frame_tokens, wl.block)
        assert ln[s] == b - a
        kref = synth.bf16_bits(np.asarray(ro.tok_k[int(g)], np.float32)).view(np.int16)
        vref = synth.bf16_bits(np.asarray(ro.tok_v[int(g)], np.float32)).view(np.int16)
        assert np.array_equal(kk[s, :ln[s]], kref), f"slot {s} block {g}: K bytes differ"
        assert np.array_equal(vv[s, :ln[s]], vref), f"slot {s} block {g}: V bytes differ"
        assert not kk[s, ln[s]:].any() and not vv[s, ln[s]:].any()
        assert np.abs(rep[s] - ro.krep[int(g)]).max() < 2e-6


def rollout_parity(name, attn_rows=None, slot_check_every=1, dense_check=False, wl=None,
                   seed=None, union=False):
    wl = wl if wl is not None else synth.WORKLOADS[name]
    seed = seed if seed is not None else synth.SEEDS[name]
    shape = shape_of(wl, route_mode=ops.PBSA_ROUTE_UNION if union else ops.PBSA_ROUTE_WINDOW)
    sch = schedule_of(wl, union)
    H, C, K = wl.heads, wl.capacity, wl.topk
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    ros = [orc.PersistentRollout(sch, wl.head_dim, keep_history=dense_check) for _ in range(H)]
    stats = dict(rows=0, near=0, resync=0)
    last = wl.measured_chunk
    for c in range(last + 1):
        q, k, v = synth.chunk_qkv(wl, seed, c)
        qd, kd, vd = dev(q), dev(k), dev(v)
        say(f"[rollout {name}] chunk {c}")
        layer.route(qd)
        torch.cuda.synchronize()
        scores = layer.scores.cpu().numpy()
        sel = layer.sel.cpu().numpy()
        bid = layer.cache.block_id.cpu().numpy()
        # the table and the routing pass the library's own host-side checks
        ops.pbsa_check_cache_table(shape, bid, layer.cache.len.cpu().numpy(), c)
        ops.pbsa_check_selection(shape, bid, sel)
        routed = []
        for h in range(H):
            ro = ros[h]
            rt = ro.select(q[:, h])
            routed.append(rt)
            assert gpu_P(layer, h, C) == ro.P
            # scores of every occupied slot against the oracle's
            col = {g: rt["scores_P"][:, i] for i, g in enumerate(rt["P"])}
            col.update({g: rt["scores_L"][:, i] for i, g in enumerate(rt["L"])})
            occ = [s for s in range(shape.slots) if bid[h, s] >= 0]
            assert sorted(int(bid[h, s]) for s in occ) == sorted(col)
            for s in occ:
                assert np.abs(scores[h, :, s] - col[int(bid[h, s])]).max() < 1e-5
            for s in range(shape.slots):
                if bid[h, s] < 0:
                    assert np.all(np.isneginf(scores[h, :, s]))
            for r in range(shape.nq):
                got = [g for g in sel[h, r] if g >= 0]
                assert all(g == -1 for g in sel[h, r, len(got):])
                exact, near = check_topk(got, rt["cand"], rt["scores_cand"][r], K)
                stats["rows"] += 1
                stats["near"] += near
        if c == last:
            layer.attend(qd, kd, vd)
            torch.cuda.synchronize()
            o = host(layer.o)
            lse = layer.lse.cpu().numpy()
            nq_rows = wl.chunk_frames * wl.frame_tokens
            for h in range(H):
                gsel = [[int(g) for g in sel[h, r] if g >= 0] for r in range(shape.nq)]
                rows = attn_rows(h, nq_rows) if attn_rows else None
                ro_, rl_ = ros[h].attend(q[:, h], k[:, h], v[:, h], gsel, rows=rows)
                idx = np.arange(nq_rows) if rows is None else np.asarray(rows)
                assert_close_attn(o[idx, h], ro_[idx], f"O head {h}")
                assert np.abs(lse[h, idx] - rl_[idx]).max() < 1e-3
                if dense_check:
                    do_, dl_ = ros[h].attend_dense(q[:, h], k[:, h], v[:, h], gsel)
                    np.testing.assert_allclose(do_, ro_, atol=1e-12, rtol=0)
            return stats, layer, ros
        layer.update(kd, vd)
        torch.cuda.synchronize()
        for h in range(H):
            ro = ros[h]
            cand, m = ro.update_candidates(routed[h])
            gp = gpu_P(layer, h, C)
            kept = [g for g in gp if g >= wl.sinks]
            exact, near = check_topk(kept, cand, m, C - wl.sinks)
            ro.update(routed[h], k[:, h], v[:, h], P_override=None if exact else gp)
            stats["resync"] += not exact
            assert gp == ro.P
            if slot_check_every and (c % slot_check_every == 0 or c == last - 1):
                check_slots(layer, ro, h, wl)
    raise AssertionError("unreachable")


def test_rollout_tiny_full_parity():
    stats, layer, ros = rollout_parity("tiny", dense_check=True)
    say(f"  tiny: {stats}")


def sampled_rows(seed):
    def pick(h, T):
        rs = np.random.default_rng(seed + h)
        # a full block, a frame-tail block (24 rows) and a random sample
        fixed = list(range(0, 64)) + list(range(1536, 1560)) + list(range(T - 24, T))
        return sorted(set(fixed) | set(rs.choice(T, 64, replace=False).tolist()))
    return pick


def test_rollout_wan_5s_parity():
    stats, _, _ = rollout_parity("wan_5s", attn_rows=sampled_rows(1), slot_check_every=2)
    say(f"  wan_5s: {stats}")
    assert stats["near"] <= 0.2 * stats["rows"]


def test_rollout_wan_20s_parity():
    stats, _, _ = rollout_parity("wan_20s", attn_rows=sampled_rows(2), slot_check_every=9)
    say(f"  wan_20s: {stats}")


def test_rollout_wan_1min_parity():
    stats, _, _ = rollout_parity("wan_1min", attn_rows=sampled_rows(3), slot_check_every=20)
    say(f"  wan_1min: {stats}")


# ---- selection variants: top-K over P_t and the window together, whole-frame sinks,
# planted directions that change with each segment
def test_rollout_tiny_union_routing_full_parity():
    stats, _, _ = rollout_parity("tiny", dense_check=True, union=True)
    say(f"  tiny union: {stats}")


def test_rollout_wan_5s_union_routing_parity():
    stats, _, _ = rollout_parity("wan_5s", attn_rows=sampled_rows(4), slot_check_every=3,
                                 union=True)
    say(f"  wan_5s union: {stats}")


def test_rollout_wan_1min_union_routing_parity():
    stats, _, _ = rollout_parity("wan_1min", attn_rows=sampled_rows(5), slot_check_every=40,
                                 union=True)
    say(f"  wan_1min union: {stats}")


def test_rollout_whole_frame_sinks_parity():
    # frame 0's 25 blocks are the sinks (S = nb): pinned in P_t, never routed or evicted
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["wan_5s"], name="frame_sinks", sinks=25)
    stats, layer, ros = rollout_parity("frame_sinks", attn_rows=sampled_rows(6),
                                       slot_check_every=3, wl=wl, seed=1006)
    for h in range(wl.heads):
        assert set(range(25)) <= set(gpu_P(layer, h, wl.capacity))
    say(f"  whole-frame sinks: {stats}")


def test_rollout_per_segment_directions_parity():
    # the planted direction changes every 6 frames: the memory must let old salient blocks
    # go as the queries turn to the new segment's direction
    wl = synth.Workload("seg_dirs", 4, 128, 64, 1560, 3, 30, 6, 64, 1, 32,
                        planted_per_segment=8, segment_frames=6, q_align=1.0, kv_shift=3.0,
                        direction_per_segment=True)
    stats, _, _ = rollout_parity("seg_dirs", attn_rows=sampled_rows(7), slot_check_every=3,
                                 wl=wl, seed=1007)
    say(f"  per-segment directions: {stats}")


@pytest.mark.parametrize("name", ["small64", "wan_5s"])
def test_route_equals_pool_then_score_topk(name):
    """pbsa_route (pooling fused into the routing launch) gives bit-identical q_rep, scores
    and selections to pbsa_pool followed by pbsa_score_topk, with and without q_rep."""
    wl = (synth.Workload("small64", 2, 64, 64, 100, 2, 8, 4, 3, 1, 3) if name == "small64"
          else synth.WORKLOADS[name])
    shape = shape_of(wl)
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    H, nq, d = wl.heads, shape.nq, wl.head_dim
    q_rep = torch.empty(H, nq, d, dtype=torch.float32, device="cuda")
    scores = torch.empty(H, nq, shape.slots, dtype=torch.float32, device="cuda")
    sel = torch.empty(H, nq, wl.topk, dtype=torch.int32, device="cuda")
    for c in range(wl.measured_chunk + 1):
        say(f"[route {name}] chunk {c}")
        q, k, v = (dev(x) for x in synth.chunk_qkv(wl, 5, c))
        ops.pbsa_pool(shape, q, shape.chunk_frames, q_rep)
        ops.pbsa_score_topk(shape, q_rep, layer.cache, scores, sel)
        layer.route(q)
        torch.cuda.synchronize()
        assert torch.equal(layer.q_rep, q_rep)
        assert torch.equal(layer.scores, scores)
        assert torch.equal(layer.sel, sel)
        layer.scores.zero_()
        layer.sel.fill_(-7)
        ops.pbsa_route(shape, q, layer.cache, None, layer.scores, layer.sel)
        torch.cuda.synchronize()
        assert torch.equal(layer.scores, scores) and torch.equal(layer.sel, sel)
        layer.update(k, v)


@pytest.mark.parametrize("head_dim", [128, 64])
def test_memory_update_pooled_rep_matches_given_rep(head_dim):
    """memory_update with chunk_rep = pbsa_pool(chunk_k) and with chunk_rep = NULL (block
    means taken in the update) leave the same cache: identical ids, lengths and K/V bytes,
    representatives equal up to fp32 rounding.  Both updates use the same scores, so that
    rounding in the representatives cannot change a selection."""
    wl = synth.Workload("rep", 2, head_dim, 64, 100, 2, 8, 4, 3, 1, 3)
    shape = shape_of(wl)
    a, b = runtime.PersistentLayer(shape), runtime.PersistentLayer(shape)
    a.reset()
    b.reset()
    k_rep = torch.empty(wl.heads, shape.nq, head_dim, dtype=torch.float32, device="cuda")
    for c in range(wl.measured_chunk + 1):
        say(f"[rep d={head_dim}] chunk {c}")
        q, k, v = (dev(x) for x in synth.chunk_qkv(wl, 91, c))
        a.route(q)
        ops.pbsa_pool(shape, k, shape.chunk_frames, k_rep)
        ops.pbsa_memory_update(shape, a.scores, a.cache, k, v, k_rep, a.workspace)
        ops.pbsa_memory_update(shape, a.scores, b.cache, k, v, None, b.workspace)
        torch.cuda.synchronize()
        assert torch.equal(a.cache.block_id, b.cache.block_id)
        assert torch.equal(a.cache.len, b.cache.len)
        assert torch.equal(a.cache.k.view(torch.int16), b.cache.k.view(torch.int16))
        assert torch.equal(a.cache.v.view(torch.int16), b.cache.v.view(torch.int16))
        occ = a.cache.block_id >= 0
        assert (a.cache.rep[occ] - b.cache.rep[occ]).abs().max().item() < 1e-6


# Degenerate shapes: no persistent memory at all (C = S = 0), a window no longer than the
# chunk, frames shorter than one block, frames an exact multiple of the block, one head.
EDGE = {
    "no_memory": synth.Workload("no_memory", 2, 64, 64, 100, 2, 8, 2, 0, 0, 2),
    "short_frames": synth.Workload("short_frames", 1, 128, 64, 40, 1, 6, 3, 2, 1, 1),
    "exact_blocks": synth.Workload("exact_blocks", 2, 128, 64, 128, 2, 8, 4, 3, 1, 3),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_rollout_edge_shapes(name):
    stats, _, _ = rollout_parity(name, wl=EDGE[name], seed=4242, dense_check=True)
    say(f"[{name}] {stats}")


def test_attn_fwd_d64_ragged_small():
    # head_dim 64, 100-token frames (64 + 36), window smaller than the history
    wl = synth.Workload("small64", 2, 64, 64, 100, 2, 8, 4, 3, 1, 3)
    shape = shape_of(wl)
    sch = schedule_of(wl)
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    ros = [orc.PersistentRollout(sch, 64, keep_history=True) for _ in range(2)]
    for c in range(wl.measured_chunk + 1):
        say(f"[small64] chunk {c}")
        q, k, v = synth.chunk_qkv(wl, 77, c)
        qd, kd, vd = dev(q), dev(k), dev(v)
        layer.route(qd)
        layer.attend(qd, kd, vd)
        torch.cuda.synchronize()
        sel = layer.sel.cpu().numpy()
        routed = []
        for h in range(2):
            rt = ros[h].select(q[:, h])
            routed.append(rt)
            gsel = [[int(g) for g in sel[h, r] if g >= 0] for r in range(shape.nq)]
            for r in range(shape.nq):
                check_topk(gsel[r], rt["L"], rt["scores_L"][r], wl.topk)
            ro_, rl_ = ros[h].attend_dense(q[:, h], k[:, h], v[:, h], gsel)
            assert_close_attn(host(layer.o)[:, h], ro_, f"O chunk {c} head {h}")
            assert np.abs(layer.lse[h].cpu().numpy() - rl_).max() < 1e-3
        layer.update(kd, vd)
        torch.cuda.synchronize()
        for h in range(2):
            ros[h].update(routed[h], k[:, h], v[:, h])
            assert gpu_P(layer, h, wl.capacity) == ros[h].P


def test_tie_goes_to_lower_id_on_gpu():
    # every window block identical: all scores tie exactly, top-K must be the K lowest ids
    wl = synth.Workload("ties", 1, 64, 64, 128, 1, 6, 3, 2, 1, 2)
    shape = shape_of(wl)
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    blk = synth.round_bf16(synth.tiny_tokens(9, (64, 1, 64)))
    kv = np.concatenate([blk, blk])        # 2 identical blocks per frame
    for c in range(5):
        q = synth.round_bf16(synth.tiny_tokens(10 + c, (128, 1, 64)))
        say(f"[ties] chunk {c}")
        layer.step(dev(q), dev(kv), dev(kv), attend=False)
    q = synth.round_bf16(synth.tiny_tokens(20, (128, 1, 64)))
    layer.route(dev(q))
    torch.cuda.synchronize()
    sel = layer.sel.cpu().numpy()
    # window = frames 2..4 (blocks 4..9), all equal -> ids 4, 5
    assert sel[0].tolist() == [[4, 5], [4, 5]]
    # the last update ranked blocks 1, 2, 3 with equal memory scores and one free slot:
    # the lowest id stays
    assert gpu_P(layer, 0, 2) == [0, 1]


# --------------------------------------------------------------------------- two-level
def decomposed_reference(q, k, v, dout, allowed, n, B, scale, qblocks=None, kv_blocks=None):
    """The oracle's attention and gradient for one head, one query block at a time.

    Each query block's rows attend exactly its own selected keys, so O, LSE and dQ of its
    rows come from masked_attention(_grad) over those keys alone, and the gradient of the
    keys and values is the sum over the query blocks of their contributions (dK = scale
    dS^T Q and dV = P^T dO are sums over query rows).  Returns O, LSE, dQ for the rows of
    `qblocks` (default: all) and dK, dV summed over every query block for the token rows of
    `kv_blocks` (default: all), as full-size arrays (other rows NaN)."""
    T, d = q.shape
    nqb = len(allowed)
    qblocks = range(nqb) if qblocks is None else qblocks
    O = np.full((T, d), np.nan)
    L = np.full(T, np.nan)
    dQ = np.full((T, d), np.nan)
    dK = np.zeros((T, d))
    dV = np.zeros((T, d))
    want_kv = None if kv_blocks is None else set(kv_blocks)
    need_q = set(qblocks)
    for r in range(nqb):
        if want_kv is not None and r not in need_q and not (want_kv & set(allowed[r])):
            continue
        a, b = orc.block_token_range(r, n, B)
        toks = np.concatenate([np.arange(*orc.block_token_range(g, n, B)) for g in allowed[r]])
        m = np.ones((b - a, len(toks)), bool)
        rq, rk, rv = orc.masked_attention_grad(q[a:b], k[toks], v[toks], m, scale, dout[a:b])
        if r in need_q:
            O[a:b], L[a:b] = orc.masked_attention(q[a:b], k[toks], v[toks], m, scale)
            dQ[a:b] = rq
        np.add.at(dK, toks, rk)
        np.add.at(dV, toks, rv)
    if want_kv is not None:
        keep = np.zeros(T, bool)
        for g in want_kv:
            keep[slice(*orc.block_token_range(g, n, B))] = True
        dK[~keep] = np.nan
        dV[~keep] = np.nan
    return O, L, dQ, dK, dV


def check_two_level_selection(wl, q, k, clip, sel, nsel, ks):
    """Every query block's two-level selection against the oracle's (frame-level near-ties:
    every valid frame set is a candidate explanation; block-level near-ties through
    check_topk); also the pooled representatives.  Returns (near-tie rows, selections)."""
    F, n, nb, H = wl.chunk_frames, wl.frame_tokens, wl.nb, wl.heads
    chunks = wl.clip_chunks
    near_rows = 0
    gsel_all = []
    for h in range(H):
        qr, _ = orc.mean_pool(q[:, h], n, wl.block)
        kr, kf = orc.mean_pool(k[:, h], n, wl.block)
        assert np.abs(clip.q_rep[h].cpu().numpy() - qr).max() < 2e-6
        assert np.abs(clip.k_rep[h].cpu().numpy() - kr).max() < 2e-6
        assert np.abs(clip.k_frame[h].cpu().numpy() - kf).max() < 2e-6
        gsel = []
        for r in range(chunks * F * nb):
            i = r // (F * nb) + 1
            got = sel[h, r, :nsel[h, r]].tolist()
            gsel.append(got)
            if i == 1:
                assert got == list(range(F * nb))
                continue
            hist, p, T_r = orc.two_level_frames(qr[r], kf, i, F, wl.top_frames, wl.scale)
            forced = {0, F * (i - 1) - 1} | {F * (i - 1) + t for t in range(F)}
            # frame-level near-ties: every valid frame set is a candidate explanation
            options = [T_r]
            if len(hist) > wl.top_frames:
                o = np.lexsort((np.asarray(hist), -p))
                tau = p[o[wl.top_frames - 1]]
                amb = [f for f, s in zip(hist, p) if abs(s - tau) <= 1e-5]
                if len(amb) > 1:
                    sure = {f for f, s in zip(hist, p) if s > tau + 1e-5}
                    import itertools
                    need = wl.top_frames - len(sure)
                    options = [sorted(sure | set(cmb) | forced)
                               for cmb in itertools.combinations(amb, need)]
                    near_rows += 1
            ok = False
            for T_opt in options:
                cand, o_ = orc.two_level_blocks(qr[r], kr, T_opt, nb, wl.scale)
                try:
                    _, near = check_topk(got, cand, o_, min(ks[i - 1], len(cand)))
                    near_rows += near
                    ok = True
                    break
                except AssertionError:
                    continue
            assert ok, f"head {h} row {r}: selection {got} not a valid two-level top-k"
        gsel_all.append(gsel)
    return near_rows, gsel_all


def two_level_check(wl, seed, grad_check="full", rows_fn=None, kv_blocks_fn=None,
                    whole_heads=()):
    F, n, nb, H, d = wl.chunk_frames, wl.frame_tokens, wl.nb, wl.heads, wl.head_dim
    chunks = wl.clip_chunks
    shape = shape_of(wl)
    q, k, v = synth.clip_qkv(wl, seed)
    T = q.shape[0]
    alphas = synth.clip_alphas(wl, seed)
    ks = runtime.cag_budgets(alphas, wl.topk, chunks)
    max_sel = max(max(ks), F * nb)
    clip = runtime.TwoLevelClip(shape, chunks, wl.top_frames, max_sel)
    qd, kd, vd = dev(q), dev(k), dev(v)
    dout = synth.clip_dout(wl, seed, T)
    dod = dev(dout)
    say(f"[two-level {wl.name}] select/forward/backward")
    clip.select(qd, kd, ks)
    clip.forward(qd, kd, vd)
    clip.backward(qd, kd, vd, dod)
    torch.cuda.synchronize()
    sel = clip.sel.cpu().numpy()
    nsel = clip.nsel.cpu().numpy()
    # the selection passes the library's own host-side check
    ops.pbsa_check_selection_2lvl(shape, chunks, sel, nsel)
    near_rows, gsel_all = check_two_level_selection(wl, q, k, clip, sel, nsel, ks)
    o = host(clip.o)
    lse = clip.lse.cpu().numpy()
    dq, dk, dv = host(clip.dq), host(clip.dk), host(clip.dv)
    for h in range(H):
        allowed = gsel_all[h]
        nqb = len(allowed)
        if grad_check == "full":
            mask = orc.block_mask(range(nqb), allowed, n, wl.block, T, T)
            ro, rl = orc.masked_attention(q[:, h], k[:, h], v[:, h], mask, wl.scale)
            assert_close_attn(o[:, h], ro, f"O head {h}")
            assert np.abs(lse[h] - rl).max() < 1e-3
            rq, rk, rv = orc.masked_attention_grad(q[:, h], k[:, h], v[:, h], mask, wl.scale,
                                                   dout[:, h])
            assert_close_attn(dq[:, h], rq, f"dQ head {h}")
            assert_close_attn(dk[:, h], rk, f"dK head {h}")
            assert_close_attn(dv[:, h], rv, f"dV head {h}")
        elif h in whole_heads or grad_check == "decomposed":
            # every row and every key of this head, one query block at a time
            ro, rl, rq, rk, rv = decomposed_reference(q[:, h], k[:, h], v[:, h], dout[:, h],
                                                      allowed, n, wl.block, wl.scale)
            assert_close_attn(o[:, h], ro, f"O head {h} (all rows)")
            assert np.abs(lse[h] - rl).max() < 1e-3
            assert_close_attn(dq[:, h], rq, f"dQ head {h} (all rows)")
            assert_close_attn(dk[:, h], rk, f"dK head {h} (all keys)")
            assert_close_attn(dv[:, h], rv, f"dV head {h} (all keys)")
        else:
            # sampled query rows: O, LSE and dQ from the rows' own selected keys
            rows = rows_fn(h, T)
            for r in sorted({(rr // n) * nb + (rr % n) // wl.block for rr in rows}):
                a, b = orc.block_token_range(r, n, wl.block)
                toks = np.concatenate([np.arange(*orc.block_token_range(g, n, wl.block))
                                       for g in allowed[r]])
                m = np.ones((b - a, len(toks)), bool)
                ro, rl = orc.masked_attention(q[a:b, h], k[toks, h], v[toks, h], m, wl.scale)
                assert_close_attn(o[a:b, h], ro, f"O head {h} qblock {r}")
                assert np.abs(lse[h, a:b] - rl).max() < 1e-3
                rq, _, _ = orc.masked_attention_grad(q[a:b, h], k[toks, h], v[toks, h], m,
                                                     wl.scale, dout[a:b, h])
                assert_close_attn(dq[a:b, h], rq, f"dQ head {h} qblock {r}")
            # sampled KV blocks: dK/dV summed over every query block that selected them
            blocks = kv_blocks_fn(h, nqb)
            _, _, _, rk, rv = decomposed_reference(q[:, h], k[:, h], v[:, h], dout[:, h],
                                                   allowed, n, wl.block, wl.scale,
                                                   qblocks=[], kv_blocks=blocks)
            for g in blocks:
                users = sum(g in allowed[r] for r in range(nqb))
                a, b = orc.block_token_range(g, n, wl.block)
                assert_close_attn(dk[a:b, h], rk[a:b], f"dK head {h} block {g} ({users} users)")
                assert_close_attn(dv[a:b, h], rv[a:b], f"dV head {h} block {g} ({users} users)")
    return near_rows


def test_two_level_small_full_gradients():
    wl = synth.Workload("train_small", 2, 128, 64, 200, 2, 0, 0, 0, 0, 6, planted_per_segment=2,
                        segment_frames=8, q_align=1.0, kv_shift=3.0, clip_chunks=4,
                        top_frames=2)
    near = two_level_check(wl, 31)
    say(f"  near-tie rows: {near}")


def test_two_level_small_d64_full_gradients():
    wl = synth.Workload("train_small64", 2, 64, 64, 100, 2, 0, 0, 0, 0, 3, clip_chunks=3,
                        top_frames=1)
    two_level_check(wl, 32)


def test_two_level_small_ragged_second_half_full_gradients():
    # 100-token frames: one full block and a 36-token tail, so the tail's second 32-key
    # half tile holds 4 rows (head_dim 128, the gathered dQ path)
    wl = synth.Workload("train_small_r", 2, 128, 64, 100, 2, 0, 0, 0, 0, 3, clip_chunks=3,
                        top_frames=1)
    two_level_check(wl, 33)


def test_two_level_wan_train_sampled():
    wl = synth.WORKLOADS["wan_train"]

    def rows(h, T):
        rs = np.random.default_rng(40 + h)
        return rs.choice(T, 6, replace=False).tolist() + [T - 1, 1559]

    def kv_blocks(h, nqb):
        # a block of the last chunk's own frames and one of the newest history frame; on
        # heads 3 and 11 also blocks of frame 0 (forced for every chunk from the second on,
        # so selected by up to 525 query blocks: their dK/dV are summed from up to six work
        # items)
        return [nqb - 3, nqb - 75 - 2] + ([0, 1, 12, 24] if h in (3, 11) else [])

    # heads 0 and 7: every row and every key, one query block at a time
    near = two_level_check(wl, synth.SEEDS["wan_train"], grad_check="sampled", rows_fn=rows,
                           kv_blocks_fn=kv_blocks, whole_heads=(0, 7))
    say(f"  near-tie rows: {near}")


def test_two_level_long_clip_split_items_full_gradients():
    # 64-token frames (one block each), 4-frame chunks, 64 chunks: 256 query blocks, top-2
    # frames with frame 0 forced and budgets up to every candidate, so frame 0's block is
    # selected by more than 2 x 96 query blocks (three dK/dV work items and their fixed-order
    # reduce); every gradient of both heads compared
    wl = synth.Workload("train_long", 2, 128, 64, 64, 4, 0, 0, 0, 0, 64, clip_chunks=64,
                        top_frames=2)
    two_level_check(wl, 34, grad_check="decomposed")


def test_two_level_selection_long_clip_row_parallel():
    # 16 chunks of 3 frames of 1560 tokens: 1200 blocks a late chunk can see, more than the
    # matrix-core selection keeps in LDS for 32 query blocks, so the row-parallel selection
    # runs; every query block of both heads against the oracle
    wl = synth.Workload("train_wide", 2, 64, 64, 1560, 3, 0, 0, 0, 0, 48, clip_chunks=16,
                        top_frames=8)
    F, nb = wl.chunk_frames, wl.nb
    q, k, _ = synth.clip_qkv(wl, 36)
    ks = runtime.cag_budgets(synth.clip_alphas(wl, 36), wl.topk, wl.clip_chunks)
    clip = runtime.TwoLevelClip(shape_of(wl), wl.clip_chunks, wl.top_frames,
                                max(max(ks), F * nb))
    say("[two-level selection, 48 frames]")
    clip.select(dev(q), dev(k), ks)
    torch.cuda.synchronize()
    sel, nsel = clip.sel.cpu().numpy(), clip.nsel.cpu().numpy()
    ops.pbsa_check_selection_2lvl(shape_of(wl), wl.clip_chunks, sel, nsel)
    near, _ = check_two_level_selection(wl, q, k, clip, sel, nsel, ks)
    say(f"  near-tie rows: {near}")


def test_bwd_is_deterministic():
    wl = synth.Workload("det", 2, 128, 64, 200, 2, 0, 0, 0, 0, 6, clip_chunks=4, top_frames=2)
    shape = shape_of(wl)
    q, k, v = synth.clip_qkv(wl, 50)
    ks = runtime.cag_budgets(synth.clip_alphas(wl, 50), wl.topk, wl.clip_chunks)
    clip = runtime.TwoLevelClip(shape, wl.clip_chunks, wl.top_frames, max(max(ks), 8))
    qd, kd, vd = dev(q), dev(k), dev(v)
    dod = dev(synth.clip_dout(wl, 50, q.shape[0]))
    say("[determinism]")
    clip.select(qd, kd, ks)
    clip.forward(qd, kd, vd)
    outs = []
    for _ in range(2):
        clip.backward(qd, kd, vd, dod)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int16).clone() for t in (clip.dq, clip.dk, clip.dv)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_head_major_inputs_give_identical_training_results():
    """q, k, v and dO stored head-major ([H][T][d]: token stride d, head stride T*d) instead
    of token-major: forward and backward read them through other strides (the backward's
    row offsets and buffer extents scale with the token stride), so the outputs must be
    bit-identical."""
    wl = synth.Workload("layout", 2, 128, 64, 200, 2, 0, 0, 0, 0, 6, clip_chunks=4, top_frames=2)
    shape = shape_of(wl)
    q, k, v = synth.clip_qkv(wl, 51)
    ks = runtime.cag_budgets(synth.clip_alphas(wl, 51), wl.topk, wl.clip_chunks)
    clip = runtime.TwoLevelClip(shape, wl.clip_chunks, wl.top_frames, max(max(ks), 8))
    qd, kd, vd = dev(q), dev(k), dev(v)
    dod = dev(synth.clip_dout(wl, 51, q.shape[0]))
    head_major = lambda x: x.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    qh, kh, vh, doh = (head_major(x) for x in (qd, kd, vd, dod))
    assert qh.stride(0) == wl.head_dim and qh.stride(1) == q.shape[0] * wl.head_dim
    say("[layout] token-major vs head-major")
    clip.select(qd, kd, ks)
    outs = []
    for a, b, c, g in ((qd, kd, vd, dod), (qh, kh, vh, doh)):
        clip.forward(a, b, c)
        clip.backward(a, b, c, g)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int16).clone() for t in (clip.o, clip.dq, clip.dk, clip.dv)]
                    + [clip.lse.clone()])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_overlapped_step_equals_sequential_calls():
    """PersistentLayer.step(overlap=True) runs the memory selection (pbsa_memory_select,
    256 threads) on a second stream beside the attention and applies it after
    (pbsa_memory_apply); over a rollout its outputs and cache must be bit-identical to
    route, attention and pbsa_memory_update (1024-thread selection) in sequence."""
    wl = synth.WORKLOADS["wan_5s"]
    shape = shape_of(wl)
    seed = synth.SEEDS["wan_5s"]
    a, b = runtime.PersistentLayer(shape), runtime.PersistentLayer(shape)
    a.reset()
    b.reset()
    for c in range(wl.measured_chunk + 2):
        say(f"[overlap] chunk {c}")
        q, k, v = (dev(x) for x in synth.chunk_qkv(wl, seed, c))
        a.step(q, k, v, overlap=True)
        b.route(q)
        b.attend(q, k, v)
        b.update(k, v)
        torch.cuda.synchronize()
        assert a.cache.chunk_index == b.cache.chunk_index == c + 1
        assert torch.equal(a.o.view(torch.int16), b.o.view(torch.int16))
        assert torch.equal(a.lse, b.lse)
        for name in ("block_id", "len", "rep"):
            assert torch.equal(getattr(a.cache, name), getattr(b.cache, name)), name
        assert torch.equal(a.cache.k.view(torch.int16), b.cache.k.view(torch.int16))
        assert torch.equal(a.cache.v.view(torch.int16), b.cache.v.view(torch.int16))
