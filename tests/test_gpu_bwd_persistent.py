"""Backward of the persistent-mode attention (pbsa_attn_bwd_persistent) against the fp64
oracle: Sparse Forcing trains with the same dynamic sparse cache it uses at inference
(English page, 2.D).

A rollout builds the cache to the measured chunk (its persistent sets checked against the
oracle's after every update, continuing from the GPU's choice inside near-ties); the chunk
is routed (the routing validated against the oracle) and attended, then the gradient of
O is taken for a seeded dO.  The oracle's gradient over its own stored blocks and the chunk
(PersistentRollout.attend_grad, i.e. masked_attention_grad on the gathered keys) is
compared element by element with dQ, the chunk's dK/dV and every cache slot's dK/dV
(mapped from slot to block through the cache's block ids; rows past a slot's length and
slots of blocks no query attends must be exactly zero).
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


def shape_of(wl, union=False):
    return ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                     wl.capacity, wl.sinks, wl.topk, wl.scale,
                     route_mode=ops.PBSA_ROUTE_UNION if union else ops.PBSA_ROUTE_WINDOW)


SMALL64 = synth.Workload("small64", 2, 64, 64, 100, 2, 8, 4, 3, 1, 3)
RAGGED128 = synth.Workload("ragged128", 3, 128, 64, 100, 2, 10, 4, 5, 1, 4)


def build(wl, seed, heads, union=False):
    shape = shape_of(wl, union)
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale, union)
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    ros = {h: orc.PersistentRollout(sch, wl.head_dim) for h in heads}
    for c in range(wl.measured_chunk):
        q, k, v = synth.chunk_qkv(wl, seed, c)
        layer.route(dev(q))
        routed = {h: ros[h].select(q[:, h]) for h in heads}
        layer.update(dev(k), dev(v))
        torch.cuda.synchronize()
        for h in heads:
            cand, m = ros[h].update_candidates(routed[h])
            gp = sorted(int(g) for g in layer.cache.block_id[h, :wl.capacity].cpu() if g >= 0)
            exact, _ = check_topk([g for g in gp if g >= wl.sinks], cand, m,
                                  wl.capacity - wl.sinks)
            ros[h].update(routed[h], k[:, h], v[:, h], P_override=None if exact else gp)
            assert gp == ros[h].P
    return shape, layer, ros


def run_bwd(shape, layer, qd, kd, vd, doutd):
    T, H, d = shape.chunk_tokens, shape.heads, shape.head_dim
    dq, dk, dv = (torch.empty(T, H, d, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    dkc, dvc = torch.empty_like(layer.cache.k), torch.empty_like(layer.cache.v)
    # stale values that a missing write would leave behind
    for t in (dq, dk, dv, dkc, dvc):
        t.fill_(7.0)
    ws = torch.empty(ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_BWD_PERSISTENT),
                     dtype=torch.uint8, device="cuda")
    ops.pbsa_attn_bwd_persistent(shape, qd, layer.cache, kd, vd, layer.sel, layer.o, layer.lse,
                                 doutd, dq, dk, dv, dkc, dvc, ws)
    return dq, dk, dv, dkc, dvc


@pytest.mark.parametrize("name,heads,union", [
    ("tiny", (0,), False), ("small64", (0, 1), False), ("ragged128", (0, 2), False),
    ("wan_5s", (4,), False), ("small64", (0, 1), True), ("ragged128", (1,), True),
    ("wan_5s", (9,), True)])
def test_persistent_backward_parity(name, heads, union):
    wl = {"small64": SMALL64, "ragged128": RAGGED128}.get(name) or synth.WORKLOADS[name]
    seed = synth.SEEDS.get(name, 77)
    say(f"[bwd persistent] {name} union={union}")
    shape, layer, ros = build(wl, seed, heads, union)
    q, k, v = synth.chunk_qkv(wl, seed, wl.measured_chunk)
    dout = synth.clip_dout(wl, seed, q.shape[0])
    qd, kd, vd, doutd = dev(q), dev(k), dev(v), dev(dout)
    layer.route(qd)
    layer.attend(qd, kd, vd)
    dq, dk, dv, dkc, dvc = run_bwd(shape, layer, qd, kd, vd, doutd)
    torch.cuda.synchronize()
    sel = layer.sel.cpu().numpy()
    bid = layer.cache.block_id.cpu().numpy()
    ln = layer.cache.len.cpu().numpy()
    for h in heads:
        rt = ros[h].select(q[:, h])
        for r in range(shape.nq):
            got = [int(g) for g in sel[h, r] if g >= 0]
            check_topk(got, rt["cand"], rt["scores_cand"][r], wl.topk)
        gsel = [[int(g) for g in sel[h, r] if g >= 0] for r in range(shape.nq)]
        rdq, rdk, rdv, rdkb, rdvb = ros[h].attend_grad(q[:, h], k[:, h], v[:, h], gsel, dout[:, h])
        assert_close_attn(dq[:, h].float().cpu().numpy(), rdq, f"dQ head {h}")
        assert_close_attn(dk[:, h].float().cpu().numpy(), rdk, f"chunk dK head {h}")
        assert_close_attn(dv[:, h].float().cpu().numpy(), rdv, f"chunk dV head {h}")
        gk = dkc[h].float().cpu().numpy()
        gv = dvc[h].float().cpu().numpy()
        got_k, got_v, ref_k, ref_v = [], [], [], []
        seen = set()
        for s in range(shape.slots):
            g = int(bid[h, s])
            if g < 0:
                assert not gk[s].any() and not gv[s].any(), f"empty slot {s} has a gradient"
                continue
            seen.add(g)
            n_ = int(ln[h, s])
            assert not gk[s, n_:].any() and not gv[s, n_:].any(), f"slot {s}: rows past len"
            got_k.append(gk[s, :n_])
            got_v.append(gv[s, :n_])
            ref_k.append(rdkb[g])
            ref_v.append(rdvb[g])
        assert seen == set(rdkb), "the cache holds other blocks than the oracle stores"
        assert_close_attn(np.concatenate(got_k), np.concatenate(ref_k), f"cache dK head {h}")
        assert_close_attn(np.concatenate(got_v), np.concatenate(ref_v), f"cache dV head {h}")
    # the same call again gives the same bits
    again = run_bwd(shape, layer, qd, kd, vd, doutd)
    torch.cuda.synchronize()
    for nm, x, y in zip(("dq", "dk", "dv", "dk_cache", "dv_cache"), (dq, dk, dv, dkc, dvc), again):
        diff = (x.view(torch.int16) != y.view(torch.int16))
        assert not diff.any(), f"{nm}: {int(diff.sum())} values differ between two calls"


def test_persistent_backward_lists_at_limit():
    """The persistent-mode backward with its per-query-block list at the boundary's limit
    (C + K + chunk blocks = 1536: the dQ pass's list full), each pair's routed sets
    disjoint and 128 window blocks routed to no query block.  dQ of sampled rows of three
    pairs against the fp64 definition; the unattended window slots' dK/dV exactly zero."""
    H, D, n, nb = 1, 128, 2048, 32
    F, W = 8, 20                     # 256 chunk blocks; 640 window blocks
    C, S, K = 1024, 1, 256
    nq = F * nb
    assert C + K + nq == 1536
    shape = ops.Shape(H, D, n, F, W, C, S, K)
    rng = np.random.default_rng(1536 * 3)
    cache = ops.Cache(shape)
    chunk = 7                        # frames 56..63; the window holds frames 36..55
    f_last = chunk * F - 1
    bid = np.full((H, C + W * nb), -1, np.int32)
    bid[0, :S] = np.arange(S)
    bid[0, S:C] = np.sort(rng.choice(np.arange(S, (f_last - W + 1) * nb), C - S, replace=False))
    for f in range(f_last - W + 1, f_last + 1):
        for j in range(nb):
            bid[0, C + (f % W) * nb + j] = f * nb + j
    kc = synth.round_bf16(rng.standard_normal((H, shape.slots, 64, D)).astype(np.float32))
    vc = synth.round_bf16(rng.standard_normal((H, shape.slots, 64, D)).astype(np.float32))
    cache.block_id.copy_(torch.from_numpy(bid))
    cache.len.copy_(torch.from_numpy(np.where(bid >= 0, 64, 0).astype(np.int32)))
    cache.k.copy_(torch.from_numpy(kc).to(torch.bfloat16))
    cache.v.copy_(torch.from_numpy(vc).to(torch.bfloat16))
    cache.chunk_index = chunk
    win = np.sort(bid[0, C:])
    sel_h = np.stack([win[:K] if r % 2 == 0 else win[K:2 * K] for r in range(nq)]).astype(np.int32)
    T = F * n
    q, k, v, do = (synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
                   for _ in range(4))
    sel = torch.from_numpy(sel_h[None]).cuda()
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o = torch.empty_like(qd)
    lse = torch.empty(H, T, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
    dkc = torch.full_like(cache.k, float("nan"))
    dvc = torch.full_like(cache.v, float("nan"))
    ws = torch.empty(ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_BWD_PERSISTENT),
                     dtype=torch.uint8, device="cuda")
    say(f"[persistent backward at the list limit] C={C} K={K} chunk blocks={nq}")
    ops.pbsa_attn_fwd(shape, qd, cache, kd, vd, sel, o, lse)
    ops.pbsa_attn_bwd_persistent(shape, qd, cache, kd, vd, sel, o, lse, dod, dq, dk, dv, dkc,
                                 dvc, ws)
    torch.cuda.synchronize()
    dqg = dq[:, 0].float().cpu().numpy()
    slot_of = {int(g): s for s, g in enumerate(bid[0])}
    q0, k0, v0, do0 = (x[:, 0].astype(np.float64) for x in (q, k, v, do))
    keys = {}
    for par in (0, 1):
        slots_ = list(range(C)) + [slot_of[int(g)] for g in sel_h[par]]
        keys[par] = (np.concatenate([kc[0, s] for s in slots_] + [k0]).astype(np.float64),
                     np.concatenate([vc[0, s] for s in slots_] + [v0]).astype(np.float64))
    rows = []
    for r in (0, 1, 128, 129, nq - 2, nq - 1):
        rows += sorted({64 * r, 64 * r + 63} | set((64 * r + rng.choice(64, 2, replace=False)).tolist()))
    got, ref = [], []
    for t in rows:
        K_, V_ = keys[(t // 64) % 2]
        dq_ref, _, _ = orc.masked_attention_grad(q0[t:t + 1], K_, V_, np.ones((1, len(K_)), bool),
                                                 shape.c().scale, do0[t:t + 1])
        got.append(dqg[t])
        ref.append(dq_ref[0])
    assert_close_attn(np.array(got), np.array(ref), f"dQ of {len(rows)} rows at the list limit")
    unused = [slot_of[int(g)] for g in win[2 * K:]]
    assert len(unused) == 128
    dkz = dkc[0, unused].float().cpu().numpy()
    dvz = dvc[0, unused].float().cpu().numpy()
    assert not dkz.any() and not dvz.any(), "unattended window slots must have zero dK/dV"
