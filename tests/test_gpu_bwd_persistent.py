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
