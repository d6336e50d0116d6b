"""The FP8 KV cache (PBSA_KV_FP8) against the fp64 oracle's reading of it.

Light Forcing (papernotes.org), "Key findings": the sparse attention deployed with FP8.
The cache keeps each block's K and V as OCP E4M3 codes with a power-of-two scale per block
and tensor.  Checked here: the attention's decode of every code against the format's
definition (bit for bit); rollouts whose persistent sets, routing, slot codes and scales
match the oracle's after every update (codes and scales bit for bit); and the attention at
the measured chunk against the oracle's attention over the decoded blocks (the stated
tolerance; the chunk's own K/V stay bf16).  The FP8-arithmetic attention (pbsa_attn_fwd_fp8)
is checked at the same chunk against the oracle's fp8_attention: element by element within
its bound on the rounding of the probabilities (plus bf16 output rounding), LSE within 1e-3.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
from block_sparse_attention_pbsa_amd import ops, runtime, synth
from parity import assert_close_attn, check_topk, say

pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)


def test_fp8_decode_matches_the_format():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] * 2, np.uint8)
    pad = (-len(codes)) % 16
    codes = np.concatenate([codes, np.zeros(pad, np.uint8)])
    n = len(codes)
    rs = np.random.default_rng(1)
    scales = (2.0 ** rs.integers(-12, 12, n // 16)).astype(np.float32)
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    ops.pbsa_probe_fp8_decode(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), out)
    torch.cuda.synchronize()
    ref = orc.e4m3_decode(codes) * np.repeat(scales.astype(np.float64), 16)
    want = synth.bf16_bits(ref.astype(np.float32)).view(np.int16)
    assert np.array_equal(synth.round_bf16(ref.astype(np.float32)).astype(np.float64), ref)
    assert np.array_equal(out.cpu().numpy(), want)


TINY128 = synth.Workload("tiny128", 1, 128, 64, 256, 1, 4, 2, 4, 1, 4)


def fp8_rollout(wl, seed, heads, rows, union=False, math8=False, slot_check_every=1):
    shape = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                      wl.capacity, wl.sinks, wl.topk, wl.scale,
                      route_mode=ops.PBSA_ROUTE_UNION if union else ops.PBSA_ROUTE_WINDOW,
                      kv_format=ops.PBSA_KV_FP8)
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale, union)
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    ros = {h: orc.PersistentRollout(sch, wl.head_dim, kv_fp8=True) for h in heads}
    last = wl.measured_chunk
    T = shape.chunk_tokens
    for c in range(last + 1):
        say(f"[fp8 {wl.name}] chunk {c}")
        q, k, v = synth.chunk_qkv(wl, seed, c)
        qd, kd, vd = dev(q), dev(k), dev(v)
        layer.route(qd)
        torch.cuda.synchronize()
        sel = layer.sel.cpu().numpy()
        routed = {}
        for h in heads:
            rt = ros[h].select(q[:, h])
            routed[h] = rt
            for r in range(shape.nq):
                got = [int(g) for g in sel[h, r] if g >= 0]
                check_topk(got, rt["cand"], rt["scores_cand"][r], wl.topk)
        if c == last:
            layer.attend(qd, kd, vd)
            torch.cuda.synchronize()
            for h in heads:
                gsel = [[int(g) for g in sel[h, r] if g >= 0] for r in range(shape.nq)]
                idx = np.arange(T) if rows is None else rows(h, T)
                o_ref, l_ref = ros[h].attend(q[:, h], k[:, h], v[:, h], gsel, rows=idx)
                o = layer.o[:, h].float().cpu().numpy()
                assert_close_attn(o[idx], o_ref[idx], f"O head {h}")
                assert np.abs(layer.lse[h].cpu().numpy()[idx] - l_ref[idx]).max() < 1e-3
            if math8:
                check_fp8_math(layer, ros, heads, rows, q, k, v, sel)
            return layer, ros
        layer.update(kd, vd)
        torch.cuda.synchronize()
        bid = layer.cache.block_id.cpu().numpy()
        kk, vv = layer.cache.k.cpu().numpy(), layer.cache.v.cpu().numpy()
        sc = layer.cache.kv_scale.cpu().numpy()
        ln = layer.cache.len.cpu().numpy()
        for h in heads:
            ro = ros[h]
            cand, m = ro.update_candidates(routed[h])
            gp = sorted(int(g) for g in bid[h, :wl.capacity] if g >= 0)
            exact, _ = check_topk([g for g in gp if g >= wl.sinks], cand, m,
                                  wl.capacity - wl.sinks)
            ro.update(routed[h], k[:, h], v[:, h], P_override=None if exact else gp)
            assert gp == ro.P
            if c % slot_check_every and c != last - 1:
                continue
            for s_ in range(shape.slots):
                g = int(bid[h, s_])
                if g < 0:
                    continue
                kc, ks, vc, vs = ro.fp8_codes[g]
                n_ = int(ln[h, s_])
                assert np.array_equal(kk[h, s_, :n_], kc), f"slot {s_} block {g}: K codes"
                assert np.array_equal(vv[h, s_, :n_], vc), f"slot {s_} block {g}: V codes"
                assert not kk[h, s_, n_:].any() and not vv[h, s_, n_:].any()
                assert sc[h, s_, 0] == ks and sc[h, s_, 1] == vs, f"slot {s_}: scales"
    raise AssertionError("unreachable")


def check_fp8_math(layer, ros, heads, rows, q, k, v, sel):
    """pbsa_attn_fwd_fp8 at the rollout's current chunk against the oracle's FP8 arithmetic."""
    shape = layer.shape
    T = shape.chunk_tokens
    ws = torch.empty(ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_FWD_FP8), dtype=torch.uint8,
                     device="cuda")
    o8 = torch.full_like(layer.o, float("nan"))
    l8 = torch.full_like(layer.lse, float("nan"))
    qd, kd, vd = dev(q), dev(k), dev(v)
    ops.pbsa_attn_fwd_fp8(shape, qd, layer.cache, kd, vd, layer.sel, o8, l8, ws)
    torch.cuda.synchronize()
    for h in heads:
        gsel = [[int(g) for g in sel[h, r] if g >= 0] for r in range(shape.nq)]
        idx = np.arange(T) if rows is None else rows(h, T)
        o_ref, l_ref, bnd = ros[h].attend_fp8(q[:, h], k[:, h], v[:, h], gsel, rows=idx)
        o = o8[:, h].float().cpu().numpy()[idx]
        err = np.abs(o - o_ref[idx])
        tol = bnd[idx] + 2.0 ** -8 * np.abs(o_ref[idx]) + 1e-4
        say(f"  fp8 arithmetic head {h}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}, "
            f"max err/tol {(err / tol).max():.3f}, mean bound {bnd[idx].mean():.3e}")
        assert np.isfinite(o).all()
        assert np.all(err <= tol), f"head {h}: FP8 O outside its bound"
        assert np.abs(l8[h].cpu().numpy()[idx] - l_ref[idx]).max() < 1e-3


def _sampled(seed):
    def pick(h, T):
        rs = np.random.default_rng(seed + h)
        fixed = list(range(0, 64)) + list(range(1536, 1560)) + list(range(T - 24, T))
        return np.array(sorted(set(fixed) | set(rs.choice(T, 64, replace=False).tolist())))
    return pick


def test_fp8_rollout_tiny128_all_rows():
    fp8_rollout(TINY128, 41, (0,), None)


def test_fp8_rollout_wan_5s():
    fp8_rollout(synth.WORKLOADS["wan_5s"], synth.SEEDS["wan_5s"], (0, 5, 11), _sampled(8))


def test_fp8_arithmetic_tiny128_all_rows():
    fp8_rollout(TINY128, 43, (0,), None, math8=True)


@pytest.mark.parametrize("history", [0, 1, 2])
def test_fp8_arithmetic_first_chunks(history):
    # an empty cache (only the chunk attends), then a cache holding only sinks and the window
    wl = dataclasses.replace(TINY128, name=f"tiny128_h{history}", history_frames=history)
    fp8_rollout(wl, 44 + history, (0,), None, math8=True)


def test_fp8_arithmetic_wan_5s():
    fp8_rollout(synth.WORKLOADS["wan_5s"], synth.SEEDS["wan_5s"], (1, 6), _sampled(10),
                math8=True)


def test_fp8_arithmetic_wan_5s_union_routing():
    # routed ids may name persistent blocks: the FP8 kernel's lookups of them
    wl = dataclasses.replace(synth.WORKLOADS["wan_5s"], name="wan_5s_union")
    fp8_rollout(wl, synth.SEEDS["wan_5s"], (4,), _sampled(11), union=True, math8=True)


def test_fp8_arithmetic_wan_1min():
    # the bench's workload: 240-frame history, capacity 256, top-64 routing
    fp8_rollout(synth.WORKLOADS["wan_1min"], synth.SEEDS["wan_1min"], (2,), _sampled(12),
                math8=True, slot_check_every=20)


def test_fp8_rollout_wan_5s_union_routing():
    wl = dataclasses.replace(synth.WORKLOADS["wan_5s"], name="wan_5s_union")
    fp8_rollout(wl, synth.SEEDS["wan_5s"], (2,), _sampled(9), union=True)


def test_fp8_cache_step_matches_bf16_routing_and_halves_bytes():
    # same seeded chunks through a bf16 and an FP8 cache: identical routing and persistent
    # sets (the representatives are the bf16 keys' means in both), half the K/V bytes
    wl = synth.WORKLOADS["wan_5s"]
    base = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                     wl.capacity, wl.sinks, wl.topk, wl.scale)
    a = runtime.PersistentLayer(base)
    b = runtime.PersistentLayer(dataclasses.replace(base, kv_format=ops.PBSA_KV_FP8))
    a.reset()
    b.reset()
    for c in range(wl.measured_chunk + 1):
        q, k, v = (dev(x) for x in synth.chunk_qkv(wl, synth.SEEDS["wan_5s"], c))
        a.step(q, k, v)
        b.step(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(a.sel, b.sel) and torch.equal(a.cache.block_id, b.cache.block_id)
        assert torch.equal(a.scores, b.scores)
    err = (a.o.float() - b.o.float()).abs()
    say(f"  fp8 vs bf16 cache: O max-abs {err.max().item():.3e} mean-abs {err.mean().item():.3e}")
    assert b.cache.k.element_size() * 2 == a.cache.k.element_size()
    assert ops.pbsa_cache_bytes(b.shape) < 0.53 * ops.pbsa_cache_bytes(a.shape)


def test_fp8_arithmetic_lists_at_capacity():
    """pbsa_attn_fwd_fp8 with its lists at the FP8 path's limit (C + K + chunk blocks = 1536)
    and each pair's routed sets disjoint, so that B's private list is as long as it can be;
    the cache holds random finite E4M3 codes with power-of-two scales per block and tensor.
    Sampled rows of three pairs against the oracle's fp8_attention within its bound."""
    H, D, n, nb = 1, 128, 2048, 32   # 32 full blocks per frame
    F, W = 8, 16                     # 256 chunk blocks; 512 window blocks
    C, S, K = 1024, 1, 256
    nq = F * nb
    assert C + K + nq == 1536
    shape = ops.Shape(H, D, n, F, W, C, S, K, kv_format=ops.PBSA_KV_FP8)
    rng = np.random.default_rng(1536)
    cache = ops.Cache(shape)
    chunk = 6                        # frames 48..55; the window holds frames 32..47
    f_last = chunk * F - 1
    bid = np.full((H, C + W * nb), -1, np.int32)
    bid[0, :S] = np.arange(S)
    bid[0, S:C] = np.sort(rng.choice(np.arange(S, (f_last - W + 1) * nb), C - S, replace=False))
    for f in range(f_last - W + 1, f_last + 1):
        for j in range(nb):
            bid[0, C + (f % W) * nb + j] = f * nb + j
    # codes with exponent fields 3..8 (magnitudes 2^-4 .. 3.75) and a random sign
    def codes(size):
        e = rng.integers(3, 9, size)
        m = rng.integers(0, 8, size)
        return ((rng.integers(0, 2, size) << 7) | (e << 3) | m).astype(np.uint8)
    kc, vc = codes((H, shape.slots, 64, D)), codes((H, shape.slots, 64, D))
    scales = np.ldexp(1.0, rng.integers(-2, 2, (H, shape.slots, 2))).astype(np.float32)
    cache.block_id.copy_(torch.from_numpy(bid))
    cache.len.copy_(torch.from_numpy(np.where(bid >= 0, 64, 0).astype(np.int32)))
    cache.k.copy_(torch.from_numpy(kc))
    cache.v.copy_(torch.from_numpy(vc))
    cache.kv_scale.copy_(torch.from_numpy(scales))
    cache.chunk_index = chunk
    win = np.sort(bid[0, C:])
    assert len(win) == 2 * K and win.min() >= 0
    sel_h = np.stack([win[:K] if r % 2 == 0 else win[K:] for r in range(nq)]).astype(np.int32)
    T = F * n
    q = synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
    k = synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
    v = synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
    ws = torch.empty(ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_FWD_FP8), dtype=torch.uint8,
                     device="cuda")
    o = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
    say(f"[fp8 arithmetic lists at capacity] C={C} chunk blocks={nq} K={K}")
    ops.pbsa_attn_fwd_fp8(shape, dev(q), cache, dev(k), dev(v), torch.from_numpy(sel_h[None]).cuda(),
                          o, lse, ws)
    torch.cuda.synchronize()
    og = o[:, 0].float().cpu().numpy()
    lg = lse[0].cpu().numpy()
    # the oracle's values: cache blocks decoded; the chunk's blocks quantized per block
    dec = lambda c, s_: orc.e4m3_decode(c) * float(s_)
    slot_of = {int(g): s for s, g in enumerate(bid[0])}
    own_k, own_v = [], []
    for b in range(nq):
        kq, ks = orc.e4m3_quantize_block(k[64 * b:64 * b + 64, 0])
        vq, vs = orc.e4m3_quantize_block(v[64 * b:64 * b + 64, 0])
        own_k.append(orc.e4m3_decode(kq) * ks)
        own_v.append(orc.e4m3_decode(vq) * vs)
    keys = {}
    for par in (0, 1):
        slots_ = list(range(C)) + [slot_of[int(g)] for g in sel_h[par]]
        keys[par] = (np.concatenate([dec(kc[0, s], scales[0, s, 0]) for s in slots_] + own_k),
                     np.concatenate([dec(vc[0, s], scales[0, s, 1]) for s in slots_] + own_v))
    rows = []
    for r in (0, 1, 128, 129, nq - 2, nq - 1):
        rows += sorted({64 * r, 64 * r + 63} | set((64 * r + rng.choice(64, 3, replace=False)).tolist()))
    worst = 0.0
    for t in rows:
        K_, V_ = keys[(t // 64) % 2]
        o_ref, l_ref, bnd = orc.fp8_attention(q[t:t + 1, 0].astype(np.float64), K_, V_,
                                              shape.c().scale)
        err = np.abs(og[t] - o_ref[0])
        tol = bnd[0] + 2.0 ** -8 * np.abs(o_ref[0]) + 1e-4
        worst = max(worst, float((err / tol).max()))
        assert np.isfinite(og[t]).all(), f"row {t}: non-finite output"
        assert np.all(err <= tol), f"row {t}: FP8 O outside its bound (max err/tol {(err / tol).max():.3f})"
        assert abs(lg[t] - l_ref[0]) < 1e-3, f"row {t}: LSE {lg[t]} vs {l_ref[0]}"
    say(f"  {len(rows)} rows at the FP8 list limit: max err/tol {worst:.3f}")
