"""Routing and memory-update selections at sizes that take the wide register paths of the
wave top-K (window of 600 blocks: 16 keys per lane; 1047 memory candidates: 32 keys per
lane), on synthetic cache states built directly, checked against the fp64 oracle.

Selections must match exactly wherever the exact score gap at the selection boundary
exceeds 1e-5 (near ties: any correct set); exact ties must go to the lower id."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_sparse_attention_pbsa_amd import ops, synth
from parity import assert_close_attn, check_topk, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


N_TOK, NB = 1600, 25  # 25 blocks per frame


def _window_state(shape, f_last, rng, drop=0.05):
    """block_id [H][slots] for a window holding frames (f_last - W, f_last] in their ring
    slots, a few slots empty, and P slots [0, C) holding the sinks and older ids."""
    H, C, S, W = shape.heads, shape.capacity, shape.sinks, shape.window_frames
    bid = np.full((H, C + W * NB), -1, np.int32)
    for h in range(H):
        old = rng.choice(np.arange(S, (f_last - W + 1) * NB), C - S, replace=False)
        bid[h, :S] = np.arange(S)
        bid[h, S:C] = np.sort(old)
        for f in range(f_last - W + 1, f_last + 1):
            for j in range(NB):
                if rng.random() >= drop:
                    bid[h, C + (f % W) * NB + j] = f * NB + j
    return bid


@pytest.mark.parametrize("topk,tie_all", [(1, False), (100, False), (600, False), (37, True)])
def test_score_topk_600_window_blocks(topk, tie_all):
    H, D = 2, 128
    shape = ops.Shape(H, D, N_TOK, 1, 24, 64, 1, topk)
    rng = np.random.default_rng(600 + topk)
    cache = ops.Cache(shape)
    bid = _window_state(shape, f_last=60, rng=rng)
    rep = rng.standard_normal((H, shape.slots, D)).astype(np.float32)
    if tie_all:
        rep[:, shape.capacity:] = rep[:, shape.capacity:shape.capacity + 1]  # one row for all
    else:
        # a few exact duplicates, so some scores tie bit for bit
        for h in range(H):
            src = rng.choice(np.arange(shape.capacity, shape.slots), 40)
            dst = rng.choice(np.arange(shape.capacity, shape.slots), 40)
            rep[h, dst] = rep[h, src]
    cache.block_id.copy_(torch.from_numpy(bid))
    cache.len.copy_(torch.from_numpy(np.where(bid >= 0, 64, 0).astype(np.int32)))
    cache.rep.copy_(torch.from_numpy(rep))
    q_rep = torch.from_numpy(rng.standard_normal((H, shape.nq, D)).astype(np.float32)).cuda()
    scores = torch.empty(H, shape.nq, shape.slots, dtype=torch.float32, device="cuda")
    sel = torch.full((H, shape.nq, topk), -7, dtype=torch.int32, device="cuda")
    say(f"[score_topk wide] K={topk} ties={tie_all}")
    ops.pbsa_score_topk(shape, q_rep, cache, scores, sel)
    torch.cuda.synchronize()
    sc, sl, qr = scores.cpu().numpy(), sel.cpu().numpy(), q_rep.cpu().numpy()
    for h in range(H):
        occ = np.nonzero(bid[h] >= 0)[0]
        exact = orc.coarse_scores(qr[h].astype(np.float64), rep[h, occ].astype(np.float64),
                                  shape.c().scale)
        assert np.abs(sc[h][:, occ] - exact).max() < 1e-5
        assert np.all(np.isneginf(sc[h][:, bid[h] < 0]))
        win = [s for s in occ if s >= shape.capacity]
        ids = bid[h, win]
        for r in range(shape.nq):
            got = [int(g) for g in sl[h, r] if g >= 0]
            assert all(g == -1 for g in sl[h, r, len(got):])
            ws = exact[r, [list(occ).index(s) for s in win]]
            check_topk(got, ids, ws, topk)
            if tie_all:
                assert got == sorted(ids)[:topk]


def test_memory_update_1047_candidates():
    H, D, C, S, W = 2, 128, 1024, 2, 4
    shape = ops.Shape(H, D, N_TOK, 1, W, C, S, 8)
    rng = np.random.default_rng(1047)
    chunk = 50                       # appending frame 50 pushes frame 46 out of the window
    cache = ops.Cache(shape)
    bid = _window_state(shape, f_last=chunk - 1, rng=rng, drop=0.0)
    ln = np.where(bid >= 0, 64, 0).astype(np.int32)
    kbits = rng.integers(0, 1 << 15, (H, shape.slots, 64, D), dtype=np.int16)
    vbits = rng.integers(0, 1 << 15, (H, shape.slots, 64, D), dtype=np.int16)
    rep = rng.standard_normal((H, shape.slots, D)).astype(np.float32)
    cache.block_id.copy_(torch.from_numpy(bid))
    cache.len.copy_(torch.from_numpy(ln))
    cache.k.view(torch.int16).copy_(torch.from_numpy(kbits))
    cache.v.view(torch.int16).copy_(torch.from_numpy(vbits))
    cache.rep.copy_(torch.from_numpy(rep))
    cache.chunk_index = chunk
    scores = rng.standard_normal((H, shape.nq, shape.slots)).astype(np.float32)
    kc = synth.round_bf16(rng.standard_normal((N_TOK, H, D)).astype(np.float32))
    vc = synth.round_bf16(rng.standard_normal((N_TOK, H, D)).astype(np.float32))
    ws = torch.empty(max(ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_MEMORY_UPDATE), 16),
                     dtype=torch.uint8, device="cuda")
    say("[memory_update wide] C=1024")
    ops.pbsa_memory_update(shape, torch.from_numpy(scores).cuda(), cache,
                           torch.from_numpy(kc).cuda().to(torch.bfloat16),
                           torch.from_numpy(vc).cuda().to(torch.bfloat16), None, ws)
    torch.cuda.synchronize()
    assert cache.chunk_index == chunk + 1
    nb2 = cache.block_id.cpu().numpy()
    k2 = cache.k.view(torch.int16).cpu().numpy()
    leave = [C + ((chunk - W) % W) * NB + j for j in range(NB)]  # ring slots of frame 46
    for h in range(H):
        P = [int(g) for g in bid[h, :C] if g >= 0]
        cols_P = [s for s in range(C) if bid[h, s] >= 0]
        ev = [int(bid[h, s]) for s in leave]
        cand, msum = orc.memory_scores(P, list(range(S)), scores[h][:, cols_P].astype(np.float64),
                                       ev, scores[h][:, leave].astype(np.float64))
        newP = sorted(int(g) for g in nb2[h, :C] if g >= 0)
        assert newP[:S] == list(range(S))
        check_topk(newP[S:], cand, msum, C - S)
        # promoted blocks carry their K bytes from the window slot they left
        slot_of = {int(g): s for s, g in enumerate(bid[h])}
        for s in range(C):
            g = int(nb2[h, s])
            if g >= 0 and slot_of.get(g, -1) != s:
                assert np.array_equal(k2[h, s], kbits[h, slot_of[g]])
        # the chunk's blocks now sit in the freed window slots
        for j, s in enumerate(leave):
            assert nb2[h, s] == chunk * NB + j
            ref = synth.bf16_bits(kc[64 * j:64 * j + 64, h]).view(np.int16)
            assert np.array_equal(k2[h, s], ref)


@pytest.mark.parametrize("topk", [300, 600])
def test_attn_fwd_long_routed_lists(topk):
    """Attention over P_t, top-300/600 routed window blocks and the chunk: the split of each
    query-block pair's routed sets (shared / A only / B only) runs over several 256-id
    rounds.  Sampled rows against the fp64 definition on the GPU's own routing."""
    H, D, n = 1, 128, 1560          # 24 full blocks + a 24-row tail per frame
    shape = ops.Shape(H, D, n, 1, 24, 64, 1, topk)
    rng = np.random.default_rng(7000 + topk)
    cache = ops.Cache(shape)
    bid = _window_state(shape, f_last=60, rng=rng)
    blen = np.where(bid >= 0, np.where(bid % NB == NB - 1, n - 64 * (NB - 1), 64), 0)
    kc = synth.round_bf16(rng.standard_normal((H, shape.slots, 64, D)).astype(np.float32))
    vc = synth.round_bf16(rng.standard_normal((H, shape.slots, 64, D)).astype(np.float32))
    for h in range(H):
        for s in range(shape.slots):
            kc[h, s, blen[h, s]:] = 0
            vc[h, s, blen[h, s]:] = 0
    rep = np.stack([kc[h].mean(axis=1) for h in range(H)]).astype(np.float32)
    cache.block_id.copy_(torch.from_numpy(bid))
    cache.len.copy_(torch.from_numpy(blen.astype(np.int32)))
    cache.k.copy_(torch.from_numpy(kc).to(torch.bfloat16))
    cache.v.copy_(torch.from_numpy(vc).to(torch.bfloat16))
    cache.rep.copy_(torch.from_numpy(rep))
    cache.chunk_index = 61
    q = synth.round_bf16(rng.standard_normal((n, H, D)).astype(np.float32))
    k = synth.round_bf16(rng.standard_normal((n, H, D)).astype(np.float32))
    v = synth.round_bf16(rng.standard_normal((n, H, D)).astype(np.float32))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    scores = torch.empty(H, shape.nq, shape.slots, dtype=torch.float32, device="cuda")
    sel = torch.empty(H, shape.nq, topk, dtype=torch.int32, device="cuda")
    o = torch.empty(n, H, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(H, n, dtype=torch.float32, device="cuda")
    say(f"[attn long lists] K={topk}")
    ops.pbsa_route(shape, dev(q), cache, None, scores, sel)
    ops.pbsa_attn_fwd(shape, dev(q), cache, dev(k), dev(v), sel, o, lse)
    torch.cuda.synchronize()
    sl = sel.cpu().numpy()
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    scale = shape.c().scale
    rows = sorted(set(rng.choice(n, 96, replace=False).tolist()) | {0, 63, 64, n - 1})
    slot_of = {int(g): s for s, g in enumerate(bid[0])}
    P = [s for s in range(shape.capacity) if bid[0, s] >= 0]
    got_o, ref_o = [], []
    for t in rows:
        r = t // 64
        picked = [slot_of[int(g)] for g in sl[0, r] if g >= 0]
        assert len(picked) == min(topk, int((bid[0, shape.capacity:] >= 0).sum()))
        kk = [kc[0, s, :blen[0, s]] for s in P + picked] + [k[:, 0]]
        vv = [vc[0, s, :blen[0, s]] for s in P + picked] + [v[:, 0]]
        K = np.concatenate(kk).astype(np.float64)
        V = np.concatenate(vv).astype(np.float64)
        o_ref, lse_ref = orc.masked_attention(q[t:t + 1, 0].astype(np.float64), K, V,
                                              np.ones((1, len(K)), bool), scale)
        got_o.append(og[t, 0])
        ref_o.append(o_ref[0])
        assert abs(lg[0, t] - lse_ref[0]) < 1e-3
    assert_close_attn(np.array(got_o), np.array(ref_o), f"O of {len(rows)} rows, K={topk}")


def test_attn_fwd_lists_at_capacity():
    """The attention's per-workgroup lists filled to their capacity: C + chunk blocks + 2 K =
    3072 entries (the most the boundary accepts, with C - sinks, the window and the chunk at
    their own limits), each pair's routed sets disjoint, so that B's private list runs to the
    last entry and every private step past it reads the empty entry kept after the lists.
    Sampled rows of both query blocks of several pairs against the fp64 definition."""
    H, D, n, nb = 1, 128, 2048, 32   # 32 full blocks per frame
    F = W = 32                       # a 32-frame chunk (1024 blocks); 1024 window blocks
    C, S, K = 1024, 1, 512           # two disjoint top-512 sets fill the window
    nq = F * nb
    assert C + nq + 2 * K == 3072
    shape = ops.Shape(H, D, n, F, W, C, S, K)
    rng = np.random.default_rng(3072)
    cache = ops.Cache(shape)
    chunk = 3                        # frames 96..127; the window holds frames 64..95
    f_last = chunk * F - 1
    bid = np.full((H, C + W * nb), -1, np.int32)
    bid[0, :S] = np.arange(S)
    bid[0, S:C] = np.sort(rng.choice(np.arange(S, (f_last - W + 1) * nb), C - S, replace=False))
    for f in range(f_last - W + 1, f_last + 1):
        for j in range(nb):
            bid[0, C + (f % W) * nb + j] = f * nb + j
    blen = np.where(bid >= 0, 64, 0).astype(np.int32)
    kc = synth.round_bf16(rng.standard_normal((H, shape.slots, 64, D)).astype(np.float32))
    vc = synth.round_bf16(rng.standard_normal((H, shape.slots, 64, D)).astype(np.float32))
    cache.block_id.copy_(torch.from_numpy(bid))
    cache.len.copy_(torch.from_numpy(blen))
    cache.k.copy_(torch.from_numpy(kc).to(torch.bfloat16))
    cache.v.copy_(torch.from_numpy(vc).to(torch.bfloat16))
    cache.chunk_index = chunk
    win = np.sort(bid[0, C:])
    assert len(win) == 2 * K and win.min() >= 0
    # even query blocks take the older half of the window, odd ones the newer half
    sel_h = np.stack([win[:K] if r % 2 == 0 else win[K:] for r in range(nq)]).astype(np.int32)
    T = F * n
    q = synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
    k = synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
    v = synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    sel = torch.from_numpy(sel_h[None]).cuda()
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(H, T, dtype=torch.float32, device="cuda")
    say(f"[attn lists at capacity] C={C} chunk blocks={nq} K={K}: {C + nq + 2 * K} list entries")
    ops.pbsa_attn_fwd(shape, dev(q), cache, dev(k), dev(v), sel, o, lse)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    scale = shape.c().scale
    slot_of = {int(g): s for s, g in enumerate(bid[0])}
    P = [s for s in range(C) if bid[0, s] >= 0]
    # the keys of an even and of an odd query block: P, its routed blocks, the whole chunk
    keys = {}
    for par in (0, 1):
        picked = [slot_of[int(g)] for g in sel_h[par]]
        keys[par] = tuple(np.concatenate([x[0, s] for s in P + picked] + [y[:, 0]])
                          .astype(np.float64) for x, y in ((kc, k), (vc, v)))
    # query blocks 0/1 (the first pair), 510/511 and the last pair; rows at both ends of
    # each block and three inside
    rows = []
    for r in (0, 1, 510, 511, nq - 2, nq - 1):
        rows += sorted({64 * r, 64 * r + 63} | set((64 * r + rng.choice(64, 3, replace=False)).tolist()))
    got_o, ref_o = [], []
    for t in rows:
        K_, V_ = keys[(t // 64) % 2]
        o_ref, lse_ref = orc.masked_attention(q[t:t + 1, 0].astype(np.float64), K_, V_,
                                              np.ones((1, len(K_)), bool), scale)
        got_o.append(og[t, 0])
        ref_o.append(o_ref[0])
        assert abs(lg[0, t] - lse_ref[0]) < 1e-3, f"row {t}: LSE {lg[0, t]} vs {lse_ref[0]}"
    assert_close_attn(np.array(got_o), np.array(ref_o), f"O of {len(rows)} rows at the list capacity")


def test_two_level_lists_at_capacity():
    """Two-level attention and its backward with the largest selections the boundary accepts
    (max_sel = 1536, so a query-block pair's lists fill the 3072-entry capacity, and the dQ
    pass's per-block list is full): the last chunk's query blocks take 1536 earlier blocks
    each, the two blocks of a pair disjoint sets; every other query block takes its own
    block only.  Sampled rows of O, LSE and dQ, and dK/dV of one block with 17 users,
    against the fp64 definition."""
    H, D, n, nb, M = 1, 128, 2048, 32, 1536
    chunks = 97                      # one frame per chunk; the last sees frames 0..96
    shape = ops.Shape(H, D, n, 1, 1, 1, 1, 1)
    nq, T = chunks * nb, chunks * n
    last = range(nq - nb, nq)        # the last chunk's query blocks
    sel_h = np.full((H, nq, M), -1, np.int32)
    nsel_h = np.ones((H, nq), np.int32)
    for r in range(nq):
        if r in last:
            sel_h[0, r] = np.arange(M) if r % 2 == 0 else np.arange(M, 2 * M)
            nsel_h[0, r] = M
        else:
            sel_h[0, r, 0] = r
    rng = np.random.default_rng(1536 * 2)
    q, k, v, do = (synth.round_bf16(rng.standard_normal((T, H, D)).astype(np.float32))
                   for _ in range(4))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    sel, nsel = torch.from_numpy(sel_h).cuda(), torch.from_numpy(nsel_h).cuda()
    o = torch.empty_like(qd)
    lse = torch.empty(H, T, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
    ws = torch.empty(ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_BWD, chunks, M),
                     dtype=torch.uint8, device="cuda")
    say(f"[two-level lists at capacity] {chunks} chunks, max_sel {M}: forward and backward")
    ops.pbsa_attn_fwd_2lvl(shape, chunks, qd, kd, vd, sel, nsel, o, lse)
    ops.pbsa_attn_bwd(shape, chunks, qd, kd, vd, o, lse, dod, sel, nsel, dq, dk, dv, ws)
    torch.cuda.synchronize()
    og, lg = o[:, 0].float().cpu().numpy(), lse[0].cpu().numpy()
    dqg, dkg, dvg = (x[:, 0].float().cpu().numpy() for x in (dq, dk, dv))
    del ws
    scale = shape.c().scale
    tok = lambda blocks: np.concatenate([np.arange(64 * g, 64 * g + 64) for g in blocks])
    keys_of = {0: tok(range(M)), 1: tok(range(M, 2 * M))}
    q0, k0, v0, do0 = (x[:, 0].astype(np.float64) for x in (q, k, v, do))
    # rows of both halves of two pairs of the last chunk, and of two own-block-only blocks
    rows = []
    for r in (nq - nb, nq - nb + 1, nq - 2, nq - 1, 5, 2000):
        rows += sorted({64 * r, 64 * r + 63} | set((64 * r + rng.choice(64, 2, replace=False)).tolist()))
    got, ref, gq, rq = [], [], [], []
    for t in rows:
        r = t // 64
        kk = keys_of[r % 2] if r in last else tok([r])
        mask = np.ones((1, len(kk)), bool)
        o_ref, l_ref = orc.masked_attention(q0[t:t + 1], k0[kk], v0[kk], mask, scale)
        dq_ref, _, _ = orc.masked_attention_grad(q0[t:t + 1], k0[kk], v0[kk], mask, scale,
                                                 do0[t:t + 1])
        got.append(og[t]); ref.append(o_ref[0]); gq.append(dqg[t]); rq.append(dq_ref[0])
        assert abs(lg[t] - l_ref[0]) < 1e-3, f"row {t}: LSE {lg[t]} vs {l_ref[0]}"
    assert_close_attn(np.array(got), np.array(ref), f"O of {len(rows)} rows, max_sel {M}")
    assert_close_attn(np.array(gq), np.array(rq), f"dQ of {len(rows)} rows, max_sel {M}")
    # dK, dV of block 5: the 16 even query blocks of the last chunk and block 5 itself
    g = 5
    users = tok([r for r in last if r % 2 == 0])
    kk = keys_of[0]
    _, rk_a, rv_a = orc.masked_attention_grad(q0[users], k0[kk], v0[kk],
                                              np.ones((len(users), len(kk)), bool), scale,
                                              do0[users])
    own = tok([g])
    _, rk_s, rv_s = orc.masked_attention_grad(q0[own], k0[own], v0[own],
                                              np.ones((64, 64), bool), scale, do0[own])
    rk = rk_a[64 * g:64 * g + 64] + rk_s
    rv = rv_a[64 * g:64 * g + 64] + rv_s
    assert_close_attn(dkg[own], rk, f"dK of block {g} (17 users)")
    assert_close_attn(dvg[own], rv, f"dV of block {g} (17 users)")
