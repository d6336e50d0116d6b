"""Pins of the fp64 oracle to facts it does not itself define.

Each check compares the oracle with something independent of its own formulas: exact
rational means, closed forms, brute force over all subsets, a library attention routine
(torch's scaled_dot_product_attention and autograd in float64), finite differences,
hand-derived fixtures under tests/golden/, and invariants the pages state.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
from block_sparse_attention_pbsa_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- pooling
def test_pool_exact_rational_means_with_ragged_tail():
    # integer tokens: exact means computed with Fractions, token by token
    n, B, d = 100, 32, 3   # blocks of 32, 32, 32 and a 4-token tail
    rs = np.random.default_rng(0)
    x = rs.integers(-50, 50, size=(2 * n, d))
    br, fr = orc.mean_pool(x, n, B)
    starts = [0, 32, 64, 96]
    ends = [32, 64, 96, 100]
    for f in range(2):
        for j in range(4):
            for c in range(d):
                toks = [Fraction(int(x[f * n + t, c])) for t in range(starts[j], ends[j])]
                assert Fraction(br[f * 4 + j, c]).limit_denominator(1000) == sum(toks) / len(toks)
        for c in range(d):
            exact = sum(Fraction(int(x[f * n + t, c])) for t in range(n)) / n
            assert Fraction(fr[f, c]).limit_denominator(1000) == exact


def test_frame_rep_is_token_mean_not_mean_of_block_reps():
    # 1560-token frame: 24 full blocks of value a, a 24-token tail of value b
    n, B = 1560, 64
    a, b = 1.0, 5.0
    x = np.full((n, 1), a)
    x[24 * 64:] = b
    br, fr = orc.mean_pool(x, n, B)
    assert br.shape == (25, 1)
    assert br[24, 0] == b and br[0, 0] == a
    assert fr[0, 0] == pytest.approx((1536 * a + 24 * b) / 1560, abs=1e-15)
    assert br[:, 0].mean() == pytest.approx(29 / 25) and abs(fr[0, 0] - 29 / 25) > 0.09


def test_pool_block_table_matches_hand_tiling():
    assert orc.blocks_per_frame(1560, 64) == 25
    assert orc.frame_block_ranges(1560, 64)[-1] == (1536, 1560)
    assert orc.block_token_range(25, 1560, 64) == (1560, 1624)      # frame 1, block 0
    assert orc.block_token_range(49, 1560, 64) == (1560 + 1536, 3120)  # frame 1 tail


# ----------------------------------------------------------------------------- scores / top-k
def test_coarse_scores_orthonormal_closed_form():
    e = np.eye(4)
    S = orc.coarse_scores(e, e[::-1], 0.5)
    assert np.array_equal(S, 0.5 * np.eye(4)[::-1])


@pytest.mark.parametrize("seed", range(20))
def test_top_ids_brute_force_over_subsets(seed):
    rs = np.random.default_rng(seed)
    m = int(rs.integers(1, 9))
    k = int(rs.integers(0, m + 2))
    vals = rs.integers(-3, 4, size=m).astype(float)   # many exact ties
    ids = rs.permutation(100)[:m]
    got = orc.top_ids(vals, ids, k)
    kk = min(k, m)

    def beats(i, j):   # i strictly ahead of j in (value desc, id asc)
        return vals[i] > vals[j] or (vals[i] == vals[j] and ids[i] < ids[j])

    winners = [set(ids[list(c)]) for c in itertools.combinations(range(m), kk)
               if all(beats(i, j) for i in c for j in range(m) if j not in c)]
    assert len(winners) == 1
    assert got == sorted(winners[0])


def test_top_ids_ties_go_to_lower_id():
    assert orc.top_ids([1.0] * 6, [9, 3, 7, 1, 5, 8], 3) == [1, 3, 5]
    assert orc.top_ids([2.0, 1.0, 2.0], [4, 0, 2], 1) == [2]


# ----------------------------------------------------------------------------- attention
def _sdpa64(q, k, v, mask, scale):
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None],
        attn_mask=torch.tensor(mask)[None], scale=scale)
    return o[0].numpy()


@pytest.mark.parametrize("seed", range(4))
def test_masked_attention_matches_library_sdpa(seed):
    rs = np.random.default_rng(seed)
    Tq, Tk, d = 37, 91, 16
    q, k, v = rs.standard_normal((Tq, d)), rs.standard_normal((Tk, d)), rs.standard_normal((Tk, d))
    mask = rs.random((Tq, Tk)) < 0.3
    mask[np.arange(Tq), rs.integers(0, Tk, Tq)] = True
    o, lse = orc.masked_attention(q, k, v, mask, 0.25)
    np.testing.assert_allclose(o, _sdpa64(q, k, v, mask, 0.25), atol=1e-12, rtol=0)
    from scipy.special import logsumexp
    ref_lse = np.array([logsumexp(0.25 * (q[t] @ k[mask[t]].T)) for t in range(Tq)])
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12, rtol=0)


def test_softmax_rows_sum_to_one_single_key_and_constant_v():
    rs = np.random.default_rng(1)
    Tq, Tk, d = 8, 20, 5
    q, k = rs.standard_normal((Tq, d)) * 3, rs.standard_normal((Tk, d)) * 3
    mask = rs.random((Tq, Tk)) < 0.5
    mask[:, 0] = True
    # V = identity: O rows are the softmax rows themselves
    o, _ = orc.masked_attention(q, k, np.eye(Tk), mask, 1.0)
    np.testing.assert_allclose(o.sum(1), 1.0, atol=1e-14)
    assert np.all(o[~mask] == 0)
    # a single allowed key: O = that key's value
    single = np.zeros((Tq, Tk), bool)
    single[np.arange(Tq), np.arange(Tq)] = True
    v = rs.standard_normal((Tk, d))
    o, lse = orc.masked_attention(q, k, v, single, 0.7)
    np.testing.assert_array_equal(o, v[:Tq])
    np.testing.assert_allclose(lse, 0.7 * np.einsum("td,td->t", q, k[:Tq]), atol=1e-13)
    # constant V: O = that constant
    o, _ = orc.masked_attention(q, k, np.tile(rs.standard_normal(d), (Tk, 1)), mask, 1.0)
    np.testing.assert_allclose(o, np.tile(o[0], (Tq, 1)), atol=1e-14)


def test_masked_attention_rejects_empty_rows():
    with pytest.raises(ValueError):
        orc.masked_attention(np.ones((2, 2)), np.ones((3, 2)), np.ones((3, 2)),
                             np.array([[1, 0, 0], [0, 0, 0]], bool), 1.0)


@pytest.mark.parametrize("seed", range(3))
def test_attention_grad_matches_autograd_and_finite_differences(seed):
    rs = np.random.default_rng(seed)
    Tq, Tk, d, scale = 9, 14, 4, 0.6
    q, k, v, do = (rs.standard_normal(s) for s in [(Tq, d), (Tk, d), (Tk, d), (Tq, d)])
    mask = rs.random((Tq, Tk)) < 0.5
    mask[:, 3] = True
    dq, dk, dv = orc.masked_attention_grad(q, k, v, mask, scale, do)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=torch.tensor(mask)[None], scale=scale)[0]
    o.backward(torch.tensor(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), atol=1e-12, rtol=0)
    # central differences on a few coordinates of each input
    eps = 1e-6

    def loss(qq, kk, vv):
        return float((orc.masked_attention(qq, kk, vv, mask, scale)[0] * do).sum())

    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in [(0, 0), (arr.shape[0] - 1, d - 1), (arr.shape[0] // 2, 1)]:
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            args_p = [p if a is arr else a for a in (q, k, v)]
            args_m = [m if a is arr else a for a in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd))


# ----------------------------------------------------------------------------- schedule
def test_tiny_schedule_matches_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "tiny_schedule.json")))
    sch = orc.Schedule(g["n"], g["B"], g["F"], g["W"], g["C"], g["S"], g["K"], 0.125)
    for row in g["chunks"]:
        c = row["c"]
        assert sch.window_frames(c) == row["window_frames"]
        assert sch.window_blocks(c) == row["window_blocks"]
        assert sch.evicted_blocks(c) == row["evicted"]
        assert sch.chunk_blocks(c) == row["chunk_blocks"]


def test_tiny_rollout_matches_hand_worked_persistent_sets():
    g = json.load(open(os.path.join(GOLDEN, "tiny_schedule.json")))
    wl = synth.WORKLOADS["tiny"]
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    ro = orc.PersistentRollout(sch, wl.head_dim)
    for c in range(wl.measured_chunk):
        q, k, v = (a[:, 0, :] for a in synth.chunk_qkv(wl, 7, c))
        routed = ro.select(q)
        cand = len([p for p in routed["P"] if p >= sch.S]) + len(sch.evicted_blocks(c))
        assert cand == g["candidates_at_update"][str(c)]
        ro.update(routed, k, v)
        if str(c) in g["persistent_after_update"]:
            assert ro.P == g["persistent_after_update"][str(c)]
    q, k, v = (a[:, 0, :] for a in synth.chunk_qkv(wl, 7, wl.measured_chunk))
    routed = ro.select(q)
    A = ro.attended_blocks(routed["sel"])
    keys = [sum(b - a for a, b in (orc.block_token_range(x, sch.n, sch.B) for x in row)) for row in A]
    assert set(keys) == {g["keys_per_query_at_chunk_4"]}
    assert (ro.chunk + 1) * sch.F * sch.n == g["dense_keys_per_query_at_chunk_4"]


def test_candidate_counts_fixture():
    g = json.load(open(os.path.join(GOLDEN, "candidate_counts.json")))
    assert orc.blocks_per_frame(1560, 64) == g["nb_wan"]
    for name, row in g["workloads"].items():
        wl = synth.WORKLOADS[name]
        sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                           wl.capacity, wl.sinks, wl.topk, wl.scale)
        c = wl.measured_chunk
        assert (wl.capacity - wl.sinks) + len(sch.evicted_blocks(c)) == row["candidates_full"]
        assert len(sch.window_blocks(c)) == row["window_blocks_full"]
        assert wl.capacity + wl.topk + wl.chunk_frames * wl.nb == row["attended_blocks_per_query_block"]


# ----------------------------------------------------------------------------- memory update
@pytest.mark.parametrize("seed", range(25))
def test_memory_update_brute_force_and_invariants(seed):
    rs = np.random.default_rng(100 + seed)
    S = int(rs.integers(0, 3))
    C = S + int(rs.integers(0, 5))
    sinks = list(range(S))
    others = sorted(rs.choice(np.arange(S, 60), size=int(rs.integers(0, C - S + 1)), replace=False).tolist())
    P = sinks + others
    E = sorted(rs.choice(np.arange(60, 90), size=int(rs.integers(0, 6)), replace=False).tolist())
    Nq = 3
    sP = rs.integers(-2, 3, size=(Nq, len(P))).astype(float)
    sE = rs.integers(-2, 3, size=(Nq, len(E))).astype(float)
    newP = orc.memory_update(P, sinks, sP, E, sE, C)
    m = {g: sP[:, i].sum() for i, g in enumerate(P)}
    m.update({g: sE[:, i].sum() for i, g in enumerate(E)})
    R = [g for g in P if g not in sinks] + E
    kk = min(C - S, len(R))
    best = None
    for comb in itertools.combinations(R, kk):
        if all(m[a] > m[b] or (m[a] == m[b] and a < b) for a in comb for b in R if b not in comb):
            assert best is None
            best = sorted(comb)
    assert newP == sorted(sinks + best)
    assert set(sinks) <= set(newP) and len(newP) <= C and len(set(newP)) == len(newP)
    if C - S >= len(R):
        assert set(newP) == set(P) | set(E)


def _rollout(wl, seed, heads=(0,), chunks=None):
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    ros = {h: orc.PersistentRollout(sch, wl.head_dim, keep_history=True) for h in heads}
    last = None
    for c in range(wl.measured_chunk + 1 if chunks is None else chunks):
        q, k, v = synth.chunk_qkv(wl, seed, c)
        for h in heads:
            routed = ros[h].select(q[:, h])
            last = (q, k, v, routed)
            if c < (wl.measured_chunk if chunks is None else chunks - 1):
                ros[h].update(routed, k[:, h], v[:, h])
    return sch, ros, last


def test_rollout_invariants_every_chunk():
    wl = synth.Workload("small", 1, 16, 8, 24, 2, 12, 4, 5, 2, 3)   # n=24 -> 3 blocks/frame
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    ro = orc.PersistentRollout(sch, wl.head_dim)
    for c in range(wl.measured_chunk):
        q, k, v = (a[:, 0] for a in synth.chunk_qkv(wl, 3, c))
        routed = ro.select(q)
        L = set(routed["L"])
        assert not (set(ro.P) & L)
        for row in routed["sel"]:
            assert row == sorted(row) and set(row) <= L and len(row) == min(sch.K, len(L))
        ro.update(routed, k, v)
        h_blocks = ro.chunk * sch.F * sch.nb
        assert set(range(sch.S)) <= set(ro.P)
        assert len(ro.P) <= sch.C and len(set(ro.P)) == len(ro.P)
        assert all(0 <= g < h_blocks for g in ro.P)
        assert not (set(ro.P) & set(sch.window_blocks(ro.chunk)))


def test_full_selection_is_textbook_block_causal_attention():
    # capacity and top-K large enough to keep everything: PBSA = dense chunk-causal attention
    wl = synth.Workload("full", 1, 8, 4, 12, 1, 5, 2, 100, 1, 100)
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    ro = orc.PersistentRollout(sch, wl.head_dim)
    Q, Kc, Vc = [], [], []
    for c in range(wl.measured_chunk + 1):
        q, k, v = (a[:, 0].astype(np.float64) for a in synth.chunk_qkv(wl, 11, c))
        Q.append(q), Kc.append(k), Vc.append(v)
        routed = ro.select(q)
        o, lse = ro.attend(q, k, v, routed["sel"])
        Kall, Vall = np.concatenate(Kc), np.concatenate(Vc)
        ref = _sdpa64(q, Kall, Vall, np.ones((len(q), len(Kall)), bool), wl.scale)
        np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
        ro.update(routed, k, v)


def test_gathered_and_dense_masked_forms_agree():
    wl = synth.WORKLOADS["tiny"]
    sch, ros, (q, k, v, routed) = _rollout(wl, 5)
    ro = ros[0]
    o1, l1 = ro.attend(q[:, 0], k[:, 0], v[:, 0], routed["sel"])
    o2, l2 = ro.attend_dense(q[:, 0], k[:, 0], v[:, 0], routed["sel"])
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-12, rtol=0)
    rows = [0, 63, 64, 200, 255]
    o3, l3 = ro.attend(q[:, 0], k[:, 0], v[:, 0], routed["sel"], rows=rows)
    np.testing.assert_allclose(o3[rows], o1[rows], atol=1e-14, rtol=0)
    assert np.isnan(o3[1]).all()


def test_planted_blocks_are_routed_and_retained():
    # strong planted direction: every planted window block is in every query block's top-K,
    # and every planted block that left the window is in P (their count is below C - S)
    wl = synth.Workload("plant", 2, 32, 16, 64, 2, 16, 4, 12, 1, 6, planted_per_segment=3,
                        segment_frames=6, q_align=2.0, kv_shift=6.0)
    seed = 21
    sch, ros, (q, k, v, routed_last) = _rollout(wl, seed, heads=(0, 1))
    planted = set(synth.planted_blocks(wl, seed, wl.history_frames + wl.chunk_frames).tolist())
    c = wl.measured_chunk
    win = set(sch.window_blocks(c))
    out_of_window = {g for g in planted if g < c * sch.F * sch.nb and g not in win}
    assert len(out_of_window) <= sch.C - sch.S
    for h in (0, 1):
        ro = ros[h]
        assert out_of_window <= set(ro.P)
        routed = ro.select(q[:, h])
        for row in routed["sel"]:
            assert (planted & win) <= set(row)


# ----------------------------------------------------------------------------- two-level
def test_two_level_reduces_to_dense_and_forces_frames():
    F, nb, n, B, d = 2, 2, 8, 4, 4
    chunks = 4
    rs = np.random.default_rng(3)
    q = rs.standard_normal((chunks * F * n, d))
    k = rs.standard_normal((chunks * F * n, d))
    qr, _ = orc.mean_pool(q, n, B)
    kr, kf = orc.mean_pool(k, n, B)
    for i in range(1, chunks + 1):
        for r in range((i - 1) * F * nb, i * F * nb):
            dense = orc.two_level_select(qr[r], kr, kf, i, F, nb, top_frames=99, k_i=10 ** 6,
                                         scale=0.5)
            assert dense == list(range(i * F * nb))
            if i >= 2:
                # one frame picked by score + the forced ones; the mask is exactly the
                # blocks of T; forced frames always present
                sel = orc.two_level_select(qr[r], kr, kf, i, F, nb, top_frames=1,
                                           k_i=10 ** 6, scale=0.5)
                frames = {g // nb for g in sel}
                forced = {0, F * (i - 1) - 1} | {F * (i - 1) + t for t in range(F)}
                assert forced <= frames and len(frames - forced) <= 1
                assert sel == [f * nb + j for f in sorted(frames) for j in range(nb)]
                best = int(np.argmax([0.5 * qr[r] @ kf[f] for f in range(F * (i - 1))]))
                assert best in frames


def test_two_level_block_topk_brute_force():
    F, nb, n, B, d = 3, 2, 8, 4, 4
    rs = np.random.default_rng(8)
    T = 4 * F * n
    q, k = rs.standard_normal((T, d)), rs.standard_normal((T, d))
    qr, _ = orc.mean_pool(q, n, B)
    kr, kf = orc.mean_pool(k, n, B)
    i, k_i = 4, 5
    for r in range((i - 1) * F * nb, i * F * nb):
        sel = orc.two_level_select(qr[r], kr, kf, i, F, nb, top_frames=2, k_i=k_i, scale=0.3)
        hist = F * (i - 1)
        fs = sorted(range(hist), key=lambda f: (-(qr[r] @ kf[f]), f))[:2]
        T_r = set(fs) | {0, hist - 1} | set(range(hist, hist + F))
        cand = [f * nb + j for f in T_r for j in range(nb)]
        sc = {g: qr[r] @ kr[g] for g in cand}
        want = sorted(sorted(cand, key=lambda g: (-sc[g], g))[:k_i])
        assert sel == want


def test_cag_budget_reading_and_identity_closed_form():
    # reading: chunk i_ref keeps k_ref blocks at alpha = 0; k_i = round(4 i (1 + alpha))
    ks = orc.cag_budgets([0.0] * 8, k_ref=32, i_ref=8)
    assert ks == [0, 8, 12, 16, 20, 24, 28, 32]
    ks = orc.cag_budgets([0.0, 1.0, 0.5, 0.25, 0.0, 0.0, 0.0, 1.0], k_ref=32, i_ref=8)
    assert ks == [0, 16, 18, 20, 20, 24, 28, 64]
    # rounding to nearest: 4*2*1.2 = 9.6 -> 10, 4*3*1.1 = 13.2 -> 13, 4*4*1.2 = 19.2 -> 19
    assert orc.cag_budgets([0.0, 0.2, 0.1, 0.2], k_ref=32, i_ref=8) == [0, 10, 13, 19]
    # equal alphas: the FLOPs identity gives s_target = s_base - alpha * beta exactly
    lq = [4680] * 8
    lk = [4680 * i for i in range(1, 9)]
    for a in (0.0, 0.3, 1.0):
        st = orc.cag_target_sparsity([a] * 8, s_base=1 - 32 / 600, beta=32 / 600, lq=lq, lk=lk)
        assert st == pytest.approx((1 - 32 / 600) - a * 32 / 600, abs=1e-12)
