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



def _dominates(col_a, col_b):
    """Column a scores at least as high as column b for every query block, higher for one."""
    return bool(np.all(col_a >= col_b) and np.any(col_a > col_b))


def _check_dominance(P, sinks, sP, E, sE, newP):
    """No candidate is dropped while a candidate it dominates is kept."""
    cols = {g: sP[:, i] for i, g in enumerate(P) if g not in sinks}
    cols.update({g: sE[:, i] for i, g in enumerate(E)})
    kept = set(newP)
    for a, ca in cols.items():
        for b, cb in cols.items():
            if a != b and _dominates(ca, cb):
                assert not (b in kept and a not in kept), (a, b)


@pytest.mark.parametrize("seed", range(30))
def test_memory_update_respects_score_dominance(seed):
    # Sparse Forcing 2.C "Dynamic Update": the blocks the chunk's queries score highest are
    # the ones promoted.  Whatever the aggregate over query blocks, a candidate that every
    # query block scores at least as high as another (and one strictly higher) is at least
    # as important, and strictly so: it is never dropped while the other is kept.  Query
    # blocks are at least as many as candidates, so that a sum over the wrong axis still
    # runs (and must fail here), and each case plants dominance pairs.
    rs = np.random.default_rng(500 + seed)
    S = int(rs.integers(0, 3))
    sinks = list(range(S))
    nP = int(rs.integers(1, 6))
    P = sinks + sorted(rs.choice(np.arange(S, 40), size=nP, replace=False).tolist())
    E = sorted(rs.choice(np.arange(40, 70), size=int(rs.integers(1, 6)), replace=False).tolist())
    C = S + int(rs.integers(1, nP + len(E)))
    ncand = nP + len(E)
    Nq = ncand + int(rs.integers(0, 4))
    sP = rs.integers(-3, 4, size=(Nq, len(P))).astype(float)
    sE = rs.integers(-3, 4, size=(Nq, len(E))).astype(float)
    # plant: a few candidates are copies of another plus non-negative bumps (one positive)
    cand = [(0, i) for i, g in enumerate(P) if g >= S] + [(1, i) for i in range(len(E))]
    for _ in range(3):
        (ta, ia), (tb, ib) = (cand[j] for j in rs.choice(len(cand), size=2, replace=False))
        src = (sP, sE)[tb][:, ib]
        bump = rs.integers(0, 2, size=Nq).astype(float)
        bump[rs.integers(0, Nq)] = 1.0
        (sP, sE)[ta][:, ia] = src + bump
    newP = orc.memory_update(P, sinks, sP, E, sE, C)
    _check_dominance(P, sinks, sP, E, sE, newP)
    # the sinks' own scores never matter
    sP2 = sP.copy()
    sP2[:, :S] = rs.integers(-100, 100, size=(Nq, S))
    assert orc.memory_update(P, sinks, sP2, E, sE, C) == newP


def test_memory_update_strict_dominance_breaks_equal_maxima():
    # Two candidates with the same best score over the query blocks; the higher id one is
    # scored higher by the other query blocks.  Only one place is free: it must go to the
    # dominating candidate, even though the tie rule favours the lower id when only the
    # best query block is looked at.
    P, sinks = [0, 5], [0]
    E = [9]
    sP = np.array([[7.0, 4.0], [0.0, 1.0], [0.0, 1.0]])   # sink 0, block 5
    sE = np.array([[4.0], [2.0], [3.0]])                     # block 9: >= block 5 everywhere
    assert orc.memory_update(P, sinks, sP, E, sE, 2) == [0, 9]
    # and with the roles swapped the lower id wins
    assert orc.memory_update([0, 9], sinks, np.array([[7.0, 4.0], [0.0, 2.0], [0.0, 3.0]]), [5],
                             np.array([[4.0], [1.0], [1.0]]), 2) == [0, 9]


def test_memory_scores_are_column_aggregates_of_the_chunk():
    # Orientation: the memory score of a candidate depends on its own column only (the
    # scores all query blocks give that candidate), never on other candidates' columns,
    # and reordering the chunk's query blocks changes nothing.
    rs = np.random.default_rng(9)
    P, sinks, E = [0, 3, 8, 12], [0], [20, 21, 22]
    Nq = 6
    sP, sE = rs.standard_normal((Nq, 4)), rs.standard_normal((Nq, 3))
    ids, m = orc.memory_scores(P, sinks, sP, E, sE)
    assert ids == [3, 8, 12, 20, 21, 22]
    perm = rs.permutation(Nq)
    _, m_perm = orc.memory_scores(P, sinks, sP[perm], E, sE[perm])
    np.testing.assert_allclose(m_perm, m, atol=1e-14, rtol=0)
    sP3 = sP.copy()
    sP3[:, 2] += 5.0      # only block 8's column changes
    _, m3 = orc.memory_scores(P, sinks, sP3, E, sE)
    changed = [i for i in range(len(ids)) if m3[i] != m[i]]
    assert changed == [1] and m3[1] > m[1]


def test_rollout_updates_respect_score_dominance():
    # the same dominance check on the candidates of every update of a small rollout (six
    # query blocks per chunk, so dominance pairs do occur among the real candidates)
    wl = synth.Workload("dom", 1, 16, 8, 24, 2, 16, 4, 4, 1, 3)
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    ro = orc.PersistentRollout(sch, wl.head_dim)
    pairs = 0
    for c in range(wl.measured_chunk):
        q, k, v = (a[:, 0] for a in synth.chunk_qkv(wl, 31, c))
        routed = ro.select(q)
        E = sch.evicted_blocks(ro.chunk)
        col = {g: i for i, g in enumerate(routed["L"])}
        sE = routed["scores_L"][:, [col[g] for g in E]] if E else np.zeros((len(q), 0))
        before = list(ro.P)
        ro.update(routed, k, v)
        _check_dominance(before, list(range(sch.S)), routed["scores_P"], E, sE, ro.P)
        cols = [routed["scores_P"][:, i] for i, g in enumerate(before) if g >= sch.S] + \
            [sE[:, i] for i in range(len(E))]
        pairs += sum(_dominates(a, b) for a in cols for b in cols if a is not b)
    assert pairs > 0

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


def test_persistent_gradient_with_full_selection_is_textbook_autograd():
    # capacity and top-K keep every block: the gradient of the persistent-mode attention is
    # the gradient of dense softmax attention over the whole history plus the chunk
    wl = synth.Workload("fullg", 1, 8, 4, 12, 1, 4, 2, 100, 1, 100)
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale)
    ro = orc.PersistentRollout(sch, wl.head_dim)
    Kc, Vc = [], []
    rs = np.random.default_rng(4)
    for c in range(wl.measured_chunk + 1):
        q, k, v = (a[:, 0].astype(np.float64) for a in synth.chunk_qkv(wl, 12, c))
        routed = ro.select(q)
        if c == wl.measured_chunk:
            do = rs.standard_normal(q.shape)
            dq, dkc, dvc, dkb, dvb = ro.attend_grad(q, k, v, routed["sel"], do)
            Kall, Vall = np.concatenate(Kc + [k]), np.concatenate(Vc + [v])
            tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, Kall, Vall))
            out = torch.nn.functional.scaled_dot_product_attention(
                tq[None], tk[None], tv[None], scale=wl.scale)[0]
            out.backward(torch.tensor(do))
            np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
            hist = c * sch.F * sch.n
            np.testing.assert_allclose(dkc, tk.grad.numpy()[hist:], atol=1e-12, rtol=0)
            np.testing.assert_allclose(dvc, tv.grad.numpy()[hist:], atol=1e-12, rtol=0)
            assert sorted(dkb) == list(range(c * sch.F * sch.nb))
            for g in dkb:
                a, b = orc.block_token_range(g, sch.n, sch.B)
                np.testing.assert_allclose(dkb[g], tk.grad.numpy()[a:b], atol=1e-12, rtol=0)
                np.testing.assert_allclose(dvb[g], tv.grad.numpy()[a:b], atol=1e-12, rtol=0)
        else:
            ro.update(routed, k, v)
            Kc.append(k)
            Vc.append(v)


def test_persistent_gradient_of_unattended_blocks_is_zero():
    # a window block that no query block routes to gets no gradient; P blocks always do
    wl = synth.WORKLOADS["tiny"]
    sch, ros, (q, k, v, routed) = _rollout(wl, 6)
    ro = ros[0]
    sel = [row[:1] for row in routed["sel"]]   # one routed block per query block
    do = np.random.default_rng(0).standard_normal((q.shape[0], wl.head_dim))
    _, _, _, dkb, dvb = ro.attend_grad(q[:, 0], k[:, 0], v[:, 0], sel, do)
    routed_any = {g for row in sel for g in row}
    for g in sch.window_blocks(ro.chunk):
        if g not in routed_any:
            assert not dkb[g].any() and not dvb[g].any()
    for g in ro.P:
        assert np.abs(dvb[g]).sum() > 0


def _rollout_sels(wl, seed, union, chunks):
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale, union)
    ro = orc.PersistentRollout(sch, wl.head_dim)
    out = []
    for c in range(chunks):
        q, k, v = (a[:, 0] for a in synth.chunk_qkv(wl, seed, c))
        rt = ro.select(q)
        o, lse = ro.attend(q, k, v, rt["sel"])
        out.append((rt, ro.attended_blocks(rt["sel"]), o, lse, list(ro.P)))
        ro.update(rt, k, v)
    return sch, out


def test_union_routing_with_only_sinks_in_memory_is_window_routing():
    # capacity = sinks: P_t holds only the sinks, so routing over P_t and the window
    # together chooses among the window alone
    wl = synth.Workload("u1", 1, 16, 8, 24, 2, 12, 4, 2, 2, 3)
    _, a = _rollout_sels(wl, 13, False, wl.measured_chunk + 1)
    _, b = _rollout_sels(wl, 13, True, wl.measured_chunk + 1)
    for (ra, aa, oa, la, pa), (rb, ab, ob, lb, pb) in zip(a, b):
        assert ra["sel"] == rb["sel"] and aa == ab and pa == pb
        np.testing.assert_array_equal(oa, ob)


def test_union_routing_full_selection_is_dense_attention():
    # top-K at least every candidate: both variants attend everything
    wl = synth.Workload("u2", 1, 8, 4, 12, 1, 5, 2, 100, 1, 100)
    _, a = _rollout_sels(wl, 14, False, wl.measured_chunk + 1)
    _, b = _rollout_sels(wl, 14, True, wl.measured_chunk + 1)
    for (ra, aa, oa, la, pa), (rb, ab, ob, lb, pb) in zip(a, b):
        assert aa == ab
        np.testing.assert_allclose(oa, ob, atol=1e-12, rtol=0)


def test_union_routing_candidates_and_invariants():
    # routing over P_t and the window: candidates are exactly the non-sink persistent
    # blocks and the window blocks; every query block attends the sinks, its K routed
    # blocks and its chunk, and no other persistent block
    wl = synth.Workload("u3", 1, 16, 8, 24, 2, 16, 4, 6, 2, 4)
    sch, out = _rollout_sels(wl, 15, True, wl.measured_chunk + 1)
    routed_p = 0
    for c, (rt, att, o, lse, P) in enumerate(out):
        sinks = [g for g in P if g < sch.S]
        assert rt["cand"] == [g for g in P if g >= sch.S] + rt["L"]
        own = set(sch.chunk_blocks(c))
        for row, a in zip(rt["sel"], att):
            assert len(row) == min(sch.K, len(rt["cand"])) and set(row) <= set(rt["cand"])
            assert set(a) == set(sinks) | set(row) | own
            routed_p += len(set(row) & set(P))
        # the best-scoring candidate of each query block is always routed
        for r, row in enumerate(rt["sel"]):
            if rt["cand"]:
                best = rt["cand"][int(np.lexsort((rt["cand"], -rt["scores_cand"][r]))[0])]
                assert best in row
    assert routed_p > 0


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
    planted = set(synth.planted_blocks(wl, seed, wl.plant_frames).tolist())
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


# ----------------------------------------------------------------------------- FP8 cache
def test_e4m3_decode_table_landmarks():
    # OCP E4M3: bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN
    v = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9 and v[0x3C] == 1.5
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and v[0xB8] == -1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)           # codes 0..126 increase strictly
    assert np.array_equal(v[0x80:0xFF], -pos)


def test_e4m3_encode_is_nearest_with_ties_to_even():
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    cv, vv = codes[fin], vals[fin]
    rs = np.random.default_rng(3)
    pos = np.sort(np.unique(vv[vv >= 0]))
    mids = (pos[1:] + pos[:-1]) / 2                      # exact ties
    ys = np.concatenate([rs.uniform(-448, 448, 4000), rs.uniform(-0.05, 0.05, 2000), mids,
                         -mids, pos, -pos])
    got = orc.e4m3_encode(ys)
    for y, g in zip(ys, got):
        d = np.abs(vv - y)
        best = cv[d == d.min()]
        if len(best) > 1:                                # a tie: the even mantissa wins
            best = best[(best & 1) == 0]
            best = best[np.signbit(orc.e4m3_decode(best)) == np.signbit(y)] if len(best) > 1 else best
        assert g in best, (y, g, best)


def test_e4m3_block_scale_is_the_smallest_power_of_two():
    rs = np.random.default_rng(4)
    for _ in range(200):
        x = rs.standard_normal((64, 8)) * 10.0 ** rs.uniform(-4, 4)
        sc = orc.e4m3_block_scale(x)
        e = np.log2(sc)
        assert e == np.round(e)
        amax = np.abs(x).max()
        assert amax <= 448 * sc and amax > 448 * sc / 2
    assert orc.e4m3_block_scale(np.zeros((3, 4))) == 1.0
    assert orc.e4m3_block_scale(np.full((1, 1), 448.0)) == 1.0
    assert orc.e4m3_block_scale(np.full((1, 1), 448.5)) == 2.0


def test_e4m3_dequantized_values_are_exact_in_bf16():
    rs = np.random.default_rng(5)
    x = synth.round_bf16(rs.standard_normal((64, 128)).astype(np.float32) * 3)
    codes, sc = orc.e4m3_quantize_block(x)
    deq = orc.e4m3_decode(codes) * sc
    assert np.array_equal(synth.round_bf16(deq.astype(np.float32)).astype(np.float64), deq)
    # relative error of the nearest code: at most half a mantissa step (2^-4)
    big = np.abs(x) >= 2.0 ** -6 * sc
    assert np.all(np.abs(deq - x)[big] <= 2.0 ** -4 * np.abs(x)[big] + 1e-30)


# ----------------------------------------------------------------------------- FP8 arithmetic
def _nearest_grid(y, grid):
    """Nearest value of a sorted grid to y, ties to the larger |mantissa| parity rule being
    irrelevant here (the test data avoid exact ties)."""
    i = np.searchsorted(grid, y)
    lo = grid[max(i - 1, 0)]
    hi = grid[min(i, len(grid) - 1)]
    return lo if abs(y - lo) <= abs(hi - y) else hi


def test_e4m3_rows_are_nearest_values_of_each_rows_own_grid():
    # brute force: each row's values against every E4M3 value times that row's own scale,
    # the scale being the smallest power of two that holds the row's max
    vals = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = np.sort(np.unique(vals[~np.isnan(vals)]))
    rs = np.random.default_rng(21)
    x = rs.standard_normal((12, 40)) * (10.0 ** rs.uniform(-3, 3, (12, 1)))
    got = orc.e4m3_rows(x)
    for t in range(x.shape[0]):
        amax = np.abs(x[t]).max()
        e = 0
        while amax > 448 * 2.0 ** e:
            e += 1
        while amax <= 448 * 2.0 ** (e - 1):
            e -= 1
        for c in range(x.shape[1]):
            assert got[t, c] == _nearest_grid(x[t, c] / 2.0 ** e, grid) * 2.0 ** e


def _c32(scale):
    # scale * log2(e) as float32 (the product and both factors rounded to float32)
    return np.float32(np.float32(scale) * np.float32(math.log2(math.e)))


def test_fp8_attention_is_base2_attention_of_the_quantized_scaled_queries():
    # x8 = E4M3 rows of float32(q) * c; torch's attention with scale ln 2 on x8 is the
    # base-2 softmax of x8 . k
    rs = np.random.default_rng(22)
    q = rs.standard_normal((6, 16))
    K = orc.e4m3_decode(rs.integers(0, 0x7E, (30, 16)).astype(np.uint8)) * 2.0 ** -4
    V = rs.standard_normal((30, 16))
    o, lse, _ = orc.fp8_attention(q, K, V, 0.25)
    x8 = orc.e4m3_rows((q.astype(np.float32) * _c32(0.25)).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(x8)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        scale=math.log(2))[0].numpy()
    assert np.abs(o - ref).max() < 1e-12
    z = math.log(2) * (x8 @ K.T)
    assert np.abs(lse - np.log(np.exp(z).sum(axis=1))).max() < 1e-12


def _simulate_fp8_pv(x8, K, V, head):
    # an implementation's rounding of p: scores t = x8 . k in exp2 units, a row offset with
    # the max mapping to 2^head (head in [3, 8.8]), p rounded to E4M3 by brute force over
    # the value grid
    vals = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = np.sort(np.unique(vals[~np.isnan(vals)]))
    t = x8 @ K.T
    out = np.empty((x8.shape[0], V.shape[1]))
    for r in range(x8.shape[0]):
        pk = np.exp2(t[r] - t[r].max() + head)
        assert pk.max() <= 448
        p8 = np.array([_nearest_grid(x, grid) for x in pk])
        out[r] = (p8 @ V) / pk.sum()
    return out


def test_fp8_attention_bound_covers_simulated_probability_rounding():
    rs = np.random.default_rng(23)
    for trial in range(6):
        q = rs.standard_normal((4, 32)) * 1.5
        K = rs.standard_normal((400, 32))
        V = rs.standard_normal((400, 32)) + (0.5 if trial % 2 else 0.0)
        o, _, bound = orc.fp8_attention(q, K, V, 0.3)
        x8 = orc.e4m3_rows((q.astype(np.float32) * _c32(0.3)).astype(np.float64))
        for head in (3.0, 4.5, 6.5, 8.5):
            sim = _simulate_fp8_pv(x8, K, V, head)
            assert np.all(np.abs(sim - o) <= bound * (1 + 1e-9) + 1e-12)


@pytest.mark.parametrize("head", [3, 5])
def test_fp8_attention_bound_needs_its_subnormal_term(head):
    # one dominant key and many keys head + 11 exp2 units below it (p = 2^-11 against the
    # max's 2^head), all with V = 1: every small p rounds to zero, so the error is
    # one-signed and equals the subnormal term; the normal-range term alone does not cover it
    scale = 1.0
    c = float(_c32(scale))
    q = np.zeros((1, 4))
    q[0, 0] = 1.0
    K = np.zeros((3001, 4))
    x0 = float(orc.e4m3_rows(np.array([[c, 0.0, 0.0, 0.0]]))[0, 0])   # the quantized c q
    K[0, 0] = 40.0                      # the dominant key
    K[1:, 0] = 40.0 - (head + 11) / x0 - np.linspace(0, 0.05, 3000)
    V = np.ones((3001, 4))
    V[0] = 0.0
    o, lse, bound = orc.fp8_attention(q, K, V, scale, head=head)
    x8 = orc.e4m3_rows((q.astype(np.float32) * _c32(scale)).astype(np.float64))
    sim = _simulate_fp8_pv(x8, K, V, float(head))
    err = np.abs(sim - o).max()
    t = x8 @ K.T
    p = np.exp2(t - t.max())
    p /= p.sum()
    normal_only = 2.0 ** -4 * (p @ np.abs(V)).max()
    assert err > normal_only                     # the subnormal range matters here
    assert err <= bound.max() * (1 + 1e-9)       # and the full bound covers it


def test_rollout_attend_fp8_quantizes_queries_and_chunk_blocks():
    # attend_fp8 = attend over the same stored blocks with the queries and the chunk's own
    # blocks replaced by their quantized values (the queries as scale * log2 e * q)
    wl = synth.Workload("pin_fp8", 1, 16, 32, 64, 1, 4, 2, 4, 1, 2)
    sch = orc.Schedule(wl.frame_tokens, wl.block, wl.chunk_frames, wl.window_frames,
                       wl.capacity, wl.sinks, wl.topk, wl.scale, False)
    ro = orc.PersistentRollout(sch, wl.head_dim, kv_fp8=True)
    for c in range(4):
        q, k, v = synth.chunk_qkv(wl, 5, c)
        rt = ro.select(q[:, 0])
        if c == 3:
            o8, l8, b8 = ro.attend_fp8(q[:, 0], k[:, 0], v[:, 0], rt["sel"])
            kq, vq = np.empty_like(k[:, 0], dtype=np.float64), np.empty_like(v[:, 0], dtype=np.float64)
            for b in range(sch.F * sch.nb):
                a0, b0 = orc.block_token_range(b, sch.n, sch.B)
                kc, ks = orc.e4m3_quantize_block(k[a0:b0, 0])
                vc, vs = orc.e4m3_quantize_block(v[a0:b0, 0])
                kq[a0:b0], vq[a0:b0] = orc.e4m3_decode(kc) * ks, orc.e4m3_decode(vc) * vs
            # attend's softmax of scale * q' . k with q' = x8 ln 2 / scale is the base-2
            # softmax of x8 . k
            x8 = orc.e4m3_rows((q[:, 0].astype(np.float32) * _c32(wl.scale)).astype(np.float64))
            o, l = ro.attend(x8 * math.log(2) / wl.scale, kq, vq, rt["sel"])
            assert np.abs(o8 - o).max() < 1e-12 and np.abs(l8 - l).max() < 1e-12
            assert np.all(b8 > 0)
            return
        ro.update(rt, k[:, 0], v[:, 0])
