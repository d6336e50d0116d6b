"""Helpers for comparing the HIP path with the fp64 oracle (not a test module)."""
from __future__ import annotations

import sys

import numpy as np

TIE = 1e-5          # score gap below which several selections are correct
ATTN_MAX = 2e-2     # max-abs error bound for bf16 outputs / gradients vs fp64
ATTN_MEAN = 2e-3    # mean-abs error bound


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def order(ids, scores):
    """Indices sorted by (score desc, id asc)."""
    return np.lexsort((np.asarray(ids), -np.asarray(scores, dtype=np.float64)))


def check_topk(got, cand_ids, cand_scores, k, tie=TIE):
    """Validate a selected id list against exact candidate scores.

    Returns (exact, near_tie).  Raises AssertionError if `got` is not a correct top-k set:
    it must hold min(k, |cand|) distinct candidates in ascending order, contain every
    candidate scoring more than tau + tie and none scoring less than tau - tie, where tau is
    the k-th best exact score.  Where no candidate lies within tie of tau the set is unique
    and must match exactly.
    """
    got = [int(g) for g in got]
    cand_ids = np.asarray(cand_ids)
    cand_scores = np.asarray(cand_scores, dtype=np.float64)
    kk = min(k, len(cand_ids))
    assert len(got) == kk, f"expected {kk} ids, got {len(got)}"
    assert got == sorted(set(got)), f"ids not ascending/unique: {got}"
    pos = {int(g): i for i, g in enumerate(cand_ids)}
    assert all(g in pos for g in got), f"ids outside the candidates: {got}"
    o = order(cand_ids, cand_scores)
    want = sorted(int(cand_ids[i]) for i in o[:kk])
    if kk == 0 or kk == len(cand_ids):
        assert got == want
        return True, False
    tau = cand_scores[o[kk - 1]]
    must_in = {int(g) for g, s in zip(cand_ids, cand_scores) if s > tau + tie}
    must_out = {int(g) for g, s in zip(cand_ids, cand_scores) if s < tau - tie}
    gs = set(got)
    assert must_in <= gs, f"missing clear winners {sorted(must_in - gs)}"
    assert not (gs & must_out), f"holds clear losers {sorted(gs & must_out)}"
    near = len(must_in) + len(must_out) < len(cand_ids) - 1 or \
        abs(cand_scores[o[kk]] - tau) <= tie
    if not near:
        assert got == want
    return got == want, near


def err_stats(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    return float(d.max()), float(d.mean()), float(rel)


def assert_close_attn(got, ref, what, max_abs=ATTN_MAX, mean_abs=ATTN_MEAN, rel_l2=1e-2):
    mx, mn, rel = err_stats(got, ref)
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mn:.3e} rel-L2 {rel:.3e}")
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{what}: non-finite values"
    assert mx <= max_abs, f"{what}: max-abs {mx} > {max_abs}"
    assert mn <= mean_abs, f"{what}: mean-abs {mn} > {mean_abs}"
    assert rel <= rel_l2, f"{what}: rel-L2 {rel} > {rel_l2}"
