"""Planted mistakes in the oracle must each fail at least one pin.

Every case below replaces one oracle function (on the CPU, for the duration of the test)
by a version with a plausible mistake -- a dropped term, a wrong sign, index or axis, a
tie broken the wrong way -- and runs the pins that should catch it.  A case passes when at
least one of those pins fails; a mistake no pin notices would mean the oracle is not
pinned where it matters.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.pbsa_oracle as po
import test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(po, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(calls):
    failed = 0
    for call in calls:
        try:
            call()
        except Exception:  # an assertion of the pin, or the mistake breaking the run
            failed += 1
    return failed


_orig = {n: getattr(po, n) for n in ("memory_scores", "top_ids", "mean_pool", "coarse_scores",
                                      "masked_attention_grad", "masked_attention",
                                      "two_level_frames", "cag_budgets", "e4m3_encode",
                                      "e4m3_block_scale")}


def _memory_negated(P, sinks, sP, E, sE):
    ids, m = _orig["memory_scores"](P, sinks, sP, E, sE)
    return ids, [-x for x in m]


def _memory_rows(P, sinks, sP, E, sE):
    # sums over the candidates of one query block instead of over the query blocks
    ids, _ = _orig["memory_scores"](P, sinks, sP, E, sE)
    full = np.concatenate([np.asarray(sP, float), np.asarray(sE, float)], axis=1)
    return ids, [full[i].sum() for i in range(len(ids))]


def _memory_max(P, sinks, sP, E, sE):
    sinks = set(sinks)
    ids, m = [], []
    for i, g in enumerate(P):
        if g not in sinks:
            ids.append(g)
            m.append(np.asarray(sP, float)[:, i].max())
    for i, g in enumerate(E):
        ids.append(g)
        m.append(np.asarray(sE, float)[:, i].max())
    return ids, m


def _top_ids_high_tie(values, ids, k):
    values = np.asarray(values, float)
    ids = np.asarray(ids)
    if k <= 0 or ids.size == 0:
        return []
    order = np.lexsort((-ids, -values))
    return sorted(int(g) for g in ids[order[:k]])


def _pool_block_mean(x, n, B):
    br, fr = _orig["mean_pool"](x, n, B)
    nb = po.blocks_per_frame(n, B)
    return br, br.reshape(-1, nb, br.shape[1]).mean(axis=1)


def _scores_no_scale(q_rep, k_rep, scale):
    return _orig["coarse_scores"](q_rep, k_rep, 1.0)


def _grad_dk_sign(q, k, v, mask, scale, dout):
    dq, dk, dv = _orig["masked_attention_grad"](q, k, v, mask, scale, dout)
    return dq, -dk, dv


def _attn_lse_log2(q, k, v, mask, scale):
    o, lse = _orig["masked_attention"](q, k, v, mask, scale)
    return o, lse / math.log(2.0)


def _frames_no_last(q_rep_row, k_frame_rep, i, F, top_frames, scale):
    hist, p, T = _orig["two_level_frames"](q_rep_row, k_frame_rep, i, F, top_frames, scale)
    top = set(po.top_ids(p, hist, top_frames))
    return hist, p, sorted(t for t in T if t != F * (i - 1) - 1 or t in top)


def _budget_floor(alphas, k_ref, i_ref):
    return [0] + [max(1, int(math.floor(k_ref * i * (1.0 + float(a)) / i_ref)))
                  for i, a in enumerate(alphas[1:], start=2)]


def _encode_truncating(y):
    # rounds the magnitude toward zero instead of to nearest
    y = np.asarray(y, float)
    codes = _orig["e4m3_encode"](y)
    vals = po.e4m3_decode(codes)
    over = np.abs(vals) > np.abs(y)
    dn = np.where(over & ((codes & 0x7F) > 0), codes - 1, codes).astype(np.uint8)
    return dn


def _encode_ties_odd(y):
    y = np.asarray(y, float)
    codes = _orig["e4m3_encode"](y)
    vals = po.e4m3_decode(codes)
    out = codes.copy()
    for i, (c, v, t) in enumerate(zip(codes.ravel(), vals.ravel(), y.ravel())):
        for nb in (int(c) - 1, int(c) + 1):
            if 0 <= nb < 256 and (nb & 0x7F) != 0x7F and (nb & 0x80) == (c & 0x80):
                if abs(po.e4m3_decode(np.uint8(nb)) - t) == abs(v - t) and nb & 1:
                    out.ravel()[i] = nb
    return out


def _scale_doubled(x):
    return 2.0 * _orig["e4m3_block_scale"](x)


def _dominance_calls():
    return [lambda s=s: pins.test_memory_update_respects_score_dominance(s) for s in range(30)] + \
        [pins.test_memory_update_strict_dominance_breaks_equal_maxima,
         pins.test_rollout_updates_respect_score_dominance]


CASES = {
    "memory score negated": ("memory_scores", _memory_negated, _dominance_calls),
    "memory score summed over the wrong axis": ("memory_scores", _memory_rows, _dominance_calls),
    "memory score max instead of aggregate": ("memory_scores", _memory_max, _dominance_calls),
    "ties to the higher id": ("top_ids", _top_ids_high_tie, lambda: [
        pins.test_top_ids_ties_go_to_lower_id] + [
        lambda s=s: pins.test_top_ids_brute_force_over_subsets(s) for s in range(20)]),
    "frame rep as mean of block reps": ("mean_pool", _pool_block_mean, lambda: [
        pins.test_frame_rep_is_token_mean_not_mean_of_block_reps]),
    "score scale dropped": ("coarse_scores", _scores_no_scale, lambda: [
        pins.test_coarse_scores_orthonormal_closed_form]),
    "dK sign flipped": ("masked_attention_grad", _grad_dk_sign, lambda: [
        lambda: pins.test_attention_grad_matches_autograd_and_finite_differences(0)]),
    "LSE in base 2": ("masked_attention", _attn_lse_log2, lambda: [
        lambda: pins.test_masked_attention_matches_library_sdpa(0)]),
    "last history frame not forced": ("two_level_frames", _frames_no_last, lambda: [
        pins.test_two_level_reduces_to_dense_and_forces_frames]),
    "budget truncated instead of rounded": ("cag_budgets", _budget_floor, lambda: [
        pins.test_cag_budget_reading_and_identity_closed_form]),
    "fp8 encode truncating": ("e4m3_encode", _encode_truncating, lambda: [
        pins.test_e4m3_encode_is_nearest_with_ties_to_even]),
    "fp8 encode ties to odd": ("e4m3_encode", _encode_ties_odd, lambda: [
        pins.test_e4m3_encode_is_nearest_with_ties_to_even]),
    "fp8 block scale one step large": ("e4m3_block_scale", _scale_doubled, lambda: [
        pins.test_e4m3_block_scale_is_the_smallest_power_of_two]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_planted_mistake_fails_a_pin(case, monkeypatch):
    name, fn, calls = CASES[case]
    _patch(monkeypatch, name, fn)
    assert _fails(calls()) > 0, f"no pin caught: {case}"


def test_pins_pass_unpatched():
    for case in sorted(CASES):
        _, _, calls = CASES[case]
        assert _fails(calls()) == 0, case
