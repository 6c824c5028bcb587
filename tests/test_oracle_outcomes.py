"""Pins of the oracle's verification-outcome distribution.

Source: "Speculative Speculative Decoding", "Method" (an outcome is the
accepted prefix length plus the bonus token's identity) and "Key claims"
(the bonus follows the residual max(p_t - p_d, 0); beta down-weights the
draft's likeliest tokens).  The closed form is checked against a brute-force
walk of the accept/reject procedure over every draft tuple, against the
oracle's own sampler, and against special cases with known answers.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

from pins import (binom_pvalue, chi2_pvalue, draft_law, exact_values, sample_categorical, softmax,
                  to_bf16_bits)


def _rows(rng, V, K, spread=1.2, noise=1.0):
    base = rng.normal(size=(K + 1, V)) * spread
    tgt = (base + noise * rng.normal(size=(K + 1, V))).astype(np.float32)
    drf = base[:K].astype(np.float32)
    return tgt, drf


def _laws(traw, draw_, T, beta):
    K = draw_.shape[0]
    Tq = float(np.float32(T))
    tz, dz = exact_values(traw), exact_values(draw_)
    p = [softmax(tz[i], Tq) for i in range(K + 1)]
    q = [draft_law(dz[i], Tq, beta) for i in range(K)]
    return p, q


def _brute_force_joint(p, q):
    """P(n = k, bonus = v) by walking the verify procedure for every draft
    tuple x (drawn with prob prod q_j(x_j)): position j accepts x_j with prob
    min(1, p_j(x_j)/q_j(x_j)); the first rejection at k emits v with the
    normalised clamped residual; after K acceptances the bonus follows p_K."""
    K = len(q)
    V = p[0].size
    joint = np.zeros((K + 1, V))
    for x in itertools.product(range(V), repeat=K):
        w = 1.0
        for j in range(K):
            w *= q[j][x[j]]
        if w == 0.0:
            continue
        reach = w
        for j in range(K):
            a = min(1.0, p[j][x[j]] / q[j][x[j]])
            rej = reach * (1.0 - a)
            if rej > 0.0:
                res = np.maximum(p[j] - q[j], 0.0)
                joint[j] += rej * res / res.sum()
            reach *= a
            if reach == 0.0:
                break
        joint[K] += reach * p[K]
    return joint


def _ranked(mass, F):
    """(tokens, masses) of the F largest positive masses, ties to the lower token."""
    order = np.lexsort((np.arange(mass.size), -mass))
    toks = np.full(F, -1, dtype=np.int32)
    vals = np.zeros(F)
    j = 0
    for v in order:
        if j == F or not mass[v] > 0.0:
            break
        toks[j], vals[j] = v, mass[v]
        j += 1
    return toks, vals


BRUTE_CASES = [
    # V, K, T, beta, dtype
    (4, 2, 1.0, 1.0, "fp32"),
    (6, 2, 0.7, 0.5, "fp32"),
    (5, 3, 1.3, 0.0, "bf16"),
    (7, 2, 0.5, 0.25, "bf16"),
    (3, 1, 2.0, 1.0, "bf16"),
]


@pytest.mark.parametrize("V,K,T,beta,dtype", BRUTE_CASES)
def test_outcomes_match_brute_force_over_drafts(oracle_mod, V, K, T, beta, dtype):
    """Pin: accept rates, the length law and the ranked residual masses equal
    what a walk of the procedure over all V^K draft tuples gives."""
    rng = np.random.default_rng(300 + V * 7 + K)
    tgt, drf = _rows(rng, V, K)
    if dtype == "bf16":
        traw, draw_ = to_bf16_bits(tgt), to_bf16_bits(drf)
    else:
        traw, draw_ = tgt, drf
    p, q = _laws(traw, draw_, T, beta)
    joint = _brute_force_joint(p, q)
    assert abs(joint.sum() - 1.0) < 1e-12
    p_len = joint.sum(axis=1)
    reach = np.cumsum(p_len[::-1])[::-1]          # P(n >= k)
    F = V + 1                                     # more slots than tokens
    res = oracle_mod.outcomes(traw[None], draw_[None], np.float32(T), beta, F=F)
    assert res["error"] == 0
    np.testing.assert_allclose(res["p_len"][0], p_len, rtol=1e-10, atol=1e-14)
    for k in range(K):
        np.testing.assert_allclose(res["accept_rate"][0, k], reach[k + 1] / reach[k], rtol=1e-10)
    for k in range(K + 1):
        toks, vals = _ranked(joint[k] / reach[k], F)
        got_t, got_m = res["top_tokens"][0, k], res["top_mass"][0, k]
        np.testing.assert_allclose(got_m, vals, rtol=1e-9, atol=1e-14)
        # tokens agree wherever the brute-force masses are not near-ties
        for f in range(F):
            if toks[f] < 0:
                assert got_t[f] == -1
                continue
            near = np.abs(joint[k] / reach[k] - vals[f]) <= 1e-9 * max(vals[f], 1e-300)
            assert near[got_t[f]], f"position {k} slot {f}"


def test_outcome_law_matches_the_sampler_chi2(oracle_mod):
    """Pin: the oracle's own sampler, run with drafts drawn from the draft
    law, realises (n, bonus) with the joint law p_len / ranked masses give."""
    rng = np.random.default_rng(77)
    V, K, T, beta = 5, 2, 0.9, 0.5
    tgt, drf = _rows(rng, V, K)
    p, q = _laws(tgt, drf, T, beta)
    ntrials = 200_000
    tokens = np.stack([sample_categorical(rng, q[i], ntrials) for i in range(K)], axis=1)
    target = np.ascontiguousarray(np.broadcast_to(tgt, (ntrials,) + tgt.shape))
    draft = np.ascontiguousarray(np.broadcast_to(drf, (ntrials,) + drf.shape))
    run = oracle_mod.spec_verify(target, draft, tokens.astype(np.int32), 91, np.float32(T), beta)
    assert run["error"] == 0
    n = run["accepted_len"]
    bonus = run["out_tokens"][np.arange(ntrials), n]
    res = oracle_mod.outcomes(tgt[None], drf[None], np.float32(T), beta, F=V)
    reach = np.concatenate(([1.0], np.cumprod(res["accept_rate"][0])))
    law = np.zeros((K + 1, V))
    for k in range(K + 1):
        for t, m in zip(res["top_tokens"][0, k], res["top_mass"][0, k]):
            if t >= 0:
                law[k, t] = reach[k] * m
    np.testing.assert_allclose(law.sum(axis=1), res["p_len"][0], rtol=1e-12)
    counts = np.zeros((K + 1, V))
    np.add.at(counts, (n, bonus), 1)
    assert chi2_pvalue(counts.ravel(), law.ravel()) > 0.01
    assert chi2_pvalue(np.bincount(n, minlength=K + 1), res["p_len"][0]) > 0.01


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_outcomes_of_identical_rows(oracle_mod, dtype):
    """Pin: a draft equal to the target accepts every position (alpha = 1),
    the length law is all on n = K, no residual is left before K, and the
    bonus slots at K are the target law's F likeliest tokens."""
    rng = np.random.default_rng(3)
    V, K, F = 50, 3, 6
    tgt = (rng.normal(size=(K + 1, V)) * 2).astype(np.float32)
    traw = to_bf16_bits(tgt) if dtype == "bf16" else tgt
    res = oracle_mod.outcomes(traw[None], np.ascontiguousarray(traw[None, :K]), np.float32(0.8), 1.0, F=F)
    assert res["error"] == 0
    np.testing.assert_allclose(res["accept_rate"][0], 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(res["p_len"][0, :K], 0.0, atol=1e-13)
    assert abs(res["p_len"][0, K] - 1.0) < 1e-13
    assert np.all(res["top_tokens"][0, :K] == -1) and np.all(res["top_mass"][0, :K] == 0.0)
    pK = softmax(exact_values(traw)[K], float(np.float32(0.8)))
    toks, vals = _ranked(pK, F)
    assert list(res["top_tokens"][0, K]) == list(toks)
    np.testing.assert_allclose(res["top_mass"][0, K], vals, rtol=1e-12)


def test_outcomes_of_disjoint_laws(oracle_mod):
    """Pin: a one-hot target the draft never proposes gives alpha = 0, so
    n = 0 surely and the bonus is the target's token with mass one."""
    V, K = 30, 2
    tgt = np.zeros((K + 1, V), dtype=np.float32)
    tgt[:, 4] = 1e4
    drf = np.zeros((K, V), dtype=np.float32)
    drf[:, 4] = -1e4
    res = oracle_mod.outcomes(tgt[None], drf[None], np.float32(1.0), 1.0, F=3)
    assert res["error"] == 0
    np.testing.assert_allclose(res["accept_rate"][0], 0.0, atol=1e-12)
    np.testing.assert_allclose(res["p_len"][0], [1.0, 0.0, 0.0], atol=1e-12)
    assert list(res["top_tokens"][0, 0]) == [4, -1, -1]
    np.testing.assert_allclose(res["top_mass"][0, 0, 0], 1.0, rtol=1e-12)


def test_outcome_edge_cases(oracle_mod):
    """Pin: K = 0 puts all mass on n = 0 with the target's top tokens;
    greedy and invalid-temperature sequences get NaN / -1 / 0, the latter
    flagged; a missing draft with K > 0 is flagged; F = 0 is allowed."""
    rng = np.random.default_rng(8)
    V = 40
    t0 = rng.normal(size=(2, 1, V)).astype(np.float32)
    res = oracle_mod.outcomes(t0, None, np.float32(1.0), 1.0, F=2)
    assert res["error"] == 0 and res["accept_rate"].shape == (2, 0)
    np.testing.assert_array_equal(res["p_len"], 1.0)
    toks, vals = _ranked(softmax(t0[1, 0], 1.0), 2)
    assert list(res["top_tokens"][1, 0]) == list(toks)
    np.testing.assert_allclose(res["top_mass"][1, 0], vals, rtol=1e-12)

    K = 2
    tgt = rng.normal(size=(3, K + 1, V)).astype(np.float32)
    drf = rng.normal(size=(3, K, V)).astype(np.float32)
    temp = np.array([0.0, np.nan, 1.0], dtype=np.float32)
    res = oracle_mod.outcomes(tgt, drf, temp, 1.0, F=3)
    assert list(res["seq_error"]) == [0, oracle_mod.ERR_TEMPERATURE, 0]
    for b in (0, 1):
        assert np.all(np.isnan(res["accept_rate"][b])) and np.all(np.isnan(res["p_len"][b]))
        assert np.all(res["top_tokens"][b] == -1) and np.all(res["top_mass"][b] == 0.0)
    assert abs(res["p_len"][2].sum() - 1.0) < 1e-12

    res = oracle_mod.outcomes(tgt, None, np.float32(1.0), 1.0, F=3)
    assert np.all(res["seq_error"] == oracle_mod.ERR_NO_DRAFT)

    res = oracle_mod.outcomes(tgt, drf, np.float32(1.0), 1.0, F=0)
    assert res["error"] == 0 and res["top_tokens"].shape == (3, K + 1, 0)


def test_residual_masses_sum_to_the_rejection_probability(oracle_mod):
    """Pin: with F = V the ranked residual masses at k < K sum to
    1 - alpha_k, and at K to one."""
    rng = np.random.default_rng(12)
    V, K = 300, 4
    tgt, drf = _rows(rng, V, K, noise=0.6)
    res = oracle_mod.outcomes(tgt[None], drf[None], np.float32(0.7), 0.3, F=V)
    assert res["error"] == 0
    sums = res["top_mass"][0].sum(axis=1)
    np.testing.assert_allclose(sums[:K], 1.0 - res["accept_rate"][0], rtol=1e-10)
    assert abs(sums[K] - 1.0) < 1e-12


def test_ranked_bonus_tokens_break_ties_to_the_lower_token(oracle_mod):
    """Pin: equal masses (from equal logits) are ranked by token, ascending,
    as a full (mass desc, token asc) sort ranks them."""
    rng = np.random.default_rng(21)
    V, K, F = 24, 1, 10
    for trial in range(20):
        tgt = rng.integers(-2, 3, size=(K + 1, V)).astype(np.float32)
        drf = rng.integers(-2, 3, size=(K, V)).astype(np.float32)
        res = oracle_mod.outcomes(tgt[None], drf[None], np.float32(1.0), 1.0, F=F)
        p, q = _laws(tgt, drf, 1.0, 1.0)
        for k, mass in ((0, np.maximum(p[0] - q[0], 0.0)), (1, p[1])):
            toks, vals = _ranked(mass, F)
            assert list(res["top_tokens"][0, k]) == list(toks), (trial, k)
            np.testing.assert_allclose(res["top_mass"][0, k], vals, rtol=1e-12, atol=1e-15)


def test_outcome_row_failures_are_all_reported(oracle_mod):
    """Pin: a sequence whose rows fail in several ways reports every failure
    (a target row with no finite logit; a beta = 0 draft row with no mass
    outside its top-4) and gets NaN / -1 / 0; other sequences are untouched."""
    rng = np.random.default_rng(31)
    V, K = 6, 2
    tgt = rng.normal(size=(2, K + 1, V)).astype(np.float32)
    drf = rng.normal(size=(2, K, V)).astype(np.float32)
    tgt[0, 0, :] = -np.inf
    drf[0, 1, 4:] = -np.inf
    res = oracle_mod.outcomes(tgt, drf, np.float32(1.0), 0.0, F=2)
    assert res["seq_error"][0] == oracle_mod.ERR_ROW | oracle_mod.ERR_DRAFT_MASS
    assert np.all(np.isnan(res["p_len"][0])) and np.all(res["top_tokens"][0] == -1)
    assert res["seq_error"][1] == 0 and abs(res["p_len"][1].sum() - 1.0) < 1e-12


# --------------------------------------------------------------------------
# Residual mass on the draft's top-4 (the tokens beta down-weights), the
# quantity behind the hit rate of SSD's speculation cache ("Key claims":
# Saguaro sampling concentrates the residual on the draft's likeliest tokens).

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_draft_top_mass_closed_forms_and_monotone_in_beta(oracle_mod, dtype):
    """Pin: sum over the draft row's top-4 of max(p - q'_beta, 0), with q'_beta
    from the pins' own draft law; at beta = 0 it is p(top-4) (q' vanishes
    there); and it never grows with beta (q'_beta on the top-4 is
    beta q / (1 - (1 - beta) q(top-4)), increasing in beta)."""
    rng = np.random.default_rng(41)
    V, K, T = 3000, 3, 0.8
    tgt, drf = _rows(rng, V, K, noise=0.7)
    traw, draw_ = (to_bf16_bits(tgt), to_bf16_bits(drf)) if dtype == "bf16" else (tgt, drf)
    prev = None
    for beta in (1.0, 0.8, 0.5, 0.2, 0.05, 0.0):
        res = oracle_mod.outcomes(traw[None], draw_[None], np.float32(T), beta, F=2)
        assert res["error"] == 0
        p, q = _laws(traw, draw_, T, beta)
        dz = exact_values(draw_)
        for k in range(K):
            top = np.lexsort((np.arange(V), -dz[k]))[:4]
            want = np.maximum(p[k] - q[k], 0.0)[top].sum()
            assert abs(res["draft_top_mass"][0, k] - want) < 1e-12
            if beta == 0.0:
                assert abs(res["draft_top_mass"][0, k] - p[k][top].sum()) < 1e-12
        if prev is not None:
            assert np.all(res["draft_top_mass"][0] >= prev - 1e-15)
        prev = res["draft_top_mass"][0]


def test_draft_top_mass_is_the_sampler_hit_rate(oracle_mod):
    """Pin: the oracle's sampler, with drafts from the beta-weighted draft
    law, emits its bonus among the draft row's top-4 with probability
    sum_k P(n = k) draft_top_mass_k / (1 - alpha_k) over rejections."""
    rng = np.random.default_rng(43)
    V, K, T, beta = 40, 2, 1.0, 0.3
    tgt, drf = _rows(rng, V, K, noise=0.8)
    p, q = _laws(tgt, drf, T, beta)
    ntrials = 200_000
    tokens = np.stack([sample_categorical(rng, q[i], ntrials) for i in range(K)], axis=1)
    target = np.ascontiguousarray(np.broadcast_to(tgt, (ntrials,) + tgt.shape))
    draft = np.ascontiguousarray(np.broadcast_to(drf, (ntrials,) + drf.shape))
    run = oracle_mod.spec_verify(target, draft, tokens.astype(np.int32), 5, np.float32(T), beta)
    n = run["accepted_len"]
    bonus = run["out_tokens"][np.arange(ntrials), n]
    res = oracle_mod.outcomes(tgt[None], drf[None], np.float32(T), beta, F=1)
    reach = np.concatenate(([1.0], np.cumprod(res["accept_rate"][0])))
    for k in range(K):
        top = set(np.lexsort((np.arange(V), -drf[k].astype(np.float64)))[:4].tolist())
        hit = np.array([b in top for b in bonus[n == k]])
        want = min(1.0, res["draft_top_mass"][0, k] / (1.0 - res["accept_rate"][0, k]))
        assert binom_pvalue(int(hit.sum()), int(hit.size), want) > 0.01, k
        assert abs((n == k).mean() - reach[k] * (1 - res["accept_rate"][0, k])) < 5e-3
