"""Pins of the CPU oracle to what the pages and mathematics fix.

Each test names what it pins.  Sources (page title, section):
  K  = "Kangaroo: Self-Speculative Decoding via Shallow Sub-Networks",
       "3. Lossless Speculative Verification" (accept rule, clamped residual,
       exact output law) and its simulation listing (one bonus token);
  G  = glossary "speculative decoding llm", "Why It Produces Identical
       Outputs" (same rule, identical output law) and "Speedup Analysis";
  S  = "Speculative Speculative Decoding", "Key claims" / "Method" (bonus from
       the residual max(p_t - p_d, 0); beta down-weights the likeliest draft
       probabilities);
  L  = "LayerSkip Guide: Early Exit & Self-Speculative Decoding",
       "2. The Drafting and Single-Pass Verification Pipeline" (greedy match).
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.special

from pins import (binom_pvalue, chi2_pvalue, draft_law, exact_values, sample_categorical,
                  softmax, to_bf16_bits, top4_by_sort)

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


# --------------------------------------------------------------------------
# Philox4x32-10 against an independent library implementation (rocRAND).

def _rocrand_philox(tmp_path, rows: np.ndarray) -> np.ndarray:
    gxx = shutil.which("g++")
    inc = "/opt/rocm/include"
    if gxx is None or not os.path.exists(os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("g++ or rocRAND headers not available")
    exe = str(tmp_path / "rr_philox")
    subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{inc}",
                    os.path.join(HERE, "rocrand_philox_probe.cpp"), "-o", exe], check=True)
    text = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()],
                    dtype=np.uint64)


def test_philox_matches_rocrand(oracle_mod, tmp_path):
    """Pin: the oracle's Philox4x32-10 equals rocRAND's on random and extreme
    (counter, key) pairs."""
    rng = np.random.default_rng(123)
    rows = rng.integers(0, 2**32, size=(2000, 6), dtype=np.uint64)
    rows[0] = 0
    rows[1] = 2**32 - 1
    rows[2] = [7, 0, 1, 0, 0, 0]  # the (b, pos, purpose, 0) counter shape
    ref = _rocrand_philox(tmp_path, rows)
    for r, want in zip(rows, ref):
        got = oracle_mod.philox4x32_10(r[:4], r[4:])
        assert [int(v) for v in got] == [int(v) for v in want]


def test_uniforms_use_first_word_and_are_uniform(oracle_mod, tmp_path):
    """Pin: u(seed, b, pos, purpose) is the first rocRAND output word of
    counter (b, pos, purpose, 0) and key (seed_lo, seed_hi), mapped into
    (0, 1] on a 2^-24 grid; over many counters it is uniform (chi-square)."""
    seeds = [0, 1, 0xDEADBEEFCAFEF00D]
    rows, us = [], []
    for s in seeds:
        for b in range(40):
            for pos in range(6):
                for purpose in (0, 1):
                    rows.append([b, pos, purpose, 0, s & 0xFFFFFFFF, s >> 32])
                    us.append(oracle_mod.uniform(s, b, pos, purpose))
    ref = _rocrand_philox(tmp_path, np.array(rows, dtype=np.uint64))
    us = np.array(us)
    grid = us * 2**24
    assert np.all(us > 0.0) and np.all(us <= 1.0)
    assert np.all(grid == np.round(grid))
    assert np.array_equal(grid.astype(np.uint64) - 1, ref[:, 0] >> np.uint64(8))
    # uniformity over 20 equal bins
    hist = np.histogram(us, bins=20, range=(0.0, 1.0))[0]
    assert chi2_pvalue(hist, np.full(20, 1 / 20)) > 0.01


# --------------------------------------------------------------------------
# Row statistics against library routines.

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [0.35, 0.7, 1.0, 1.9])
def test_lognorm_matches_scipy_logsumexp(oracle_mod, dtype, T):
    """Pin: L = log sum exp(z / T) equals scipy.special.logsumexp."""
    rng = np.random.default_rng(5)
    for V in (1, 7, 1000, 32000):
        z = (rng.normal(size=V) * 4).astype(np.float32)
        z[rng.integers(0, V)] = -np.inf if V > 1 else z[0]
        raw = to_bf16_bits(z) if dtype == "bf16" else z
        zz = exact_values(raw)
        want = scipy.special.logsumexp(zz / np.float64(np.float32(T)))
        got = oracle_mod.row_lognorm(raw, np.float32(T))
        assert abs(got - want) <= 1e-12 * max(1.0, abs(want))
        assert oracle_mod.row_max(raw) == np.max(zz)


def test_argmax_and_top4_match_sorting_with_ties(oracle_mod):
    """Pin: argmax is numpy's (first index on ties); the top-4 is the first 4
    entries of a full (value desc, index asc) sort."""
    rng = np.random.default_rng(9)
    for trial in range(300):
        V = int(rng.integers(1, 40))
        z = rng.integers(-3, 4, size=V).astype(np.float32)  # many ties
        for raw in (z, to_bf16_bits(z)):
            assert oracle_mod.row_argmax(raw) == int(np.argmax(z))
            assert oracle_mod.row_top4(raw) == [int(i) for i in top4_by_sort(z)]


def test_beta_draft_law_invariants(oracle_mod):
    """Pin (S, reading of beta): the weighted draft law sums to one, equals
    softmax(z/T) at beta = 1, is zero on the top-4 at beta = 0, and keeps the
    softmax's ratios inside and outside the top-4 with a factor beta between."""
    rng = np.random.default_rng(11)
    for V in (5, 6, 50, 3000):
        z = (rng.normal(size=V) * 2).astype(np.float32)
        T = 0.8
        p = softmax(z, np.float32(T))
        top = top4_by_sort(z)
        rest = np.setdiff1d(np.arange(V), top)
        for beta in (1.0, 0.5, 0.1, 0.0):
            q = np.exp(oracle_mod.draft_logprobs(z, np.float32(T), beta))
            assert abs(q.sum() - 1.0) < 1e-12
            if beta == 1.0:
                np.testing.assert_allclose(q, p, rtol=1e-12, atol=0)
                continue
            r_rest = q[rest] / p[rest]
            np.testing.assert_allclose(r_rest, r_rest[0], rtol=1e-12)
            if beta == 0.0:
                assert np.all(q[top] == 0.0)
            else:
                np.testing.assert_allclose(q[top] / p[top], beta * r_rest[0], rtol=1e-12)


# --------------------------------------------------------------------------
# The output law: losslessness and the accept probability.

def _fixed_rows(rng, V, K, spread=1.5, noise=0.9):
    base = rng.normal(size=(K + 1, V)) * spread
    tgt = (base + noise * rng.normal(size=(K + 1, V))).astype(np.float32)
    drf = base[:K].astype(np.float32)
    return tgt, drf


def _run_trials(oracle_mod, tgt, drf, T, beta, dtype, ntrials, seed, rng):
    K1, V = tgt.shape
    K = K1 - 1
    if dtype == "bf16":
        traw, draw_ = to_bf16_bits(tgt), to_bf16_bits(drf)
    else:
        traw, draw_ = tgt, drf
    tz, dz = exact_values(traw), exact_values(draw_)
    Tq = float(np.float32(T))
    p = [softmax(tz[i], Tq) for i in range(K + 1)]
    q = [draft_law(dz[i], Tq, beta) for i in range(K)]
    tokens = np.stack([sample_categorical(rng, q[i], ntrials) for i in range(K)], axis=1)
    target = np.ascontiguousarray(np.broadcast_to(traw, (ntrials,) + traw.shape))
    draft = np.ascontiguousarray(np.broadcast_to(draw_, (ntrials,) + draw_.shape))
    res = oracle_mod.spec_verify(target, draft, tokens.astype(np.int32), seed, np.float32(T), beta)
    assert res["error"] == 0
    return res, p, q, tokens


LAW_CASES = [
    # V, K, T, beta, dtype
    (8, 2, 1.0, 1.0, "fp32"),
    (16, 2, 0.5, 0.5, "fp32"),
    (12, 1, 2.0, 0.0, "bf16"),
    (6, 2, 0.7, 0.5, "bf16"),
]


@pytest.mark.slow
@pytest.mark.parametrize("V,K,T,beta,dtype", LAW_CASES)
def test_output_law_is_target_law_chi2(oracle_mod, V, K, T, beta, dtype):
    """Pin (K, G: the emitted tokens follow the target law): over 10^6
    trials with drafts drawn from the (beta-weighted) draft law, the token
    emitted at every reached position i follows p_i (chi-square p > 0.01),
    and the accept probability at position i is sum_v min(p_i, q_i)."""
    rng = np.random.default_rng(1000 + V * 10 + K)
    tgt, drf = _fixed_rows(rng, V, K)
    ntrials = 1_000_000
    res, p, q, tokens = _run_trials(oracle_mod, tgt, drf, T, beta, dtype, ntrials, 77, rng)
    n = res["accepted_len"]
    out = res["out_tokens"]
    for i in range(K + 1):
        reached = n >= i
        y = out[reached, i]
        assert np.all(y >= 0)
        counts = np.bincount(y, minlength=V)
        assert chi2_pvalue(counts, p[i]) > 0.01, f"position {i}"
        if i < K:
            alpha = np.minimum(p[i], q[i]).sum()
            assert binom_pvalue(int((n[reached] > i).sum()), int(reached.sum()), alpha) > 0.01
    # accepted prefix equals the drafts; padding after the bonus
    for b in range(0, ntrials, 9973):
        k = n[b]
        assert list(out[b, :k]) == list(tokens[b, :k])
        assert np.all(out[b, k + 1:] == -1)


@pytest.mark.slow
def test_joint_law_small_case(oracle_mod):
    """Pin: for V=3, K=2 the joint law of (n, y_0..y_n) equals the product of
    min(p_j, q_j) over accepted positions times the clamped residual (or p_K
    after K acceptances), over all 3 + 9 + 27 cells."""
    rng = np.random.default_rng(42)
    V, K, T = 3, 2, 0.9
    tgt, drf = _fixed_rows(rng, V, K, spread=1.0, noise=1.0)
    res, p, q, _ = _run_trials(oracle_mod, tgt, drf, T, 1.0, "fp32", 1_000_000, 5, rng)
    n, out = res["accepted_len"], res["out_tokens"]
    cells, probs, counts = {}, [], []
    keyed = {}
    for b_n, row in zip(n, out):
        key = (int(b_n),) + tuple(int(t) for t in row[: b_n + 1])
        keyed[key] = keyed.get(key, 0) + 1
    for k in range(K + 1):
        for ys in np.ndindex(*([V] * (k + 1))):
            pr = 1.0
            for j in range(k):
                pr *= min(p[j][ys[j]], q[j][ys[j]])
            last = ys[k]
            pr *= max(p[k][last] - q[k][last], 0.0) if k < K else p[K][last]
            cells[(k,) + ys] = pr
    assert abs(sum(cells.values()) - 1.0) < 1e-12
    assert set(keyed) <= set(cells)
    for key, pr in cells.items():
        probs.append(pr)
        counts.append(keyed.get(key, 0))
    assert chi2_pvalue(np.array(counts), np.array(probs)) > 0.01


def test_glossary_example_alpha_070_k5(oracle_mod):
    """Pin (G, "Speedup Analysis"): with acceptance 0.7 at each of K=5
    positions, the mean number of accepted drafts is sum_{k=1..5} 0.7^k and
    tokens per step is one more.  The glossary's printed "~3.5" equals
    alpha*K, not this expectation (recorded in the golden fixture)."""
    with open(os.path.join(GOLDEN, "glossary_alpha070_k5.json")) as f:
        gold = json.load(f)
    alpha, K = gold["alpha"], gold["K"]
    # V=2: p = (0.5, 0.5), q = (0.8, 0.2) gives sum min(p, q) = 0.7 exactly in law
    tgt = np.zeros((K + 1, 2), dtype=np.float32)
    drf = np.tile(np.array([np.log(0.8), np.log(0.2)], dtype=np.float32), (K, 1))
    rng = np.random.default_rng(3)
    ntr = 400_000
    res, p, q, _ = _run_trials(oracle_mod, tgt, drf, 1.0, 1.0, "fp32", ntr, 11, rng)
    a = np.minimum(p[0], q[0]).sum()
    assert abs(a - alpha) < 1e-6
    n = res["accepted_len"].astype(np.float64)
    want = sum(a ** k for k in range(1, K + 1))
    assert abs(want - 1.94117) < 1e-5  # 0.7 + 0.49 + 0.343 + 0.2401 + 0.16807
    sd = n.std() / np.sqrt(ntr)
    assert abs(n.mean() - want) < 4 * sd
    assert abs(gold["page_printed"] - alpha * K) < 1e-9


# --------------------------------------------------------------------------
# Deterministic special cases.

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_identical_rows_accept_everything(oracle_mod, dtype):
    """Pin (ratio p/q = 1): when draft rows equal target rows every draft is
    accepted and the bonus comes from target row K."""
    rng = np.random.default_rng(21)
    B, K, V = 64, 5, 300
    tgt = (rng.normal(size=(B, K + 1, V)) * 3).astype(np.float32)
    traw = to_bf16_bits(tgt) if dtype == "bf16" else tgt
    draw_ = np.ascontiguousarray(traw[:, :K])
    temps = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, K)).astype(np.int32)
    res = oracle_mod.spec_verify(traw, draw_, tokens, 99, temps, 1.0)
    assert np.all(res["accepted_len"] == K)
    assert np.array_equal(res["out_tokens"][:, :K], tokens)
    # bonus = inverse CDF of softmax(row K / T) at u(seed, b, K, BONUS)
    tz = exact_values(traw)
    for b in range(B):
        if res["margin_bonus"][b] < 1e-9:
            continue
        cdf = np.cumsum(softmax(tz[b, K], temps[b]))
        u = oracle_mod.uniform(99, b, K, 1)
        want = int(np.searchsorted(cdf, u * cdf[-1], side="left"))
        assert res["out_tokens"][b, K] == want


def test_one_hot_target_always_rejects(oracle_mod):
    """Pin: a target law concentrated on a != x rejects x and emits a."""
    rng = np.random.default_rng(4)
    B, K, V = 200, 3, 40
    tgt = np.full((B, K + 1, V), -60.0, dtype=np.float32)
    a = rng.integers(0, V, size=(B, K + 1))
    for b in range(B):
        for i in range(K + 1):
            tgt[b, i, a[b, i]] = 60.0
    drf = (rng.normal(size=(B, K, V))).astype(np.float32)
    tokens = (a[:, :K] + 1 + rng.integers(0, V - 1, size=(B, K))) % V
    res = oracle_mod.spec_verify(tgt, drf, tokens.astype(np.int32), 1, 1.0, 1.0)
    assert np.all(res["accepted_len"] == 0)
    assert np.array_equal(res["out_tokens"][:, 0], a[:, 0])


@pytest.mark.slow
def test_one_hot_draft_textbook_rejection(oracle_mod):
    """Pin: a draft law concentrated on x accepts with probability p_t(x); on
    rejection the bonus follows p_t with x removed and renormalised."""
    rng = np.random.default_rng(8)
    V, K, ntr = 10, 1, 400_000
    tz = (rng.normal(size=(K + 1, V)) * 1.2).astype(np.float32)
    x = 3
    dz = np.full((K, V), -80.0, dtype=np.float32)
    dz[0, x] = 80.0
    target = np.ascontiguousarray(np.broadcast_to(tz, (ntr, K + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(dz, (ntr, K, V)))
    tokens = np.full((ntr, K), x, dtype=np.int32)
    res = oracle_mod.spec_verify(target, draft, tokens, 17, 1.0, 1.0)
    p0 = softmax(tz[0], 1.0)
    n = res["accepted_len"]
    assert binom_pvalue(int((n == 1).sum()), ntr, p0[x]) > 0.01
    rej = res["out_tokens"][n == 0, 0]
    law = p0.copy()
    law[x] = 0.0
    law /= law.sum()
    assert chi2_pvalue(np.bincount(rej, minlength=V), law) > 0.01


def test_greedy_matches_argmax_agreement(oracle_mod):
    """Pin (L): at T = 0 drafts are accepted while they equal the target
    argmax (numpy's, first index on ties); the first mismatch, or position K,
    emits the target argmax.  Drafts are never read (None)."""
    rng = np.random.default_rng(31)
    B, K, V = 500, 4, 9
    tgt = rng.integers(-2, 3, size=(B, K + 1, V)).astype(np.float32)  # many ties
    am = tgt.argmax(axis=2)
    tokens = np.where(rng.random((B, K)) < 0.7, am[:, :K], rng.integers(0, V, size=(B, K)))
    for raw in (tgt, to_bf16_bits(tgt)):
        res = oracle_mod.spec_verify(raw, None, tokens.astype(np.int32), 0, 0.0, 0.5)
        for b in range(B):
            n = 0
            while n < K and tokens[b, n] == am[b, n]:
                n += 1
            assert res["accepted_len"][b] == n
            assert list(res["out_tokens"][b, :n]) == list(tokens[b, :n])
            assert res["out_tokens"][b, n] == am[b, n]
            assert np.all(res["out_tokens"][b, n + 1:] == -1)


def test_out_of_range_token_is_rejected_and_flagged(oracle_mod):
    rng = np.random.default_rng(2)
    B, K, V = 4, 3, 50
    tgt = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    drf = np.ascontiguousarray(tgt[:, :K])  # identical rows: would accept all
    tokens = rng.integers(0, V, size=(B, K)).astype(np.int32)
    tokens[1, 1] = V
    tokens[2, 0] = -1
    res = oracle_mod.spec_verify(tgt, drf, tokens, 0, 1.0, 1.0)
    assert res["error"] & oracle_mod.ERR_TOKEN
    assert list(res["accepted_len"]) == [K, 1, 0, K]
    assert list(res["seq_error"]) == [0, 1, 1, 0]


def test_invalid_temperature_flags_sequence(oracle_mod):
    rng = np.random.default_rng(2)
    B, K, V = 4, 2, 20
    tgt = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    drf = rng.normal(size=(B, K, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, K)).astype(np.int32)
    temps = np.array([1.0, -1.0, np.nan, np.inf], dtype=np.float32)
    res = oracle_mod.spec_verify(tgt, drf, tokens, 0, temps, 1.0)
    assert list(res["seq_error"]) == [0, 2, 2, 2]
    assert np.all(res["out_tokens"][1:] == -1) and np.all(res["accepted_len"][1:] == 0)
    assert res["out_tokens"][0, res["accepted_len"][0]] >= 0


def test_results_do_not_depend_on_thread_count(oracle_mod):
    rng = np.random.default_rng(6)
    B, K, V = 33, 3, 257
    tgt = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    drf = rng.normal(size=(B, K, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, K)).astype(np.int32)
    a = oracle_mod.spec_verify(tgt, drf, tokens, 5, 0.8, 0.5, nthreads=1)
    b = oracle_mod.spec_verify(tgt, drf, tokens, 5, 0.8, 0.5, nthreads=4)
    for key in ("accepted_len", "out_tokens", "seq_error"):
        assert np.array_equal(a[key], b[key])
    for key in ("p_target", "p_draft", "residual_mass"):
        assert np.array_equal(a[key], b[key], equal_nan=True)


# --------------------------------------------------------------------------
# Ragged draft lengths (K: the drafter stops early, so a round carries
# K_b <= K drafts) and the exported draft confidence.

def _ragged_batch(rng, B, K, V, dtype):
    tgt = (rng.normal(size=(B, K + 1, V)) * 2).astype(np.float32)
    drf = (tgt[:, :K] + 0.6 * rng.normal(size=(B, K, V))).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    am = drf.argmax(axis=2)
    tok = np.where(rng.random((B, K)) < 0.5, am, tok).astype(np.int32)
    kb = rng.integers(0, K + 1, size=B).astype(np.int32)
    # rows past a sequence's drafts must never be read: poison them
    for b in range(B):
        tgt[b, kb[b] + 1:] = np.nan
        drf[b, kb[b]:] = np.nan
    if dtype == "bf16":
        return to_bf16_bits(tgt), to_bf16_bits(drf), tok, kb
    return tgt, drf, tok, kb


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("beta", [1.0, 0.5])
def test_ragged_sequence_equals_its_truncation(oracle_mod, dtype, beta):
    """Pin (ragged lengths reduce to the plain case): sequence b with K_b
    drafts gives exactly what the K = K_b verify gives on its truncated rows
    (same uniforms: keyed by b, position and purpose), greedy and sampling,
    and never reads the rows past K_b (they hold NaN here)."""
    rng = np.random.default_rng(61 if dtype == "fp32" else 62)
    B, K, V = 40, 5, 300
    tgt, drf, tok, kb = _ragged_batch(rng, B, K, V, dtype)
    temps = rng.choice([0.0, 0.6, 1.0, 1.4], size=B).astype(np.float32)
    res = oracle_mod.spec_verify(tgt, drf, tok, 9, temps, beta, draft_len=kb)
    assert res["error"] & ~oracle_mod.ERR_TOKEN == 0
    for b in range(B):
        k = int(kb[b])
        one = oracle_mod.spec_verify(tgt[b:b + 1, :k + 1], drf[b:b + 1, :k], tok[b:b + 1, :k], 9,
                                     temps[b:b + 1], beta, seq_ids=np.array([b]))
        assert res["accepted_len"][b] == one["accepted_len"][0]
        assert list(res["out_tokens"][b, :k + 1]) == list(one["out_tokens"][0])
        assert np.all(res["out_tokens"][b, k + 1:] == -1)
        assert res["seq_error"][b] == one["seq_error"][0]
        for key in ("p_target", "p_draft", "margin_accept", "draft_conf"):
            assert np.array_equal(res[key][b, :k], one[key][0], equal_nan=True), key
            assert np.all(np.isnan(res[key][b, k:])), key
        for key in ("residual_mass", "margin_bonus"):
            assert np.array_equal(res[key][b:b + 1], one[key], equal_nan=True), key


def test_ragged_length_out_of_range_fails_the_sequence(oracle_mod):
    rng = np.random.default_rng(63)
    B, K, V = 4, 3, 64
    tgt = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    drf = rng.normal(size=(B, K, V)).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    res = oracle_mod.spec_verify(tgt, drf, tok, 0, 1.0, 1.0, draft_len=np.array([3, -1, 4, 0]))
    assert list(res["seq_error"]) == [0, oracle_mod.ERR_DRAFT_LEN, oracle_mod.ERR_DRAFT_LEN, 0]
    assert np.all(res["out_tokens"][1:3] == -1) and np.all(res["accepted_len"][1:3] == 0)
    # K_b = 0: no draft to test, the bonus comes from target row 0
    assert res["accepted_len"][3] == 0 and res["out_tokens"][3, 0] >= 0
    assert np.all(res["out_tokens"][3, 1:] == -1)


@pytest.mark.slow
def test_ragged_output_law_chi2(oracle_mod):
    """Pin (closed-form law per sequence, K): with drafts drawn from the draft
    law and each trial drafting K_b in {0, 1, 2} of K = 2 positions, the
    token emitted at every reached position i <= K_b follows p_i (chi-square
    p > 0.01), the accept probability at i < K_b is sum_v min(p_i, q_i), and
    a trial stops at K_b at the latest."""
    rng = np.random.default_rng(64)
    V, K, T, beta = 10, 2, 0.8, 0.5
    tgt, drf = _fixed_rows(rng, V, K)
    tz, dz = exact_values(tgt), exact_values(drf)
    Tq = float(np.float32(T))
    p = [softmax(tz[i], Tq) for i in range(K + 1)]
    q = [draft_law(dz[i], Tq, beta) for i in range(K)]
    ntrials = 600_000
    tokens = np.stack([sample_categorical(rng, q[i], ntrials) for i in range(K)], axis=1)
    kb = rng.integers(0, K + 1, size=ntrials).astype(np.int32)
    target = np.ascontiguousarray(np.broadcast_to(tgt, (ntrials,) + tgt.shape))
    draft = np.ascontiguousarray(np.broadcast_to(drf, (ntrials,) + drf.shape))
    res = oracle_mod.spec_verify(target, draft, tokens.astype(np.int32), 31, np.float32(T), beta,
                                 draft_len=kb)
    assert res["error"] == 0
    n, out = res["accepted_len"], res["out_tokens"]
    assert np.all(n <= kb)
    for k in range(K + 1):
        grp = kb == k
        for i in range(k + 1):
            reached = grp & (n >= i)
            y = out[reached, i]
            assert np.all(y >= 0)
            assert chi2_pvalue(np.bincount(y, minlength=V), p[i]) > 0.01, (k, i)
            if i < k:
                alpha = np.minimum(p[i], q[i]).sum()
                assert binom_pvalue(int((n[reached] > i).sum()), int(reached.sum()), alpha) > 0.01


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_draft_confidence_is_the_softmax_maximum(oracle_mod, dtype):
    """Pin (library routine): the exported draft confidence of position i is
    max_v softmax(z_d / T) of draft row i (scipy), before the beta
    re-weighting, for every drafted position (reached or not); NaN past K_b,
    for greedy sequences and for failed ones."""
    rng = np.random.default_rng(65)
    B, K, V = 12, 4, 777
    tgt, drf, tok, kb = _ragged_batch(rng, B, K, V, dtype)
    temps = np.array([0.5, 1.0, 1.7, 0.0] * 3, dtype=np.float32)
    temps[5] = -1.0  # invalid: the sequence fails
    for beta in (1.0, 0.3):
        res = oracle_mod.spec_verify(tgt, drf, tok, 4, temps, beta, draft_len=kb)
        conf = res["draft_conf"]
        dz = exact_values(drf)
        for b in range(B):
            for i in range(K):
                if i >= kb[b] or temps[b] <= 0.0:
                    assert np.isnan(conf[b, i]), (b, i)
                    continue
                want = softmax(dz[b, i], float(np.float32(temps[b]))).max()
                assert abs(conf[b, i] - want) <= 1e-12 * want, (b, i, conf[b, i], want)


# --------------------------------------------------------------------------
# Replayed decisions: the parity rule lets two finite-precision paths differ
# at a decision within rounding of its threshold, and then compares the rest
# of the sequence with the oracle replaying that decision the other way.  The
# replay is pinned against ordinary runs on inputs that force the same
# outcome through the method itself: an out-of-range draft token is rejected
# (ratio 0), and a draft token the draft law gives no mass is accepted (ratio
# +inf).  Neither substitution changes any row, so the rest of the sequence
# must come out the same.

def _replay_batch(rng, B, K, V, dtype):
    tgt = (rng.normal(size=(B, K + 1, V)) * 2).astype(np.float32)
    drf = (tgt[:, :K] + 0.7 * rng.normal(size=(B, K, V))).astype(np.float32)
    drf[:, :, V - 1] = -np.inf  # token V-1: no draft mass, always accepted when drafted
    tok = rng.integers(0, V - 1, size=(B, K)).astype(np.int32)
    am = drf.argmax(axis=2)
    tok = np.where(rng.random((B, K)) < 0.6, am, tok).astype(np.int32)
    if dtype == "bf16":
        return to_bf16_bits(tgt), to_bf16_bits(drf), tok
    return tgt, drf, tok


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("beta", [1.0, 0.5])
def test_forced_decisions_equal_token_substitutions(oracle_mod, dtype, beta):
    """Pin (K, accept rule): replaying an accepted position m as a rejection
    gives what the oracle gives with x_m out of range; replaying the rejected
    position n as an acceptance gives what it gives with x_n replaced by a
    token of zero draft mass (up to that token itself)."""
    rng = np.random.default_rng(66 if dtype == "fp32" else 67)
    B, K, V = 160, 4, 61
    tgt, drf, tok = _replay_batch(rng, B, K, V, dtype)
    temps = rng.uniform(0.5, 1.5, size=B).astype(np.float32)
    base = oracle_mod.spec_verify(tgt, drf, tok, 21, temps, beta)
    assert base["error"] == 0
    n = base["accepted_len"]
    assert (n > 0).sum() > 40 and (n < K).sum() > 40
    checked_rej = checked_acc = 0
    for b in range(B):
        ids = np.array([b])
        sl = slice(b, b + 1)
        if n[b] > 0:  # replay an accepted position as a rejection
            m = int(rng.integers(0, n[b]))
            force = np.zeros((1, K), bool)
            force[0, m] = True
            got = oracle_mod.spec_verify(tgt[sl], drf[sl], tok[sl], 21, temps[sl], beta, seq_ids=ids,
                                         force=force)
            t2 = tok[sl].copy()
            t2[0, m] = -1
            want = oracle_mod.spec_verify(tgt[sl], drf[sl], t2, 21, temps[sl], beta, seq_ids=ids)
            assert want["seq_error"][0] == oracle_mod.ERR_TOKEN and got["seq_error"][0] == 0
            assert got["accepted_len"][0] == m == want["accepted_len"][0]
            assert np.array_equal(got["out_tokens"], want["out_tokens"])
            for key in ("residual_mass", "margin_bonus"):
                assert np.array_equal(got[key], want[key]), key
            assert np.array_equal(got["p_target"][0, :m], want["p_target"][0, :m])
            checked_rej += 1
        if n[b] < K:  # replay the rejection at n as an acceptance
            m = int(n[b])
            force = np.zeros((1, K), bool)
            force[0, m] = True
            got = oracle_mod.spec_verify(tgt[sl], drf[sl], tok[sl], 21, temps[sl], beta, seq_ids=ids,
                                         force=force)
            t2 = tok[sl].copy()
            t2[0, m] = V - 1
            want = oracle_mod.spec_verify(tgt[sl], drf[sl], t2, 21, temps[sl], beta, seq_ids=ids)
            assert got["accepted_len"][0] == want["accepted_len"][0] > m
            g_out, w_out = got["out_tokens"][0].copy(), want["out_tokens"][0].copy()
            assert g_out[m] == tok[b, m] and w_out[m] == V - 1
            g_out[m] = w_out[m] = 0
            assert np.array_equal(g_out, w_out)
            for key in ("residual_mass", "margin_bonus"):
                assert np.array_equal(got[key], want[key]), key
            for key in ("p_target", "p_draft", "margin_accept"):
                assert np.array_equal(got[key][0, m + 1:], want[key][0, m + 1:], equal_nan=True), key
            checked_acc += 1
    assert checked_rej > 40 and checked_acc > 40


# --------------------------------------------------------------------------
# Zero residual mass after a rejection (reading of a case the pages leave
# open: the residual max(p_t - q', 0) can only vanish through rounding, and
# the bonus is then drawn from p_t of that position).  Reached on purpose by
# underflow: every token but one has logit -800 in the target row and -790 in
# the draft row, so both laws put all their mass (1 in double precision) on
# the one finite-mass token d, a drafted token x != d has ratio e^-10 (bf16:
# e^-8) and is rejected for almost every u, and the clamped residual is 0 at
# every token.  p_t of that position is then the point mass at d: the bonus
# must be d, and the reported mass C(V-1) of the bonus draw is 1.

def _underflow_case(rng, B, K, V, dtype):
    tgt = np.full((B, K + 1, V), -800.0, dtype=np.float32)
    drf = np.full((B, K, V), -790.0, dtype=np.float32)
    dom = rng.integers(0, V, size=(B, K + 1))
    tok = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for i in range(K + 1):
            tgt[b, i, dom[b, i]] = 0.0
            if i < K:
                drf[b, i, dom[b, i]] = 0.0
                tok[b, i] = (dom[b, i] + 1 + int(rng.integers(0, V - 1))) % V
    if dtype == "bf16":
        return to_bf16_bits(tgt), to_bf16_bits(drf), tok, dom
    return tgt, drf, tok, dom


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V,K", [(2, 1), (2, 3), (5000, 2)])
def test_zero_residual_mass_draws_from_target(oracle_mod, dtype, V, K):
    rng = np.random.default_rng(V + K)
    B = 48
    tgt, drf, tok, dom = _underflow_case(rng, B, K, V, dtype)
    tz, dz = exact_values(tgt), exact_values(drf)
    u = oracle_mod.uniforms(3, B, K + 1)[:, :, 0]
    res = oracle_mod.spec_verify(tgt, drf, tok, 3, np.float32(1.0), 1.0)
    assert res["error"] == 0
    for b in range(B):
        # the accept scan by the rule itself: ratio = p_t(x) / q(x) in log form
        n = K
        for i in range(K):
            x = tok[b, i]
            lt = tz[b, i, x] - scipy.special.logsumexp(tz[b, i])
            ld = dz[b, i, x] - scipy.special.logsumexp(dz[b, i])
            if not u[b, i] <= np.exp(lt - ld):
                n = i
                break
        assert res["accepted_len"][b] == n
        assert n < K  # ratio e^-10 (bf16: e^-8): every sequence rejects here
        # the case is reached: the clamped residual has no mass in double ...
        r = np.maximum(softmax(tz[b, n], 1.0) - softmax(dz[b, n], 1.0), 0.0)
        assert r.sum() == 0.0
        # ... and p_t of that position is the point mass at the finite token
        assert softmax(tz[b, n], 1.0)[dom[b, n]] == 1.0
        assert res["out_tokens"][b, n] == dom[b, n]
        assert np.all(res["out_tokens"][b, n + 1:] == -1)
        assert res["residual_mass"][b] == 1.0
