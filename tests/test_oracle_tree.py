"""Pins of the oracle's tree (multi-draft) verification.

The rule is recursive rejection sampling over a token tree (Miao et al.,
"SpecInfer", ASPLOS'24; the pages name tree-based speculative decoding in
"Speculative Speculative Decoding", Key claims, without a rule).  It is pinned
to the chain verify step (a chain-shaped tree is that step, uniforms
included) and to losslessness: with the children of every context drawn
i.i.d. from its draft law, each emitted token follows the target's
conditional law.
"""
from __future__ import annotations

import numpy as np
import pytest

from pins import chi2_pvalue, sample_categorical, softmax, to_bf16_bits


def _chain(B, N):
    return np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [0.0, 0.6, 1.0, 1.7])
def test_chain_tree_is_the_chain_verify_step(oracle_mod, dtype, T):
    """Pin: parent[i] = i - 1 reproduces spec_verify with K = N exactly."""
    rng = np.random.default_rng(int(T * 10) + (dtype == "bf16"))
    B, N, V = 400, 5, 50
    base = rng.normal(size=(B, N + 1, V)) * 1.5
    tgt = (base + 0.5 * rng.normal(size=base.shape)).astype(np.float32)
    drf = base[:, :N].astype(np.float32)
    tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    if T == 0.0:  # make some drafts the argmax so greedy runs go deep
        am = np.argmax(tgt[:, :N], axis=2)
        pick = rng.random((B, N)) < 0.7
        tok[pick] = am[pick]
    traw, draw_ = (to_bf16_bits(tgt), to_bf16_bits(drf)) if dtype == "bf16" else (tgt, drf)
    for seed in (0, 12345):
        chain = oracle_mod.spec_verify(traw, draw_, tok, seed, np.float32(T), 1.0)
        tree = oracle_mod.spec_verify_tree(traw, draw_, _chain(B, N), tok, seed, np.float32(T))
        assert np.array_equal(chain["accepted_len"], tree["accepted_len"])
        assert np.array_equal(chain["out_tokens"], tree["out_tokens"])
        d = tree["accepted_len"]
        for b in range(B):
            assert list(tree["path"][b, :d[b]]) == list(range(d[b]))
            assert np.all(tree["path"][b, d[b]:] == -1)


def _lossless_case(rng, V):
    """Per-prefix target and draft laws of a depth-2 token tree (tables
    indexed by the prefix tokens)."""
    pz_root = rng.normal(size=V) * 1.2
    qz_root = pz_root + rng.normal(size=V)
    pz1 = rng.normal(size=(V, V)) * 1.2           # target after y1
    qz1 = pz1 + rng.normal(size=(V, V))            # draft after y1
    pz2 = rng.normal(size=(V, V, V)) * 1.2        # target after (y1, y2)
    return pz_root, qz_root, pz1, qz1, pz2


@pytest.mark.slow
@pytest.mark.parametrize("k1,k2", [(3, 2), (2, 3)])
def test_tree_output_law_is_target_law_chi2(oracle_mod, k1, k2):
    """Pin (losslessness): a depth-2 tree whose root has k1 children drawn
    i.i.d. from the root's draft law and whose every child has k2 children
    drawn i.i.d. from its own draft law.  Over 3e5 trials: y1 follows the
    root target law; after an accepted y1, y2 follows the target law after
    y1; after two accepted, the bonus follows the target law after (y1, y2)."""
    rng = np.random.default_rng(100 + 10 * k1 + k2)
    V, T = 6, 1.0
    pz_root, qz_root, pz1, qz1, pz2 = _lossless_case(rng, V)
    p_root, q_root = softmax(pz_root, T), softmax(qz_root, T)
    p1 = np.array([softmax(pz1[y], T) for y in range(V)])
    q1 = np.array([softmax(qz1[y], T) for y in range(V)])
    p2 = np.array([[softmax(pz2[a, c], T) for c in range(V)] for a in range(V)])
    trials = 300_000
    N = k1 + k1 * k2
    parent = np.empty(N, dtype=np.int32)
    parent[:k1] = -1
    for i in range(k1):
        parent[k1 + i * k2: k1 + (i + 1) * k2] = i
    parents = np.tile(parent, (trials, 1))
    tok = np.empty((trials, N), dtype=np.int32)
    for i in range(k1):
        tok[:, i] = sample_categorical(rng, q_root, trials)
    cdf1 = np.cumsum(q1, axis=1)
    for i in range(k1):
        y = tok[:, i]
        u = rng.random((trials, k2))
        for j in range(k2):
            col = k1 + i * k2 + j
            tok[:, col] = np.minimum((u[:, j:j + 1] > cdf1[y]).sum(axis=1), V - 1)
    tgt = np.empty((trials, N + 1, V), dtype=np.float32)
    drf = np.zeros((trials, N, V), dtype=np.float32)
    tgt[:, 0] = pz_root
    drf[:, 0] = qz_root
    for i in range(k1):
        y = tok[:, i]
        tgt[:, 1 + i] = pz1[y]
        drf[:, 1 + i] = qz1[y]
        for j in range(k2):
            col = k1 + i * k2 + j
            tgt[:, 1 + col] = pz2[y, tok[:, col]]
    res = oracle_mod.spec_verify_tree(tgt, drf, parents, tok, 77, np.float32(T))
    assert res["error"] == 0
    d, out = res["accepted_len"], res["out_tokens"]
    assert np.all(d <= 2)
    assert chi2_pvalue(np.bincount(out[:, 0], minlength=V), p_root) > 0.01
    for y in range(V):
        sel = (d >= 1) & (out[:, 0] == y)
        if sel.sum() > 2000:
            assert chi2_pvalue(np.bincount(out[sel, 1], minlength=V), p1[y]) > 0.01, y
    for a in range(V):
        for c in range(V):
            sel = (d == 2) & (out[:, 0] == a) & (out[:, 1] == c)
            if sel.sum() > 2000:
                assert chi2_pvalue(np.bincount(out[sel, 2], minlength=V), p2[a, c]) > 0.01, (a, c)
    # a wider root accepts more often than one draft would: sum over siblings
    acc1 = (d >= 1).mean()
    single = np.minimum(p_root, q_root).sum()
    assert acc1 > single


def test_greedy_takes_the_first_matching_child(oracle_mod):
    """Pin: greedy mode walks to the first child (in node order) whose token
    is the argmax of its context's target row, and emits the argmax where no
    child matches."""
    V = 10
    tgt = np.zeros((1, 6, V), dtype=np.float32)
    am = [3, 7, 1, 5, 2, 8]                # argmax of each context row
    for c, a in enumerate(am):
        tgt[0, c, a] = 5.0
    drf = np.zeros((1, 5, V), dtype=np.float32)
    # root children: nodes 0 (token 4), 1 (token 3 = match), 2 (token 3, never tried)
    # node 1's children: node 3 (token 9), node 4 (token 2): no match (argmax of context 2 is 1)
    parent = np.array([[-1, -1, -1, 1, 1]], dtype=np.int32)
    tok = np.array([[4, 3, 3, 9, 2]], dtype=np.int32)
    r = oracle_mod.spec_verify_tree(tgt, drf, parent, tok, 0, np.float32(0.0))
    assert r["accepted_len"][0] == 1
    assert list(r["out_tokens"][0]) == [3, am[2], -1, -1, -1, -1]
    assert list(r["path"][0]) == [1, -1, -1, -1, -1]
    tok[0, 4] = am[2]                      # now node 4 matches under node 1
    r = oracle_mod.spec_verify_tree(tgt, drf, parent, tok, 0, np.float32(0.0))
    assert list(r["path"][0][:2]) == [1, 4]
    assert list(r["out_tokens"][0][:3]) == [3, am[2], am[5]]


def test_identical_laws_accept_the_first_child(oracle_mod):
    """Pin: where every draft row equals its target row the first child of
    every context is accepted (ratio 1), so the walk follows first children
    to a leaf."""
    rng = np.random.default_rng(5)
    B, V = 50, 40
    parent = np.array([-1, -1, 0, 0, 2, 1], dtype=np.int32)
    N = parent.size
    z = rng.normal(size=(B, N + 1, V)).astype(np.float32)
    tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    r = oracle_mod.spec_verify_tree(z, np.ascontiguousarray(z[:, :N]), np.tile(parent, (B, 1)), tok, 3,
                                    np.float32(0.9))
    assert np.all(r["accepted_len"] == 3)
    assert np.all(r["path"][:, :3] == [0, 2, 4])


def test_tree_error_paths(oracle_mod):
    rng = np.random.default_rng(6)
    B, N, V = 5, 4, 30
    tgt = rng.normal(size=(B, N + 1, V)).astype(np.float32)
    drf = rng.normal(size=(B, N, V)).astype(np.float32)
    parent = np.tile(np.array([-1, 0, 0, 2], dtype=np.int32), (B, 1))
    tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    parent[1, 2] = 2                        # not an earlier node
    tgt[2, 0] = -np.inf                     # the root row has no finite logit
    tok[3, :] = V + 5                       # every token out of range: all rejected
    temps = np.array([1.0, 1.0, 1.0, 1.0, np.nan], np.float32)
    r = oracle_mod.spec_verify_tree(tgt, drf, parent, tok, 1, temps)
    e = r["seq_error"]
    assert e[0] == 0
    assert e[1] == oracle_mod.ERR_TREE and np.all(r["out_tokens"][1] == -1)
    assert e[2] == oracle_mod.ERR_ROW and np.all(r["out_tokens"][2] == -1)
    assert e[3] == oracle_mod.ERR_TOKEN and r["accepted_len"][3] == 0 and r["out_tokens"][3, 0] >= 0
    assert e[4] == oracle_mod.ERR_TEMPERATURE
    r = oracle_mod.spec_verify_tree(tgt, None, parent, tok, 1, np.float32(1.0))
    assert np.all(r["seq_error"][[0, 2, 3]] == oracle_mod.ERR_NO_DRAFT)


def test_forced_node_decisions_equal_token_substitutions(oracle_mod):
    """Pin (replayed near-ties, as for the chain): replaying an accepted node
    as a rejection gives what the walk gives with that node's token out of
    range (ratio 0: rejected, and the law still takes its residual); replaying
    a rejected node as an acceptance gives what it gives with that node's
    token replaced by one of zero draft mass (ratio +inf), up to that token.
    Neither substitution changes a row, so the rest of the walk must agree;
    forcing a chain tree equals forcing the chain verify step."""
    rng = np.random.default_rng(71)
    B, V = 120, 41
    parent = np.array([-1, -1, -1, 0, 0, 1, 3, 3, 5], dtype=np.int32)
    N = parent.size
    tgt = (rng.normal(size=(B, N + 1, V)) * 1.5).astype(np.float32)
    drf = (tgt[:, :N] + 0.8 * rng.normal(size=(B, N, V))).astype(np.float32)
    drf[:, :, V - 1] = -np.inf  # token V-1 has no draft mass in any context
    tok = rng.integers(0, V - 1, size=(B, N)).astype(np.int32)
    temps = rng.uniform(0.6, 1.4, size=B).astype(np.float32)
    par = np.tile(parent, (B, 1))
    base = oracle_mod.spec_verify_tree(tgt, drf, par, tok, 5, temps)
    assert base["error"] == 0
    n_rej = n_acc = 0
    for b in range(B):
        sl, ids = slice(b, b + 1), np.array([b])
        tested = np.flatnonzero(~np.isnan(base["node_margin"][b]))
        on_path = set(int(j) for j in base["path"][b] if j >= 0)
        for j in tested:
            force = np.zeros((1, N), bool)
            force[0, j] = True
            got = oracle_mod.spec_verify_tree(tgt[sl], drf[sl], par[sl], tok[sl], 5, temps[sl],
                                              seq_ids=ids, force=force)
            t2 = tok[sl].copy()
            t2[0, j] = -1 if j in on_path else V - 1
            want = oracle_mod.spec_verify_tree(tgt[sl], drf[sl], par[sl], t2, 5, temps[sl], seq_ids=ids)
            assert np.array_equal(got["path"], want["path"])
            assert got["accepted_len"][0] == want["accepted_len"][0]
            go, wo = got["out_tokens"][0].copy(), want["out_tokens"][0].copy()
            if j not in on_path:  # the replayed acceptance emits node j's own token
                d = list(got["path"][0]).index(j)
                assert go[d] == tok[b, j] and wo[d] == V - 1
                go[d] = wo[d] = 0
                n_acc += 1
            else:
                n_rej += 1
            assert np.array_equal(go, wo)
            assert np.array_equal(got["bonus_margin"], want["bonus_margin"])
    assert n_rej > 50 and n_acc > 50
    # a chain: forcing the tree equals forcing the chain verify step
    chain = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    force = rng.random((B, N)) < 0.2
    dch = np.ascontiguousarray(drf[:, :N])
    a = oracle_mod.spec_verify(tgt, dch, tok, 8, temps, 1.0, force=force)
    t = oracle_mod.spec_verify_tree(tgt, dch, chain, tok, 8, temps, force=force)
    assert np.array_equal(a["accepted_len"], t["accepted_len"])
    assert np.array_equal(a["out_tokens"], t["out_tokens"])


def test_repeated_rejections_match_high_precision(oracle_mod):
    """Pin (the recursion itself, evaluated exactly): siblings that all carry
    the token x of a draft law equal to the target law except at x, which the
    draft favours.  Each rejection of x leaves the residual max(r - q, 0)
    proportional to p off x, its mass multiplying into a factor ~1e-14 of p
    after four rejections: a case where subtracting r - q in double leaves
    nothing but rounding.  The recursion r <- max(r - q, 0) / sum max(r - q, 0)
    is carried out in 60-digit decimal arithmetic from the same logits, and the
    oracle's bonus token and its CDF interval must agree with it."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    rng = np.random.default_rng(92)
    B, V, N = 64, 5003, 4
    parent = np.tile(np.array([-1] * N, dtype=np.int32), (B, 1))
    tgt = rng.normal(size=(B, N + 1, V)).astype(np.float32)
    drf = tgt[:, :N].copy()
    x = rng.integers(0, V, size=B)
    drf[np.arange(B), 0, x] += np.float32(np.log1p(2e-3 * V / 1.65))  # ~1e-3 of draft mass moved to x
    tok = np.repeat(x[:, None], N, axis=1).astype(np.int32)
    res = oracle_mod.spec_verify_tree(tgt, drf, parent, tok, 11, np.ones(B, np.float32))
    assert res["error"] == 0
    checked = 0
    for b in range(B):
        if res["accepted_len"][b] != 0:
            continue  # the first sibling was accepted (ratio ~0.14)
        zt = [Decimal(float(v)) for v in tgt[b, 0]]
        zd = [Decimal(float(v)) for v in drf[b, 0]]
        et = [v.exp() for v in zt]
        ed = [v.exp() for v in zd]
        st, sd = sum(et), sum(ed)
        p = [v / st for v in et]
        q = [v / sd for v in ed]
        r = p
        for j in range(N):  # every sibling carries x: all rejected (ratio 0 after the first)
            dlt = [max(ri - qi, Decimal(0)) for ri, qi in zip(r, q)]
            z = sum(dlt)
            if z > 0:
                r = [v / z for v in dlt]
        Z = sum(r)
        u = Decimal(oracle_mod.uniform(11, b, 0, 1))
        c = Decimal(0)
        want = None
        for v in range(V):
            lo = c / Z
            c += r[v]
            if c >= u * Z:
                want, want_lo, want_hi = v, lo, c / Z
                break
        got = oracle_mod.spec_verify_tree(tgt[b:b + 1], drf[b:b + 1], parent[b:b + 1], tok[b:b + 1], 11,
                                          np.ones(1, np.float32), seq_ids=np.array([b]),
                                          probe=np.array([want]))
        assert res["out_tokens"][b, 0] == want, (b, res["out_tokens"][b, 0], want)
        assert abs(got["probe_cdf"][0, 0] - float(want_lo)) < 1e-12
        assert abs(got["probe_cdf"][0, 1] - float(want_hi)) < 1e-12
        checked += 1
    assert checked > 40
