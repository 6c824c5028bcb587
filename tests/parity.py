"""Element-by-element comparison of the HIP path's outputs with the oracle's.

The rule ("Kangaroo: Self-Speculative Decoding via Shallow Sub-Networks",
"3. Lossless Speculative Verification": for fixed inputs and uniforms the
verify step is a deterministic function, so two correct finite-precision
implementations can differ only at a decision within rounding of its
threshold): accepted_len and out_tokens must match exactly, except that a
sampling sequence may diverge at a decision the oracle took within `margin`
of its threshold (|u - ratio| for an accept test; for the bonus, u within
`margin` of the ends of the GPU token's CDF interval).  Each such divergence
is one excused flip, and the comparison goes on: an accept test is replayed
by the oracle the way the GPU decided it (its `force` argument) and the rest
of the sequence -- later accept tests, the bonus, the diagnostics -- is
compared with that replay; after a bonus flip the diagnostics are still
compared.  Excused accept-test flips must be at most `flip_rate` of the
decisions, with no allowance: below 1/flip_rate decisions that means none;
the rate of excused bonus flips is measured and bounded by the census
(tests/test_gpu_census.py, >= 10^5 decisions per workload).  Greedy and
failed sequences allow no excuse.  Diagnostic probabilities must agree
within `ptol` where both paths evaluated them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from pins import draft_law, exact_values, softmax


@dataclass
class Report:
    sequences: int = 0
    decisions: int = 0
    flips: int = 0
    flips_accept: int = 0
    flips_bonus: int = 0
    failures: list = field(default_factory=list)
    max_p_err: float = 0.0
    max_z_err: float = 0.0
    max_z_rel: float = 0.0

    def merge(self, other: "Report") -> None:
        self.sequences += other.sequences
        self.decisions += other.decisions
        self.flips += other.flips
        self.flips_accept += other.flips_accept
        self.flips_bonus += other.flips_bonus
        self.failures += other.failures
        self.max_p_err = max(self.max_p_err, other.max_p_err)
        self.max_z_err = max(self.max_z_err, other.max_z_err)
        self.max_z_rel = max(self.max_z_rel, other.max_z_rel)

    def check(self, flip_rate: float = 1e-5, bonus_rate: float | None = None) -> None:
        """No failure; excused accept-test flips at most flip_rate of the
        decisions, with no allowance (below 1/flip_rate decisions: none).
        Excused bonus-draw flips: at most bonus_rate of the decisions when
        given (the census, over >= 10^5 decisions per workload, where a rate
        means something); otherwise at most one -- each is checked to be a
        near-tie of the exact law (u within the margin of the GPU token's
        CDF interval), and an inverse CDF over ~10^5 tokens meets such
        near-ties at a rate the census measures, not a test of a few hundred
        decisions."""
        assert not self.failures, "\n".join(self.failures[:20])
        assert self.flips_accept <= flip_rate * self.decisions, (self.flips_accept, self.decisions)
        if bonus_rate is None:
            assert self.flips_bonus <= 1, (self.flips_bonus, self.decisions)
        else:
            assert self.flips_bonus <= bonus_rate * self.decisions, (self.flips_bonus, self.decisions)

    def record(self) -> dict:
        return {"sequences": self.sequences, "decisions": self.decisions, "flips": self.flips,
                "flips_accept": self.flips_accept, "flips_bonus": self.flips_bonus,
                "flip_rate": self.flips / max(1, self.decisions),
                "max_abs_p_err": self.max_p_err, "max_abs_residual_mass_err": self.max_z_err,
                "max_rel_residual_mass_err": self.max_z_rel}


def _draft_len(h, b) -> int:
    dl = h.get("draft_len")
    return int(dl[b]) if dl is not None else h["tokens"].shape[1]


def _bonus_within_margin(h, b, n, tok_g, u, margin) -> bool:
    """Is u within `margin` of the ends of token tok_g's CDF interval under
    the residual law at position n (computed with library routines)?"""
    T = float(h["temperature"][b])
    K = _draft_len(h, b)
    tz = exact_values(h["target"][b, n])
    if n < K:
        dz = exact_values(h["draft"][b, n])
        r = np.maximum(softmax(tz, T) - draft_law(dz, T, h["beta"]), 0.0)
    else:
        r = softmax(tz, T)
    c = np.cumsum(r)
    Z = c[-1]
    if not (0 <= tok_g < r.size) or Z <= 0:
        return False
    lo = (c[tok_g - 1] if tok_g > 0 else 0.0) / Z
    hi = c[tok_g] / Z
    return (lo - margin) <= u <= (hi + margin)


def _replay(oracle_mod, h, b, gb, seed, force) -> dict:
    """The oracle on sequence b alone, with the accept tests in `force`
    reversed (uniforms keyed by the global index gb)."""
    sl = slice(b, b + 1)
    dl = h.get("draft_len")
    o = oracle_mod.spec_verify(h["target"][sl], None if h["draft"] is None else h["draft"][sl],
                               h["tokens"][sl], seed, h["temperature"][sl], h["beta"],
                               seq_ids=np.array([gb]), draft_len=None if dl is None else dl[sl],
                               force=force[None, :])
    return {k: (v[0] if isinstance(v, np.ndarray) else v) for k, v in o.items()}


def compare(gpu: dict, orc: dict, h: dict, seed: int, oracle_mod, seq_ids=None,
            margin: float = 1e-6, ptol: float = 1e-5) -> Report:
    """gpu: numpy arrays accepted_len, out_tokens (+ optional p_target,
    p_draft, residual_mass, draft_conf, error_word); orc: oracle.spec_verify
    result on the same inputs h (numpy host inputs, with draft_len for ragged
    calls); seq_ids: the global index of each row of h (uniforms are keyed by
    it).  The draft confidence depends on no decision: it is compared at every
    position of every sequence."""
    rep = Report()
    B, K1 = orc["out_tokens"].shape
    K = K1 - 1
    temps = h["temperature"]
    for b in range(B):
        rep.sequences += 1
        gb = int(seq_ids[b]) if seq_ids is not None else b
        o = {k: (v[b] if isinstance(v, np.ndarray) else v) for k, v in orc.items()}
        n_g = int(gpu["accepted_len"][b])
        out_g = gpu["out_tokens"][b]
        tag = f"seq {gb}"
        Kb = _draft_len(h, b)
        if "draft_conf" in gpu:
            for i in range(K):
                co, cg = o["draft_conf"][i], gpu["draft_conf"][b, i]
                if np.isnan(co) or np.isnan(cg):
                    if not (np.isnan(co) and np.isnan(cg)):
                        rep.failures.append(f"{tag}: draft_conf[{i}] {cg} vs oracle {co}")
                    continue
                err = abs(float(cg) - float(co))
                rep.max_p_err = max(rep.max_p_err, err)
                if not err <= ptol:
                    rep.failures.append(f"{tag}: draft_conf[{i}] {cg} vs {co}")
        if o["seq_error"] != 0 or temps[b] == 0.0:
            n_o = int(o["accepted_len"])
            if n_o != n_g or not np.array_equal(o["out_tokens"], out_g):
                rep.failures.append(f"{tag}: exact mismatch n {n_o}/{n_g} out {o['out_tokens']}/{out_g}")
            rep.decisions += min(n_o + 1, K1)
            continue
        force = np.zeros(K, dtype=bool)
        counted = False
        while True:
            n_o = int(o["accepted_len"])
            if not counted:  # the accept tests the oracle performs, plus the bonus draw
                rep.decisions += (n_o + 1 if n_o < Kb else Kb) + 1
                counted = True
            m = min(n_o, n_g)
            if not np.array_equal(out_g[:m], h["tokens"][b, :m]):
                rep.failures.append(f"{tag}: accepted prefix differs from drafts")
                break
            if n_g < K and not np.all(out_g[n_g + 1:] == -1):
                rep.failures.append(f"{tag}: padding after the bonus is not -1: {out_g}")
                break
            if n_o != n_g:
                mg = o["margin_accept"][m]
                if mg < margin and not force[m]:
                    rep.flips += 1
                    rep.flips_accept += 1
                    force[m] = True  # replay the GPU's outcome there, compare the rest
                    o = _replay(oracle_mod, h, b, gb, seed, force)
                    if int(o["accepted_len"]) > n_o:  # the replay reaches further decisions
                        rep.decisions += int(o["accepted_len"]) - n_o
                    continue
                rep.failures.append(f"{tag}: accept decision at {m} differs (n {n_o}/{n_g}), "
                                    f"oracle margin {mg:.3g}")
                break
            if out_g[n_o] != o["out_tokens"][n_o]:
                mgb = o["margin_bonus"]
                if mgb < margin and _bonus_within_margin(
                        h, b, n_o, int(out_g[n_o]), oracle_mod.uniform(seed, gb, n_o, 1), margin):
                    rep.flips += 1
                    rep.flips_bonus += 1
                else:
                    rep.failures.append(f"{tag}: bonus {out_g[n_o]} vs oracle {o['out_tokens'][n_o]} "
                                        f"at n={n_o}, oracle margin {mgb:.3g}")
                    break
            # diagnostics (they depend on no bonus draw)
            for key in ("p_target", "p_draft"):
                if key in gpu:
                    for i in range(min(n_o + 1, K)):
                        po, pg = o[key][i], gpu[key][b, i]
                        if np.isnan(po):
                            if not np.isnan(pg):
                                rep.failures.append(f"{tag}: {key}[{i}] {pg} where oracle has NaN")
                            continue
                        err = abs(float(pg) - float(po))
                        rep.max_p_err = max(rep.max_p_err, err)
                        if not err <= ptol:
                            rep.failures.append(f"{tag}: {key}[{i}] {pg} vs {po}")
            if "residual_mass" in gpu:
                zo, zg = float(o["residual_mass"]), float(gpu["residual_mass"][b])
                err = abs(zg - zo)
                rep.max_z_err = max(rep.max_z_err, err)
                if zo > 0:
                    rep.max_z_rel = max(rep.max_z_rel, err / zo)
                if not err <= ptol:
                    rep.failures.append(f"{tag}: residual mass {zg} vs {zo}")
            break
    if "error_word" in gpu and seq_ids is None:
        want = int(np.bitwise_or.reduce(orc["seq_error"])) if B else 0
        if int(gpu["error_word"]) != want:
            rep.failures.append(f"error word {int(gpu['error_word'])} vs oracle {want}")
    return rep


def _tree_replay(oracle_mod, h, b, gb, seed, force, probe=None) -> dict:
    sl = slice(b, b + 1)
    o = oracle_mod.spec_verify_tree(h["target"][sl], None if h["draft"] is None else h["draft"][sl],
                                    h["parent"][sl], h["tokens"][sl], seed, h["temperature"][sl],
                                    seq_ids=np.array([gb]), force=force[None, :],
                                    probe=None if probe is None else np.array([probe]))
    return {k: (v[0] if isinstance(v, np.ndarray) else v) for k, v in o.items()}


def compare_tree(gpu: dict, orc: dict, h: dict, seed: int, oracle_mod, seq_ids=None,
                 margin: float = 1e-6) -> Report:
    """Tree verification under the rule of compare(): accepted_len, path and
    out_tokens exact, except that a sampling sequence may diverge at a node's
    accept test whose oracle margin |u - ratio| is below `margin` (the oracle
    then replays the GPU's outcome there and the rest of the walk is
    compared), or at the bonus when u lies within `margin` of the ends of the
    GPU token's CDF interval under the oracle's final law.  Decisions = the
    node tests the oracle takes plus the bonus draw."""
    rep = Report()
    B, N = h["tokens"].shape
    temps = h["temperature"]
    for b in range(B):
        rep.sequences += 1
        gb = int(seq_ids[b]) if seq_ids is not None else b
        o = {k: (v[b] if isinstance(v, np.ndarray) else v) for k, v in orc.items()}
        d_g = int(gpu["accepted_len"][b])
        path_g, out_g = gpu["path"][b], gpu["out_tokens"][b]
        tag = f"tree seq {gb}"
        if (int(o["seq_error"]) & ~1) != 0 or temps[b] == 0.0:
            same = (d_g == int(o["accepted_len"]) and np.array_equal(path_g, o["path"])
                    and np.array_equal(out_g, o["out_tokens"]))
            if not same:
                rep.failures.append(f"{tag}: exact mismatch n {int(o['accepted_len'])}/{d_g} "
                                    f"out {list(o['out_tokens'])}/{list(out_g)}")
            rep.decisions += int(o["accepted_len"]) + 1
            continue
        force = np.zeros(N, dtype=bool)
        counted = 0
        while True:
            tested = int(np.sum(~np.isnan(o["node_margin"])))
            rep.decisions += max(0, tested - counted) + (1 if counted == 0 else 0)
            counted = max(counted, tested)
            d_o = int(o["accepted_len"])
            k = 0
            while k < min(d_o, d_g) and path_g[k] == o["path"][k]:
                k += 1
            if k < max(d_o, d_g):
                # the walks part at depth k: the first child the two decided differently
                gk = int(path_g[k]) if k < d_g else -1
                ok = int(o["path"][k]) if k < d_o else -1
                j = ok if gk < 0 else gk if ok < 0 else min(gk, ok)
                mg = o["node_margin"][j]
                if not np.isnan(mg) and mg < margin and not force[j]:
                    rep.flips += 1
                    rep.flips_accept += 1
                    force[j] = True
                    o = _tree_replay(oracle_mod, h, b, gb, seed, force)
                    continue
                rep.failures.append(f"{tag}: node {j} decided differently (depth {k}, path "
                                    f"{list(path_g[:d_g])} vs {list(o['path'][:d_o])}), margin {mg:.3g}")
                break
            if not np.array_equal(out_g[:d_g], h["tokens"][b, path_g[:d_g]]):
                rep.failures.append(f"{tag}: accepted tokens are not the path's")
                break
            if not np.all(out_g[d_g + 1:] == -1) or not np.all(path_g[d_g:] == -1):
                rep.failures.append(f"{tag}: padding is not -1")
                break
            if out_g[d_g] != o["out_tokens"][d_g]:
                ok = False
                if o["bonus_margin"] < margin:
                    p = _tree_replay(oracle_mod, h, b, gb, seed, force, probe=int(out_g[d_g]))
                    lo, hi = p["probe_cdf"]
                    u = oracle_mod.uniform(seed, gb, d_g, 1)
                    ok = bool(lo - margin <= u <= hi + margin)
                if ok:
                    rep.flips += 1
                    rep.flips_bonus += 1
                else:
                    rep.failures.append(f"{tag}: bonus {out_g[d_g]} vs oracle {o['out_tokens'][d_g]}, "
                                        f"margin {o['bonus_margin']:.3g}")
            break
    return rep
