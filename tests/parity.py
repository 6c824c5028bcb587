"""Element-by-element comparison of the HIP path's outputs with the oracle's.

The rule: accepted_len and out_tokens must match exactly, except that the
first divergence of a sampling sequence may sit at a decision the oracle took
within `margin` of its threshold (|u - ratio| for an accept test; for the
bonus, u within `margin` of C(v)/Z at the GPU's token).  Each such divergence
is one excused flip.  Greedy sequences and failed sequences allow no excuse.
Diagnostic probabilities must agree within `ptol` where both paths evaluated
them.
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
    failures: list = field(default_factory=list)
    max_p_err: float = 0.0
    max_z_err: float = 0.0

    def merge(self, other: "Report") -> None:
        self.sequences += other.sequences
        self.decisions += other.decisions
        self.flips += other.flips
        self.failures += other.failures
        self.max_p_err = max(self.max_p_err, other.max_p_err)
        self.max_z_err = max(self.max_z_err, other.max_z_err)

    def check(self, flip_rate: float = 1e-5) -> None:
        assert not self.failures, "\n".join(self.failures[:20])
        assert self.flips <= flip_rate * self.decisions + 1, (self.flips, self.decisions)


def _draft_len(h, b) -> int:
    dl = h.get("draft_len")
    return int(dl[b]) if dl is not None else h["tokens"].shape[1]


def _bonus_within_margin(h, b, n, tok_g, u, Z_o, margin) -> bool:
    """Is u within `margin` of the oracle-law CDF interval of token tok_g?"""
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


def compare(gpu: dict, orc: dict, h: dict, seed: int, seq_ids=None, margin: float = 1e-6,
            ptol: float = 1e-5, uniform=None) -> Report:
    """gpu: numpy arrays accepted_len, out_tokens (+ optional p_target,
    p_draft, residual_mass, draft_conf, error_word); orc: oracle.spec_verify
    result on the same inputs h (numpy host inputs, with draft_len for ragged
    calls); uniform(b, pos, purpose) gives the oracle's uniforms for the
    excusal check of bonus draws.  The draft confidence depends on no
    decision: it is compared at every position of every sequence."""
    rep = Report()
    B, K1 = orc["out_tokens"].shape
    K = K1 - 1
    temps = h["temperature"]
    for b in range(B):
        rep.sequences += 1
        gb = int(seq_ids[b]) if seq_ids is not None else b
        n_o, n_g = int(orc["accepted_len"][b]), int(gpu["accepted_len"][b])
        out_o, out_g = orc["out_tokens"][b], gpu["out_tokens"][b]
        tag = f"seq {gb}"
        Kb = _draft_len(h, b)
        if "draft_conf" in gpu:
            for i in range(K):
                co, cg = orc["draft_conf"][b, i], gpu["draft_conf"][b, i]
                if np.isnan(co) or np.isnan(cg):
                    if not (np.isnan(co) and np.isnan(cg)):
                        rep.failures.append(f"{tag}: draft_conf[{i}] {cg} vs oracle {co}")
                    continue
                err = abs(float(cg) - float(co))
                rep.max_p_err = max(rep.max_p_err, err)
                if not err <= ptol:
                    rep.failures.append(f"{tag}: draft_conf[{i}] {cg} vs {co}")
        if orc["seq_error"][b] != 0 or temps[b] == 0.0:
            if n_o != n_g or not np.array_equal(out_o, out_g):
                rep.failures.append(f"{tag}: exact mismatch n {n_o}/{n_g} out {out_o}/{out_g}")
            rep.decisions += min(n_o + 1, K1)
            continue
        rep.decisions += (n_o + 1 if n_o < Kb else Kb) + 1
        m = min(n_o, n_g)
        if not np.array_equal(out_g[:m], h["tokens"][b, :m]):
            rep.failures.append(f"{tag}: accepted prefix differs from drafts")
            continue
        if n_g < K and not np.all(out_g[n_g + 1:] == -1):
            rep.failures.append(f"{tag}: padding after the bonus is not -1: {out_g}")
        if n_o != n_g:
            mg = orc["margin_accept"][b, m]
            if mg < margin:
                rep.flips += 1
            else:
                rep.failures.append(f"{tag}: accept decision at {m} differs (n {n_o}/{n_g}), "
                                    f"oracle margin {mg:.3g}")
            continue
        if out_g[n_o] != out_o[n_o]:
            mgb = orc["margin_bonus"][b]
            ok = False
            if mgb < margin and uniform is not None:
                ok = _bonus_within_margin(h, b, n_o, int(out_g[n_o]), uniform(gb, n_o, 1),
                                          orc["residual_mass"][b], margin)
            if ok:
                rep.flips += 1
            else:
                rep.failures.append(f"{tag}: bonus {out_g[n_o]} vs oracle {out_o[n_o]} at n={n_o}, "
                                    f"oracle margin {mgb:.3g}")
            continue
        # diagnostics on the common path
        for key in ("p_target", "p_draft"):
            if key in gpu:
                for i in range(min(n_o + 1, K)):
                    po, pg = orc[key][b, i], gpu[key][b, i]
                    if np.isnan(po):
                        if not np.isnan(pg):
                            rep.failures.append(f"{tag}: {key}[{i}] {pg} where oracle has NaN")
                        continue
                    err = abs(float(pg) - float(po))
                    rep.max_p_err = max(rep.max_p_err, err)
                    if not err <= ptol:
                        rep.failures.append(f"{tag}: {key}[{i}] {pg} vs {po}")
        if "residual_mass" in gpu:
            zo, zg = orc["residual_mass"][b], gpu["residual_mass"][b]
            err = abs(float(zg) - float(zo))
            rep.max_z_err = max(rep.max_z_err, err)
            if not err <= ptol:
                rep.failures.append(f"{tag}: residual mass {zg} vs {zo}")
    if "error_word" in gpu and seq_ids is None:
        want = int(np.bitwise_or.reduce(orc["seq_error"])) if B else 0
        if int(gpu["error_word"]) != want:
            rep.failures.append(f"error word {int(gpu['error_word'])} vs oracle {want}")
    return rep
