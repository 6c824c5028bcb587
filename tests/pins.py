"""Shared helpers for the oracle pins: laws computed with library routines
(scipy softmax, numpy sorting) and chi-square checks.  Nothing here calls the
HIP library."""
from __future__ import annotations

import numpy as np
import scipy.special
import scipy.stats
import torch


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (nearest-even) and return the bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def exact_values(raw: np.ndarray) -> np.ndarray:
    if raw.dtype == np.uint16:
        return bf16_bits_to_f64(raw)
    return raw.astype(np.float64)


def softmax(z: np.ndarray, T: float) -> np.ndarray:
    return scipy.special.softmax(np.asarray(z, dtype=np.float64) / float(T))


def top4_by_sort(z: np.ndarray) -> np.ndarray:
    """Indices of the 4 largest values, ties to the lower index (full sort)."""
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(z.size), -z))
    return order[: min(4, z.size)]


def draft_law(z: np.ndarray, T: float, beta: float) -> np.ndarray:
    """Draft law with the top-4 probabilities multiplied by beta, renormalised."""
    p = softmax(z, T)
    if beta >= 1.0:
        return p
    w = np.ones_like(p)
    w[top4_by_sort(z)] = beta
    q = w * p
    return q / q.sum()


def sample_categorical(rng: np.random.Generator, probs: np.ndarray, n: int) -> np.ndarray:
    cdf = np.cumsum(probs)
    cdf /= cdf[-1]
    return np.minimum(np.searchsorted(cdf, rng.random(n), side="right"), probs.size - 1)


def chi2_pvalue(observed: np.ndarray, expected_probs: np.ndarray) -> float:
    """Pearson chi-square of counts against a law; cells expecting < 5 are pooled."""
    observed = np.asarray(observed, dtype=np.float64)
    n = observed.sum()
    exp = np.asarray(expected_probs, dtype=np.float64) * n
    big = exp >= 5.0
    obs_c = list(observed[big])
    exp_c = list(exp[big])
    if (~big).any():
        obs_c.append(observed[~big].sum())
        exp_c.append(exp[~big].sum())
    obs_c = np.array(obs_c)
    exp_c = np.array(exp_c)
    keep = exp_c > 0
    if (obs_c[~keep] > 0).any():
        return 0.0  # mass where the law has none
    obs_c, exp_c = obs_c[keep], exp_c[keep]
    if obs_c.size < 2:
        return 1.0
    exp_c *= obs_c.sum() / exp_c.sum()
    return float(scipy.stats.chisquare(obs_c, exp_c).pvalue)


def binom_pvalue(k: int, n: int, p: float) -> float:
    return float(scipy.stats.binomtest(int(k), int(n), float(p)).pvalue)
