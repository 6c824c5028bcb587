"""Double-precision CPU oracle of the speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the library or its binding.  The C
source (``specverify_oracle.c``) shares no code with the HIP path; this module
only marshals numpy arrays into it with ctypes.

What each function follows is cited in the C source.  Every function here is
pinned by ``tests/test_oracle_pins.py`` except the zero-residual-mass fallback,
which is "parity unpinned" (it can only be reached through rounding).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "specverify_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
ACCEPT = 0
BONUS = 1

ERR_TOKEN = 1
ERR_TEMPERATURE = 2
ERR_ROW = 4
ERR_DRAFT_MASS = 8
ERR_NO_DRAFT = 16
ERR_DRAFT_LEN = 32
ERR_TREE = 64

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE double, OpenMP over sequences)."""
    cmd = [
        "gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
        "-fPIC", "-shared", _SRC, "-o", _LIB_PATH + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, u32, u64, f64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double
    lib.oracle_philox4x32_10.argtypes = [P, P, P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_uniform.argtypes = [u64, u32, u32, u32]
    lib.oracle_uniform.restype = f64
    lib.oracle_row_max.argtypes = [P, i32, i32]
    lib.oracle_row_max.restype = f64
    lib.oracle_row_argmax.argtypes = [P, i32, i32]
    lib.oracle_row_argmax.restype = i32
    lib.oracle_row_lognorm.argtypes = [P, i32, i32, f64]
    lib.oracle_row_lognorm.restype = f64
    lib.oracle_row_top4.argtypes = [P, i32, i32, P]
    lib.oracle_row_top4.restype = i32
    lib.oracle_draft_logprobs.argtypes = [P, i32, i32, f64, f64, P]
    lib.oracle_draft_logprobs.restype = i32
    lib.oracle_spec_verify.argtypes = [P, P, P, i32, i32, i32, i32, u64, P, f64,
                                       P, P, P, P, P, P, P, P, P, i32]
    lib.oracle_spec_verify_ragged.argtypes = [P, P, P, P, i32, i32, i32, i32, u64, P, f64,
                                              P, P, P, P, P, P, P, P, P, P, P, i32]
    lib.oracle_spec_verify_ragged.restype = i32
    lib.oracle_spec_verify_outcomes.argtypes = [P, P, i32, i32, i32, i32, P, f64, i32, P, P, P, P, P,
                                                P, i32]
    lib.oracle_spec_verify_outcomes.restype = i32
    lib.oracle_spec_verify_tree.argtypes = [P, P, P, P, i32, i32, i32, i32, u64, P, P, P, P, P, P, P,
                                            P, P, P, P, i32]
    lib.oracle_spec_verify_tree.restype = i32
    lib.oracle_uniforms.argtypes = [u64, i32, i32, P]
    lib.oracle_uniforms.restype = None
    lib.oracle_spec_verify.restype = i32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_raw(logits: np.ndarray) -> tuple[np.ndarray, int]:
    """Accept float32 arrays, or uint16 arrays holding bf16 bit patterns."""
    if logits.dtype == np.float32:
        return np.ascontiguousarray(logits), F32
    if logits.dtype == np.uint16:
        return np.ascontiguousarray(logits), BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {logits.dtype}")


def philox4x32_10(ctr, key) -> np.ndarray:
    lib = _load()
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, b: int, pos: int, purpose: int) -> float:
    return float(_load().oracle_uniform(seed, b, pos, purpose))


def uniforms(seed: int, B: int, P: int) -> np.ndarray:
    """u(seed, b, pos, purpose) as a [B, P, 2] float64 array."""
    out = np.zeros((B, P, 2), dtype=np.float64)
    _load().oracle_uniforms(int(seed) & (2**64 - 1), B, P, _ptr(out))
    return out


def row_max(row: np.ndarray) -> float:
    raw, dt = _as_raw(row)
    return float(_load().oracle_row_max(_ptr(raw), dt, raw.shape[-1]))


def row_argmax(row: np.ndarray) -> int:
    raw, dt = _as_raw(row)
    return int(_load().oracle_row_argmax(_ptr(raw), dt, raw.shape[-1]))


def row_lognorm(row: np.ndarray, T: float) -> float:
    """log sum_v exp(z_v / T)."""
    raw, dt = _as_raw(row)
    return float(_load().oracle_row_lognorm(_ptr(raw), dt, raw.shape[-1], float(T)))


def row_top4(row: np.ndarray) -> list[int]:
    raw, dt = _as_raw(row)
    idx = np.zeros(4, dtype=np.int32)
    n = _load().oracle_row_top4(_ptr(raw), dt, raw.shape[-1], _ptr(idx))
    return [int(i) for i in idx[:n]]


def draft_logprobs(row: np.ndarray, T: float, beta: float) -> np.ndarray:
    raw, dt = _as_raw(row)
    out = np.zeros(raw.shape[-1], dtype=np.float64)
    err = _load().oracle_draft_logprobs(_ptr(raw), dt, raw.shape[-1], float(T), float(beta),
                                        _ptr(out))
    if err:
        raise ValueError(f"oracle_draft_logprobs error bits {err}")
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def spec_verify(target: np.ndarray, draft: np.ndarray | None, tokens: np.ndarray, seed: int,
                temperature, beta: float = 1.0, nthreads: int = 0,
                seq_ids: np.ndarray | None = None, draft_len: np.ndarray | None = None,
                force: np.ndarray | None = None) -> dict:
    """Run the oracle on a whole batch.

    target: [B, K+1, V] float32 or uint16 (bf16 bits); draft: [B, K, V] same
    dtype, or None when every temperature is 0; tokens: [B, K] int32;
    temperature: scalar or [B] float32.  Returns a dict of numpy arrays:
    accepted_len [B], out_tokens [B, K+1], p_target / p_draft / margin_accept
    [B, K], residual_mass / margin_bonus / seq_error [B], and error (int).
    seq_ids [B] gives the global sequence index each row's uniforms are keyed
    by (default 0..B-1), so a sample of a larger batch can be verified alone.
    draft_len [B] (default K for every sequence) gives ragged draft lengths
    K_b <= K; draft_conf [B, K] is the draft confidence max_v p_d (NaN past
    K_b, for greedy and for failed sequences).  force [B, K] (bool) reverses
    the outcome of those accept tests (parity checks replay a near-tie the
    other implementation decided the other way).
    """
    lib = _load()
    t_raw, dt = _as_raw(target)
    B, K1, V = t_raw.shape
    K = K1 - 1
    if draft is not None:
        d_raw, dt2 = _as_raw(draft)
        assert dt2 == dt and d_raw.shape == (B, K, V)
    else:
        d_raw = None
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(B, K))
    temp = np.asarray(temperature, dtype=np.float32)
    if temp.ndim == 0:
        temp = np.full(B, temp, dtype=np.float32)
    temp = np.ascontiguousarray(temp)
    assert temp.shape == (B,)
    if seq_ids is not None:
        seq_ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
        assert seq_ids.shape == (B,)
    res = {
        "accepted_len": np.zeros(B, dtype=np.int32),
        "out_tokens": np.zeros((B, K + 1), dtype=np.int32),
        "p_target": np.zeros((B, K), dtype=np.float64),
        "p_draft": np.zeros((B, K), dtype=np.float64),
        "residual_mass": np.zeros(B, dtype=np.float64),
        "margin_accept": np.zeros((B, K), dtype=np.float64),
        "margin_bonus": np.zeros(B, dtype=np.float64),
        "seq_error": np.zeros(B, dtype=np.int32),
        "draft_conf": np.zeros((B, K), dtype=np.float64),
    }
    if draft_len is not None:
        draft_len = np.ascontiguousarray(np.asarray(draft_len, dtype=np.int32))
        assert draft_len.shape == (B,)
    if force is not None:
        force = np.ascontiguousarray(np.asarray(force, dtype=bool).reshape(B, K).astype(np.uint8))
    err = lib.oracle_spec_verify_ragged(
        _ptr(t_raw), _ptr(d_raw), _ptr(tok), _ptr(draft_len), B, K, V, dt, int(seed) & (2**64 - 1),
        _ptr(temp), float(beta), _ptr(res["accepted_len"]), _ptr(res["out_tokens"]),
        _ptr(res["p_target"]), _ptr(res["p_draft"]), _ptr(res["residual_mass"]),
        _ptr(res["margin_accept"]), _ptr(res["margin_bonus"]), _ptr(res["seq_error"]),
        _ptr(res["draft_conf"]), _ptr(seq_ids), _ptr(force), int(nthreads))
    res["error"] = int(err)
    return res


def outcomes(target: np.ndarray, draft: np.ndarray | None, temperature, beta: float = 1.0,
             F: int = 4, nthreads: int = 0) -> dict:
    """Verification-outcome distribution of every sequence (see the C source):
    accept_rate [B, K], p_len [B, K+1], top_tokens [B, K+1, F] int32,
    top_mass [B, K+1, F], draft_top_mass [B, K] (residual mass on each draft
    row's top-4), seq_error [B], error (int)."""
    lib = _load()
    t_raw, dt = _as_raw(target)
    B, K1, V = t_raw.shape
    K = K1 - 1
    d_raw = None
    if draft is not None:
        d_raw, dt2 = _as_raw(draft)
        assert dt2 == dt and d_raw.shape == (B, K, V)
    temp = np.asarray(temperature, dtype=np.float32)
    if temp.ndim == 0:
        temp = np.full(B, temp, dtype=np.float32)
    temp = np.ascontiguousarray(temp)
    res = {
        "accept_rate": np.zeros((B, K), dtype=np.float64),
        "p_len": np.zeros((B, K + 1), dtype=np.float64),
        "top_tokens": np.zeros((B, K + 1, F), dtype=np.int32),
        "top_mass": np.zeros((B, K + 1, F), dtype=np.float64),
        "draft_top_mass": np.zeros((B, K), dtype=np.float64),
        "seq_error": np.zeros(B, dtype=np.int32),
    }
    err = lib.oracle_spec_verify_outcomes(
        _ptr(t_raw), _ptr(d_raw), B, K, V, dt, _ptr(temp), float(beta), int(F), _ptr(res["accept_rate"]),
        _ptr(res["p_len"]), _ptr(res["top_tokens"]), _ptr(res["top_mass"]),
        _ptr(res["draft_top_mass"]) if K > 0 and d_raw is not None else None, _ptr(res["seq_error"]),
        int(nthreads))
    if K > 0 and d_raw is None:
        res["draft_top_mass"][:] = np.nan
    res["error"] = int(err)
    return res


def spec_verify_tree(target: np.ndarray, draft: np.ndarray | None, parent: np.ndarray,
                     tokens: np.ndarray, seed: int, temperature, seq_ids=None,
                     nthreads: int = 0, force: np.ndarray | None = None,
                     probe: np.ndarray | None = None) -> dict:
    """Tree verification of every sequence (see the C source): target
    [B, N+1, V], draft [B, N, V] (row c: the law the children of context c
    were drawn from), parent and tokens [B, N] int32.  Returns accepted_len
    [B], out_tokens [B, N+1], path [B, N], node_margin [B, N] (|u - ratio| of
    each node tested, NaN otherwise), bonus_margin [B], seq_error [B], error.
    force [B, N] (bool) reverses the outcome of those nodes' tests; probe [B]
    names a token whose CDF interval under the final law is returned as
    probe_cdf [B, 2]."""
    lib = _load()
    t_raw, dt = _as_raw(target)
    B, N1, V = t_raw.shape
    N = N1 - 1
    d_raw = None
    if draft is not None:
        d_raw, dt2 = _as_raw(draft)
        assert dt2 == dt and d_raw.shape == (B, N, V)
    parent = np.ascontiguousarray(parent, dtype=np.int32).reshape(B, N)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, N)
    temp = np.asarray(temperature, dtype=np.float32)
    if temp.ndim == 0:
        temp = np.full(B, temp, dtype=np.float32)
    temp = np.ascontiguousarray(temp)
    ids = None if seq_ids is None else np.ascontiguousarray(seq_ids, dtype=np.int32)
    if force is not None:
        force = np.ascontiguousarray(np.asarray(force, dtype=bool).reshape(B, N).astype(np.uint8))
    res = {"accepted_len": np.zeros(B, dtype=np.int32),
           "out_tokens": np.zeros((B, N + 1), dtype=np.int32),
           "path": np.zeros((B, N), dtype=np.int32),
           "node_margin": np.zeros((B, N), dtype=np.float64),
           "bonus_margin": np.zeros(B, dtype=np.float64),
           "seq_error": np.zeros(B, dtype=np.int32)}
    if probe is not None:
        probe = np.ascontiguousarray(np.asarray(probe, dtype=np.int32).reshape(B))
        res["probe_cdf"] = np.full((B, 2), np.nan)
    err = lib.oracle_spec_verify_tree(
        _ptr(t_raw), _ptr(d_raw), _ptr(parent), _ptr(tokens), B, N, V, dt, int(seed) & (2**64 - 1),
        _ptr(temp), _ptr(res["accepted_len"]), _ptr(res["out_tokens"]), _ptr(res["path"]),
        _ptr(res["node_margin"]), _ptr(res["bonus_margin"]), _ptr(res["seq_error"]), _ptr(ids),
        _ptr(force), _ptr(probe), _ptr(res.get("probe_cdf")), int(nthreads))
    res["error"] = int(err)
    return res
