"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Inputs are seeded and synthetic (workload.gen); the oracle runs on host copies
of the very same bytes.  Sizes span many chunks and ragged tails while keeping
the oracle to seconds; the full-size workloads are checked on sampled
sequences in the launch configuration the benchmark times.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from parity import Report, compare
from pins import to_bf16_bits
from workload import WORKLOADS, make_inputs, to_numpy_inputs

pytestmark = pytest.mark.gpu

_SKIP = not torch.cuda.is_available()


@pytest.fixture(scope="module")
def sv():
    if _SKIP:
        pytest.skip("no GPU")
    import draft_token_verification_03_amd as sv
    sv.load_library()
    return sv


def _say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()




def run_gpu(sv, inp: dict, seed: int, draft_none: bool = False,
            workspace=None) -> dict:
    acc, out, aux = sv.spec_verify(inp["target"], None if draft_none else inp["draft"],
                                   inp["tokens"], seed, inp["temperature"], inp["beta"], aux=True,
                                   workspace=workspace, draft_len=inp.get("draft_len"))
    torch.cuda.synchronize()
    res = {"accepted_len": acc.cpu().numpy(), "out_tokens": out.cpu().numpy()}
    for k, v in aux.items():
        res[k] = v.cpu().numpy()
    res["error_word"] = int(res["error_word"][0])
    return res


def run_both(sv, oracle_mod, inp: dict, seed: int, ptol: float, draft_none: bool = False) -> Report:
    g = run_gpu(sv, inp, seed, draft_none)
    h = to_numpy_inputs(inp)
    if draft_none:
        h["draft"] = None
    o = oracle_mod.spec_verify(h["target"], h["draft"], h["tokens"], seed, h["temperature"],
                               h["beta"], draft_len=h.get("draft_len"))
    return compare(g, o, h, seed, oracle_mod, ptol=ptol)


def _ptol(dtype: str) -> float:
    return 1e-5 if dtype == "fp32" else 2e-3


# ---------------------------------------------------------------------------

def test_uniforms_match_oracle(sv, oracle_mod):
    for seed in (0, 1, 0xDEADBEEFCAFEF00D):
        _say(f"uniforms seed={seed}")
        g = sv.uniforms(seed, 2000, 250).cpu().numpy().astype(np.float64)
        o = oracle_mod.uniforms(seed, 2000, 250)
        assert np.array_equal(g, o)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_row_stats_match_oracle(sv, oracle_mod, dtype):
    rng = np.random.default_rng(7)
    for V in (1, 2, 7, 999, 4097, 32000, 128256, 152067):
        rows = 6
        z = (rng.normal(size=(rows, V)) * 4 - 1.1 * np.log1p(rng.permutation(V))).astype(np.float32)
        if V > 3:
            z[1, rng.integers(0, V, size=max(1, V // 3))] = -np.inf
            z[2, :] = np.round(z[2, :])  # ties for the argmax rows
        temps = np.array([0.7, 1.0, 0.0, 1.3, 0.0, 0.45], dtype=np.float32)
        raw = to_bf16_bits(z) if dtype == "bf16" else z
        _say(f"row_stats dtype={dtype} V={V}")
        t = torch.from_numpy(raw.view(np.int16) if dtype == "bf16" else raw)
        t = t.view(torch.bfloat16) if dtype == "bf16" else t
        mx, ls, am = sv.row_stats(t.cuda(), torch.from_numpy(temps).cuda())
        mx, ls, am = mx.cpu().numpy(), ls.cpu().numpy(), am.cpu().numpy()
        for r in range(rows):
            want_m = oracle_mod.row_max(raw[r])
            assert mx[r] == want_m, (V, r)
            if temps[r] == 0.0:
                assert am[r] == oracle_mod.row_argmax(raw[r]), (V, r)
            else:
                L_o = oracle_mod.row_lognorm(raw[r], float(temps[r]))
                L_g = float(mx[r]) / float(temps[r]) + float(ls[r])
                assert abs(L_g - L_o) <= 1e-6 + 1e-12 * abs(L_o), (V, r, L_g, L_o)


@pytest.mark.parametrize("name,B,seeds", [
    ("C1", 1, 200), ("C2", 8, 25), ("C3", 64, 6), ("C4", 30, 4), ("C5", 24, 4),
])
def test_workload_parity_reduced(sv, oracle_mod, name, B, seeds):
    """Each named workload at full vocabulary and a batch the oracle finishes
    in seconds, over several input and Philox seeds."""
    w = WORKLOADS[name].sized(B=B)
    rep = Report()
    for s in range(seeds):
        _say(f"parity {name} B={B} seed={s}")
        inp = make_inputs(w, seed=100 + s, device="cuda")
        rep.merge(run_both(sv, oracle_mod, inp, seed=s, ptol=_ptol(w.dtype),
                           draft_none=w.greedy))
    _say(f"{name}: {rep.sequences} seqs {rep.decisions} decisions {rep.flips} flips "
         f"max|dp| {rep.max_p_err:.2e} max|dZ| {rep.max_z_err:.2e}")
    rep.check()


# ---------------------------------------------------------------------------
# Edge cases.

def _inputs_from_numpy(tgt, drf, tokens, temps, beta, dtype):
    if dtype == "bf16":
        t = torch.from_numpy(to_bf16_bits(tgt).view(np.int16)).view(torch.bfloat16)
        d = None if drf is None else torch.from_numpy(to_bf16_bits(drf).view(np.int16)).view(
            torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(tgt, dtype=np.float32))
        d = None if drf is None else torch.from_numpy(np.ascontiguousarray(drf, dtype=np.float32))
    return {"target": t.cuda(), "draft": None if d is None else d.cuda(),
            "tokens": torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).cuda(),
            "temperature": torch.from_numpy(np.asarray(temps, dtype=np.float32)).cuda(),
            "beta": float(beta)}


def _random_case(rng, B, K, V, spread=3.0, noise=0.7, argmax_frac=0.5):
    base = rng.normal(size=(B, K + 1, V)) * spread
    tgt = (base + noise * rng.normal(size=(B, K + 1, V))).astype(np.float32)
    drf = base[:, :K].astype(np.float32)
    tokens = rng.integers(0, V, size=(B, K)).astype(np.int32)
    # drafts partly the draft argmax so acceptance is non-trivial
    am = drf.argmax(axis=2) if K else np.zeros((B, 0), dtype=np.int64)
    pick = rng.random((B, K)) < argmax_frac
    tokens = np.where(pick, am, tokens).astype(np.int32)
    return tgt, drf, tokens


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 5, 9, 31, 257, 2049, 10007, 70001])
def test_ragged_and_tiny_vocab(sv, oracle_mod, dtype, V):
    rng = np.random.default_rng(V)
    B, K = 24, 3
    tgt, drf, tok = _random_case(rng, B, K, V)
    temps = rng.choice([0.0, 0.6, 1.0, 1.7], size=B).astype(np.float32)
    for beta in (1.0, 0.5, 0.0):
        if beta == 0.0 and V <= 4:
            continue  # every draft token down-weighted to zero: undefined draft law
        _say(f"ragged dtype={dtype} V={V} beta={beta}")
        inp = _inputs_from_numpy(tgt, drf, tok, temps, beta, dtype)
        run_both(sv, oracle_mod, inp, seed=V, ptol=_ptol(dtype)).check()


@pytest.mark.parametrize("K", [0, 1, 2, 7, 16, 20])
def test_draft_lengths(sv, oracle_mod, K):
    rng = np.random.default_rng(40 + K)
    B, V = 40, 3001
    tgt, drf, tok = _random_case(rng, B, K, V)
    temps = rng.uniform(0.5, 1.2, size=B).astype(np.float32)
    temps[::5] = 0.0
    for dtype in ("fp32", "bf16"):
        _say(f"draft-length K={K} dtype={dtype}")
        inp = _inputs_from_numpy(tgt, drf, tok, temps, 0.5, dtype)
        run_both(sv, oracle_mod, inp, seed=K, ptol=_ptol(dtype)).check()


def _shaped_draft_rows(rng, K, V):
    """Draft rows whose top-4 forms in every way a streaming pass can meet:
    rising and falling rows (every element, or none, a new entry), constant
    rows and repeated maxima (ties broken by index), the top at the ragged
    tail, signed zeros at the top, rows of mostly -inf, and Zipf-like rows."""
    rows = np.empty((K, V), dtype=np.float32)
    for i in range(K):
        s = i % 8
        if s == 0:
            r = np.linspace(-6.0, 6.0, V)
        elif s == 1:
            r = np.linspace(6.0, -6.0, V)
        elif s == 2:
            r = np.zeros(V)
        elif s == 3:
            r = rng.normal(size=V)
            r[-7:] = 5.0 + np.arange(7) * 0.25
        elif s == 4:
            r = rng.normal(size=V) * 2
            r[rng.choice(V, size=6, replace=False)] = r.max() + 1.0
        elif s == 5:
            r = np.full(V, -1.0)
            pos = rng.choice(V, size=6, replace=False)
            r[pos[:3]] = -0.0
            r[pos[3:]] = 0.0
        elif s == 6:
            r = np.full(V, -np.inf)
            r[rng.choice(V, size=2, replace=False)] = rng.normal(size=2)
        else:
            r = rng.normal(size=V) * 3 - 1.1 * np.log1p(rng.permutation(V))
        rows[i] = r
    return rows


def _top4_indices(row):
    order = np.lexsort((np.arange(row.size), -row.astype(np.float64)))
    return order[:4]


@pytest.mark.parametrize("B,V", [(3, 70001), (16, 9001), (32, 20011), (128, 20011)])
def test_weighted_draft_rows_of_every_shape(sv, oracle_mod, B, V):
    """Beta-weighted draft rows: top-4 selection under ties, rising rows and
    ragged tails, with many chunks per row (few sequences: merged per wave),
    three and two chunks (merged per position thread) and one chunk."""
    rng = np.random.default_rng(B + V)
    K = 8
    drf = np.stack([_shaped_draft_rows(rng, K, V) for _ in range(B)])
    tgt = np.concatenate([drf, rng.normal(size=(B, 1, V)).astype(np.float32) * 2], axis=1)
    tgt[:, :K] += (0.5 * rng.normal(size=(B, K, V))).astype(np.float32)
    tgt[:, 6::8] = np.where(np.isinf(drf[:, 6::8]), 0.0, tgt[:, 6::8])  # targets stay finite
    temps = rng.uniform(0.5, 1.2, size=B).astype(np.float32)
    for dtype in ("fp32", "bf16"):
        d_used = to_bf16_bits(drf).view(np.uint16).astype(np.uint32) if dtype == "bf16" else None
        tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
        for b in range(B):
            for i in range(K):
                row = drf[b, i] if d_used is None else (d_used[b, i] << 16).view(np.float32)
                if rng.random() < 0.6:
                    tok[b, i] = _top4_indices(row)[rng.integers(0, 4)]
        for beta in (0.5, 0.05):
            _say(f"weighted shapes B={B} V={V} dtype={dtype} beta={beta}")
            inp = _inputs_from_numpy(tgt, drf, tok, temps, beta, dtype)
            run_both(sv, oracle_mod, inp, seed=B, ptol=_ptol(dtype)).check()


@pytest.mark.parametrize("B,V", [(5, 30011), (40, 3001), (300, 2053)])
def test_ragged_draft_lengths(sv, oracle_mod, B, V):
    """Ragged draft lengths (spec_verify_ragged): K_b in [0, K] per sequence,
    mixed greedy and sampling, beta on and off, many, a few and one chunk per
    row; rows past K_b hold NaN (they must never be read); lengths outside
    [0, K] fail their sequence."""
    rng = np.random.default_rng(B * 7 + V)
    K = 5
    tgt, drf, tok = _random_case(rng, B, K, V)
    kb = rng.integers(0, K + 1, size=B).astype(np.int32)
    kb[:3] = [0, K, 2]
    if B > 10:
        kb[7], kb[9] = -1, K + 1
    for b in range(B):
        if 0 <= kb[b] <= K:
            tgt[b, kb[b] + 1:] = np.nan
            drf[b, kb[b]:] = np.nan
    temps = rng.choice([0.0, 0.6, 1.0, 1.3], size=B).astype(np.float32)
    for dtype in ("fp32", "bf16"):
        for beta in (1.0, 0.5):
            _say(f"ragged lengths B={B} V={V} dtype={dtype} beta={beta}")
            inp = _inputs_from_numpy(tgt, drf, tok, temps, beta, dtype)
            inp["draft_len"] = torch.from_numpy(kb).cuda()
            rep = run_both(sv, oracle_mod, inp, seed=B, ptol=_ptol(dtype))
            rep.check()


def test_ragged_without_draft_logits(sv, oracle_mod):
    """No draft logits: greedy sequences, and sampling sequences that drafted
    nothing (K_b = 0, bonus from target row 0); a sampling sequence with
    K_b > 0 fails."""
    rng = np.random.default_rng(77)
    B, K, V = 12, 4, 5003
    tgt, drf, tok = _random_case(rng, B, K, V)
    kb = np.array([0, 0, 3, 4, 0, 1, 0, 2, 0, 4, 0, 3], dtype=np.int32)
    temps = np.array([0.8, 1.0, 0.0, 0.0, 0.7, 0.9, 1.2, 0.0, 0.5, 0.0, 1.0, 0.0], np.float32)
    for dtype in ("fp32", "bf16"):
        _say(f"ragged without drafts dtype={dtype}")
        inp = _inputs_from_numpy(tgt, drf, tok, temps, 1.0, dtype)
        inp["draft_len"] = torch.from_numpy(kb).cuda()
        rep = run_both(sv, oracle_mod, inp, seed=3, ptol=_ptol(dtype), draft_none=True)
        rep.check()
        g = run_gpu(sv, inp, seed=3, draft_none=True)
        assert g["error_word"] & sv.SV_ERR_NO_DRAFT  # sequence 5 samples with K_b = 1
        assert np.all(g["out_tokens"][5] == -1)


@pytest.mark.parametrize("B,K,V", [(1, 3, 32000), (3, 4, 5003), (64, 4, 20011), (200, 2, 4099)])
def test_greedy_only_calls(sv, oracle_mod, B, K, V):
    """No draft logits and no ragged lengths: the streaming pass takes only the
    argmax of target rows, with its own grid and chunking (up to 31 chunks a
    row here, merged through LDS); greedy sequences match the oracle, and a
    sampling sequence fails with SV_ERR_NO_DRAFT and emits -1."""
    rng = np.random.default_rng(B * 7 + K)
    tgt, drf, tok = _random_case(rng, B, K, V)
    am = tgt[:, :K].argmax(axis=2)
    tok = np.where(rng.random((B, K)) < 0.7, am, tok).astype(np.int32)  # deep greedy runs
    temps = np.where(rng.random(B) < 0.25, 0.9, 0.0).astype(np.float32)
    temps[0] = 0.0
    for dtype in ("fp32", "bf16"):
        _say(f"greedy-only B={B} K={K} V={V} dtype={dtype}")
        inp = _inputs_from_numpy(tgt, drf, tok, temps, 1.0, dtype)
        rep = run_both(sv, oracle_mod, inp, seed=1, ptol=_ptol(dtype), draft_none=True)
        rep.check()
        g = run_gpu(sv, inp, seed=1, draft_none=True)
        samp = temps > 0
        if samp.any():
            assert g["error_word"] & sv.SV_ERR_NO_DRAFT
            assert np.all(g["out_tokens"][samp] == -1)
        assert np.all(g["out_tokens"][~samp][:, 0] >= 0)


def test_identical_rows_accept_all_and_masked_vocab(sv, oracle_mod):
    rng = np.random.default_rng(3)
    B, K, V = 16, 5, 50000
    tgt = (rng.normal(size=(B, K + 1, V)) * 3).astype(np.float32)
    tgt[:, :, rng.integers(0, V, size=V // 4)] = -np.inf  # masked tokens
    drf = np.ascontiguousarray(tgt[:, :K])
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    for dtype in ("fp32", "bf16"):
        _say(f"identical rows dtype={dtype}")
        inp = _inputs_from_numpy(tgt, drf, tok, np.full(B, 0.8, np.float32), 1.0, dtype)
        g = run_gpu(sv, inp, seed=9)
        assert np.all(g["accepted_len"] == K)
        run_both(sv, oracle_mod, inp, seed=9, ptol=_ptol(dtype)).check()


def test_error_paths(sv, oracle_mod):
    rng = np.random.default_rng(5)
    B, K, V = 8, 3, 777
    tgt, drf, tok = _random_case(rng, B, K, V)
    tok[1, 0] = V          # out of range
    tok[2, 1] = -3         # out of range
    temps = np.array([1.0, 1.0, 1.0, -1.0, np.nan, np.inf, 0.0, 0.9], dtype=np.float32)
    tgt[7, 1, :] = -np.inf  # a row without a finite maximum
    for dtype in ("fp32", "bf16"):
        _say(f"error paths dtype={dtype}")
        inp = _inputs_from_numpy(tgt, drf, tok, temps, 1.0, dtype)
        rep = run_both(sv, oracle_mod, inp, seed=1, ptol=_ptol(dtype))
        rep.check()
    # no draft logits while a sequence samples
    inp = _inputs_from_numpy(tgt, None, tok, np.array([0.0] * 7 + [1.0], np.float32), 1.0, "fp32")
    g = run_gpu(sv, inp, seed=0, draft_none=True)
    assert g["error_word"] & sv.SV_ERR_NO_DRAFT
    assert np.all(g["out_tokens"][7] == -1)


def test_extreme_logits_and_unaligned_rows(sv, oracle_mod):
    # Logits spanning +-1600 (exp underflow everywhere but the top).  Drafts are
    # the draft argmax, i.e. draws from the near one-hot draft law: a token the
    # draft law gives ~0 mass would be rejected against a residual that is pure
    # cancellation noise (p_t and q' both ~1 at a shared argmax), a draw that no
    # finite precision, fp64 included, resolves.
    rng = np.random.default_rng(8)
    B, K, V = 12, 4, 6001
    tgt, drf, tok = _random_case(rng, B, K, V, spread=400.0, noise=30.0, argmax_frac=1.0)
    temps = rng.uniform(0.3, 2.0, size=B).astype(np.float32)
    for dtype in ("fp32", "bf16"):
        _say(f"extreme/unaligned dtype={dtype}")
        inp = _inputs_from_numpy(tgt, drf, tok, temps, 0.5, dtype)
        run_both(sv, oracle_mod, inp, seed=2, ptol=_ptol(dtype)).check()
        # the same rows one element into a larger buffer: no row is 16-byte aligned
        for key in ("target", "draft"):
            t = inp[key]
            big = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
            big[1:].copy_(t.reshape(-1))
            inp[key] = big[1:].view(t.shape)
        run_both(sv, oracle_mod, inp, seed=2, ptol=_ptol(dtype)).check()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_small_residual_mass_is_accurate(sv, oracle_mod, dtype):
    """Draft rows equal the target rows except that the drafted token x gets a
    draft probability ~1e-4 where the target gives it ~1e-9: x is rejected and
    the residual, p_t minus a draft law that differs from it by ~1e-4, has mass
    Z ~ 1e-4.  Z and the bonus draw must keep their relative accuracy."""
    rng = np.random.default_rng(17)
    B, K, V = 256, 2, 5000
    tgt = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    x = rng.integers(0, V, size=(B, K))
    for b in range(B):
        for i in range(K):
            tgt[b, i, x[b, i]] = -20.0
    drf = np.ascontiguousarray(tgt[:, :K]).copy()
    for b in range(B):
        for i in range(K):
            drf[b, i, x[b, i]] = np.float32(np.log(1e-4 * V * 1.65))  # q'(x) ~ 1e-4
    _say(f"small residual mass dtype={dtype}")
    inp = _inputs_from_numpy(tgt, drf, x.astype(np.int32), np.full(B, 1.0, np.float32), 1.0, dtype)
    g = run_gpu(sv, inp, seed=4)
    h = to_numpy_inputs(inp)
    o = oracle_mod.spec_verify(h["target"], h["draft"], h["tokens"], 4, h["temperature"], h["beta"])
    rej = o["accepted_len"] < K
    assert rej.mean() > 0.9
    zo, zg = o["residual_mass"][rej], g["residual_mass"][rej].astype(np.float64)
    assert np.all(zo < 1e-3)
    np.testing.assert_allclose(zg, zo, rtol=1e-5)  # fp32 subtraction would be ~1e-3
    compare(g, o, h, 4, oracle_mod, ptol=_ptol(dtype)).check()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_repeatable_and_scratch_contents_do_not_matter(sv, dtype):
    """Repeated calls give bit-identical outputs -- tokens and every
    diagnostic float -- whatever the workspace holds before the call, with
    beta-weighted draft rows (the top-4 the streaming pass keeps out of its
    sums) and plain ones."""
    for beta in (0.5, 1.0):
        w = WORKLOADS["C5"].sized(B=64, V=20011, dtype=dtype, beta=beta)
        inp = make_inputs(w, seed=1, device="cuda")
        ws = sv.alloc_workspace(w.B, w.K, w.V, inp["target"].dtype, "cuda")
        ref = None
        for rep in range(20):
            _say(f"repeatable dtype={dtype} beta={beta} call {rep}")
            ws.fill_(0xFF if rep % 2 else 0x00)
            acc, out, aux = sv.spec_verify(inp["target"], inp["draft"], inp["tokens"], 5,
                                           inp["temperature"], inp["beta"], workspace=ws, aux=True)
            cur = [acc.cpu().numpy(), out.cpu().numpy()] + [
                aux[k].cpu().numpy().view(np.uint32) for k in ("p_target", "p_draft", "residual_mass",
                                                                "draft_conf")]
            if ref is None:
                ref = cur
            for x, y in zip(ref, cur):
                assert np.array_equal(x, y)


def _underflow_case(rng, B, K, V):
    """Every token but one has logit -800 in the target row and -790 in the
    draft row: both laws are the point mass at the one finite token d (in
    double and single precision), a drafted token x != d has ratio e^-10
    (bf16: e^-8) and is rejected, and the clamped residual is 0 everywhere."""
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
    return tgt, drf, tok, dom


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,K,V", [(8, 1, 2), (16, 3, 5000), (4, 2, 128256), (300, 2, 2053)])
def test_zero_residual_mass_draws_from_target(sv, oracle_mod, dtype, B, K, V):
    """A rejection whose residual max(p_t - q', 0) has no mass (reached by
    underflow): the bonus comes from p_t of that position, the point mass at
    its one finite token, and the reported mass C(V-1) of that draw is 1 --
    on the GPU as in the oracle, with one and many chunks and slots a row."""
    rng = np.random.default_rng(B + K + V)
    tgt, drf, tok, dom = _underflow_case(rng, B, K, V)
    _say(f"zero residual mass dtype={dtype} B={B} K={K} V={V}")
    inp = _inputs_from_numpy(tgt, drf, tok, np.ones(B, np.float32), 1.0, dtype)
    g = run_gpu(sv, inp, seed=3)
    assert np.all(g["accepted_len"] == 0)
    assert np.array_equal(g["out_tokens"][:, 0], dom[:, 0])
    assert np.all(g["out_tokens"][:, 1:] == -1)
    assert np.all(g["residual_mass"] == 1.0)
    assert g["error_word"] == 0
    run_both(sv, oracle_mod, inp, seed=3, ptol=_ptol(dtype)).check()


def test_workspace_reused_across_batch_sizes(sv, oracle_mod):
    """Back-to-back calls of different batch sizes on one workspace each match
    the oracle."""
    w = WORKLOADS["C2"].sized(B=40, V=9001)
    ws = sv.alloc_workspace(w.B, w.K, w.V, torch.bfloat16, "cuda")
    for i, B in enumerate((40, 3, 17, 40, 1)):
        inp = make_inputs(w.sized(B=B), seed=60 + i, device="cuda")
        g = run_gpu(sv, inp, seed=i, workspace=ws)
        h = to_numpy_inputs(inp)
        o = oracle_mod.spec_verify(h["target"], h["draft"], h["tokens"], i, h["temperature"],
                                   h["beta"])
        compare(g, o, h, i, oracle_mod, ptol=2e-3).check()


def test_batch_beyond_one_sub_batch(sv, oracle_mod):
    """More sequences than one sub-batch of launches holds (8192): the call is
    split into sub-batches that reuse the workspace; the uniforms stay keyed
    on each sequence's index in the call."""
    w = WORKLOADS["C5"].sized(B=9000, V=301)
    inp = make_inputs(w, seed=71, device="cuda")
    g = run_gpu(sv, inp, seed=5)
    h = to_numpy_inputs(inp)
    o = oracle_mod.spec_verify(h["target"], h["draft"], h["tokens"], 5, h["temperature"], h["beta"])
    compare(g, o, h, 5, oracle_mod, ptol=1e-5).check()


def test_stream_probe_runs_and_is_timed(sv):
    """The read-floor probe (a measurement aid) enqueues, stamps its events and
    leaves the logits untouched."""
    rng = np.random.default_rng(11)
    B, K, V = 4, 3, 10007
    tgt, drf, tok = _random_case(rng, B, K, V)
    for dtype in ("fp32", "bf16"):
        inp = _inputs_from_numpy(tgt, drf, tok, np.ones(B, np.float32), 1.0, dtype)
        before = inp["target"].clone()
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record()
        ev[1].record()
        for draft in (inp["draft"], None):
            sv.stream_probe(inp["target"], draft, events=ev)
            torch.cuda.synchronize()
            assert ev[0].elapsed_time(ev[1]) > 0.0
        assert torch.equal(before, inp["target"])


def test_empty_batch(sv):
    t = torch.empty((0, 3, 10), dtype=torch.float32, device="cuda")
    d = torch.empty((0, 2, 10), dtype=torch.float32, device="cuda")
    tok = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    acc, out = sv.spec_verify(t, d, tok, 0, torch.empty(0, device="cuda"), 1.0,
                              workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert acc.numel() == 0 and out.shape == (0, 3)
