"""GPU parity of tree verification (spec_verify_tree) against the oracle,
through the C-ABI.

Rule (tests/parity.py, compare_tree): accepted_len, path and out_tokens match
the oracle exactly, except that a sampling sequence may part from it at a
node's accept test within 1e-6 of its threshold (the oracle then replays the
GPU's outcome and the rest of the walk is compared) or at a bonus draw with u
within 1e-6 of the GPU token's CDF interval; such flips must be at most 1e-5
of the decisions.  Greedy and failed sequences allow no excuse.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from parity import compare_tree
from workload import WORKLOADS, make_tree_inputs

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


def _raw(x):
    if x is None:
        return None
    x = x.contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def run_gpu(sv, inp, seed, draft_none=False):
    acc, out, path, ew = sv.spec_verify_tree(inp["target"], None if draft_none else inp["draft"],
                                             inp["parent"], inp["tokens"], seed, inp["temperature"])
    torch.cuda.synchronize()
    return {"accepted_len": acc.cpu().numpy(), "out_tokens": out.cpu().numpy(),
            "path": path.cpu().numpy(), "error_word": int(ew.item())}


def host(inp, draft_none=False) -> dict:
    return {"target": _raw(inp["target"]), "draft": None if draft_none else _raw(inp["draft"]),
            "parent": inp["parent"].cpu().numpy(), "tokens": inp["tokens"].cpu().numpy(),
            "temperature": inp["temperature"].cpu().numpy()}


def run_oracle(oracle_mod, h, seed, ids=None):
    return oracle_mod.spec_verify_tree(h["target"], h["draft"], h["parent"], h["tokens"], seed,
                                       h["temperature"], seq_ids=ids)


def check(oracle_mod, g, inp, seed, draft_none=False, ids=None, gpu_ids=None):
    """Compare the GPU's walk with the oracle's (rows `ids` of the batch when
    given; the GPU outputs are indexed by `gpu_ids`, default the same) and
    return the report, after asserting the rule."""
    h = host(inp, draft_none)
    o = run_oracle(oracle_mod, h, seed, ids=ids)
    gs = g if gpu_ids is None else {k: (v[gpu_ids] if isinstance(v, np.ndarray) else v) for k, v in g.items()}
    rep = compare_tree(gs, o, h, seed, oracle_mod, seq_ids=ids)
    rep.check()
    return rep, o


SHAPES = [(4, 2, 1), (3, 3), (1, 1, 1, 1, 1), (6,), (2, 2, 2, 2)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("name,V", [("C2", 30011), ("C5", 20011), ("C4", 152064)])
def test_tree_matches_oracle(sv, oracle_mod, shape, name, V):
    """Tree shapes from a chain to a wide root, bf16 and fp32, aligned and
    unaligned rows, fixed and per-sequence temperatures."""
    w = WORKLOADS[name].sized(B=10 if V > 100000 else 24, V=V, beta=1.0)
    for s in range(2):
        _say(f"tree {name} V={V} shape={shape} seed={s}")
        inp = make_tree_inputs(w, shape, seed=50 + s, device="cuda")
        g = run_gpu(sv, inp, seed=s)
        rep, o = check(oracle_mod, g, inp, s)
        assert g["error_word"] == o["error"]
        _say(f"  decisions {rep.decisions} excused flips {rep.flips}")


def test_chain_tree_equals_chain_verify_on_gpu(sv, oracle_mod):
    """A chain-shaped tree through spec_verify_tree gives what spec_verify
    gives with K = N on the same rows and seed: both follow the oracle under
    the same rule, and with the residual formed the same way they agree."""
    w = WORKLOADS["C4"].sized(B=64, V=20011)
    N = 5
    inp = make_tree_inputs(w, (1,) * N, seed=9, device="cuda")
    g = run_gpu(sv, inp, seed=4)
    acc, out = sv.spec_verify(inp["target"], inp["draft"], inp["tokens"], 4, inp["temperature"], 1.0)
    check(oracle_mod, g, inp, 4)
    same = (acc.cpu().numpy() == g["accepted_len"]) & np.all(out.cpu().numpy() == g["out_tokens"], axis=1)
    assert same.all()


def test_greedy_trees_are_exact(sv, oracle_mod):
    w = WORKLOADS["C3"].sized(B=48, V=128256)
    for shape in ((4, 2, 1), (2, 2, 2)):
        inp = make_tree_inputs(w, shape, seed=3, device="cuda")
        # make some children the target argmax so that greedy walks go deep
        am = torch.argmax(inp["target"][:, :-1].float(), dim=2).to(torch.int32)
        par = inp["parent"]
        pick = torch.rand(par.shape, device="cuda") < 0.5
        inp["tokens"] = torch.where(pick, torch.gather(am, 1, (par + 1).long()), inp["tokens"]).contiguous()
        for draft_none in (False, True):
            _say(f"greedy trees shape={shape} draft_none={draft_none}")
            g = run_gpu(sv, inp, seed=0, draft_none=draft_none)
            rep, o = check(oracle_mod, g, inp, 0, draft_none=draft_none)
            assert rep.flips == 0
            assert g["error_word"] == o["error"]
        assert (g["accepted_len"] > 0).mean() > 0.3


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 9, 257, 4099])
def test_tiny_and_odd_vocabularies(sv, oracle_mod, dtype, V):
    w = WORKLOADS["C5" if dtype == "fp32" else "C2"].sized(B=16, V=V, beta=1.0)
    _say(f"tree tiny vocab dtype={dtype} V={V}")
    inp = make_tree_inputs(w, (3, 2), seed=V, device="cuda")
    g = run_gpu(sv, inp, seed=1)
    check(oracle_mod, g, inp, 1)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("tiles", [1, 2, 3, 4])
def test_aligned_rows_of_few_tiles(sv, oracle_mod, dtype, tiles):
    """Aligned rows (V a multiple of the 16-byte vector) stream through the
    walk's LDS ring: rows of one to four tile steps (1024 vectors each), the
    last one full or holding a single vector, so that the ring's fill loads
    repeat the last tile's addresses and the final tile's lanes past the row
    are masked."""
    vec = 4 if dtype == "fp32" else 8
    for last in (1024, 1):
        V = ((tiles - 1) * 1024 + last) * vec
        w = WORKLOADS["C5" if dtype == "fp32" else "C2"].sized(B=12, V=V, beta=1.0)
        _say(f"tree aligned rows dtype={dtype} tiles={tiles} V={V}")
        inp = make_tree_inputs(w, (3, 2, 1), seed=V + tiles, device="cuda")
        g = run_gpu(sv, inp, seed=3)
        check(oracle_mod, g, inp, 3)


def test_tree_error_paths(sv, oracle_mod):
    w = WORKLOADS["C5"].sized(B=6, V=3001, beta=1.0)
    inp = make_tree_inputs(w, (2, 2), seed=5, device="cuda")
    inp["parent"][1, 3] = 5                       # not an earlier node
    inp["target"][2, 0] = float("-inf")           # the root row has no finite logit
    inp["tokens"][3] = w.V + 7                    # every token out of range
    t = inp["temperature"].clone()
    t[4] = float("nan")
    t[5] = 0.0
    inp["temperature"] = t
    _say("tree error paths")
    g = run_gpu(sv, inp, seed=2)
    rep, o = check(oracle_mod, g, inp, 2)
    assert rep.flips == 0
    assert g["error_word"] == o["error"]
    assert g["error_word"] & sv.SV_ERR_TREE and g["error_word"] & sv.SV_ERR_ROW
    assert g["error_word"] & sv.SV_ERR_TOKEN and g["error_word"] & sv.SV_ERR_TEMPERATURE
    g = run_gpu(sv, inp, seed=2, draft_none=True)
    assert g["error_word"] & sv.SV_ERR_NO_DRAFT
    assert np.all(g["out_tokens"][0] == -1)


def test_no_nodes_draws_from_the_root(sv, oracle_mod):
    w = WORKLOADS["C2"].sized(B=32, V=9001)
    inp = make_tree_inputs(w, (), seed=8, device="cuda")
    assert inp["parent"].shape == (32, 0)
    g = run_gpu(sv, inp, seed=3, draft_none=True)
    check(oracle_mod, g, inp, 3, draft_none=True)
    assert np.all(g["accepted_len"] == 0) and np.all(g["out_tokens"][:, 0] >= 0)


def test_tree_full_size(sv, oracle_mod):
    """A C4-sized batch of (4, 2, 1) trees in one launch: every sequence
    re-verified by the oracle (with its Philox index in the call), and the
    properties that hold at any size."""
    w = WORKLOADS["C4"].sized(beta=1.0)
    shape = (4, 2, 1)
    inp = make_tree_inputs(w, shape, seed=11, device="cuda")
    _say(f"tree full size {w.tag()} shape={shape}")
    g = run_gpu(sv, inp, seed=6)
    rep, _ = check(oracle_mod, g, inp, 6)
    _say(f"  decisions {rep.decisions} excused flips {rep.flips}")
    # properties at any size: a path follows parent links, tokens are the nodes'
    par = inp["parent"][0].cpu().numpy()
    tok = inp["tokens"].cpu().numpy()
    for b in range(w.B):
        d = g["accepted_len"][b]
        prev = -1
        for k in range(d):
            node = g["path"][b, k]
            assert par[node] == prev and g["out_tokens"][b, k] == tok[b, node]
            prev = node
        assert 0 <= g["out_tokens"][b, d] < w.V and np.all(g["out_tokens"][b, d + 1:] == -1)
    assert g["error_word"] == 0


def test_largest_trees_and_mixed_modes(sv, oracle_mod):
    """N = 128 nodes (the maximum): a random tree (each node's parent drawn
    from the earlier nodes and the root) and a 128-deep chain, with greedy
    and sampling sequences in one batch."""
    rng = np.random.default_rng(77)
    B, N, V = 12, 128, 257
    for kind in ("random", "chain"):
        if kind == "random":
            par = np.array([[rng.integers(-1, i) for i in range(N)] for _ in range(B)], dtype=np.int32)
        else:
            par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
        base = rng.normal(size=(B, N + 1, V)) * 1.2
        tgt = (base + 0.3 * rng.normal(size=base.shape)).astype(np.float32)
        drf = base[:, :N].astype(np.float32)
        tok = np.empty((B, N), dtype=np.int32)
        for b in range(B):
            for i in range(N):
                q = np.exp(drf[b, par[b, i] + 1] - drf[b, par[b, i] + 1].max())
                tok[b, i] = rng.choice(V, p=q / q.sum())
        temps = np.where(np.arange(B) % 3 == 0, 0.0, 0.9).astype(np.float32)
        inp = {"target": torch.from_numpy(tgt).cuda(), "draft": torch.from_numpy(drf).cuda(),
               "parent": torch.from_numpy(par).cuda(), "tokens": torch.from_numpy(tok).cuda(),
               "temperature": torch.from_numpy(temps).cuda()}
        _say(f"largest trees {kind}")
        g = run_gpu(sv, inp, seed=5)
        _, o = check(oracle_mod, g, inp, 5)
        assert g["error_word"] == o["error"]
        if kind == "chain":
            assert g["accepted_len"].max() > 8


def test_tree_residual_keeps_relative_accuracy(sv, oracle_mod):
    """Siblings whose draft law nearly equals the target law: after a
    rejection the next law is the residual of two close laws, whose mass is
    small (~1e-3) and must keep its relative accuracy for the next sibling's
    test and the bonus to follow the oracle at the 1e-6 margin."""
    rng = np.random.default_rng(91)
    B, V = 64, 5003
    parent = np.array([-1, -1, -1, -1], dtype=np.int32)
    N = parent.size
    for dtype in ("fp32", "bf16"):
        tgt = rng.normal(size=(B, N + 1, V)).astype(np.float32)
        drf = tgt[:, :N].copy()
        # the draft moves 1e-3 of mass away from one token of each row
        x = rng.integers(0, V, size=(B, N))
        for b in range(B):
            drf[b, 0, x[b, 0]] += np.float32(np.log1p(2e-3 * V / 1.65))
        tok = np.where(rng.random((B, N)) < 0.7, x[:, :1].repeat(N, 1), rng.integers(0, V, size=(B, N)))
        if dtype == "bf16":
            tt = torch.from_numpy(tgt).to(torch.bfloat16)
            dd = torch.from_numpy(drf).to(torch.bfloat16)
        else:
            tt, dd = torch.from_numpy(tgt), torch.from_numpy(drf)
        inp = {"target": tt.contiguous().cuda(), "draft": dd.contiguous().cuda(),
               "parent": torch.from_numpy(np.tile(parent, (B, 1))).cuda(),
               "tokens": torch.from_numpy(tok.astype(np.int32)).contiguous().cuda(),
               "temperature": torch.ones(B, device="cuda")}
        _say(f"tree small residual dtype={dtype}")
        g = run_gpu(sv, inp, seed=7)
        rep, _ = check(oracle_mod, g, inp, 7)
        _say(f"  decisions {rep.decisions} excused flips {rep.flips}")
