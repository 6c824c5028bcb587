"""The verify step under HIP graph capture.

The library enqueues only kernels on the caller's stream (no allocation, no
memset, no copy, no synchronisation), so a call can be captured into a graph
and replayed.  Each case captures one call (spec_verify through a bound
Verifier with its workspace, and spec_verify_noalloc with the library's
static scratch), then replays the graph several times with the program's own
eager work in between: the outputs, the workspace and the diagnostics are
overwritten with garbage before each replay, and every replay must give the
eager call's outputs bit for bit (the captured seed is fixed).
"""
from __future__ import annotations

import pytest
import torch

from workload import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

_SKIP = not torch.cuda.is_available()
REPLAYS = 4


@pytest.fixture(scope="module")
def sv():
    if _SKIP:
        pytest.skip("no GPU")
    import draft_token_verification_03_amd as sv
    sv.load_library()
    return sv


CASES = [("C2", 16, 20011, 1.0), ("C5", 24, 12007, 0.5), ("C3", 16, 9001, 1.0), ("C4", 20, 8192, 1.0)]


@pytest.mark.parametrize("name,B,V,beta", CASES)
def test_captured_verify_replays_exactly(sv, name, B, V, beta):
    w = WORKLOADS[name].sized(B=B, V=V, beta=beta)
    inp = make_inputs(w, seed=31 + B, device="cuda")
    draft = None if w.greedy else inp["draft"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    v = sv.Verifier(inp["target"], draft, inp["tokens"], inp["temperature"], inp["beta"], stream=s,
                    aux=not w.greedy)
    with torch.cuda.stream(s):
        res = v(5)
    s.synchronize()
    ref = [x.clone() for x in res[:2]]
    ref_aux = {k: t.clone() for k, t in v.aux.items()} if v.aux is not None else None

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        v(5)
    workspace = v._keep[4]
    for r in range(REPLAYS):
        # eager work of the program between replays: garbage everywhere
        v.accepted_len.fill_(-7)
        v.out_tokens.fill_(-7)
        workspace.random_(0, 256)
        if v.aux is not None:
            for t in v.aux.values():
                t.fill_(123)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(v.accepted_len, ref[0]), r
        assert torch.equal(v.out_tokens, ref[1]), r
        if ref_aux is not None:
            for k, t in v.aux.items():
                assert torch.equal(torch.nan_to_num(t, nan=-1.0), torch.nan_to_num(ref_aux[k], nan=-1.0)), (r, k)


@pytest.mark.parametrize("name,B,V,beta", CASES[:2])
def test_captured_noalloc_replays_exactly(sv, name, B, V, beta):
    w = WORKLOADS[name].sized(B=B, V=V, beta=beta)
    inp = make_inputs(w, seed=41 + B, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, w.K + 1), dtype=torch.int32, device="cuda")
    ref_acc, ref_out = sv.spec_verify(inp["target"], inp["draft"], inp["tokens"], 9, inp["temperature"],
                                      inp["beta"])
    torch.cuda.synchronize()

    def call():
        sv.spec_verify_noalloc(inp["target"], inp["draft"], inp["tokens"], 9, inp["temperature"],
                               inp["beta"], acc, out, stream=s)

    with torch.cuda.stream(s):
        call()  # the first call on a device takes the scratch's address: outside the capture
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for r in range(REPLAYS):
        acc.fill_(-7)
        out.fill_(-7)
        # another (eager) call on the same scratch in between, with other inputs
        other = make_inputs(w, seed=500 + r, device="cuda")
        sv.spec_verify_noalloc(other["target"], other["draft"], other["tokens"], r, other["temperature"],
                               other["beta"], torch.empty_like(acc), torch.empty_like(out))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(acc, ref_acc), r
        assert torch.equal(out, ref_out), r
