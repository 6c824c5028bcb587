"""spec_verify_noalloc (the verify step on the library's static scratch, for
callers that cannot allocate) against spec_verify with a workspace, through
the C ABI: bit-identical outputs on two calls in a row, the second with a
smaller batch, and sizes beyond the scratch rejected before anything is
enqueued."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from workload import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

_SKIP = not torch.cuda.is_available()


@pytest.fixture(scope="module")
def sv():
    if _SKIP:
        pytest.skip("no GPU")
    import draft_token_verification_03_amd as sv
    sv.load_library()
    return sv


def _aux(B, K, dev):
    return {"p_target": torch.empty((B, K), dtype=torch.float32, device=dev),
            "p_draft": torch.empty((B, K), dtype=torch.float32, device=dev),
            "residual_mass": torch.empty((B,), dtype=torch.float32, device=dev),
            "draft_conf": torch.empty((B, K), dtype=torch.float32, device=dev),
            "error_word": torch.zeros((1,), dtype=torch.int32, device=dev)}


def _bits(t):
    x = t.cpu().numpy()
    return x.view(np.uint32) if x.dtype == np.float32 else x


@pytest.mark.parametrize("name", ["C5", "C4", "C3"])
def test_noalloc_matches_spec_verify(sv, name):
    w = WORKLOADS[name]
    for B, seed in ((w.B, 3), (max(1, w.B // 8), 4)):  # a full batch, then a smaller one
        print(f"noalloc {name} B={B} seed={seed}", flush=True)
        sys.stdout.flush()
        inp = make_inputs(w.sized(B=B), seed=seed, device="cuda")
        draft = None if w.greedy else inp["draft"]
        acc, out, aux = sv.spec_verify(inp["target"], draft, inp["tokens"], seed, inp["temperature"],
                                       inp["beta"], aux=True)
        acc2 = torch.full_like(acc, -7)
        out2 = torch.full_like(out, -7)
        aux2 = _aux(B, w.K, "cuda")
        sv.spec_verify_noalloc(inp["target"], draft, inp["tokens"], seed, inp["temperature"], inp["beta"],
                               acc2, out2, aux=aux2)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc2.cpu().numpy())
        assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())
        for key in ("p_target", "p_draft", "residual_mass", "draft_conf", "error_word"):
            assert np.array_equal(_bits(aux[key]), _bits(aux2[key])), key


def test_noalloc_rejects_sizes_beyond_its_scratch(sv):
    """Sizes whose workspace exceeds the static scratch return SV_ESCRATCH
    before any pointer is used (NULL buffers here)."""
    cap = sv.noalloc_max_scratch()
    assert cap == 32 << 20
    B, K, V = 8192, 128, 152064
    assert sv.workspace_size(B, K, V, torch.bfloat16) > cap
    lib = sv.load_library()
    fake = 1 << 20  # never dereferenced: the call returns before any launch
    st = lib.spec_verify_noalloc(fake, fake, fake, B, K, V, sv.SV_BF16, 0, fake, 1.0, fake, fake, None, None)
    assert st == sv.SV_ESCRATCH
    assert "scratch" in sv.status_str(st)
