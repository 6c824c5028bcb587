"""The C-ABI boundary on the CPU: the library loads, exports every function
include/*.h declares, sizes workspaces, and rejects invalid arguments with a
status code before anything reaches the GPU (no compute call is made here)."""
from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import draft_token_verification_03_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        from draft_token_verification_03_amd import build
        build.build()
    return sv.load_library()


def declared_functions() -> set[str]:
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M):
            name = m.group(1)
            if name not in ("defined",):
                names.add(name)
    return names


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert {"spec_verify", "spec_verify_workspace_size", "spec_verify_row_stats",
            "spec_verify_uniforms", "spec_verify_status_str"} <= names


def test_every_declared_symbol_is_exported(lib):
    import draft_token_verification_03_amd as sv
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert set(sv.EXPORTED) <= declared_functions()


def test_status_strings(lib):
    import draft_token_verification_03_amd as sv
    for code in (sv.SV_OK, sv.SV_EINVAL, sv.SV_EWORKSPACE, sv.SV_EHIP):
        assert sv.status_str(code).startswith("SV_")
    assert sv.status_str(12345) == "unknown status"


def test_workspace_size(lib):
    f = lib.spec_verify_workspace_size
    assert f(8, 5, 128256, 1) > 0
    assert f(8, 5, 128256, 1) % 256 == 0
    assert f(512, 5, 128256, 0) >= f(8, 5, 128256, 0)
    assert f(1, 0, 7, 0) > 0          # K = 0 (plain sampling) is allowed
    assert f(-1, 5, 100, 0) == 0
    assert f(1, -1, 100, 0) == 0
    assert f(1, 129, 100, 0) == 0     # K above the documented maximum
    assert f(1, 4, 0, 0) == 0
    assert f(1, 4, 100, 7) == 0


# fake but well-aligned device addresses: validation must reject before use
A = 0x7F0000000000


def _call(lib, **kw):
    args = dict(target=A, draft=A + 0x100000, tokens=A + 0x200000, B=2, K=3, V=1000, dtype=1,
                seed=0, temperature=A + 0x300000, beta=1.0, acc=A + 0x400000,
                out=A + 0x500000, ws=A + 0x600000, wsbytes=1 << 30, aux=None, stream=None)
    args.update(kw)
    return lib.spec_verify(args["target"], args["draft"], args["tokens"], args["B"], args["K"],
                           args["V"], args["dtype"], args["seed"], args["temperature"],
                           args["beta"], args["acc"], args["out"], args["ws"], args["wsbytes"],
                           args["aux"], args["stream"])


@pytest.mark.parametrize("bad", [
    dict(B=-1), dict(K=-1), dict(K=129), dict(V=0), dict(V=-5), dict(dtype=2),
    dict(beta=1.5), dict(beta=-0.1), dict(beta=float("nan")),
    dict(target=None), dict(temperature=None), dict(acc=None), dict(out=None),
    dict(tokens=None), dict(target=A + 1), dict(draft=A + 0x100001),
    dict(target=A + 2, dtype=0),
])
def test_invalid_arguments_rejected(lib, bad):
    import draft_token_verification_03_amd as sv
    assert _call(lib, **bad) == sv.SV_EINVAL


@pytest.mark.parametrize("bad", [dict(ws=None), dict(ws=A + 0x600010), dict(wsbytes=16)])
def test_bad_workspace_rejected(lib, bad):
    import draft_token_verification_03_amd as sv
    assert _call(lib, **bad) == sv.SV_EWORKSPACE


def test_empty_batch_is_a_noop(lib):
    import draft_token_verification_03_amd as sv
    # B == 0 returns before touching any pointer, even NULL ones
    assert _call(lib, B=0, target=None, draft=None, tokens=None, temperature=None, acc=None,
                 out=None, ws=None, wsbytes=0) == sv.SV_OK


def test_tokens_may_be_null_when_no_drafts(lib):
    import draft_token_verification_03_amd as sv
    # K == 0 with NULL tokens passes validation up to the workspace check
    assert _call(lib, K=0, tokens=None, draft=None, ws=None) == sv.SV_EWORKSPACE


def test_row_stats_and_uniforms_validation(lib):
    import draft_token_verification_03_amd as sv
    P = ctypes.c_void_p
    assert lib.spec_verify_row_stats(P(A), -1, 10, 0, P(A), P(A), P(A), P(A), P(A), 1 << 20,
                                     None) == sv.SV_EINVAL
    assert lib.spec_verify_row_stats(None, 4, 10, 0, P(A), P(A), P(A), P(A), P(A), 1 << 20,
                                     None) == sv.SV_EINVAL
    assert lib.spec_verify_row_stats(P(A), 4, 10, 0, P(A), P(A), P(A), P(A), None, 0,
                                     None) == sv.SV_EWORKSPACE
    assert lib.spec_verify_row_stats(P(A), 0, 10, 0, None, None, None, None, None, 0,
                                     None) == sv.SV_OK
    assert lib.spec_verify_uniforms(0, -1, 3, P(A), None) == sv.SV_EINVAL
    assert lib.spec_verify_uniforms(0, 4, 3, None, None) == sv.SV_EINVAL
    assert lib.spec_verify_uniforms(0, 0, 3, None, None) == sv.SV_OK


def test_binding_fails_loudly_without_library(tmp_path):
    import draft_token_verification_03_amd as sv
    saved = sv._lib
    sv._lib = None
    try:
        with pytest.raises(sv.SpecVerifyError):
            sv.load_library(str(tmp_path / "missing.so"))
    finally:
        sv._lib = saved


def test_outcomes_validation(lib):
    """spec_verify_outcomes and its workspace size reject bad arguments
    before any launch."""
    import draft_token_verification_03_amd as sv
    P = ctypes.c_void_p
    ws = lib.spec_verify_outcomes_workspace_size
    assert ws(8, 5, 1000, 1, 8) > 0 and ws(8, 5, 1000, 1, 8) % 256 == 0
    assert ws(8, 5, 1000, 1, 32) > ws(8, 5, 1000, 1, 0) > 0
    assert ws(8, 5, 1000, 1, 33) == 0 and ws(8, 5, 1000, 1, -1) == 0 and ws(-1, 5, 1000, 1, 8) == 0

    def call(**kw):
        a = dict(t=P(A), d=P(A + 0x100000), B=2, K=3, V=1000, dt=1, temp=P(A + 0x200000), beta=1.0, F=4,
                 ar=P(A + 0x300000), pl=P(A + 0x400000), tt=P(A + 0x500000), tm=P(A + 0x600000), dtm=None,
                 ew=None, w=P(A + 0x700000), wb=1 << 30)
        a.update(kw)
        return lib.spec_verify_outcomes(a["t"], a["d"], a["B"], a["K"], a["V"], a["dt"], a["temp"],
                                        ctypes.c_float(a["beta"]), a["F"], a["ar"], a["pl"], a["tt"], a["tm"],
                                        a["dtm"], a["ew"], a["w"], a["wb"], None, None, None)
    for bad in (dict(F=33), dict(F=-1), dict(beta=float("nan")), dict(beta=2.0), dict(K=129), dict(V=0),
                dict(dt=3), dict(t=None), dict(temp=None), dict(pl=None), dict(ar=None), dict(tt=None),
                dict(tm=None), dict(t=P(A + 1))):
        assert call(**bad) == sv.SV_EINVAL, bad
    assert call(w=None) == sv.SV_EWORKSPACE
    assert call(wb=64) == sv.SV_EWORKSPACE
    assert call(B=0, t=None, temp=None, pl=None, ar=None, tt=None, tm=None, w=None, wb=0) == sv.SV_OK
    # F == 0 needs no ranked outputs; K == 0 needs no accept rates (stops at the workspace check)
    assert call(F=0, tt=None, tm=None, w=None) == sv.SV_EWORKSPACE
    assert call(K=0, ar=None, d=None, w=None) == sv.SV_EWORKSPACE


def test_tree_validation(lib):
    """spec_verify_tree rejects bad arguments before any launch."""
    import draft_token_verification_03_amd as sv
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(t=P(A), d=P(A + 0x100000), par=P(A + 0x200000), tok=P(A + 0x300000), B=2, N=5, V=1000, dt=1,
                 temp=P(A + 0x400000), acc=P(A + 0x500000), out=P(A + 0x600000), path=P(A + 0x700000))
        a.update(kw)
        return lib.spec_verify_tree(a["t"], a["d"], a["par"], a["tok"], a["B"], a["N"], a["V"], a["dt"], 0,
                                    a["temp"], a["acc"], a["out"], a["path"], None, None, None, None)
    for bad in (dict(B=-1), dict(N=-1), dict(N=129), dict(V=0), dict(dt=2), dict(t=None), dict(temp=None),
                dict(acc=None), dict(out=None), dict(par=None), dict(tok=None), dict(path=None),
                dict(t=P(A + 1)), dict(d=P(A + 0x100001)), dict(V=1 << 25)):
        assert call(**bad) == sv.SV_EINVAL, bad
    assert call(B=0, t=None, temp=None, acc=None, out=None, par=None, tok=None, path=None) == sv.SV_OK


def test_noalloc_validation(lib):
    """spec_verify_noalloc validates like spec_verify and rejects sizes whose
    workspace exceeds its static scratch with SV_ESCRATCH, all before any
    pointer is used or anything is enqueued (no device call is made here)."""
    import draft_token_verification_03_amd as sv
    f = lib.spec_verify_noalloc
    assert lib.spec_verify_noalloc_max_scratch() == 32 << 20
    # B == 0: a no-op even with NULL buffers
    assert f(None, None, None, 0, 4, 100, sv.SV_F32, 0, None, 1.0, None, None, None, None) == sv.SV_OK
    fake = 1 << 20
    args = dict(t=fake, d=fake, tok=fake, B=4, K=3, V=1000, dt=sv.SV_F32, T=fake, beta=1.0, acc=fake, out=fake)

    def call(**kw):
        a = {**args, **kw}
        return f(a["t"], a["d"], a["tok"], a["B"], a["K"], a["V"], a["dt"], 0, a["T"], a["beta"], a["acc"],
                 a["out"], None, None)

    for bad in (dict(B=-1), dict(K=129), dict(V=0), dict(dt=5), dict(beta=2.0), dict(t=None), dict(acc=None),
                dict(t=fake + 2)):
        assert call(**bad) == sv.SV_EINVAL, bad
    assert call(B=8192, K=128, V=152064, dt=sv.SV_BF16) == sv.SV_ESCRATCH
    assert sv.status_str(sv.SV_ESCRATCH).startswith("SV_ESCRATCH")
