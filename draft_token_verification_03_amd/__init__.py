"""Python binding of libspecverify, the speculative-sampling verify step for
AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the verify step runs in the HIP
kernels of ``libspecverify.so`` (built in-tree by ``build.py``).  PyTorch is
used for device memory and the current stream.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_F32 = 0
SV_BF16 = 1
SV_OK = 0
SV_EINVAL = -1
SV_EWORKSPACE = -2
SV_EHIP = -3
SV_ESCRATCH = -4

SV_ERR_TOKEN = 1
SV_ERR_TEMPERATURE = 2
SV_ERR_ROW = 4
SV_ERR_DRAFT_MASS = 8
SV_ERR_NO_DRAFT = 16
SV_ERR_DRAFT_LEN = 32
SV_ERR_TREE = 64
MAX_TREE_NODES = 128

EXPORTED = ("spec_verify", "spec_verify_ragged", "spec_verify_workspace_size", "spec_verify_row_stats",
            "spec_verify_uniforms", "spec_verify_stream_probe", "spec_verify_outcomes",
            "spec_verify_outcomes_workspace_size", "spec_verify_tree", "spec_verify_status_str",
            "spec_verify_noalloc", "spec_verify_noalloc_max_scratch")
MAX_OUTCOME_F = 32


class SpecVerifyError(RuntimeError):
    pass


class _Aux(ctypes.Structure):
    _fields_ = [("p_target", ctypes.c_void_p), ("p_draft", ctypes.c_void_p),
                ("residual_mass", ctypes.c_void_p), ("error_word", ctypes.c_void_p),
                ("pass_begin", ctypes.c_void_p), ("pass_end", ctypes.c_void_p),
                ("draft_conf", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecverify.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise SpecVerifyError(
            f"{path} is missing: build it with `python -m draft_token_verification_03_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.spec_verify_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_workspace_size.restype = sz
    lib.spec_verify.argtypes = [P, P, P, i32, i32, i32, i32, u64, P, f32, P, P, P, sz,
                                ctypes.POINTER(_Aux), P]
    lib.spec_verify.restype = i32
    lib.spec_verify_ragged.argtypes = [P, P, P, P, i32, i32, i32, i32, u64, P, f32, P, P, P, sz,
                                       ctypes.POINTER(_Aux), P]
    lib.spec_verify_ragged.restype = i32
    lib.spec_verify_row_stats.argtypes = [P, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.spec_verify_row_stats.restype = i32
    lib.spec_verify_uniforms.argtypes = [u64, i32, i32, P, P]
    lib.spec_verify_uniforms.restype = i32
    lib.spec_verify_stream_probe.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P]
    lib.spec_verify_stream_probe.restype = i32
    lib.spec_verify_outcomes_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.spec_verify_outcomes_workspace_size.restype = sz
    lib.spec_verify_outcomes.argtypes = [P, P, i32, i32, i32, i32, P, f32, i32, P, P, P, P, P, P, P,
                                         sz, P, P, P]
    lib.spec_verify_outcomes.restype = i32
    lib.spec_verify_tree.argtypes = [P, P, P, P, i32, i32, i32, i32, u64, P, P, P, P, P, P, P, P]
    lib.spec_verify_tree.restype = i32
    lib.spec_verify_noalloc.argtypes = [P, P, P, i32, i32, i32, i32, u64, P, f32, P, P,
                                        ctypes.POINTER(_Aux), P]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_verify_noalloc_max_scratch.argtypes = []
    lib.spec_verify_noalloc_max_scratch.restype = sz
    lib.spec_verify_status_str.argtypes = [i32]
    lib.spec_verify_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().spec_verify_status_str(int(status)).decode()


def _check(status: int) -> None:
    if status != SV_OK:
        raise SpecVerifyError(status_str(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_size(B: int, K: int, V: int, dtype: torch.dtype) -> int:
    code = SV_F32 if dtype == torch.float32 else SV_BF16
    return int(load_library().spec_verify_workspace_size(B, K, V, code))


def alloc_workspace(B: int, K: int, V: int, dtype: torch.dtype, device) -> torch.Tensor:
    """A workspace for these sizes (scratch: its contents do not matter)."""
    n = workspace_size(B, K, V, dtype)
    if n == 0:
        raise SpecVerifyError("invalid sizes for a workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


class Verifier:
    """One verify step with its buffers bound once, for loops that run the
    step repeatedly (a decode loop, a benchmark): each call only marshals the
    seed and enqueues the kernels.

    target [B, K+1, V] and draft [B, K, V] (or None if every temperature is 0)
    are contiguous float32 or bfloat16 CUDA tensors; tokens [B, K] int32;
    temperature a float or a [B] float32 tensor (0 = greedy); beta in [0, 1].
    The outputs accepted_len [B] and out_tokens [B, K+1] (int32) are
    allocated unless passed in, and so is the workspace.  With aux=True the
    diagnostics p_target, p_draft, residual_mass, draft_conf and error_word
    are written too (error_word is cleared before every call).  draft_len, a
    [B] int32 tensor, gives ragged draft lengths K_b <= K
    (spec_verify_ragged).
    """

    def __init__(self, target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor,
                 temperature, beta: float = 1.0, *, workspace: torch.Tensor | None = None,
                 accepted_len: torch.Tensor | None = None, out_tokens: torch.Tensor | None = None,
                 aux: bool = False, stream=None, draft_len: torch.Tensor | None = None):
        if target.dim() != 3:
            raise ValueError("target must be [B, K+1, V]")
        B, K1, V = target.shape
        K = K1 - 1
        dev = target.device
        code = _dtype_code(target)
        if not target.is_contiguous():
            raise ValueError("target must be contiguous")
        if draft is not None:
            if draft.shape != (B, K, V) or draft.dtype != target.dtype or not draft.is_contiguous():
                raise ValueError("draft must be a contiguous [B, K, V] tensor of the target's dtype")
        if tokens.shape != (B, K) or tokens.dtype != torch.int32 or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous [B, K] int32 tensor")
        if draft_len is not None and (draft_len.shape != (B,) or draft_len.dtype != torch.int32
                                      or not draft_len.is_contiguous()):
            raise ValueError("draft_len must be a contiguous [B] int32 tensor")
        if not torch.is_tensor(temperature):
            temperature = torch.full((B,), float(temperature), dtype=torch.float32, device=dev)
        if temperature.shape != (B,) or temperature.dtype != torch.float32:
            raise ValueError("temperature must be a [B] float32 tensor")
        temperature = temperature.contiguous()
        if workspace is None:
            workspace = alloc_workspace(B, K, V, target.dtype, dev)
        if accepted_len is None:
            accepted_len = torch.empty(B, dtype=torch.int32, device=dev)
        if out_tokens is None:
            out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        self.shape = (B, K, V)
        self.accepted_len, self.out_tokens = accepted_len, out_tokens
        # keep every buffer alive for as long as the bound call
        self._keep = (target, draft, tokens, temperature, workspace, draft_len)
        self.aux = None
        self._aux = _Aux()
        if aux:
            self.aux = {
                "p_target": torch.empty((B, K), dtype=torch.float32, device=dev),
                "p_draft": torch.empty((B, K), dtype=torch.float32, device=dev),
                "residual_mass": torch.empty((B,), dtype=torch.float32, device=dev),
                "error_word": torch.zeros((1,), dtype=torch.int32, device=dev),
                "draft_conf": torch.empty((B, K), dtype=torch.float32, device=dev),
            }
            self._aux.p_target = self.aux["p_target"].data_ptr()
            self._aux.p_draft = self.aux["p_draft"].data_ptr()
            self._aux.residual_mass = self.aux["residual_mass"].data_ptr()
            self._aux.error_word = self.aux["error_word"].data_ptr()
            self._aux.draft_conf = self.aux["draft_conf"].data_ptr()
        if draft_len is None:
            self._fn = load_library().spec_verify
            self._head = (_ptr(target), _ptr(draft), _ptr(tokens), B, K, V, code)
        else:
            self._fn = load_library().spec_verify_ragged
            self._head = (_ptr(target), _ptr(draft), _ptr(tokens), _ptr(draft_len), B, K, V, code)
        self._mid = (_ptr(temperature), ctypes.c_float(float(beta)), _ptr(accepted_len),
                     _ptr(out_tokens), _ptr(workspace), workspace.numel())
        self._stream = _stream(stream)

    def __call__(self, seed: int, pass_events=None):
        """Enqueue one verify step with this Philox seed; returns
        (accepted_len, out_tokens), plus the diagnostics dict when bound with
        aux=True.  pass_events, a pair of torch.cuda.Event that have been
        recorded once (so that they exist), are recorded on the stream right
        before and after the streaming-pass launch."""
        aux = self._aux
        if self.aux is not None:
            self.aux["error_word"].zero_()
        if pass_events is not None:
            aux.pass_begin = pass_events[0].cuda_event
            aux.pass_end = pass_events[1].cuda_event
        else:
            aux.pass_begin = aux.pass_end = None
        use_aux = self.aux is not None or pass_events is not None
        _check(self._fn(*self._head, int(seed) & (2**64 - 1), *self._mid,
                        ctypes.byref(aux) if use_aux else None, self._stream))
        if self.aux is not None:
            return self.accepted_len, self.out_tokens, self.aux
        return self.accepted_len, self.out_tokens


def spec_verify(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor,
                seed: int, temperature, beta: float = 1.0, *, workspace: torch.Tensor | None = None,
                accepted_len: torch.Tensor | None = None, out_tokens: torch.Tensor | None = None,
                aux: bool = False, stream=None, draft_len: torch.Tensor | None = None):
    """Verify K drafted tokens per sequence (one call of the C entry point).

    Arguments as for Verifier.  Returns (accepted_len [B] int32, out_tokens
    [B, K+1] int32), plus a dict of diagnostics (p_target, p_draft,
    residual_mass, draft_conf, error_word) if aux=True.  The work is enqueued
    on `stream` (default: the current stream); a workspace of at least
    workspace_size(B, K, V, dtype) bytes may be passed in (e.g. from
    alloc_workspace) to avoid an allocation per call.  draft_len [B] int32
    gives ragged draft lengths (spec_verify_ragged).
    """
    return Verifier(target, draft, tokens, temperature, beta, workspace=workspace,
                    accepted_len=accepted_len, out_tokens=out_tokens, aux=aux, stream=stream,
                    draft_len=draft_len)(seed)


def spec_verify_noalloc(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor,
                        seed: int, temperature: torch.Tensor, beta: float, accepted_len: torch.Tensor,
                        out_tokens: torch.Tensor, *, aux: dict | None = None, stream=None) -> None:
    """The verify step through spec_verify_noalloc: no workspace, the
    library's static scratch instead, for callers that cannot allocate device
    memory.  Every buffer is the caller's: target [B, K+1, V], draft [B, K, V]
    or None, tokens [B, K] int32, temperature [B] float32, accepted_len [B]
    and out_tokens [B, K+1] int32 (written), and optionally aux, a dict of
    p_target [B, K], p_draft [B, K], residual_mass [B], draft_conf [B, K]
    (float32) and error_word [1] (int32, OR-ed into) tensors.  Nothing is
    allocated here; calls on one GPU must not overlap in time."""
    B, K1, V = target.shape
    a = None
    if aux is not None:
        a = _Aux()
        for key in ("p_target", "p_draft", "residual_mass", "error_word", "draft_conf"):
            if aux.get(key) is not None:
                setattr(a, key, aux[key].data_ptr())
    _check(load_library().spec_verify_noalloc(
        _ptr(target), _ptr(draft), _ptr(tokens), B, K1 - 1, V, _dtype_code(target),
        int(seed) & (2**64 - 1), _ptr(temperature), ctypes.c_float(float(beta)), _ptr(accepted_len),
        _ptr(out_tokens), ctypes.byref(a) if a is not None else None, _stream(stream)))


def noalloc_max_scratch() -> int:
    """Bytes of spec_verify_noalloc's static scratch."""
    return int(load_library().spec_verify_noalloc_max_scratch())


def row_stats(logits: torch.Tensor, temperature, *, stream=None):
    """Streaming-pass statistics of each row of a [rows, V] tensor:
    (max [rows] f32, ln sum exp((z - max)/T) [rows] f64, argmax [rows] i32);
    rows with T == 0 get the argmax and a NaN log-sum."""
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [rows, V] tensor")
    rows, V = logits.shape
    dev = logits.device
    code = _dtype_code(logits)
    if not torch.is_tensor(temperature):
        temperature = torch.full((rows,), float(temperature), dtype=torch.float32, device=dev)
    temperature = temperature.contiguous()
    ws = alloc_workspace(max(rows, 1), 0, V, logits.dtype, dev)
    mx = torch.empty(rows, dtype=torch.float32, device=dev)
    ls = torch.empty(rows, dtype=torch.float64, device=dev)
    am = torch.empty(rows, dtype=torch.int32, device=dev)
    _check(load_library().spec_verify_row_stats(
        _ptr(logits), rows, V, code, _ptr(temperature), _ptr(mx), _ptr(ls), _ptr(am), _ptr(ws),
        ws.numel(), _stream(stream)))
    return mx, ls, am


def stream_probe(target: torch.Tensor, draft, *, sink=None, events=None, stream=None) -> None:
    """The streaming pass over these logits with its arithmetic taken out (a
    measurement aid: its duration is the read floor of the pass).  `events`:
    optional (begin, end) torch.cuda.Event pair stamped with the kernel's
    start and end."""
    B, K1, V = target.shape
    code = _dtype_code(target)
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=target.device)
    b_ev = e_ev = None
    if events is not None:
        b_ev, e_ev = events[0].cuda_event, events[1].cuda_event
    _check(load_library().spec_verify_stream_probe(
        _ptr(target), _ptr(draft) if draft is not None else None, B, K1 - 1, V, code, _ptr(sink),
        b_ev, e_ev, _stream(stream)))


def uniforms(seed: int, B: int, P: int, *, device="cuda", stream=None) -> torch.Tensor:
    """u(b, pos, purpose) as a [B, P, 2] float32 tensor."""
    out = torch.empty((B, P, 2), dtype=torch.float32, device=device)
    _check(load_library().spec_verify_uniforms(int(seed) & (2**64 - 1), B, P, _ptr(out),
                                               _stream(stream)))
    return out


def outcomes_workspace_size(B: int, K: int, V: int, dtype: torch.dtype, F: int) -> int:
    code = SV_F32 if dtype == torch.float32 else SV_BF16
    return int(load_library().spec_verify_outcomes_workspace_size(B, K, V, code, F))


class Outcomes:
    """The verification-outcome distribution (spec_verify_outcomes) with its
    buffers bound once, for repeated calls.

    target [B, K+1, V] and draft [B, K, V] (or None) are contiguous float32 or
    bfloat16 CUDA tensors; temperature a float or a [B] float32 tensor; beta in
    [0, 1]; F ranked bonus tokens per position (0..32).  Each call returns a
    dict of accept_rate [B, K], p_len [B, K+1], top_tokens [B, K+1, F] int32,
    top_mass [B, K+1, F] (float32) and error_word [1] int32 (cleared before
    every call); with draft_top=True also draft_top_mass [B, K], the residual
    mass on each draft row's top-4.
    """

    def __init__(self, target: torch.Tensor, draft: torch.Tensor | None, temperature,
                 beta: float = 1.0, F: int = 8, *, workspace: torch.Tensor | None = None,
                 stream=None, draft_top: bool = False):
        if target.dim() != 3 or not target.is_contiguous():
            raise ValueError("target must be a contiguous [B, K+1, V] tensor")
        B, K1, V = target.shape
        K = K1 - 1
        dev = target.device
        code = _dtype_code(target)
        if draft is not None:
            if draft.shape != (B, K, V) or draft.dtype != target.dtype or not draft.is_contiguous():
                raise ValueError("draft must be a contiguous [B, K, V] tensor of the target's dtype")
        if not 0 <= F <= MAX_OUTCOME_F:
            raise ValueError(f"F must be in [0, {MAX_OUTCOME_F}]")
        if not torch.is_tensor(temperature):
            temperature = torch.full((B,), float(temperature), dtype=torch.float32, device=dev)
        if temperature.shape != (B,) or temperature.dtype != torch.float32:
            raise ValueError("temperature must be a [B] float32 tensor")
        temperature = temperature.contiguous()
        if workspace is None:
            n = outcomes_workspace_size(max(B, 1), K, V, target.dtype, F)
            if n == 0:
                raise SpecVerifyError("invalid sizes for a workspace")
            workspace = torch.empty(n, dtype=torch.uint8, device=dev)
        self.out = {
            "accept_rate": torch.empty((B, K), dtype=torch.float32, device=dev),
            "p_len": torch.empty((B, K + 1), dtype=torch.float32, device=dev),
            "top_tokens": torch.empty((B, K + 1, F), dtype=torch.int32, device=dev),
            "top_mass": torch.empty((B, K + 1, F), dtype=torch.float32, device=dev),
            "error_word": torch.zeros((1,), dtype=torch.int32, device=dev),
        }
        if draft_top:
            self.out["draft_top_mass"] = torch.empty((B, K), dtype=torch.float32, device=dev)
        o = self.out
        self._keep = (target, draft, temperature, workspace)
        self._args = (_ptr(target), _ptr(draft), B, K, V, code, _ptr(temperature),
                      ctypes.c_float(float(beta)), int(F), _ptr(o["accept_rate"]), _ptr(o["p_len"]),
                      _ptr(o["top_tokens"]), _ptr(o["top_mass"]), _ptr(o.get("draft_top_mass")),
                      _ptr(o["error_word"]), _ptr(workspace), workspace.numel())
        self._stream = _stream(stream)

    def __call__(self, pass_events=None) -> dict:
        """Enqueue the call; pass_events, a pair of recorded torch.cuda.Event,
        are stamped with the start and end of the outcome-pass kernel."""
        self.out["error_word"].zero_()
        b_ev = e_ev = None
        if pass_events is not None:
            b_ev, e_ev = pass_events[0].cuda_event, pass_events[1].cuda_event
        _check(load_library().spec_verify_outcomes(*self._args, b_ev, e_ev, self._stream))
        return self.out


def outcomes(target: torch.Tensor, draft: torch.Tensor | None, temperature, beta: float = 1.0,
             F: int = 8, *, workspace: torch.Tensor | None = None, stream=None,
             draft_top: bool = False) -> dict:
    """Verification-outcome distribution of every sequence: accept rates
    alpha_j, the law of the accepted length and the F likeliest bonus tokens
    of each position with their residual masses, and with draft_top=True the
    residual mass on each draft row's top-4 (see Outcomes)."""
    return Outcomes(target, draft, temperature, beta, F, workspace=workspace, stream=stream,
                    draft_top=draft_top)()


class TreeVerifier:
    """Tree (multi-draft) verification (spec_verify_tree) with its buffers
    bound once.  target [B, N+1, V] (row c: target logits after context c,
    context 0 the root and context i + 1 node i), draft [B, N, V] (row c: the
    draft logits the children of context c were drawn from; None if every
    temperature is 0), parent and tokens [B, N] int32 (parent[i] in
    [-1, i-1]), temperature a float or [B] float32 tensor.  Each call returns
    (accepted_len [B], out_tokens [B, N+1], path [B, N], error_word [1]);
    error_word is cleared before every call."""

    def __init__(self, target: torch.Tensor, draft: torch.Tensor | None, parent: torch.Tensor,
                 tokens: torch.Tensor, temperature, *, stream=None):
        if target.dim() != 3 or not target.is_contiguous():
            raise ValueError("target must be a contiguous [B, N+1, V] tensor")
        B, N1, V = target.shape
        N = N1 - 1
        dev = target.device
        code = _dtype_code(target)
        if draft is not None and (draft.shape != (B, N, V) or draft.dtype != target.dtype
                                  or not draft.is_contiguous()):
            raise ValueError("draft must be a contiguous [B, N, V] tensor of the target's dtype")
        for name, x in (("parent", parent), ("tokens", tokens)):
            if x.shape != (B, N) or x.dtype != torch.int32 or not x.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [B, N] int32 tensor")
        if not torch.is_tensor(temperature):
            temperature = torch.full((B,), float(temperature), dtype=torch.float32, device=dev)
        temperature = temperature.contiguous()
        self.accepted_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
        self.path = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.error_word = torch.zeros((1,), dtype=torch.int32, device=dev)
        self._keep = (target, draft, parent, tokens, temperature)
        self._head = (_ptr(target), _ptr(draft), _ptr(parent), _ptr(tokens), B, N, V, code)
        self._tail = (_ptr(temperature), _ptr(self.accepted_len), _ptr(self.out_tokens), _ptr(self.path),
                      _ptr(self.error_word))
        self._stream = _stream(stream)

    def __call__(self, seed: int, pass_events=None):
        self.error_word.zero_()
        b_ev = e_ev = None
        if pass_events is not None:
            b_ev, e_ev = pass_events[0].cuda_event, pass_events[1].cuda_event
        _check(load_library().spec_verify_tree(*self._head, int(seed) & (2**64 - 1), *self._tail, b_ev,
                                               e_ev, self._stream))
        return self.accepted_len, self.out_tokens, self.path, self.error_word


def spec_verify_tree(target: torch.Tensor, draft: torch.Tensor | None, parent: torch.Tensor,
                     tokens: torch.Tensor, seed: int, temperature, *, stream=None):
    """Verify a token tree per sequence (see TreeVerifier); returns
    (accepted_len, out_tokens, path, error_word)."""
    return TreeVerifier(target, draft, parent, tokens, temperature, stream=stream)(seed)
