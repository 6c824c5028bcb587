"""Synthetic verify-step inputs.

Recipe (per sequence b and position i in [0, K]):
  base[b, i, v]   = 3 * N(0, 1) - s * ln(rank[b, i, v]),  s = 1.1,
                    rank = 1 + a uniformly random permutation of the vocabulary
                    (a Zipf(s) log-pmf over randomly permuted token ids);
  draft[b, i]     = base[b, i]                     for i < K;
  target[b, i]    = base[b, i] + sigma_b * N(0, 1)  for i <= K;
  both cast to the workload dtype (bf16 by round-to-nearest-even).
Drafted tokens are sampled from the draft law at the sequence temperature,
softmax(draft / T), after multiplying the probabilities of the 4 largest draft
logits (ties to the lower id) by beta and renormalising when beta < 1; at
T == 0 the drafted token is the draft argmax (first index on ties).  The draft
sampler uses the Gumbel-max trick in float64.

These logits stand in for the verify-pass outputs of Llama-3-sized (V=128256)
and Qwen-sized (V=152064) vocabularies; no dataset item is used.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    dtype: str                 # "fp32" or "bf16"
    temperature: float | None  # None: per-sequence U[t_lo, t_hi]
    sigma: float               # target noise sd
    beta: float = 1.0          # 1.0 = off
    t_lo: float = 0.0
    t_hi: float = 0.0
    identical_every: int = 0   # sequences b % identical_every == 0 get sigma 0
    zipf_s: float = 1.1

    def sized(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def greedy(self) -> bool:
        return self.temperature == 0.0

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def algorithmic_bytes(self) -> int:
        """Bytes the method must read once: every target row and, when
        sampling, every draft row (greedy reads target rows only), plus the
        int32 drafted tokens, temperatures and outputs."""
        rows = self.B * (self.K + 1) + (0 if self.greedy else self.B * self.K)
        small = 4 * (self.B * self.K + self.B + self.B + self.B * (self.K + 1))
        return rows * self.V * self.elt_bytes + small

    def stream_bytes(self) -> int:
        """Bytes the streaming pass must read once: the logit rows alone."""
        rows = self.B * (self.K + 1) + (0 if self.greedy else self.B * self.K)
        return rows * self.V * self.elt_bytes

    def tag(self) -> str:
        t = "Tgreedy" if self.greedy else (f"T{self.temperature:g}" if self.temperature
                                           else f"TU[{self.t_lo:g},{self.t_hi:g}]")
        s = f"B{self.B}_K{self.K}_V{self.V}_{self.dtype}_{t}"
        if self.beta < 1.0:
            s += f"_beta{self.beta:g}"
        return s


WORKLOADS: dict[str, Workload] = {
    "C1": Workload("C1", B=1, K=4, V=32000, dtype="fp32", temperature=1.0, sigma=0.5),
    "C2": Workload("C2", B=8, K=5, V=128256, dtype="bf16", temperature=0.7, sigma=0.8),
    "C3": Workload("C3", B=64, K=4, V=128256, dtype="bf16", temperature=0.0, sigma=1.0),
    "C4": Workload("C4", B=256, K=7, V=152064, dtype="bf16", temperature=1.0, sigma=0.4,
                   identical_every=10),
    "C5": Workload("C5", B=512, K=5, V=128256, dtype="fp32", temperature=None, sigma=0.6,
                   beta=0.5, t_lo=0.5, t_hi=1.2),
}


def _torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


@torch.no_grad()
def make_inputs(w: Workload, seed: int = 0, device: str | torch.device = "cpu",
                rows_per_batch: int = 256) -> dict:
    """Fabricate one batch of inputs on `device`.

    Returns dict(target [B,K+1,V], draft [B,K,V] (workload dtype), tokens
    [B,K] int32, temperature [B] float32, beta float).  Deterministic for a
    given (workload, seed, device type).
    """
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + 17)
    B, K, V = w.B, w.K, w.V
    dt = _torch_dtype(w.dtype)
    target = torch.empty((B, K + 1, V), dtype=dt, device=device)
    draft = torch.empty((B, K, V), dtype=dt, device=device)

    sig = torch.full((B,), float(w.sigma), dtype=torch.float32, device=device)
    if w.identical_every:
        sig[::w.identical_every] = 0.0

    flat_t = target.view(B * (K + 1), V)
    nrows = B * (K + 1)
    for r0 in range(0, nrows, rows_per_batch):
        r1 = min(nrows, r0 + rows_per_batch)
        n = r1 - r0
        keys = torch.rand((n, V), generator=g, device=device)
        perm = torch.argsort(keys, dim=1)          # a random permutation per row
        base = 3.0 * torch.randn((n, V), generator=g, device=device)
        base -= w.zipf_s * torch.log1p(perm.to(torch.float32))
        noise = torch.randn((n, V), generator=g, device=device)
        rows = torch.arange(r0, r1, device=device)
        b_idx = rows // (K + 1)
        i_idx = rows % (K + 1)
        tgt = base + sig[b_idx].unsqueeze(1) * noise
        # identical rows must stay bitwise identical after the cast
        same = (sig[b_idx] == 0.0).unsqueeze(1)
        tgt = torch.where(same, base, tgt)
        flat_t[r0:r1] = tgt.to(dt)
        is_draft = i_idx < K
        if bool(is_draft.any()):
            dst = (b_idx * K + i_idx)[is_draft]
            draft.view(B * K, V)[dst] = base[is_draft].to(dt)
        del keys, perm, base, noise, tgt

    if w.temperature is None:
        temp = (w.t_lo + (w.t_hi - w.t_lo) * torch.rand((B,), generator=g, device=device,
                                                          dtype=torch.float64)).to(torch.float32)
    else:
        temp = torch.full((B,), float(w.temperature), dtype=torch.float32, device=device)

    tokens = sample_drafts(draft, temp, w.beta, g)
    return {"target": target, "draft": draft, "tokens": tokens, "temperature": temp,
            "beta": float(w.beta)}


@torch.no_grad()
def sample_drafts(draft: torch.Tensor, temp: torch.Tensor, beta: float,
                  g: torch.Generator, rows_per_batch: int = 256) -> torch.Tensor:
    """Draw one drafted token per draft row from the (beta-weighted) draft law
    at the sequence temperature; argmax where the temperature is 0."""
    B, K, V = draft.shape
    device = draft.device
    out = torch.empty((B * K,), dtype=torch.int32, device=device)
    flat = draft.view(B * K, V)
    tb = temp.to(torch.float64).repeat_interleave(K)
    for r0 in range(0, B * K, rows_per_batch):
        r1 = min(B * K, r0 + rows_per_batch)
        z = flat[r0:r1].to(torch.float64)
        t = tb[r0:r1]
        greedy = t == 0.0
        u = torch.rand(z.shape, generator=g, device=device, dtype=torch.float64)
        gumbel = -torch.log(-torch.log(u.clamp_min(1e-300)))
        safe_t = torch.where(greedy, torch.ones_like(t), t)
        score = z / safe_t.unsqueeze(1) + gumbel
        if beta < 1.0:
            order = torch.sort(z, dim=1, descending=True, stable=True).indices[:, :4]
            logw = torch.zeros_like(z)
            lb = float(np.log(beta)) if beta > 0.0 else float("-inf")
            logw.scatter_(1, order, lb)
            score = score + logw
        pick = torch.argmax(score, dim=1)
        pick = torch.where(greedy, torch.argmax(z, dim=1), pick)
        out[r0:r1] = pick.to(torch.int32)
    return out.view(B, K)


def ragged_lengths(w, seed: int, device) -> torch.Tensor:
    """Per-sequence draft counts K_b ~ U{0..K} (a drafter that stops early, as
    Kangaroo's confidence exit does), seeded; int32 [B] on `device`."""
    g = torch.Generator().manual_seed(1_000_003 * (seed + 1) + w.B)
    return torch.randint(0, w.K + 1, (w.B,), generator=g, dtype=torch.int32).to(device)


def ragged_rows(w, draft_len) -> int:
    """Logit rows a ragged call reads: K_b + 1 target rows, and K_b draft rows
    when sampling."""
    kb = int(draft_len.sum().item())
    return kb + w.B + (0 if w.greedy else kb)


def to_numpy_inputs(inp: dict, b0: int = 0, b1: int | None = None) -> dict:
    """Host copies for the oracle: float32 arrays, or uint16 arrays holding
    bf16 bit patterns (sequences b0..b1 only)."""
    def raw(x):
        x = x[b0:b1].contiguous().cpu()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16)
        return x.numpy()
    return {
        "target": raw(inp["target"]),
        "draft": raw(inp["draft"]) if inp.get("draft") is not None else None,
        "tokens": inp["tokens"][b0:b1].contiguous().cpu().numpy(),
        "temperature": inp["temperature"][b0:b1].contiguous().cpu().numpy(),
        "beta": inp["beta"],
        "draft_len": (inp["draft_len"][b0:b1].contiguous().cpu().numpy()
                      if inp.get("draft_len") is not None else None),
    }


def tree_parents(shape) -> np.ndarray:
    """Parents of a token tree given its branching per depth, nodes numbered
    breadth-first: shape (4, 2, 1) is a root with 4 children, each with 2
    children, each with 1 child (N = 4 + 8 + 8 = 20)."""
    parents = []
    level = [-1]
    for k in shape:
        nxt = []
        for p in level:
            for _ in range(k):
                parents.append(p)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.array(parents, dtype=np.int32)


@torch.no_grad()
def make_tree_inputs(w: Workload, shape, seed: int = 0, device: str | torch.device = "cpu",
                     rows_per_batch: int = 256) -> dict:
    """One batch of tree-verification inputs: every context c (the root and
    each node) has base logits with the workload's recipe; target row c =
    base + sigma_b N(0, 1), draft row c = base (contexts 0..N-1); the children
    of context c get tokens drawn i.i.d. from its draft law at the sequence
    temperature (argmax where it is 0).  Returns dict(target [B, N+1, V],
    draft [B, N, V], parent [B, N], tokens [B, N], temperature [B])."""
    device = torch.device(device)
    parent_np = tree_parents(shape)
    N = parent_np.size
    chain = w.sized(K=N)
    inp = make_inputs(chain, seed=seed, device=device, rows_per_batch=rows_per_batch)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 7919 + 3)
    B, V = w.B, w.V
    parent = torch.from_numpy(parent_np).to(device).unsqueeze(0).repeat(B, 1).contiguous()
    # node i's token comes from the draft row of its parent's context
    ctx = torch.from_numpy(parent_np.astype(np.int64) + 1).to(device)
    tokens = torch.empty((B, N), dtype=torch.int32, device=device)
    temp = inp["temperature"].to(torch.float64)
    for i in range(N):
        z = inp["draft"][:, int(ctx[i])].to(torch.float64)
        greedy = temp == 0.0
        u = torch.rand(z.shape, generator=g, device=device, dtype=torch.float64)
        gumbel = -torch.log(-torch.log(u.clamp_min(1e-300)))
        t = torch.where(greedy, torch.ones_like(temp), temp).unsqueeze(1)
        pick = torch.argmax(z / t + gumbel, dim=1)
        pick = torch.where(greedy, torch.argmax(z, dim=1), pick)
        tokens[:, i] = pick.to(torch.int32)
    return {"target": inp["target"], "draft": inp["draft"], "parent": parent, "tokens": tokens,
            "temperature": inp["temperature"]}
