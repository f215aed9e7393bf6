"""Seeded synthetic inputs for the tree-drafting hot path.

This module only draws random numbers with stated recipes: drafter logits of a
given shape and entropy mix, prior logits for a latent mixture, the per-query
verify-latency table C(N) of a roofline model with fixed constants, and
"target model" argmax tokens for the nodes of a tree.  It computes no softmax,
no top-k, no path score, no tree, no mask and no acceptance: those belong to
the HIP library and to the CPU reference, which both consume what is drawn
here.  Both sides import this module and nothing else in common.

Stand-ins: the pages evaluate trained drafters (Qwen3 / Llama-3.1 targets) on
math, code and chat prompts.  None of that is available, so logits are drawn
with the vocabulary sizes of those targets and with one dominant token per row
whose margin varies, so row entropy spans nearly-deterministic to flat.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"
DTYPE_CODE = {F32: 0, BF16: 1}
TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, logits recipe and tree parameters."""

    name: str
    B: int          # queries
    b: int          # drafted block length (positions per query)
    V: int          # vocabulary size
    dtype: str      # storage type of the logits
    k: int          # candidates kept per position
    nmax: int       # node budget (non-root nodes)
    nmin: int       # smallest budget the online controller may stop at
    online: bool    # stop at the peak of S(N) instead of a fixed budget
    seed: int
    recipe: str     # "gauss_bump" or "rowmax_peak"
    peak_lo: float = 0.0
    peak_hi: float = 0.0
    K: int = 1      # latent branches (mixture workloads only)

    @property
    def rows(self) -> int:
        return self.B * self.K * self.b

    @property
    def logit_bytes(self) -> int:
        return self.rows * self.V * (4 if self.dtype == F32 else 2)


WORKLOADS = {
    # 1 query, 4 positions, V=1024 fp32; N(0, variance 2) plus +6 on one token.
    "tiny": Workload("tiny", 1, 4, 1024, F32, 4, 32, 1, False, 1001, "gauss_bump"),
    # 64 queries x 16 positions over a Qwen3-sized vocabulary, bf16.
    "main": Workload("main", 64, 16, 151936, BF16, 8, 64, 1, False, 1002,
                     "rowmax_peak", 2.0, 10.0),
    # budget-controller sweep over a Llama-3.1-sized vocabulary, fp32.
    "sweep": Workload("sweep", 256, 16, 128256, F32, 4, 256, 1, True, 1003, "gauss_bump"),
    # the sweep's shape and budget with the main workload's peaked rows, where
    # N* lands deep in the budget (a labelled extra sweep).
    "sweep_peaks": Workload("sweep_peaks", 256, 16, 128256, F32, 4, 256, 1, True, 1013,
                            "rowmax_peak", 2.0, 10.0),
    # single query latency case with confident rows.
    "latency": Workload("latency", 1, 16, 151936, BF16, 16, 128, 1, True, 1004,
                        "rowmax_peak", 6.0, 12.0),
    # latent mixture: 8 branches per query.
    "mixture": Workload("mixture", 128, 16, 151936, BF16, 8, 64, 1, False, 1005,
                        "rowmax_peak", 2.0, 10.0, K=8),
}


@dataclasses.dataclass(frozen=True)
class VerifyWorkload:
    """One attention layer of the verify pass over a batch of drafted trees:
    S sequences, T = N + 1 tree tokens each, behind contexts drawn uniformly
    from [ctx_lo, ctx_hi] (the contexts of the latency table below), with the
    target's head shape (Qwen3-8B: 32 query heads, 8 KV heads of 128)."""

    name: str
    S: int
    T: int
    Hq: int
    Hkv: int
    ctx_lo: int
    ctx_hi: int
    seed: int
    D: int = 128

    @property
    def lmax(self) -> int:
        return (self.ctx_hi + self.T + 31) // 32 * 32


VERIFY_WORKLOADS = {
    # the trees of the main workload (64 queries, N = 64) verified in one pass
    "verify": VerifyWorkload("verify", 64, 65, 32, 8, 512, 8192, 1006),
}


def make_verify_contexts(vw: VerifyWorkload) -> np.ndarray:
    """Cached tokens per sequence, uniform on [ctx_lo, ctx_hi] (int32 [S])."""
    rng = np.random.default_rng(vw.seed)
    return rng.integers(vw.ctx_lo, vw.ctx_hi + 1, size=vw.S).astype(np.int32)


def make_verify_tensors(vw: VerifyWorkload, device="cpu", seed: int | None = None):
    """Random bf16 layer inputs: qkv rows [S*T, (Hq+2Hkv)*D] and the KV cache,
    k [S, Hkv, Lmax, D] and v in 32-slot tiles [S, Hkv, Lmax/32, D, 32], every
    element N(0, 1) rounded to bf16."""
    g = _gen(vw.seed if seed is None else seed, device)
    C = (vw.Hq + 2 * vw.Hkv) * vw.D
    L = vw.lmax

    def normal(*shape):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        return t.normal_(0.0, 1.0, generator=g)

    return (normal(vw.S * vw.T, C), normal(vw.S, vw.Hkv, L, vw.D),
            normal(vw.S, vw.Hkv, L // 32, vw.D, 32))


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(wl, **changes)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _fill_rows(out: torch.Tensor, wl: Workload, g: torch.Generator) -> None:
    """Fill out[..., V] (any leading shape) in place with one recipe."""
    dev = out.device
    lead = out.shape[:-1]
    nrows = int(np.prod(lead)) if len(lead) else 1
    V = out.shape[-1]
    flat = out.reshape(nrows, V)
    if wl.recipe == "gauss_bump":
        # N(0, 2): variance 2, i.e. standard deviation sqrt(2); then +6 on one
        # uniformly chosen token per row.
        base = torch.randn((nrows, V), generator=g, device=dev, dtype=torch.float32)
        base.mul_(math.sqrt(2.0))
        tok = torch.randint(0, V, (nrows,), generator=g, device=dev)
        rows = torch.arange(nrows, device=dev)
        base[rows, tok] += 6.0
    elif wl.recipe == "rowmax_peak":
        # 3 * N(0,1) background; one uniformly chosen token per row is lifted
        # to (row maximum + U(lo, hi)), so the margin of the dominant token,
        # and with it the row entropy, varies from row to row.
        base = torch.randn((nrows, V), generator=g, device=dev, dtype=torch.float32)
        base.mul_(3.0)
        tok = torch.randint(0, V, (nrows,), generator=g, device=dev)
        lift = torch.rand((nrows,), generator=g, device=dev, dtype=torch.float32)
        lift = wl.peak_lo + (wl.peak_hi - wl.peak_lo) * lift
        rows = torch.arange(nrows, device=dev)
        base[rows, tok] = base.max(dim=1).values + lift
    else:
        raise ValueError(f"unknown recipe {wl.recipe!r}")
    flat.copy_(base.to(out.dtype))   # bf16 by round-to-nearest-even


def make_logits(wl: Workload, device="cpu", seed: int | None = None,
                chunk_rows: int = 4096) -> torch.Tensor:
    """Drafter logits: [B, b, V] (or [B, K, b, V] when K > 1), in wl.dtype.

    Rows are generated in chunks so that large workloads never hold a full
    fp32 copy.  The same (workload, seed, device type) always gives the same
    tensor.
    """
    g = _gen(wl.seed if seed is None else seed, device)
    shape = (wl.B, wl.b, wl.V) if wl.K == 1 else (wl.B, wl.K, wl.b, wl.V)
    out = torch.empty(shape, dtype=TORCH_DTYPE[wl.dtype], device=device)
    flat = out.view(-1, wl.V)
    for r0 in range(0, flat.shape[0], chunk_rows):
        _fill_rows(flat[r0:r0 + chunk_rows], wl, g)
    return out


def make_prior_logits(wl: Workload, device="cpu", seed: int | None = None) -> torch.Tensor:
    """Latent-branch prior logits [B, K], fp32, N(0, 1)."""
    g = _gen((wl.seed if seed is None else seed) + 7919, device)
    return torch.randn((wl.B, wl.K), generator=g, device=device, dtype=torch.float32)


# ---------------------------------------------------------------------------
# Verify-latency table C(N) = T_draft + max(bytes(N)/BW, flops(N)/peak) + c0.
# Constants describe an 8B-parameter, Qwen3-8B-shaped target (36 layers,
# 8 KV heads of 128, 32 query heads), fp16 weights and KV cache.  N counts
# non-root nodes, so the verifier processes N+1 tokens.
# ---------------------------------------------------------------------------
LATENCY_A100 = dict(bw=2.039e12, peak=312e12)
LATENCY_MI355X = dict(bw=8.0e12, peak=2.5e15)


def make_cost_table(B: int, nmax: int, seed: int, bw: float, peak: float,
                    n_params: float = 8.0e9, layers: int = 36, kv_heads: int = 8,
                    q_heads: int = 32, head_dim: int = 128, c0: float = 30e-6,
                    ctx_lo: int = 512, ctx_hi: int = 8192) -> tuple[np.ndarray, np.ndarray]:
    """Per-query latency table [B, nmax+1] in seconds (float64) and contexts.

    Each query draws its own context length uniformly from [ctx_lo, ctx_hi].
    """
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=B).astype(np.float64)
    w_bytes = 2.0 * n_params
    kv_per_token = 2.0 * layers * kv_heads * head_dim * 2.0
    t_draft = 0.1 * w_bytes / bw
    n = np.arange(nmax + 1, dtype=np.float64)[None, :]
    tokens = n + 1.0
    keys = ctx[:, None] + n + 1.0
    nbytes = w_bytes + kv_per_token * keys
    flops = 2.0 * n_params * tokens + 4.0 * layers * q_heads * head_dim * tokens * keys
    cost = t_draft + np.maximum(nbytes / bw, flops / peak) + c0
    return np.ascontiguousarray(cost, dtype=np.float64), ctx


# ---------------------------------------------------------------------------
# Synthetic target-model argmax per tree node.  A node's target token is a
# pure function of (seed, query, the node's token path), so two trees that
# share a prefix see the same targets on it.  With probability p_match the
# target agrees with the drafter's most likely token at the next position
# (passed in as top1[B, b]); otherwise it is uniform over the vocabulary.
# Nodes at the last position always draw uniformly.  splitmix64 (Steele,
# Lea & Flood, "Fast splittable pseudorandom number generators", 2014) is the
# hash.
# ---------------------------------------------------------------------------
_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def make_targets(parent: np.ndarray, token: np.ndarray, depth: np.ndarray,
                 n_nodes: np.ndarray, top1: np.ndarray, V: int, seed: int,
                 p_match: float = 0.7) -> np.ndarray:
    """target[B, nmax+1] int32 for the nodes 0..n_nodes[q] of each tree."""
    parent = np.asarray(parent)
    B, width = parent.shape
    b = top1.shape[1]
    out = np.zeros((B, width), dtype=np.int32)
    for q in range(B):
        h = [0] * width
        h[0] = splitmix64(splitmix64(seed & _M64) ^ q)
        for i in range(int(n_nodes[q]) + 1):
            if i > 0:
                h[i] = splitmix64(h[int(parent[q, i])] ^ (int(token[q, i]) + 1))
            d = int(depth[q, i])
            u = (h[i] >> 11) * (1.0 / (1 << 53))
            if d < b and u < p_match:
                out[q, i] = int(top1[q, d])
            else:
                out[q, i] = splitmix64(h[i] ^ 0xD1B54A32D192ED03) % V
    return out
