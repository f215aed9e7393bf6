"""A tree-structured verifier forward pass with random weights, for measuring
T_verify(N) on this GPU.

Bastion page (gist.science), Methodology 3: the budget controller weighs
A_hat(T_N) against the verify latency of a tree of N non-root nodes, from a
roofline model calibrated on observed runtimes; Experimental results: the
target checks the whole tree in one forward pass.  Timing needs no trained
weights, so this module builds a target of the pages' main model's shape
(Qwen3-8B: 36 layers, hidden 4096, 32 query heads and 8 KV heads of 128,
MLP 12288, vocabulary 151936, rotary base 1e6) with random bf16 weights and
runs one verification pass of N+1 tree tokens over a KV cache of ctx tokens:

  per layer: RMSNorm -> q/k/v projection -> per-head RMSNorm of q and k ->
  bastion_tree_attention (rotary embedding at the tree's position ids, cache
  append, ancestor-masked attention) -> output projection + residual ->
  RMSNorm -> gate/up projection -> SiLU(gate) * up -> down projection +
  residual; then the final RMSNorm and the vocabulary projection.

The projections are plain GEMMs (hipBLASLt through torch's linear, weights
stored [out, in]); the
tree-specific step is the library's attention layer.  The pass is captured
in a HIP graph once per (N, ctx) so that host launch overhead stays out of
the measured time.
"""
from __future__ import annotations

import dataclasses

import torch

from block_diffusion_tree_amd import binding


@dataclasses.dataclass(frozen=True)
class TargetShape:
    layers: int = 36
    hidden: int = 4096
    q_heads: int = 32
    kv_heads: int = 8
    head_dim: int = 128
    intermediate: int = 12288
    vocab: int = 151936
    rope_theta: float = 1.0e6
    eps: float = 1e-6

    @property
    def qkv_cols(self) -> int:
        return (self.q_heads + 2 * self.kv_heads) * self.head_dim

    def matmul_params(self) -> int:
        """Parameters every token multiplies through (all projections)."""
        h, i = self.hidden, self.intermediate
        per_layer = h * self.qkv_cols + self.q_heads * self.head_dim * h + h * 2 * i + i * h
        return self.layers * per_layer + h * self.vocab

    def weight_bytes(self) -> int:
        return 2 * self.matmul_params()

    def kv_bytes_per_token(self) -> int:
        return 2 * self.layers * self.kv_heads * self.head_dim * 2

    def flops(self, n: int, ctx: int) -> float:
        """Dense flops of verifying n non-root nodes (n + 1 tokens) behind ctx
        cached tokens: every projection, plus q.k and p.v over ctx + n + 1 keys."""
        t = n + 1
        attn = 4.0 * self.layers * self.q_heads * self.head_dim * t * (ctx + t)
        return 2.0 * self.matmul_params() * t + attn

    def bytes(self, n: int, ctx: int) -> float:
        """Bytes a verification pass must move at least: the weights once and
        the KV cache of ctx + n + 1 tokens once."""
        return float(self.weight_bytes() + self.kv_bytes_per_token() * (ctx + n + 1))


QWEN3_8B = TargetShape()


class RandomTarget:
    """Random bf16 weights of a TargetShape and a KV cache of up to lmax
    tokens per layer, on one GPU (about 17.7 GB for the Qwen3-8B shape)."""

    def __init__(self, shape: TargetShape = QWEN3_8B, lmax: int = 9216, device="cuda", seed=0):
        s = shape
        self.shape = s
        self.device = torch.device(device)
        self.lmax = (lmax + 31) // 32 * 32
        g = torch.Generator(device=self.device)
        g.manual_seed(seed)

        def w(*dims, scale=0.02):
            t = torch.empty(dims, dtype=torch.bfloat16, device=self.device)
            t.normal_(0.0, scale, generator=g)
            return t

        self.embed = w(s.vocab, s.hidden, scale=1.0)
        self.layers = []
        for _ in range(s.layers):
            self.layers.append(dict(
                w_qkv=w(s.qkv_cols, s.hidden), w_o=w(s.hidden, s.q_heads * s.head_dim),
                w_gu=w(2 * s.intermediate, s.hidden), w_d=w(s.hidden, s.intermediate),
                n_in=torch.ones(s.hidden, dtype=torch.bfloat16, device=self.device),
                n_post=torch.ones(s.hidden, dtype=torch.bfloat16, device=self.device),
                n_q=torch.ones(s.head_dim, dtype=torch.bfloat16, device=self.device),
                n_k=torch.ones(s.head_dim, dtype=torch.bfloat16, device=self.device),
                kc=w(1, s.kv_heads, self.lmax, s.head_dim, scale=1.0),
                vc=w(1, s.kv_heads, self.lmax // 32, s.head_dim, 32, scale=1.0)))
        self.n_final = torch.ones(s.hidden, dtype=torch.bfloat16, device=self.device)
        self.lm_head = w(s.vocab, s.hidden)
        self.inv_freq = binding.rope_inv_freq(s.rope_theta, s.head_dim, self.device)

    def forward(self, tokens, ctx_len, position_ids, mask, attn_ws, max_ctx=-1):
        """One verification pass: tokens [T] int64, ctx_len [1] int32,
        position_ids [1, T] int32, mask [1, T, W] int32 ancestor rows.
        Returns the logits [T, vocab] (bf16)."""
        s = self.shape
        T = tokens.shape[0]
        F = torch.nn.functional
        x = self.embed[tokens]
        nh = s.q_heads + s.kv_heads
        for L in self.layers:
            h = F.rms_norm(x, (s.hidden,), L["n_in"], s.eps)
            qkv = F.linear(h, L["w_qkv"])
            heads = qkv.view(T, -1, s.head_dim)
            heads[:, :s.q_heads] = F.rms_norm(heads[:, :s.q_heads], (s.head_dim,), L["n_q"], s.eps)
            heads[:, s.q_heads:nh] = F.rms_norm(heads[:, s.q_heads:nh], (s.head_dim,), L["n_k"],
                                                s.eps)
            a = binding.tree_attention(qkv, 1, T, s.q_heads, s.kv_heads, L["kc"], L["vc"], ctx_len,
                                       position_ids, mask, self.inv_freq, ws=attn_ws,
                                       max_ctx=max_ctx)
            x = x + F.linear(a, L["w_o"])
            h = F.rms_norm(x, (s.hidden,), L["n_post"], s.eps)
            gu = F.linear(h, L["w_gu"])
            x = x + F.linear(F.silu(gu[:, :s.intermediate]) * gu[:, s.intermediate:], L["w_d"])
        return F.linear(F.rms_norm(x, (s.hidden,), self.n_final, s.eps), self.lm_head)


class VerifyPass:
    """The verification pass of one (tree, context) captured in a HIP graph:
    fixed input buffers, replay() reruns it."""

    def __init__(self, target: RandomTarget, parent, ctx: int, seed: int = 0):
        """parent [N+1] int32 (GPU): a prefix-closed tree in pop order (parent
        of node 0 is -1); ctx: cached tokens in front of the root."""
        dev = target.device
        self.target = target
        self.T = int(parent.shape[0])
        n = self.T - 1
        par = parent.view(1, -1).to(torch.int32).contiguous()
        nn = torch.tensor([n], dtype=torch.int32, device=dev)
        self.ctx = int(ctx)
        self.ctx_len = torch.tensor([ctx], dtype=torch.int32, device=dev)
        # the verifier's inputs from the tree: ancestor rows and positions
        if n >= 1:
            self.mask, self.pos = binding.tree_mask(par, nn, self.ctx_len)
        else:   # the root alone (bastion_tree_mask takes budgets of at least 1)
            self.mask = torch.ones((1, 1, 1), dtype=torch.int32, device=dev)
            self.pos = self.ctx_len.view(1, 1).clone()
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        self.tokens = torch.randint(0, target.shape.vocab, (self.T,), generator=g, device=dev)
        need = binding._vlib().bastion_tree_attention_workspace_bytes(
            1, self.T, target.shape.q_heads, target.shape.kv_heads, target.lmax)
        self.attn_ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self.graph = None
        self.logits = None

    def eager(self):
        return self.target.forward(self.tokens, self.ctx_len, self.pos, self.mask, self.attn_ws,
                                   self.ctx)

    def capture(self):
        s = torch.cuda.Stream(self.target.device)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.eager()          # warm: library and BLAS handles, allocator pool
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.logits = self.eager()
        torch.cuda.synchronize()
        return self

    def replay(self):
        self.graph.replay()
        return self.logits
