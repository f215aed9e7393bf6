"""GPU parity of bastion_tree_attention (the tree's consumer) against the
float64 reference of oracle/verify_oracle.py.

Tolerance, from the kernel's arithmetic: scores and softmax are float32 and
the probabilities enter the value product rounded to bf16 (relative error at
most 2^-9 each), so an output element can move by up to 2^-9 of the largest
|v| it averages; the output itself is rounded to bf16 (2^-9 relative); the
rotated q and k are rounded to bf16 from float32 here and from float64 in
the reference, which rarely picks the neighbouring bf16 value.  Bound used:
|gpu - ref| <= 2^-8 max|v| + 2^-8 |ref|.  Cached v slots are copied
exactly; rotated k slots may differ by one bf16 step in rare elements."""
import numpy as np
import pytest
import torch

from block_diffusion_tree_amd import binding, synth
from oracle import verify_oracle as vo
import gpu_common as gc
from test_oracle_verify import make_case

pytestmark = pytest.mark.gpu


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to("cuda")


def run_case(S, T, Hq, Hkv, Lmax, ctx, parents, seed, poison=True, mask_pos=None, max_ctx=-1):
    gc.require_gpu()
    rng = np.random.default_rng(seed)
    qkv, kc, vc, ctxa, pos, mask, inv = make_case(rng, S, T, Hq, Hkv, Lmax, ctx, parents)
    if mask_pos is not None:
        mask, pos = mask_pos
    # the reference sees the contexts the launch bound leaves
    ctx_ref = ctxa if max_ctx < 0 else np.minimum(ctxa, max_ctx).astype(np.int32)
    ref, kc_ref, vc_ref = vo.tree_attention(qkv, S, T, Hq, Hkv, 128, kc, vc, ctx_ref, pos, mask,
                                            inv)
    kcd = to_dev(kc, torch.bfloat16)
    vcd = to_dev(vc, torch.bfloat16)
    if poison:
        # slots past each sequence's keys hold NaN: nothing may read them
        for s in range(S):
            end = min(max(int(ctx_ref[s]), 0), Lmax - T) + T
            kcd[s, :, end:, :] = float("nan")
            vcd[s, :, :, end:] = float("nan")
    # the library's v cache is tiled: [S, Hkv, Lmax/32, D, 32]
    vcd = vcd.view(S, Hkv, 128, Lmax // 32, 32).permute(0, 1, 3, 2, 4).contiguous()
    out = binding.tree_attention(to_dev(qkv, torch.bfloat16), S, T, Hq, Hkv, kcd, vcd,
                                 to_dev(ctxa, torch.int32), to_dev(pos, torch.int32),
                                 to_dev(mask.view(np.int32), torch.int32),
                                 to_dev(inv, torch.float32), max_ctx=max_ctx)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    vmax = np.abs(qkv[:, (Hq + Hkv) * 128:(Hq + 2 * Hkv) * 128]).max()
    vmax = max(vmax, np.abs(vc[..., :max(ctx) if max(ctx) > 0 else 1]).max())
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * vmax + 2.0 ** -8 * np.abs(ref)
    assert np.isfinite(got).all()
    assert (err <= bound).all(), f"max err {err.max()} (bound at worst {bound[err > bound].min()})"
    # caches: v copied exactly, rotated k within one bf16 step
    kg = kcd.double().cpu().numpy()
    vg = vcd.permute(0, 1, 3, 2, 4).reshape(S, Hkv, 128, Lmax).double().cpu().numpy()
    for s in range(S):
        c = min(max(int(ctx_ref[s]), 0), Lmax - T)
        assert np.array_equal(vg[s, :, :, :c + T], vc_ref[s, :, :, :c + T])
        dk = np.abs(kg[s, :, c:c + T, :] - kc_ref[s, :, c:c + T, :])
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(kc_ref[s, :, c:c + T, :]), 1e-30))) - 7)
        assert (dk <= ulp).all()
        assert (dk > 0).mean() < 1e-3
    return got, ref


def random_parents(rng, S, T):
    return [[-1] + [int(rng.integers(0, i)) for i in range(1, T)] for _ in range(S)]


@pytest.mark.parametrize("S,T,Hq,Hkv,Lmax,ctx", [
    (2, 9, 8, 2, 64, [5, 0]),            # one key split: output written directly
    (1, 65, 32, 8, 1024, [700]),         # Qwen3-8B heads, N = 64, splits combined
    (3, 33, 16, 16, 512, [0, 300, 40]),  # no grouping
    (1, 129, 16, 1, 256, [100]),         # one KV head for 16 query heads
    (2, 17, 4, 2, 96, [90, 200]),        # contexts past the cache are clamped
    (2, 21, 6, 2, 512, [100, 7]),        # 3 query heads per KV head: tiles straddle tokens
    (3, 1, 32, 8, 4096, [4000, 0, 37]),  # the root alone (N = 0)
])
def test_tree_attention_matches_reference(S, T, Hq, Hkv, Lmax, ctx):
    rng = np.random.default_rng(T)
    run_case(S, T, Hq, Hkv, Lmax, ctx, random_parents(rng, S, T), seed=T + S)


def test_tree_attention_launch_bound():
    """A host bound of the contexts sizes the launch; contexts above it are
    clamped to it (here 300 of 700 cached tokens are used)."""
    rng = np.random.default_rng(8)
    run_case(2, 33, 8, 2, 1024, [700, 120], random_parents(rng, 2, 33), seed=8, max_ctx=300)
    run_case(2, 33, 8, 2, 1024, [700, 120], random_parents(rng, 2, 33), seed=9, max_ctx=700)


def test_tree_attention_large_tree():
    """N = 256 (1028 query rows per KV head, 17 row tiles) behind 2000 tokens."""
    rng = np.random.default_rng(5)
    run_case(1, 257, 32, 8, 2304, [2000], random_parents(rng, 1, 257), seed=5)


def test_tree_attention_consumes_build_trees_outputs():
    """The mask and position ids come straight from bastion_build_trees
    (pos_base = the context length): the layer's input is the library's
    own verifier input."""
    gc.require_gpu()
    wl = synth.scaled(synth.WORKLOADS["main"], B=2, V=20000, nmax=40)
    x = gc.device_logits(wl)
    ctx = torch.tensor([333, 17], dtype=torch.int32, device="cuda")
    g = binding.build_trees(x, k=wl.k, nmax=wl.nmax, pos_base=ctx)
    torch.cuda.synchronize()
    parent = gc.np_(g["parent"])
    T = wl.nmax + 1
    assert (gc.np_(g["n_nodes"]) == wl.nmax).all()
    mask = gc.np_(g["mask"]).view(np.uint32)
    pos = gc.np_(g["position_ids"])
    parents = [[int(p) for p in parent[s]] for s in range(2)]
    run_case(2, T, 8, 2, 512, [333, 17], parents, seed=11, mask_pos=(mask, pos))


def test_tree_attention_verify_workload_sampled():
    """The benchmark's layer: the main workload's 64 trees (built by
    bastion_build_trees from its logits, pos_base = the contexts) behind
    contexts U[512, 8192] in an 8288-slot cache, launched as the benchmark
    launches it (max_ctx 8192: two chunks of keys for the longer contexts);
    the float64 reference on three sequences (the shortest context, one in
    two chunks, the longest)."""
    gc.require_gpu()
    vw = synth.VERIFY_WORKLOADS["verify"]
    wl = synth.WORKLOADS["main"]
    ctx_np = synth.make_verify_contexts(vw)
    ctx = torch.from_numpy(ctx_np).to("cuda")
    x = synth.make_logits(wl, device="cuda")
    trees = binding.build_trees(x, k=wl.k, nmax=wl.nmax, pos_base=ctx)
    del x
    qkv, kc, vc = synth.make_verify_tensors(vw, device="cuda")
    inv = binding.rope_inv_freq(1.0e6, vw.D, "cuda")
    out = binding.tree_attention(qkv, vw.S, vw.T, vw.Hq, vw.Hkv, kc, vc, ctx,
                                 trees["position_ids"], trees["mask"], inv, max_ctx=vw.ctx_hi)
    torch.cuda.synchronize()
    mask = gc.np_(trees["mask"]).view(np.uint32)
    pos = gc.np_(trees["position_ids"])
    order = np.argsort(ctx_np)
    pick = [int(order[0]), int(order[np.searchsorted(ctx_np[order], 4500)]), int(order[-1])]
    T, D = vw.T, vw.D
    for s in pick:
        rows = qkv[s * T:(s + 1) * T].double().cpu().numpy()
        kcs = kc[s:s + 1].double().cpu().numpy()
        vcs = vc[s:s + 1].permute(0, 1, 3, 2, 4).reshape(1, vw.Hkv, D, vw.lmax).double().cpu().numpy()
        ref, _, _ = vo.tree_attention(rows, 1, T, vw.Hq, vw.Hkv, D, kcs, vcs, ctx_np[s:s + 1],
                                      pos[s:s + 1], mask[s:s + 1], inv.cpu().numpy())
        got = out[s * T:(s + 1) * T].double().cpu().numpy()
        vmax = max(np.abs(rows[:, (vw.Hq + vw.Hkv) * D:]).max(), np.abs(vcs).max())
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * vmax + 2.0 ** -8 * np.abs(ref)
        assert (err <= bound).all(), f"sequence {s} (ctx {ctx_np[s]}): max err {err.max()}"
