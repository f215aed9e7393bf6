"""GPU parity of the sampled variants: per-node draws from the target at a
temperature (bastion_sample_nodes) against the reference's draws from the
same counter-based uniforms, the target-sampling walk (bastion_accept fed
the draws), and the DBlast branch draw (bastion_mixture_sample).

The kernel scores l/T + g in float32, the reference in float64; where two
tokens' scores agree to float32 rounding either is a correct draw, so a
different draw must score within 1e-5 of the reference's best."""
import math

import numpy as np
import pytest
import torch

from block_diffusion_tree_amd import binding, synth
from oracle import oracle
import gpu_common as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gc.require_gpu()


def check_draws(logits, n_nodes, T, seed):
    g = gc.np_(binding.sample_nodes(logits, n_nodes, T, seed))
    host = oracle.host_logits(logits)
    ref, score = oracle.sample_nodes(host, gc.np_(n_nodes), T, seed)
    lf = host.astype(np.float32) if host.dtype == np.float32 else \
        (host.astype(np.uint32) << 16).view(np.float32)
    nn = gc.np_(n_nodes)
    diff = 0
    for q in range(g.shape[0]):
        assert (g[q, nn[q] + 1:] == -1).all()
        for i in range(nn[q] + 1):
            if g[q, i] == ref[q, i]:
                continue
            diff += 1
            x = int(g[q, i])
            l = float(lf[q, i, x])
            s = l if T == 0 else l / T - math.log(-math.log(oracle.uniform_at(seed, q, i, x)))
            assert s >= score[q, i] - 1e-5 * (1 + abs(score[q, i])), (q, i, x, s, score[q, i])
    return g, diff


@pytest.mark.parametrize("T", [0.0, 0.7, 1.0, 1.5])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_node_draws_match_reference(T, dtype):
    wl = synth.scaled(synth.WORKLOADS["main"], B=4, b=41, V=30011, dtype=dtype)
    x = synth.make_logits(wl, seed=40).to("cuda")            # [4, 41, V]: 41 node rows
    n_nodes = torch.tensor([40, 13, 0, 27], dtype=torch.int32, device="cuda")
    g, diff = check_draws(x, n_nodes, T, seed=2024)
    assert diff <= 1


def test_target_sampling_walk_on_built_trees():
    """Trees from bastion_build_trees, target logits per node, draws at
    T = 0.8, and the walk: bastion_accept fed the draws equals the reference
    walk fed the same draws."""
    wl = synth.scaled(synth.WORKLOADS["main"], B=8, V=20000, nmax=64)
    x = gc.device_logits(wl)
    t = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    tw = synth.scaled(synth.WORKLOADS["main"], B=8, b=wl.nmax + 1, V=20000)
    target_logits = synth.make_logits(tw, seed=41).to("cuda")   # [8, 65, V]
    draws, _ = check_draws(target_logits, t["n_nodes"], 0.8, seed=5)
    d = torch.from_numpy(draws).to("cuda")
    alen, anodes, bonus = binding.accept(t["parent"], t["token"], t["n_nodes"], wl.b, d)
    torch.cuda.synchronize()
    ra, rn, rb = oracle.accept(gc.np_(t["parent"]), gc.np_(t["token"]), gc.np_(t["n_nodes"]),
                               wl.b, draws)
    assert (gc.np_(alen) == ra).all() and (gc.np_(anodes) == rn).all()
    assert (gc.np_(bonus) == rb).all()


@pytest.mark.parametrize("T", [0.0, 0.5, 1.0, 3.0])
def test_branch_draw_matches_reference(T):
    B, K, b = 300, 8, 16
    g = torch.Generator().manual_seed(7)
    prior = torch.randn(B, K, generator=g)
    prior[:5, 2] = prior[:5, 6] = 4.0                            # ties for T = 0
    u = torch.rand(B, generator=g, dtype=torch.float64)
    chains = torch.randint(0, 151936, (B, K, b), generator=g, dtype=torch.int32)
    z, draft = binding.mixture_sample(prior.cuda(), T, u.cuda(), chains.cuda())
    torch.cuda.synchronize()
    rz, rd = oracle.mixture_sample(prior.numpy(), T, u.numpy(), chains.numpy())
    assert (gc.np_(z) == rz).all() and (gc.np_(draft) == rd).all()
