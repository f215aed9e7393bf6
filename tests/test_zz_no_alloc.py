"""bastion_build_trees_noalloc (the entry point that allocates nothing and
keeps its scratch in a per-GPU device array) against bastion_build_trees on
the same inputs: two calls in a row, the second with a smaller input, each
bit-identical to the workspace call."""
import ctypes as C

import pytest
import torch

from block_diffusion_tree_amd import binding, synth
import gpu_common as gc

pytestmark = pytest.mark.gpu


def _same(a, b):
    for f in a:
        assert torch.equal(a[f], b[f]), f


def test_noalloc_matches_workspace_call_twice():
    gc.require_gpu()
    big = synth.WORKLOADS["main"]
    small = synth.scaled(synth.WORKLOADS["sweep"], B=8, V=30011)
    xb = gc.device_logits(big)
    xs = gc.device_logits(small)
    cost, _ = synth.make_cost_table(small.B, small.nmax, seed=3, **synth.LATENCY_A100)
    cost = torch.from_numpy(cost).to("cuda")
    print(f"noalloc: main workload {tuple(xb.shape)}", flush=True)
    a1 = binding.build_trees_noalloc(xb, k=big.k, nmax=big.nmax)
    r1 = binding.build_trees(xb, k=big.k, nmax=big.nmax)
    torch.cuda.synchronize()
    _same(a1, r1)
    print(f"noalloc: smaller online input {tuple(xs.shape)}", flush=True)
    a2 = binding.build_trees_noalloc(xs, k=small.k, nmax=small.nmax, cost=cost)
    r2 = binding.build_trees(xs, k=small.k, nmax=small.nmax, cost=cost)
    torch.cuda.synchronize()
    _same(a2, r2)
    # and against the reference, once
    ref = gc.oracle.softmax_topk(gc.oracle.host_logits(xs), k=small.k)
    gc.check_rows(a2, ref)
    gc.check_tree(a2, small.b, small.k, small.nmax, 1, gc.np_(cost), 1.0,
                  gc.expected_row_status(ref))
    gc.check_mask(a2)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A plan whose scratch exceeds the array (forced 64 segments over 16384
    rows) is refused before anything is launched."""
    gc.require_gpu()
    L = binding.lib()
    L.bastion_noalloc_scratch_bytes.restype = C.c_size_t
    assert L.bastion_noalloc_scratch_bytes() == 4 << 20
    x = torch.zeros((1024, 16, 8192), dtype=torch.bfloat16, device="cuda")
    binding.set_tuning(segments=64)
    try:
        with pytest.raises(binding.BastionError) as e:
            binding.build_trees_noalloc(x, k=8, nmax=16)
        assert e.value.status == binding.EUNSUPPORTED
    finally:
        binding.set_tuning(0, -1)
