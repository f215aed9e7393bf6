"""The tree-structured verify pass (block_diffusion_tree_amd.verifier) on a
small random target: its HIP-graph replays give the eager logits, and a
node's logits depend on its own path only (Bastion page, Experimental
results: the whole tree is verified in one pass, each node conditioned on
its ancestors through the ancestor mask)."""
import pytest
import torch

from block_diffusion_tree_amd import verifier
import gpu_common as gc

pytestmark = pytest.mark.gpu

SMALL = verifier.TargetShape(layers=2, hidden=512, q_heads=4, kv_heads=2, head_dim=128,
                             intermediate=1024, vocab=1000)


def test_graph_replays_match_eager_pass():
    gc.require_gpu()
    tgt = verifier.RandomTarget(SMALL, lmax=256, seed=1)
    parent = torch.tensor([-1, 0, 0, 1, 1, 2, 3], dtype=torch.int32, device="cuda")
    vp = verifier.VerifyPass(tgt, parent, ctx=50, seed=2)
    ref = vp.eager().clone()
    vp.capture()
    for _ in range(3):
        got = vp.replay()
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        vp.eager()
        torch.cuda.synchronize()
    assert torch.isfinite(ref.float()).all()


def test_a_node_sees_its_path_only():
    gc.require_gpu()
    tgt = verifier.RandomTarget(SMALL, lmax=256, seed=3)
    parent = torch.tensor([-1, 0, 0, 1, 1, 2, 3], dtype=torch.int32, device="cuda")
    vp = verifier.VerifyPass(tgt, parent, ctx=40, seed=4)
    a = vp.eager().clone()
    # other tokens for the nodes off the path 0 -> 1 -> 3 -> 6
    vp.tokens[[2, 4, 5]] = (vp.tokens[[2, 4, 5]] + 17) % SMALL.vocab
    b = vp.eager().clone()
    torch.cuda.synchronize()
    for i in (0, 1, 3, 6):
        assert torch.equal(a[i], b[i]), i
    for i in (2, 4, 5):
        assert not torch.equal(a[i], b[i]), i
