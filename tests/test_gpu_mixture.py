"""GPU parity of bastion_mixture_score (DBlast latent mixture) against the CPU
reference: prior weights and q_dep within 1e-5 relative, chains and candidate
unions exact, candidate q within 1e-5, and the mixture tree exact against the
reference tree fed the GPU's own weights and candidate q."""
import numpy as np
import pytest
import torch

from block_diffusion_tree_amd import binding, synth
from oracle import oracle
import gpu_common as gc

pytestmark = pytest.mark.gpu

RTOL = 1e-5


@pytest.fixture(autouse=True)
def _gpu():
    gc.require_gpu()


def check_mixture(x, prior, k, nmax, with_tree=True, queries=None):
    """Full parity of one call (or of the listed queries of it)."""
    mo, tr = binding.mixture_score(x, prior, k=k, nmax=nmax, with_tree=with_tree)
    torch.cuda.synchronize()
    sel = slice(None) if queries is None else queries
    xs, ps = x[sel], prior[sel]
    ref = oracle.mixture(oracle.host_logits(xs), gc.np_(ps), k=k)
    g = {n: gc.np_(t)[sel] for n, t in mo.items()}
    assert np.allclose(g["prior_q"], ref["prior_w"], rtol=RTOL, atol=0), "prior weights differ"
    st = ref["row_status"]
    good_q = (st == oracle.OK).all(axis=(1, 2))
    assert (g["chain_tokens"] == ref["chain_tokens"]).all(), "chain tokens differ"
    assert np.allclose(g["qdep_chain"], ref["qdep_chain"], rtol=RTOL, atol=1e-300), \
        f"q_dep max rel err {np.max(np.abs(g['qdep_chain'] - ref['qdep_chain']) / np.maximum(ref['qdep_chain'], 1e-300))}"
    assert (g["cand_count"] == ref["cand_count"]).all(), "candidate counts differ"
    assert (g["cand_tokens"] == ref["cand_tokens"]).all(), "candidate tokens differ"
    assert np.allclose(g["cand_q"], ref["cand_p"], rtol=RTOL, atol=1e-30), "candidate q differs"
    rows = oracle.softmax_topk(oracle.host_logits(xs).reshape(-1, x.shape[-1]), k=k)
    good_r = rows["row_status"] == oracle.OK
    assert (g["row_max"].reshape(-1)[good_r] ==
            rows["row_max"][good_r].astype(np.float32)).all(), "row max differs"
    rs = rows["row_sum"][good_r]
    assert np.allclose(g["row_sum"].reshape(-1)[good_r].astype(np.float64), rs, rtol=RTOL, atol=0)
    if not with_tree:
        assert tr is None
        return mo, tr, ref
    t = {n: gc.np_(v)[sel] for n, v in tr.items()}
    rt = oracle.mixture_tree(g["prior_q"], g["cand_count"], g["cand_tokens"], g["cand_q"],
                             nmax=nmax, row_status=st)
    for f in ("n_nodes", "qstatus", "parent", "depth", "token"):
        assert (t[f] == rt[f]).all(), f"{f} differs at {np.argwhere(t[f] != rt[f])[:5].tolist()}"
    assert (t["rho"].view(np.uint32) == rt["rho"].view(np.uint32)).all(), "score differs"
    assert (t["ahat"] == rt["ahat"]).all(), "ahat differs"
    mask, pos = oracle.tree_mask(t["parent"], t["n_nodes"])
    assert (t["mask"].view(np.uint32) == mask).all(), "mask differs"
    assert (t["position_ids"] == pos).all(), "position ids differ"
    assert good_q.sum() == (t["qstatus"] != oracle.BAD_LOGITS).sum()
    return mo, tr, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_mixture_full_parity(dtype):
    wl = synth.scaled(synth.WORKLOADS["mixture"], B=3, K=3, b=5, V=3001, k=4, nmax=24,
                      dtype=dtype)
    x = gc.device_logits(wl, seed=21)
    prior = synth.make_prior_logits(wl).to("cuda")
    check_mixture(x, prior, wl.k, wl.nmax)


def test_mixture_workload_slice_full_parity():
    """Four queries of the latent-mixture workload's shape (K=8, b=16,
    V=151936 bf16, k=8, N=64)."""
    wl = synth.scaled(synth.WORKLOADS["mixture"], B=4)
    x = gc.device_logits(wl)
    prior = synth.make_prior_logits(wl).to("cuda")
    mo, tr, _ = check_mixture(x, prior, wl.k, wl.nmax)
    assert (gc.np_(tr["qstatus"]) == 0).all()


def test_mixture_full_workload_full_parity():
    """The whole latent-mixture workload in one call (the benchmark's launch),
    every query checked: rows, chains, q_dep, candidate unions and q, and
    every mixture tree, mask and position."""
    wl = synth.WORKLOADS["mixture"]
    x = synth.make_logits(wl, device="cuda")
    prior = synth.make_prior_logits(wl, device="cuda")
    mo, tr, _ = check_mixture(x, prior, wl.k, wl.nmax)
    assert (gc.np_(tr["qstatus"]) == 0).all()
    del x
    torch.cuda.empty_cache()


def test_single_branch_equals_plain_tree():
    """K = 1: weight 1, score = r = rho, candidates = the row's top-k, so the
    mixture tree is the plain best-first tree."""
    wl = synth.scaled(synth.WORKLOADS["main"], B=3, b=6, V=5000, nmax=40)
    x = gc.device_logits(wl, seed=5)
    prior = torch.zeros((wl.B, 1), dtype=torch.float32, device="cuda")
    mo, tr = binding.mixture_score(x.unsqueeze(1).contiguous(), prior, k=wl.k, nmax=wl.nmax)
    plain = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    torch.cuda.synchronize()
    for f in ("parent", "depth", "token", "rho", "ahat", "n_nodes", "qstatus", "mask"):
        assert torch.equal(tr[f], plain[f]), f


def test_bad_branch_row_and_no_tree():
    wl = synth.scaled(synth.WORKLOADS["mixture"], B=3, K=2, b=3, V=700, k=3, nmax=10,
                      dtype="f32")
    x = synth.make_logits(wl, seed=9)
    x[1, 1, 2, 17] = float("nan")
    x = x.to("cuda")
    prior = synth.make_prior_logits(wl).to("cuda")
    mo, tr, ref = check_mixture(x, prior, wl.k, wl.nmax)
    qs = gc.np_(tr["qstatus"])
    assert qs[1] == oracle.BAD_LOGITS and qs[0] != oracle.BAD_LOGITS and qs[2] != oracle.BAD_LOGITS
    assert (gc.np_(mo["chain_tokens"])[1] == -1).all()
    check_mixture(x, prior, wl.k, wl.nmax, with_tree=False)


def test_many_ties_across_branches():
    """Small integer logits: equal q inside and across branches."""
    torch.manual_seed(4)
    x = torch.randint(-3, 4, (3, 4, 6, 257)).float().to("cuda")
    prior = torch.randint(-1, 2, (3, 4)).float().to("cuda")
    check_mixture(x, prior, 5, 50)


@pytest.mark.parametrize("shape", [
    dict(B=4, K=8, b=5, V=3000, k=12, nmax=40),     # unions of up to 96 ids
    dict(B=2, K=16, b=2, V=5000, k=20, nmax=30),    # unions of up to 320 ids
])
def test_wide_unions_full_parity(shape):
    """Unions wider than one wave (the first-occurrence and rank path)."""
    wl = synth.scaled(synth.WORKLOADS["mixture"], dtype="f32", **shape)
    x = synth.make_logits(wl, seed=12).to("cuda")
    prior = synth.make_prior_logits(wl).to("cuda")
    check_mixture(x, prior, wl.k, wl.nmax)
