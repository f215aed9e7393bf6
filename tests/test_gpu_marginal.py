"""GPU parity of bastion_mixture_marginal (candidates from the latent
mixture's marginal sum_z w_z q_i(x|z), then the mixture tree over them)
against the float64 reference.

The kernel ranks tokens by a float32 marginal and the reference by a float64
one, so where two tokens' marginals agree to a few float32 roundings either
order is correct: the test compares the sorted top-k marginal values (1e-5
relative), the ids wherever the reference's values are apart by more than
that (the reference's (k+1)-th value bounds the last slot), every branch's
q of the selected tokens (1e-5), and the tree exactly against the reference
tree fed the GPU's own weights, candidates and q."""
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


def check_marginal(x, prior, k, nmax, with_tree=True):
    mo, tr = binding.mixture_marginal(x, prior, k=k, nmax=nmax, with_tree=with_tree)
    torch.cuda.synchronize()
    g = {n: gc.np_(t) for n, t in mo.items()}
    ref = oracle.mixture_marginal(oracle.host_logits(x), gc.np_(prior), k + 1)
    assert np.allclose(g["prior_q"], ref["prior_w"], rtol=RTOL, atol=0), "prior weights differ"
    st = ref["row_status"]
    good_q = (st == oracle.OK).all(axis=(1, 2))
    B, b = g["marg_ids"].shape[:2]
    for qq in range(B):
        if not good_q[qq]:
            assert (g["marg_ids"][qq] == -1).all() and (g["marg_q"][qq] == 0).all()
            continue
        for i in range(b):
            gi, gm = g["marg_ids"][qq, i], g["marg_q"][qq, i].astype(np.float64)
            ri, rm = ref["marg_ids"][qq, i], ref["marg_p"][qq, i]
            assert len(set(gi.tolist())) == k and (gi >= 0).all()
            assert np.allclose(gm, rm[:k], rtol=RTOL, atol=1e-30), f"marginals differ at {qq},{i}"
            for j in range(k):
                near = [abs(rm[j] - rm[jj]) <= 4 * RTOL * rm[j] for jj in (j - 1, j + 1)
                        if 0 <= jj <= k]
                if not any(near):
                    assert gi[j] == ri[j], f"candidate {j} differs at {qq},{i}"
                    assert np.allclose(g["cand_q"][qq, i, j], ref["cand_p"][qq, i, j], rtol=RTOL,
                                       atol=1e-30), f"branch q differs at {qq},{i},{j}"
    rows = oracle.softmax_topk(oracle.host_logits(x).reshape(-1, x.shape[-1]), k=1)
    good_r = rows["row_status"] == oracle.OK
    assert (g["row_max"].reshape(-1)[good_r] == rows["row_max"][good_r].astype(np.float32)).all()
    assert np.allclose(g["row_sum"].reshape(-1)[good_r].astype(np.float64),
                       rows["row_sum"][good_r], rtol=RTOL, atol=0)
    if not with_tree:
        assert tr is None
        return mo, tr
    t = {n: gc.np_(v) for n, v in tr.items()}
    cnt = np.full((B, b), k, np.int32)
    rt = oracle.mixture_tree(g["prior_q"], cnt, g["marg_ids"], g["cand_q"], nmax=nmax,
                             row_status=st)
    for f in ("n_nodes", "qstatus", "parent", "depth", "token"):
        assert (t[f] == rt[f]).all(), f"{f} differs at {np.argwhere(t[f] != rt[f])[:5].tolist()}"
    assert (t["rho"].view(np.uint32) == rt["rho"].view(np.uint32)).all(), "score differs"
    assert (t["ahat"] == rt["ahat"]).all(), "ahat differs"
    mask, pos = oracle.tree_mask(t["parent"], t["n_nodes"])
    assert (t["mask"].view(np.uint32) == mask).all() and (t["position_ids"] == pos).all()
    return mo, tr


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_marginal_full_parity(dtype):
    wl = synth.scaled(synth.WORKLOADS["mixture"], B=3, K=3, b=5, V=3001, k=4, nmax=24, dtype=dtype)
    x = gc.device_logits(wl, seed=31)
    prior = synth.make_prior_logits(wl).to("cuda")
    check_marginal(x, prior, wl.k, wl.nmax)


def test_unaligned_rows_and_ties():
    """Rows that do not start on 16 bytes (V = 3001 bf16) take the element
    path; integer logits make many exactly equal marginals."""
    torch.manual_seed(6)
    x = torch.randint(-3, 4, (2, 4, 3, 3001)).to(torch.bfloat16).to("cuda")
    prior = torch.randint(-1, 2, (2, 4)).float().to("cuda")
    check_marginal(x, prior, 6, 30)


def test_marginal_workload_full_parity():
    """The latent-mixture workload (B=128, K=8, b=16, V=151936 bf16, k=8,
    N=64) in one call, every query and position checked."""
    wl = synth.WORKLOADS["mixture"]
    x = synth.make_logits(wl, device="cuda")
    prior = synth.make_prior_logits(wl, device="cuda")
    mo, tr = check_marginal(x, prior, wl.k, wl.nmax)
    assert (gc.np_(tr["qstatus"]) == 0).all()
    del x
    torch.cuda.empty_cache()


def test_single_branch_marginal_is_the_plain_tree():
    """K = 1: the marginal is the row's softmax, its top-k the row's top-k,
    and the mixture tree over them the plain best-first tree."""
    wl = synth.scaled(synth.WORKLOADS["main"], B=3, b=6, V=5000, nmax=40)
    x = gc.device_logits(wl, seed=5)
    prior = torch.zeros((wl.B, 1), dtype=torch.float32, device="cuda")
    mo, tr = binding.mixture_marginal(x.unsqueeze(1).contiguous(), prior, k=wl.k, nmax=wl.nmax)
    plain = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    torch.cuda.synchronize()
    assert torch.equal(mo["marg_ids"], plain["topk_ids"])
    for f in ("parent", "depth", "token", "rho", "ahat", "n_nodes", "qstatus", "mask"):
        assert torch.equal(tr[f], plain[f]), f


def test_bad_branch_row_and_no_tree():
    wl = synth.scaled(synth.WORKLOADS["mixture"], B=3, K=2, b=3, V=700, k=3, nmax=10, dtype="f32")
    x = synth.make_logits(wl, seed=9)
    x[2, 0, 1, 5] = float("inf")
    x = x.to("cuda")
    prior = synth.make_prior_logits(wl).to("cuda")
    mo, tr = check_marginal(x, prior, wl.k, wl.nmax)
    assert gc.np_(tr["qstatus"]).tolist()[2] == oracle.BAD_LOGITS
    check_marginal(x, prior, wl.k, wl.nmax, with_tree=False)
