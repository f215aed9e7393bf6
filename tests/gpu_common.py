"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the CPU reference on the same inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

from block_diffusion_tree_amd import binding, synth
from oracle import oracle

# softmax probabilities: 1e-5 relative, with an absolute floor far below any
# probability that can matter (float32 exp flushes results under ~1e-38).
Q_RTOL = 1e-5
Q_ATOL = 1e-30


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()


def np_(t):
    return t.detach().cpu().numpy()


def check_rows(g, ref, rows_ok=None):
    """GPU row outputs vs the reference's float64 softmax/top-k."""
    st = ref["row_status"].reshape(-1)
    gi = np_(g["topk_ids"]).reshape(st.size, -1)
    gq = np_(g["topk_q"]).reshape(st.size, -1)
    good = st == oracle.OK
    assert (gi[good] == ref["topk_ids"].reshape(st.size, -1)[good]).all(), "top-k ids differ"
    rq = ref["topk_p"].reshape(st.size, -1)[good]
    assert np.allclose(gq[good], rq, rtol=Q_RTOL, atol=Q_ATOL), \
        f"q max rel err {np.max(np.abs(gq[good] - rq) / np.maximum(rq, 1e-300))}"
    gm = np_(g["row_max"]).reshape(-1)[good]
    assert (gm == ref["row_max"].reshape(-1)[good].astype(np.float32)).all(), "row max differs"
    gs = np_(g["row_sum"]).reshape(-1)[good].astype(np.float64)
    rs = ref["row_sum"].reshape(-1)[good]
    assert np.allclose(gs, rs, rtol=Q_RTOL, atol=0), \
        f"row sum max rel err {np.max(np.abs(gs - rs) / rs)}"
    assert (gi[~good] == -1).all()


def check_tree(g, wl_b, k, nmax, nmin=1, cost=None, l_ar=1.0, row_status=None):
    """GPU tree vs the reference fed the GPU's own top-k ids and q."""
    ids = np_(g["topk_ids"])
    q = np_(g["topk_q"])
    ref = oracle.best_first(ids, q, nmax=nmax, nmin=nmin, cost=cost, l_ar=l_ar,
                            row_status=row_status)
    for f in ("n_nodes", "qstatus", "parent", "depth", "token"):
        a, r = np_(g[f]), ref[f]
        assert (a == r).all(), f"{f} differs at {np.argwhere(a != r)[:5].tolist()}"
    assert (np_(g["rho"]).view(np.uint32) == ref["rho"].view(np.uint32)).all(), "rho differs"
    ga = np_(g["ahat"])
    assert np.allclose(ga, ref["ahat"], rtol=1e-12, atol=0), "ahat differs"
    return ref


def check_mask(g, pos_base=None):
    mask, pos = oracle.tree_mask(np_(g["parent"]), np_(g["n_nodes"]),
                                 None if pos_base is None else np_(pos_base))
    assert (np_(g["mask"]).view(np.uint32) == mask).all(), "mask differs"
    assert (np_(g["position_ids"]) == pos).all(), "position ids differ"


def run_and_check(logits, k, nmax, nmin=1, cost=None, l_ar=1.0, pos_base=None, ref_rows=None):
    """Full parity of one bastion_build_trees call; returns (gpu, reference rows)."""
    g = binding.build_trees(logits, k=k, nmax=nmax, nmin=nmin, cost=cost, l_ar=l_ar,
                            pos_base=pos_base)
    torch.cuda.synchronize()
    if ref_rows is None:
        ref_rows = oracle.softmax_topk(oracle.host_logits(logits), k=k)
    check_rows(g, ref_rows)
    cost_h = None if cost is None else np_(cost)
    check_tree(g, logits.shape[1], k, nmax, nmin, cost_h, l_ar, ref_rows["row_status"])
    check_mask(g, pos_base)
    return g, ref_rows


def device_logits(wl, seed=None):
    return synth.make_logits(wl, seed=seed).to("cuda")
