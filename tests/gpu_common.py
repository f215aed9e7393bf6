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


# The library refuses rows whose maximum logit exceeds 2^20 in magnitude
# (BASTION_Q_RANGE, a float32 range limit of the library, not of the method);
# the reference computes their softmax.  Such rows are expected refused.
RANGE_LIMIT = 2.0 ** 20


def expected_row_status(ref):
    """The reference's row status with the library's range limit applied."""
    st = np.array(ref["row_status"], copy=True)
    big = (st == oracle.OK) & (np.abs(ref["row_max"]) > RANGE_LIMIT)
    st[big] = binding.Q_RANGE
    return st


def check_rows(g, ref):
    """GPU row outputs vs the reference's float64 softmax/top-k."""
    st = expected_row_status(ref).reshape(-1)
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
    if row_status is not None:
        # queries refused only for the range limit report BASTION_Q_RANGE
        rs = np.asarray(row_status).reshape(ids.shape[0], -1)
        only_range = (rs == binding.Q_RANGE).any(axis=1) & ~(rs == oracle.BAD_LOGITS).any(axis=1)
        ref["qstatus"][only_range] = binding.Q_RANGE
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
    check_tree(g, logits.shape[1], k, nmax, nmin, cost_h, l_ar, expected_row_status(ref_rows))
    check_mask(g, pos_base)
    return g, ref_rows


def device_logits(wl, seed=None):
    return synth.make_logits(wl, seed=seed).to("cuda")
