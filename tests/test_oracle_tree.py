"""Pins of the reference's best-first tree: the pages' worked example,
exhaustive optimality, an independent full sort, invariants, special cases
and a Monte-Carlo check that ties A_hat to the acceptance walk."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tree_inputs(rng, B, b, k, ties=False):
    """Random candidate lists: ids distinct per row, q sorted descending."""
    ids = np.empty((B, b, k), np.int32)
    q = np.empty((B, b, k), np.float32)
    for qq in range(B):
        for p in range(b):
            ids[qq, p] = rng.choice(1000, size=k, replace=False)
            if ties:
                v = rng.integers(1, 4, size=k).astype(np.float64) / 8.0
            else:
                v = rng.dirichlet(np.ones(k + 2))[:k]
            order = np.lexsort((ids[qq, p], -v))   # q desc, id asc on ties
            ids[qq, p] = ids[qq, p][order]
            q[qq, p] = v[order].astype(np.float32)
    return ids, q


def paths_of(tree, qq):
    n = int(tree["n_nodes"][qq])
    par, tok = tree["parent"][qq], tree["token"][qq]
    out = []
    for i in range(1, n + 1):
        path, j = [], i
        while j != 0:
            path.append(int(tok[j]))
            j = int(par[j])
        out.append(path[::-1])
    return out


def test_lay_example(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "lay_toy.json")))
    ids = np.array(g["ids"], np.int32)[None]
    q = np.array(g["q"], np.float32)[None]
    t2 = oracle_mod.best_first(ids[:, :1], q[:, :1], nmax=2)
    assert t2["token"][0, 1:3].tolist() == g["expect_n2"]["tokens_in_pop_order"]
    assert np.allclose(t2["ahat"][0], g["expect_n2"]["ahat"], atol=g["tolerance"])
    full = oracle_mod.best_first(ids, q, nmax=6)
    assert paths_of(full, 0) == g["expect_full"]["paths_in_pop_order"]
    assert np.allclose(full["rho"][0, 1:], g["expect_full"]["rho"], atol=g["tolerance"])
    assert full["ahat"][0, 6] == pytest.approx(g["expect_full"]["ahat_full"], abs=g["tolerance"])


@pytest.mark.parametrize("k,b,nmax_n", [(3, 3, 7), (4, 4, 6), (2, 5, 7)])
def test_best_first_is_optimal_by_enumeration(oracle_mod, k, b, nmax_n):
    rng = np.random.default_rng(10 + k * b)
    for trial in range(3):
        ids, q = tree_inputs(rng, 1, b, k, ties=(trial == 2))
        t = oracle_mod.best_first(ids, q, nmax=nmax_n)
        for N in range(1, nmax_n + 1):
            best, count = pins.max_subtree_sum(ids[0], q[0], N)
            assert count > 0
            assert t["ahat"][0, N] == pytest.approx(best, rel=1e-12, abs=0)


@pytest.mark.parametrize("ties", [False, True])
def test_pop_order_equals_full_sort(oracle_mod, ties):
    rng = np.random.default_rng(3 + ties)
    b, k = 4, 4
    ids, q = tree_inputs(rng, 2, b, k, ties=ties)
    nmax = 4 + 16 + 64 + 256
    t = oracle_mod.best_first(ids, q, nmax=nmax)
    for qq in range(2):
        ref = pins.sorted_candidates(ids[qq], q[qq])
        assert int(t["n_nodes"][qq]) == len(ref) == nmax
        assert paths_of(t, qq) == [list(n["tokens"]) for n in ref]
        assert t["rho"][qq, 1:].tolist() == [float(n["rho"]) for n in ref]
        assert t["qstatus"][qq] == oracle_mod.OK


def check_invariants(t, ids, q, b, nmax):
    B = ids.shape[0]
    for qq in range(B):
        n = int(t["n_nodes"][qq])
        par, dep, tok, rho, ah = (t[x][qq] for x in ("parent", "depth", "token", "rho", "ahat"))
        assert par[0] == -1 and dep[0] == 0 and tok[0] == -1 and rho[0] == 1.0 and ah[0] == 1.0
        for i in range(1, n + 1):
            p = int(par[i])
            assert 0 <= p < i
            assert dep[i] == dep[p] + 1 <= b
            row = dep[i] - 1
            js = np.nonzero(ids[qq, row] == tok[i])[0]
            assert len(js) == 1
            assert rho[i] == pins.f32mul(rho[p], q[qq, row, js[0]])
            assert rho[i] <= rho[i - 1] or i == 1      # pops never increase
            assert rho[i] <= 1.0
            assert ah[i] == ah[i - 1] + float(rho[i])
        sib = {}
        for i in range(1, n + 1):
            sib.setdefault(int(par[i]), []).append(int(tok[i]))
        for v in sib.values():
            assert len(v) == len(set(v))
        for i in range(n + 1, nmax + 1):
            assert par[i] == -1 and dep[i] == -1 and tok[i] == -1 and rho[i] == 0 and ah[i] == 0


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 10 ** 6), b=st.integers(1, 6), k=st.integers(1, 6),
       nmax=st.integers(1, 40), ties=st.booleans())
def test_invariants_and_nesting(oracle_mod, seed, b, k, nmax, ties):
    rng = np.random.default_rng(seed)
    ids, q = tree_inputs(rng, 3, b, k, ties=ties)
    t = oracle_mod.best_first(ids, q, nmax=nmax)
    check_invariants(t, ids, q, b, nmax)
    total = sum(k ** d for d in range(1, b + 1))
    assert (t["n_nodes"] == min(nmax, total)).all()
    if total < nmax:
        assert (t["qstatus"] == oracle_mod.EXHAUSTED).all()
    # T_N is a prefix of T_{N+1}
    t2 = oracle_mod.best_first(ids, q, nmax=nmax + 1)
    for f in ("parent", "depth", "token", "rho", "ahat"):
        assert (t2[f][:, :nmax + 1] == t[f]).all()


def test_k1_is_greedy_chain(oracle_mod):
    rng = np.random.default_rng(5)
    ids, q = tree_inputs(rng, 2, 7, 1)
    t = oracle_mod.best_first(ids, q, nmax=20)
    assert t["n_nodes"].tolist() == [7, 7]
    for qq in range(2):
        assert t["parent"][qq, 1:8].tolist() == list(range(7))
        assert t["token"][qq, 1:8].tolist() == ids[qq, :, 0].tolist()
        r = np.float32(1.0)
        for d in range(7):
            r = pins.f32mul(r, q[qq, d, 0])
            assert t["rho"][qq, d + 1] == r


def test_b1_is_star(oracle_mod):
    rng = np.random.default_rng(6)
    ids, q = tree_inputs(rng, 1, 1, 6)
    t = oracle_mod.best_first(ids, q, nmax=4)
    assert t["parent"][0, 1:5].tolist() == [0, 0, 0, 0]
    assert t["token"][0, 1:5].tolist() == ids[0, 0, :4].tolist()


def test_uniform_q_gives_level_order(oracle_mod):
    b, k = 3, 3
    ids = np.tile(np.array([30, 10, 20], np.int32), (1, b, 1))
    q = np.full((1, b, k), 1.0 / 3.0, np.float32)
    t = oracle_mod.best_first(ids, q, nmax=3 + 9 + 27)
    dep = t["depth"][0, 1:]
    assert (np.diff(dep) >= 0).all()
    assert t["token"][0, 1:4].tolist() == [10, 20, 30]   # token asc on ties
    # the full tree carries the whole mass of every level: A_hat = 1 + b * 1
    assert t["ahat"][0, -1] == pytest.approx(1.0 + b, rel=1e-6)


def test_expected_accept_equals_ahat_minus_one(oracle_mod):
    """If each node's target is drawn from the drafter's own full-vocabulary
    marginal at the next position, independently per node, the greedy walk
    reaches node i with probability rho(i); so E[accept_len] = A_hat - 1."""
    from block_diffusion_tree_amd import synth
    wl = synth.WORKLOADS["tiny"]
    x = synth.make_logits(wl).numpy()
    sm = oracle_mod.softmax_topk(x, k=wl.V)           # full distributions
    ids = sm["topk_ids"][:, :, :wl.k]
    q = sm["topk_p"][:, :, :wl.k].astype(np.float32)
    N = wl.nmax
    t = oracle_mod.best_first(ids, q, nmax=N)
    n = int(t["n_nodes"][0])
    trials = 100_000
    rng = np.random.default_rng(77)
    target = np.zeros((trials, N + 1), np.int32)
    for i in range(n + 1):
        d = int(t["depth"][0, i])
        if d < wl.b:
            pfull = np.zeros(wl.V)
            pfull[sm["topk_ids"][0, d]] = sm["topk_p"][0, d]
            target[:, i] = rng.choice(wl.V, size=trials, p=pfull / pfull.sum())
        else:
            target[:, i] = rng.integers(0, wl.V, size=trials)
    rep = lambda a: np.repeat(a[:1], trials, axis=0)
    alen, _, _ = oracle_mod.accept(rep(t["parent"]), rep(t["token"]), rep(t["n_nodes"]),
                                   wl.b, target)
    mean, sd = alen.mean(), alen.std() / np.sqrt(trials)
    expect = t["ahat"][0, n] - 1.0
    assert abs(mean - expect) < 5 * sd + 1e-6, (mean, expect, sd)
