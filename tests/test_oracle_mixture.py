"""Pins of the reference's latent-mixture path: normalisation over all
sequences, the K=1 reduction to the factorised proposal, identical branches,
candidate unions, and best-first optimality of the mixture tree."""
import itertools
import math

import numpy as np
import pytest

import pins


def rand_branch_logits(rng, B, K, b, V, scale=2.0):
    return (rng.standard_normal((B, K, b, V)) * scale).astype(np.float32)


def test_qdep_sums_to_one_over_all_sequences(oracle_mod):
    rng = np.random.default_rng(0)
    B, K, b, V = 2, 2, 3, 4
    x = rand_branch_logits(rng, B, K, b, V)
    prior = rng.standard_normal((B, K)).astype(np.float32)
    seqs = pins.enumerate_sequences(V, b)
    allseq = np.repeat(seqs[None], B, axis=0)
    qd = oracle_mod.qdep_sequences(x, prior, allseq)
    assert np.allclose(qd.sum(axis=1), 1.0, rtol=0, atol=1e-13)


def test_prior_weights_closed_form(oracle_mod):
    rng = np.random.default_rng(1)
    x = rand_branch_logits(rng, 3, 2, 2, 16)
    prior = np.array([[0.3, -1.2], [5.0, 5.0], [-2.0, 1.0]], np.float32)
    m = oracle_mod.mixture(x, prior, k=3)
    for qq in range(3):
        a, b = float(prior[qq, 0]), float(prior[qq, 1])
        w0 = 1.0 / (1.0 + math.exp(b - a))
        assert m["prior_w"][qq, 0] == pytest.approx(w0, rel=1e-14)
        assert m["prior_w"][qq].sum() == pytest.approx(1.0, abs=1e-15)


def test_k1_reduces_to_factorised_proposal(oracle_mod):
    """K = 1: q_dep of the greedy chain is the product of each position's top
    probability, and the mixture tree equals the plain best-first tree."""
    rng = np.random.default_rng(2)
    B, b, V, k = 3, 5, 64, 4
    x = rand_branch_logits(rng, B, 1, b, V)
    prior = rng.standard_normal((B, 1)).astype(np.float32)
    m = oracle_mod.mixture(x, prior, k=k)
    sm = oracle_mod.softmax_topk(x[:, 0], k=k)
    assert (m["chain_tokens"][:, 0] == sm["topk_ids"][:, :, 0]).all()
    assert np.allclose(m["qdep_chain"][:, 0], np.prod(sm["topk_p"][:, :, 0], axis=1), rtol=1e-13)
    q32 = sm["topk_p"].astype(np.float32)
    plain = oracle_mod.best_first(sm["topk_ids"], q32, nmax=40)
    # mixture candidates are the same tokens, listed in ascending id order
    cand_q = np.zeros((B, b, k, 1), np.float32)
    for qq in range(B):
        for i in range(b):
            for c in range(k):
                tok = m["cand_tokens"][qq, i, c]
                j = int(np.nonzero(sm["topk_ids"][qq, i] == tok)[0][0])
                cand_q[qq, i, c, 0] = q32[qq, i, j]
    mt = oracle_mod.mixture_tree(np.ones((B, 1), np.float32), m["cand_count"],
                                 m["cand_tokens"], cand_q, nmax=40)
    for f in ("parent", "depth", "token", "rho", "ahat", "n_nodes"):
        assert (mt[f] == plain[f]).all(), f


def test_identical_branches_ignore_the_prior(oracle_mod):
    rng = np.random.default_rng(3)
    one = rand_branch_logits(rng, 2, 1, 4, 32)
    x = np.repeat(one, 3, axis=1)
    prior = rng.standard_normal((2, 3)).astype(np.float32)
    m = oracle_mod.mixture(x, prior, k=2)
    sm = oracle_mod.softmax_topk(one[:, 0], k=1)
    expect = np.prod(sm["topk_p"][:, :, 0], axis=1)
    for z in range(3):
        assert np.allclose(m["qdep_chain"][:, z], expect, rtol=1e-13)


def test_candidate_union_and_probabilities(oracle_mod):
    rng = np.random.default_rng(4)
    B, K, b, V, k = 2, 3, 3, 40, 4
    x = np.round(rand_branch_logits(rng, B, K, b, V))   # ties
    prior = rng.standard_normal((B, K)).astype(np.float32)
    m = oracle_mod.mixture(x, prior, k=k)
    for qq in range(B):
        for i in range(b):
            union = set()
            for z in range(K):
                ids = np.arange(V)
                union |= set(np.lexsort((ids, -x[qq, z, i].astype(np.float64)))[:k].tolist())
            cnt = int(m["cand_count"][qq, i])
            assert m["cand_tokens"][qq, i, :cnt].tolist() == sorted(union)
            assert (m["cand_tokens"][qq, i, cnt:] == -1).all()
            for z in range(K):
                row = x[qq, z, i].astype(np.float64)
                p = np.exp(row - row.max())
                p /= p.sum()
                assert np.allclose(m["cand_p"][qq, i, :cnt, z], p[sorted(union)], rtol=1e-13)


def mixture_inputs(rng, B, K, b, C):
    w = rng.dirichlet(np.ones(K), size=B).astype(np.float32)
    cnt = np.full((B, b), C, np.int32)
    toks = np.stack([np.stack([np.sort(rng.choice(500, C, replace=False)) for _ in range(b)])
                     for _ in range(B)]).astype(np.int32)
    cq = rng.dirichlet(np.ones(C + 1), size=(B, b, K))[..., :C]   # [B,b,K,C]
    cq = np.ascontiguousarray(np.transpose(cq, (0, 1, 3, 2))).astype(np.float32)
    return w, cnt, toks, cq


def test_mixture_tree_is_optimal_by_enumeration(oracle_mod):
    """rho_mix is non-increasing along paths, so best-first maximises the sum
    of scores over prefix-closed trees of each size."""
    rng = np.random.default_rng(5)
    B, K, b, C = 2, 3, 3, 3
    w, cnt, toks, cq = mixture_inputs(rng, B, K, b, C)
    t = oracle_mod.mixture_tree(w, cnt, toks, cq, nmax=7)
    for qq in range(B):
        score = {(): np.float32(1.0)}
        r = {(): np.ones(K, np.float32)}
        for path in itertools.chain.from_iterable(
                itertools.product(range(C), repeat=d) for d in range(1, b + 1)):
            d = len(path) - 1
            rv = (r[path[:-1]] * cq[qq, d, path[-1]]).astype(np.float32)
            r[path] = rv
            acc = np.float32(0.0)
            for z in range(K):
                acc = pins.fmaf_exact(w[qq, z], rv[z], acc)
            score[path] = acc
        for N in range(1, 8):
            best = -1.0
            # enumerate prefix-closed subsets of size N
            def rec(total, frontier, remaining):
                nonlocal best
                if remaining == 0:
                    best = max(best, total)
                    return
                for idx, node in enumerate(frontier):
                    kids = [node + (c,) for c in range(C)] if len(node) < b else []
                    rec(total + float(score[node]), frontier[idx + 1:] + kids, remaining - 1)
            rec(1.0, [(c,) for c in range(C)], N)
            assert t["ahat"][qq, N] == pytest.approx(best, rel=1e-12)


def test_full_mixture_tree_mass(oracle_mod):
    """When the candidates are the whole vocabulary, each level of the full
    tree carries total mass 1, so A_hat of the full tree is b + 1."""
    rng = np.random.default_rng(6)
    B, K, b, V = 2, 2, 3, 4
    x = rand_branch_logits(rng, B, K, b, V)
    prior = rng.standard_normal((B, K)).astype(np.float32)
    m = oracle_mod.mixture(x, prior, k=V)
    full = V + V ** 2 + V ** 3
    cq = np.ascontiguousarray(m["cand_p"].astype(np.float32))
    t = oracle_mod.mixture_tree(m["prior_w"].astype(np.float32), m["cand_count"],
                                m["cand_tokens"], cq, nmax=full)
    assert t["n_nodes"].tolist() == [full, full]
    assert np.allclose(t["ahat"][:, full], 1.0 + b, rtol=1e-5)
    assert (np.diff(t["rho"][:, 1:], axis=1) <= 0).all()


def test_qdep_one_hot_disjoint_branches(oracle_mod):
    """Branches that put all their mass on one token per position, on tokens
    no other branch uses (every other entry -inf): chain z gets probability 1
    from branch z and 0 from every other branch, so its q_dep is exactly the
    prior weight w_z (DBlast page, Methodology 1, the latent-mixture
    q_dep).  Holds for several K and b with an unequal prior."""
    for K, b in ((2, 2), (3, 4), (4, 3)):
        V = K * b + 5
        B = 2
        x = np.full((B, K, b, V), -np.inf, np.float32)
        for qq in range(B):
            for z in range(K):
                for i in range(b):
                    x[qq, z, i, (z * b + i + qq) % V] = 1.5 + z
        prior = np.array([[0.7 * z - 0.4 * z * z + qq for z in range(K)] for qq in range(B)],
                         np.float32)
        m = oracle_mod.mixture(x, prior, k=1)
        for qq in range(B):
            e = np.exp(prior[qq].astype(np.float64) - prior[qq].max())
            w = e / e.sum()
            assert len(set(np.round(w, 12))) == K   # the prior is unequal
            for z in range(K):
                assert m["chain_tokens"][qq, z].tolist() == [(z * b + i + qq) % V
                                                            for i in range(b)]
                assert m["qdep_chain"][qq, z] == pytest.approx(w[z], rel=1e-14)


def test_qdep_two_branches_by_hand(oracle_mod):
    """K = 2, b = 2, V = 2 with logits ln(n) chosen so that every probability
    is a small fraction (two-entry softmax = sigmoid of the difference):

      branch 0: position 0 p = (1/4, 3/4), position 1 p = (2/3, 1/3) -> chain (1, 0)
      branch 1: position 0 p = (4/5, 1/5), position 1 p = (1/10, 9/10) -> chain (0, 1)
      prior weights (1/4, 3/4)

    q_dep(chain 0) = 1/4 * 3/4 * 2/3 + 3/4 * 1/5 * 1/10 = 0.14 and
    q_dep(chain 1) = 1/4 * 1/4 * 1/3 + 3/4 * 4/5 * 9/10 = 0.5608333...
    Scoring a chain on its own branch only would give 0.5 and 0.72; swapping
    the chain and branch indices 0.1875 and 0.44."""
    ln = np.log
    x = np.array([[[[0.0, ln(3)], [ln(2), 0.0]],
                   [[ln(4), 0.0], [0.0, ln(9)]]]], np.float32)
    prior = np.array([[0.0, ln(3)]], np.float32)
    m = oracle_mod.mixture(x, prior, k=1)
    assert m["chain_tokens"][0].tolist() == [[1, 0], [0, 1]]
    expect = [1 / 4 * 3 / 4 * 2 / 3 + 3 / 4 * 1 / 5 * 1 / 10,
              1 / 4 * 1 / 4 * 1 / 3 + 3 / 4 * 4 / 5 * 9 / 10]
    # float32 rounding of ln(n) moves each probability by < 1e-7 relative
    assert m["qdep_chain"][0].tolist() == pytest.approx(expect, rel=1e-6)
    # the same sequences scored by the sequence routine
    qs = oracle_mod.qdep_sequences(x, prior, m["chain_tokens"])
    assert qs[0].tolist() == pytest.approx(expect, rel=1e-6)


def test_qdep_sequences_by_hand(oracle_mod):
    """The sequence routine on every sequence of the hand example above,
    each written out as w_0 p_0(s) + w_1 p_1(s)."""
    ln = np.log
    x = np.array([[[[0.0, ln(3)], [ln(2), 0.0]],
                   [[ln(4), 0.0], [0.0, ln(9)]]]], np.float32)
    prior = np.array([[0.0, ln(3)]], np.float32)
    p = {0: [[1 / 4, 3 / 4], [2 / 3, 1 / 3]], 1: [[4 / 5, 1 / 5], [1 / 10, 9 / 10]]}
    w = [1 / 4, 3 / 4]
    seqs = np.array([[[0, 0], [0, 1], [1, 0], [1, 1]]], np.int32)
    got = oracle_mod.qdep_sequences(x, prior, seqs)[0]
    for s, (a, c) in enumerate(seqs[0].tolist()):
        want = w[0] * p[0][0][a] * p[0][1][c] + w[1] * p[1][0][a] * p[1][1][c]
        assert got[s] == pytest.approx(want, rel=1e-6)
    assert got.sum() == pytest.approx(1.0, abs=1e-14)


def test_qdep_random_branches_match_sequence_routine(oracle_mod):
    """Distinct random branches (K = 3, b = 3): the chain scores equal the
    sequence routine run on the chains, and a brute-force double sum over
    the float64 softmax of every row."""
    rng = np.random.default_rng(11)
    B, K, b, V = 2, 3, 3, 7
    x = rand_branch_logits(rng, B, K, b, V, scale=1.5)
    prior = np.array([[0.3, -1.1, 0.9], [2.0, 0.0, -0.5]], np.float32)
    m = oracle_mod.mixture(x, prior, k=2)
    qs = oracle_mod.qdep_sequences(x, prior, m["chain_tokens"])
    assert np.allclose(m["qdep_chain"], qs, rtol=1e-14, atol=0)
    xd = x.astype(np.float64)
    p = np.exp(xd - xd.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    for qq in range(B):
        w = np.exp(prior[qq].astype(np.float64) - prior[qq].max())
        w /= w.sum()
        for z in range(K):
            chain = m["chain_tokens"][qq, z]
            assert chain.tolist() == [int(np.argmax(x[qq, z, i])) for i in range(b)]
            want = sum(w[zp] * np.prod([p[qq, zp, i, chain[i]] for i in range(b)])
                       for zp in range(K))
            assert m["qdep_chain"][qq, z] == pytest.approx(want, rel=1e-12)


# ---- candidates from the mixture marginal -----------------------------------

def numpy_marginal(x, prior):
    """sum_z w_z softmax(row z) in float64 with numpy (an independent route)."""
    xd = x.astype(np.float64)
    p = np.exp(xd - xd.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)                     # [B,K,b,V]
    pr = prior.astype(np.float64)
    w = np.exp(pr - pr.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)                      # [B,K]
    return np.einsum("bz,bziv->biv", w, p), p, w


def test_marginal_matches_numpy_and_lexsort(oracle_mod):
    rng = np.random.default_rng(21)
    B, K, b, V, k = 2, 3, 4, 50, 6
    x = np.round(rand_branch_logits(rng, B, K, b, V) * 2) / 2   # ties in the logits
    prior = rng.standard_normal((B, K)).astype(np.float32)
    r = oracle_mod.mixture_marginal(x, prior, k)
    m, p, w = numpy_marginal(x, prior)
    assert np.allclose(r["prior_w"], w, rtol=1e-14)
    for qq in range(B):
        for i in range(b):
            ids = np.arange(V)
            # the ranking of numpy's marginal, rounded so that equal mixtures
            # of tied logits compare equal
            want = np.lexsort((ids, -np.round(m[qq, i], 12)))[:k]
            assert r["marg_ids"][qq, i].tolist() == want.tolist()
            assert np.allclose(r["marg_p"][qq, i], m[qq, i, want], rtol=1e-12)
            assert np.allclose(r["cand_p"][qq, i], p[qq][:, i][:, want].T, rtol=1e-12)


def test_marginal_sums_to_one_and_k1_is_the_plain_topk(oracle_mod):
    rng = np.random.default_rng(22)
    x = rand_branch_logits(rng, 2, 3, 2, 12)
    prior = rng.standard_normal((2, 3)).astype(np.float32)
    r = oracle_mod.mixture_marginal(x, prior, 12)           # k = V: every token
    assert np.allclose(r["marg_p"].sum(axis=-1), 1.0, rtol=0, atol=1e-14)
    # one branch: the marginal is that branch's softmax, its top-k the row's
    one = rand_branch_logits(rng, 2, 1, 3, 40)
    r1 = oracle_mod.mixture_marginal(one, np.zeros((2, 1), np.float32), 5)
    sm = oracle_mod.softmax_topk(one[:, 0], k=5)
    assert (r1["marg_ids"] == sm["topk_ids"]).all()
    assert np.allclose(r1["marg_p"], sm["topk_p"], rtol=1e-13)


def test_marginal_of_disjoint_one_hot_branches_is_the_prior(oracle_mod):
    """Branch z puts all its mass on token t_z: m(t_z) = w_z, so the
    candidates are the branches' tokens in prior order (then token order)."""
    K, b, V = 4, 2, 30
    x = np.full((1, K, b, V), -np.inf, np.float32)
    toks = [[7, 3], [1, 9], [20, 2], [5, 11]]
    for z in range(K):
        for i in range(b):
            x[0, z, i, toks[z][i]] = 0.5 * z
    prior = np.array([[0.3, 1.2, -0.4, 1.2]], np.float32)   # branches 1 and 3 tie
    r = oracle_mod.mixture_marginal(x, prior, 4)
    w = np.exp(prior[0].astype(np.float64) - 1.2)
    w /= w.sum()
    for i in range(b):
        order = sorted(range(K), key=lambda z: (-w[z], toks[z][i]))
        assert r["marg_ids"][0, i].tolist() == [toks[z][i] for z in order]
        assert np.allclose(r["marg_p"][0, i], [w[z] for z in order], rtol=1e-14)
