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
