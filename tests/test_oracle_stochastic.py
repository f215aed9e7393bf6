"""Pins of the reference's stochastic variants: the counter-based uniforms
are uniform, Gumbel-max draws follow softmax(l / T) (and the argmax at
T = 0), the target-sampling walk commits tokens with the target's own
conditional distributions, and the branch draw follows softmax(prior / T)."""
import numpy as np
import pytest

from oracle import oracle


def binom_ok(count, n, p, sig=5.0):
    return abs(count - n * p) <= sig * np.sqrt(n * p * (1 - p)) + 1


def test_uniforms_are_uniform_and_inside_the_unit_interval():
    rng = np.random.default_rng(0)
    us = np.array([oracle.uniform_at(int(rng.integers(2 ** 32)), int(rng.integers(1000)),
                                     int(rng.integers(1000)), int(rng.integers(200000)))
                   for _ in range(40000)])
    assert (us > 0).all() and (us < 1).all()
    hist = np.histogram(us, bins=20, range=(0, 1))[0]
    assert all(binom_ok(c, len(us), 1 / 20) for c in hist)
    # the same counter gives the same number; a neighbouring token another
    assert oracle.uniform_at(7, 3, 2, 11) == oracle.uniform_at(7, 3, 2, 11)
    assert oracle.uniform_at(7, 3, 2, 11) != oracle.uniform_at(7, 3, 2, 12)


@pytest.mark.parametrize("T", [0.7, 1.0, 1.5])
def test_gumbel_max_draws_follow_the_tempered_softmax(T):
    l = np.array([1.0, 0.2, -0.5, 1.3, 0.0], np.float32)
    n = 30000
    logits = np.broadcast_to(l, (n, 1, 5)).copy()
    s, _ = oracle.sample_nodes(logits, np.zeros(n, np.int32), T, seed=1234)
    p = np.exp(l.astype(np.float64) / T)
    p /= p.sum()
    counts = np.bincount(s[:, 0], minlength=5)
    assert all(binom_ok(counts[v], n, p[v]) for v in range(5)), (counts / n, p)


def test_zero_temperature_is_the_argmax_and_padding_is_untouched():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((4, 6, 50)).astype(np.float32)
    logits[:, :, 7] = logits[:, :, 9] = 10.0                # ties: the smaller token
    nn = np.array([5, 2, 0, 3], np.int32)
    s, sc = oracle.sample_nodes(logits, nn, 0.0, seed=9)
    for q in range(4):
        assert (s[q, :nn[q] + 1] == 7).all() and (s[q, nn[q] + 1:] == -1).all()
        assert (sc[q, :nn[q] + 1] == 10.0).all()


def test_target_sampling_walk_commits_the_targets_conditionals():
    """Root with children of tokens 0 and 2 (V = 3), child 1 (token 0) with
    a child of token 1.  The first committed token is the root's draw; given
    it is 0 (a child), the second is that child's draw."""
    V, T, n = 3, 1.2, 30000
    parent = np.array([-1, 0, 0, 1], np.int32)
    token = np.array([-1, 0, 2, 1], np.int32)
    rows = np.array([[0.3, -0.2, 0.5], [-1.0, 0.8, 0.1], [0.0, 0.0, 0.0], [0.2, 0.2, 0.9]],
                    np.float32)
    logits = np.broadcast_to(rows, (n, 4, V)).copy()
    nn = np.full(n, 3, np.int32)
    s, _ = oracle.sample_nodes(logits, nn, T, seed=77)
    alen, anodes, bonus = oracle.accept(np.broadcast_to(parent, (n, 4)),
                                        np.broadcast_to(token, (n, 4)), nn, 2, s)
    first = np.where(alen >= 1, token[anodes[:, 1].clip(0)], bonus)
    p0 = np.exp(rows[0] / T)
    p0 /= p0.sum()
    c0 = np.bincount(first, minlength=V)
    assert all(binom_ok(c0[v], n, p0[v]) for v in range(V))
    took0 = first == 0
    second = np.where(alen[took0] >= 2, token[anodes[took0, 2].clip(0)], bonus[took0])
    p1 = np.exp(rows[1] / T)
    p1 /= p1.sum()
    c1 = np.bincount(second, minlength=V)
    assert all(binom_ok(c1[v], took0.sum(), p1[v]) for v in range(V))
    # a child whose token is the draw is always taken
    assert ((alen >= 1) == np.isin(s[:, 0], [0, 2])).all()


@pytest.mark.parametrize("T", [0.0, 0.5, 1.0, 40.0])
def test_branch_draw_follows_the_tempered_prior(T):
    K, b, M = 4, 3, 4000
    prior = np.array([[0.2, 1.1, -0.3, 1.1]], np.float32)
    u = (np.arange(M) + 0.5) / M                      # a grid of uniforms
    chains = np.arange(K * b, dtype=np.int32).reshape(1, K, b)
    z, draft = oracle.mixture_sample(np.repeat(prior, M, 0), T, u, np.repeat(chains, M, 0))
    counts = np.bincount(z, minlength=K) / M
    if T == 0.0:
        assert (z == 1).all()                          # argmax, ties to the smaller index
    else:
        w = np.exp(prior[0].astype(np.float64) / T)
        w /= w.sum()
        assert np.allclose(counts, w, atol=1.5 / M)
    assert (draft == chains[0][z]).all()
