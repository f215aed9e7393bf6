"""Pins of the reference's budget controller, mask/positions and greedy
acceptance."""
import numpy as np
import pytest

import pins
from test_oracle_tree import tree_inputs


def test_budget_hand_example(oracle_mod):
    # S = A*L/C = [1, 1.5833, 1.8, 1.5]: first strict decrease after n = 2
    ahat = np.array([[1.0, 1.9, 2.7, 3.0]])
    cost = np.array([1.0, 1.2, 1.5, 2.0])
    nstar, s = oracle_mod.budget_select(ahat, [3], nmin=1, cost=cost)
    assert nstar.tolist() == [2]
    assert s[0].tolist() == pytest.approx([1.0, 1.9 / 1.2, 1.8, 1.5], rel=1e-15)
    nstar, _ = oracle_mod.budget_select(ahat, [3], nmin=3, cost=cost)
    assert nstar.tolist() == [3]


def test_budget_plateau_continues(oracle_mod):
    # "until S starts to decrease": equal S is not a decrease, so the rule
    # runs to the end of a plateau (the largest maximiser of S).
    ahat = np.array([[1.0, 2.0, 3.0, 3.5, 3.6]])
    cost = np.array([1.0, 2.0, 3.0, 3.5, 4.0])
    nstar, s = oracle_mod.budget_select(ahat, [4], nmin=1, cost=cost)
    assert s[0, :4].tolist() == [1.0, 1.0, 1.0, 1.0]
    assert nstar.tolist() == [3]


def test_constant_cost_never_stops_early(oracle_mod):
    rng = np.random.default_rng(0)
    ids, q = tree_inputs(rng, 4, 5, 3)
    nmax = 50
    cost = np.full(nmax + 1, 2.5e-3)
    t = oracle_mod.best_first(ids, q, nmax=nmax, nmin=1, cost=cost)
    assert t["n_nodes"].tolist() == [nmax] * 4


def test_zero_mass_stops_at_nmin(oracle_mod):
    ids = np.arange(2 * 4 * 3, dtype=np.int32).reshape(2, 4, 3)
    q = np.zeros((2, 4, 3), np.float32)
    cost = 1.0 + np.arange(31, dtype=np.float64)      # increasing latency
    for nmin in (0, 1, 5):
        t = oracle_mod.best_first(ids, q, nmax=30, nmin=nmin, cost=cost)
        assert t["n_nodes"].tolist() == [nmin, nmin]


def test_online_stop_is_largest_argmax(oracle_mod):
    """A_hat is concave and non-decreasing, C is convex and increasing, so
    S = A_hat/C rises then falls: the first strict decrease is the largest
    maximiser of S."""
    from block_diffusion_tree_amd import synth
    rng = np.random.default_rng(1)
    B, b, k, nmax = 24, 16, 4, 256
    for style in ("flat", "peaked"):
        if style == "flat":
            ids, q = tree_inputs(rng, B, b, k)
        else:
            ids, q = tree_inputs(rng, B, b, k)
            q[:, :, 0] = np.float32(0.9) + q[:, :, 0] * np.float32(0.09)
        for consts in (synth.LATENCY_A100, synth.LATENCY_MI355X):
            cost, _ = synth.make_cost_table(B, nmax, seed=5, **consts)
            full = oracle_mod.best_first(ids, q, nmax=nmax)
            online = oracle_mod.best_first(ids, q, nmax=nmax, nmin=1, cost=cost)
            for qq in range(B):
                n_av = int(full["n_nodes"][qq])
                S = full["ahat"][qq, :n_av + 1] / cost[qq, :n_av + 1]
                cand = np.arange(1, n_av + 1)
                smax = S[1:].max()
                largest = int(cand[S[1:] == smax].max())
                assert int(online["n_nodes"][qq]) == largest
                # the online tree is the prefix of the full one
                n = largest
                assert (online["token"][qq, :n + 1] == full["token"][qq, :n + 1]).all()


def test_mask_is_transitive_closure(oracle_mod):
    rng = np.random.default_rng(2)
    ids, q = tree_inputs(rng, 5, 6, 3)
    for nmax in (1, 31, 32, 33, 70):
        t = oracle_mod.best_first(ids, q, nmax=nmax)
        pos_base = rng.integers(0, 5000, size=5).astype(np.int32)
        mask, pos = oracle_mod.tree_mask(t["parent"], t["n_nodes"], pos_base)
        W = (nmax + 1 + 31) // 32
        assert mask.shape == (5, nmax + 1, W)
        for qq in range(5):
            n = int(t["n_nodes"][qq])
            A = pins.closure_mask(t["parent"][qq], n)
            bits = np.unpackbits(mask[qq].view(np.uint8), bitorder="little", axis=1)
            bits = bits[:, :nmax + 1].astype(bool)
            assert (bits[:n + 1, :n + 1] == A).all()
            assert not bits[:n + 1, n + 1:].any()
            assert not bits[n + 1:].any()
            assert (bits[:n + 1].sum(axis=1) == t["depth"][qq, :n + 1] + 1).all()
            assert (pos[qq, :n + 1] == pos_base[qq] + t["depth"][qq, :n + 1]).all()
            assert (pos[qq, n + 1:] == -1).all()


def test_mask_stops_at_malformed_links(oracle_mod):
    parent = np.array([[-1, 0, 5, 1, 7]], np.int32)   # node 2 -> 5 is not a parent
    mask, pos = oracle_mod.tree_mask(parent, [4])
    rows = mask[0, :, 0].tolist()
    assert rows == [0b1, 0b11, 0b100, 0b1011, 0b10000]
    assert pos[0].tolist() == [0, 1, 0, 2, 0]


def test_accept_matches_brute_force(oracle_mod):
    rng = np.random.default_rng(3)
    b, k, nmax = 5, 3, 40
    ids, q = tree_inputs(rng, 30, b, k, ties=True)
    t = oracle_mod.best_first(ids, q, nmax=nmax)
    # targets: mostly follow existing children so that long accepts occur
    target = np.zeros((30, nmax + 1), np.int32)
    for qq in range(30):
        for i in range(nmax + 1):
            kids = [j for j in range(1, nmax + 1) if t["parent"][qq, j] == i]
            if kids and rng.random() < 0.8:
                target[qq, i] = t["token"][qq, rng.choice(kids)]
            else:
                target[qq, i] = rng.integers(0, 1000)
    alen, anodes, bonus = oracle_mod.accept(t["parent"], t["token"], t["n_nodes"], b, target)
    for qq in range(30):
        L, path, bon = pins.accept_brute(t["parent"][qq], t["token"][qq],
                                         int(t["n_nodes"][qq]), target[qq], b)
        assert alen[qq] == L
        assert anodes[qq, :L + 1].tolist() == path
        assert (anodes[qq, L + 1:] == -1).all()
        assert bonus[qq] == bon
    assert alen.max() >= 3


def test_accept_degenerate(oracle_mod):
    parent = np.array([[-1, 0, 1, -1]], np.int32)
    token = np.array([[-1, 7, 8, -1]], np.int32)
    # no match at the root
    alen, anodes, bonus = oracle_mod.accept(parent, token, [2], 4, np.array([[3, 8, 9, 0]]))
    assert alen.tolist() == [0] and anodes[0].tolist() == [0, -1, -1, -1, -1]
    assert bonus.tolist() == [3]
    # full chain then bonus
    alen, anodes, bonus = oracle_mod.accept(parent, token, [2], 4, np.array([[7, 8, 9, 0]]))
    assert alen.tolist() == [2] and anodes[0, :3].tolist() == [0, 1, 2] and bonus.tolist() == [9]
    # empty tree (a bad query): only the root
    alen, _, bonus = oracle_mod.accept(parent, token, [0], 4, np.array([[7, 8, 9, 0]]))
    assert alen.tolist() == [0] and bonus.tolist() == [7]
