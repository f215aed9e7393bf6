"""Pins of the reference's softmax and top-k against closed forms, special
cases, invariants and an independent sort (np.lexsort)."""
import math

import numpy as np
import pytest


def rows_f32(*rows):
    return np.array(rows, dtype=np.float32)


def test_sum_to_one_and_ratio_closed_form(oracle_mod):
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((5, 64)) * 4).astype(np.float32)
    r = oracle_mod.softmax_topk(x, k=64)
    p = r["topk_p"]
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    # p_i / p_j = exp(l_i - l_j) for any two tokens
    for row in range(5):
        ids = r["topk_ids"][row]
        li = x[row, ids].astype(np.float64)
        ratio = p[row, :-1] / p[row, 1:]
        assert np.allclose(ratio, np.exp(li[:-1] - li[1:]), rtol=1e-12, atol=0)


def test_two_token_sigmoid(oracle_mod):
    x = rows_f32([0.25, -1.5], [3.0, 3.0], [-7.0, 2.0])
    r = oracle_mod.softmax_topk(x, k=2)
    for row in range(3):
        a, b = float(x[row, 0]), float(x[row, 1])
        p0 = 1.0 / (1.0 + math.exp(b - a))
        got = dict(zip(r["topk_ids"][row].tolist(), r["topk_p"][row].tolist()))
        assert got[0] == pytest.approx(p0, rel=1e-14)
        assert got[1] == pytest.approx(1.0 - p0, rel=1e-13)


def test_log_linear_row_closed_form(oracle_mod):
    # l_v = log(v+1): M = log(V), S = sum (v+1)/V = (V+1)/2, p_v = 2(v+1)/(V(V+1))
    V = 50
    x = np.log(np.arange(1, V + 1, dtype=np.float64)).astype(np.float32)[None, :]
    r = oracle_mod.softmax_topk(x, k=3)
    xl = x.astype(np.float64)[0]
    M = xl.max()
    assert r["row_max"][0] == M
    assert r["row_sum"][0] == pytest.approx(np.exp(xl - M).sum(), rel=1e-14)
    assert r["row_sum"][0] == pytest.approx((V + 1) / 2.0, rel=1e-6)   # float32 logs
    assert r["topk_ids"][0].tolist() == [V - 1, V - 2, V - 3]
    assert r["topk_p"][0][0] == pytest.approx(2.0 * V / (V * (V + 1)), rel=1e-6)


def test_one_finite_entry_is_certain(oracle_mod):
    x = np.full((1, 33), -np.inf, dtype=np.float32)
    x[0, 20] = 3.5
    r = oracle_mod.softmax_topk(x, k=3)
    assert r["row_status"][0] == oracle_mod.OK
    assert r["topk_ids"][0].tolist() == [20, 0, 1]     # -inf ties by id
    assert r["topk_p"][0].tolist() == [1.0, 0.0, 0.0]


def test_uniform_and_shift_invariance(oracle_mod):
    V = 1000
    x = np.zeros((1, V), np.float32)
    r = oracle_mod.softmax_topk(x, k=4)
    assert r["topk_ids"][0].tolist() == [0, 1, 2, 3]
    assert np.allclose(r["topk_p"][0], 1.0 / V, rtol=1e-14)
    rng = np.random.default_rng(1)
    y = rng.standard_normal((3, 300)).astype(np.float32)
    a = oracle_mod.softmax_topk(y, k=5)
    # large logits: without the max subtraction exp() would overflow
    b = oracle_mod.softmax_topk(y + np.float32(1000.0), k=5)
    assert (a["topk_ids"] == b["topk_ids"]).all()
    assert np.allclose(a["topk_p"], b["topk_p"], rtol=2e-4)   # float32 re-rounding of y+1000


def test_topk_matches_lexsort_with_ties(oracle_mod):
    rng = np.random.default_rng(2)
    x = rng.integers(-3, 4, size=(40, 97)).astype(np.float32)   # many exact ties
    for k in (1, 4, 8, 32):
        r = oracle_mod.softmax_topk(x, k=k)
        for row in range(x.shape[0]):
            ids = np.arange(x.shape[1])
            ref = np.lexsort((ids, -x[row].astype(np.float64)))[:k]
            assert r["topk_ids"][row].tolist() == ref.tolist()


def test_bf16_decode(oracle_mod):
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x4049 = 3.140625, 0xFF80 = -inf
    bits = np.array([[0x3F80, 0xC000, 0x4049, 0xFF80]], dtype=np.uint16)
    r = oracle_mod.softmax_topk(bits, k=4)
    assert r["row_max"][0] == 3.140625
    assert r["topk_ids"][0].tolist() == [2, 0, 1, 3]
    xs = np.array([1.0, -2.0, 3.140625])
    S = np.exp(xs - 3.140625).sum()
    assert r["row_sum"][0] == pytest.approx(S, rel=1e-15)


@pytest.mark.parametrize("bad", ["nan", "posinf", "allneginf"])
def test_bad_rows(oracle_mod, bad):
    x = np.zeros((2, 16), np.float32)
    if bad == "nan":
        x[1, 3] = np.nan
    elif bad == "posinf":
        x[1, 3] = np.inf
    else:
        x[1, :] = -np.inf
    r = oracle_mod.softmax_topk(x, k=2)
    assert r["row_status"].tolist() == [0, 1]
    assert r["topk_ids"][1].tolist() == [-1, -1]


def test_large_logits_are_a_plain_softmax(oracle_mod):
    """Logits far from zero are valid input: the softmax only sees
    differences, so integer logits shifted by 2^21 or 2^23 (exact in float32)
    give the same ids and probabilities as the unshifted row."""
    rng = np.random.default_rng(9)
    y = rng.integers(-6, 7, size=(4, 50)).astype(np.float32)
    a = oracle_mod.softmax_topk(y, k=6)
    for shift in (2.0 ** 21, -(2.0 ** 21), 2.0 ** 23):
        r = oracle_mod.softmax_topk(y + np.float32(shift), k=6)
        assert (r["row_status"] == 0).all()
        assert (r["topk_ids"] == a["topk_ids"]).all()
        assert np.allclose(r["topk_p"], a["topk_p"], rtol=1e-13, atol=0)
        assert np.allclose(r["row_sum"], a["row_sum"], rtol=1e-13, atol=0)
