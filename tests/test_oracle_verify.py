"""Pins of the reference tree attention (oracle/verify_oracle.py): bf16
rounding against torch's conversion, the rotary embedding's identities,
and the masked attention against torch's scaled-dot-product attention with
a mask built independently by walking parent links."""
import math

import numpy as np
import pytest
import torch

from oracle import verify_oracle as vo


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 0.0]])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(vo.bf16_round(x.astype(np.float64)), want)


def test_rotation_identities():
    rng = np.random.default_rng(1)
    D = 16
    x = rng.standard_normal((5, D))
    inv = np.array([2.0 ** -j for j in range(D // 2)], np.float32)   # exact fp32 angles
    # position 0 is the identity
    assert np.array_equal(vo.rotate(x, np.zeros(5, np.int64), inv, round_bf16=False), x)
    # every pair keeps its norm
    y = vo.rotate(x, np.arange(5) * 37, inv, round_bf16=False)
    n = lambda a: a[:, :D // 2] ** 2 + a[:, D // 2:] ** 2
    assert np.allclose(n(y), n(x), rtol=1e-13)
    # scores depend on the position difference only
    q, k = x[0], x[1]
    for m, nn, sh in ((3, 11, 100), (0, 7, 4096), (50, 2, 333)):
        a = vo.rotate(q, m, inv, False) @ vo.rotate(k, nn, inv, False)
        b = vo.rotate(q, m + sh, inv, False) @ vo.rotate(k, nn + sh, inv, False)
        assert a == pytest.approx(b, rel=1e-12, abs=1e-12)
    # a quarter turn maps (x1, x2) to (-x2, x1)
    qt = vo.rotate(np.array([1.0, 2.0]), 1, np.array([math.pi / 2], np.float32), False)
    assert np.allclose(qt, [-2.0, 1.0], atol=1e-7)


def make_case(rng, S, T, Hq, Hkv, Lmax, ctx, parents, D=128):
    """Random bf16-valued inputs; parents[s][i] (i >= 1) the tree's links."""
    C = (Hq + 2 * Hkv) * D
    qkv = vo.bf16_round(rng.standard_normal((S * T, C)))
    kc = vo.bf16_round(rng.standard_normal((S, Hkv, Lmax, D)))
    vc = vo.bf16_round(rng.standard_normal((S, Hkv, D, Lmax)))
    W = (T + 31) // 32
    mask = np.zeros((S, T, W), np.uint32)
    pos = np.zeros((S, T), np.int32)
    for s in range(S):
        for i in range(T):
            j, depth = i, 0
            mask[s, i, j // 32] |= np.uint32(1 << (j % 32))
            while j > 0:
                j = parents[s][j]
                mask[s, i, j // 32] |= np.uint32(1 << (j % 32))
                depth += 1
            pos[s, i] = ctx[s] + depth
    inv = (1.0e6 ** (-2.0 * np.arange(D // 2) / D)).astype(np.float32)
    return qkv, kc, vc, np.array(ctx, np.int32), pos, mask, inv


def sdpa_reference(qkv, S, T, Hq, Hkv, kc, vc, ctx, pos, parents, inv, D=128):
    """The same layer through torch's scaled_dot_product_attention (float64),
    with the visibility mask built from the parent links."""
    G = Hq // Hkv
    outs = []
    for s in range(S):
        c = int(ctx[s])
        rows = qkv[s * T:(s + 1) * T]
        q = vo.rotate(rows[:, :Hq * D].reshape(T, Hq, D), pos[s][:, None], inv)
        k = vo.rotate(rows[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D), pos[s][:, None], inv)
        v = rows[:, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(T, Hkv, D)
        K = np.concatenate([kc[s][:, :c, :].transpose(1, 0, 2), k], axis=0)    # [c+T, Hkv, D]
        V = np.concatenate([vc[s][:, :, :c].transpose(2, 0, 1), v], axis=0)
        allow = np.zeros((T, c + T), bool)
        allow[:, :c] = True
        for i in range(T):
            j = i
            allow[i, c + j] = True
            while j > 0:
                j = parents[s][j]
                allow[i, c + j] = True
        qt = torch.from_numpy(q.transpose(1, 0, 2))[None]                      # [1, Hq, T, D]
        kt = torch.from_numpy(K.transpose(1, 0, 2)).repeat_interleave(G, 0)[None]
        vt = torch.from_numpy(V.transpose(1, 0, 2)).repeat_interleave(G, 0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(allow)[None, None], scale=1.0 / math.sqrt(D))
        outs.append(o[0].permute(1, 0, 2).reshape(T, Hq * D).numpy())
    return np.concatenate(outs, axis=0)


@pytest.mark.parametrize("S,T,Hq,Hkv,ctx", [(2, 7, 4, 2, [5, 0]), (1, 9, 4, 1, [12]),
                                             (2, 5, 2, 2, [0, 3])])
def test_tree_attention_equals_sdpa_with_ancestor_mask(S, T, Hq, Hkv, ctx):
    rng = np.random.default_rng(S * 100 + T)
    Lmax = 32
    parents = [[-1] + [int(rng.integers(0, i)) for i in range(1, T)] for _ in range(S)]
    qkv, kc, vc, ctxa, pos, mask, inv = make_case(rng, S, T, Hq, Hkv, Lmax, ctx, parents)
    out, kc2, vc2 = vo.tree_attention(qkv, S, T, Hq, Hkv, 128, kc, vc, ctxa, pos, mask, inv)
    ref = sdpa_reference(qkv, S, T, Hq, Hkv, kc, vc, ctxa, pos, parents, inv)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # the tree tokens' v landed in their slots unchanged
    for s in range(S):
        for t in range(T):
            assert np.array_equal(vc2[s, :, :, ctx[s] + t],
                                  qkv[s * T + t, (Hq + Hkv) * 128:].reshape(Hkv, 128))


def test_single_visible_key_and_uniform_scores():
    rng = np.random.default_rng(3)
    S, T, Hq, Hkv, Lmax = 1, 3, 2, 1, 16
    parents = [[-1, 0, 1]]
    qkv, kc, vc, ctx, pos, mask, inv = make_case(rng, S, T, Hq, Hkv, Lmax, [0], parents)
    out, _, _ = vo.tree_attention(qkv, S, T, Hq, Hkv, 128, kc, vc, ctx, pos, mask, inv)
    v_root = qkv[0, (Hq + Hkv) * 128:(Hq + 2 * Hkv) * 128]
    # the root sees itself only: its output is its own v, exactly
    assert np.array_equal(out[0, :128], v_root) and np.array_equal(out[0, 128:], v_root)
    # zero queries give every visible key the same weight: the mean of v
    qkv2 = qkv.copy()
    qkv2[:, :Hq * 128] = 0.0
    ctx5 = np.array([5], np.int32)
    qkv2_, kc5, vc5, _, pos5, mask5, _ = make_case(rng, S, T, Hq, Hkv, Lmax, [5], parents)
    qkv2_[:, :Hq * 128] = 0.0
    out2, _, vcx = vo.tree_attention(qkv2_, S, T, Hq, Hkv, 128, kc5, vc5, ctx5, pos5, mask5, inv)
    want = vcx[0, 0][:, :5 + 3].mean(axis=1)   # token 2 sees the 5 cached and all 3 tree tokens
    assert np.allclose(out2[2, :128], want, rtol=1e-13, atol=1e-15)


def test_context_is_clamped_to_the_cache():
    rng = np.random.default_rng(4)
    S, T, Hq, Hkv, Lmax = 1, 4, 2, 1, 8
    parents = [[-1, 0, 0, 1]]
    qkv, kc, vc, _, pos, mask, inv = make_case(rng, S, T, Hq, Hkv, Lmax, [4], parents)
    a, _, _ = vo.tree_attention(qkv, S, T, Hq, Hkv, 128, kc, vc, np.array([100], np.int32), pos,
                                mask, inv)
    b, _, _ = vo.tree_attention(qkv, S, T, Hq, Hkv, 128, kc, vc, np.array([4], np.int32), pos,
                                mask, inv)
    assert np.array_equal(a, b)
