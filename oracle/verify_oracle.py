"""Plain CPU reference of the tree's consumer: one attention layer of a
tree-structured verifier, in float64 with numpy.

TEST INFRASTRUCTURE ONLY: imported by the tests and by nothing in the
product path; it imports nothing from the HIP library or its binding.

Source: "Bastion: Budget-Aware Speculative Decoding with Tree-structured
Block Diffusion Drafting", gist.science, Experimental results (the target
verifies the drafted tree in one forward pass) and Methodology 3 (that
pass's latency is what the budget controller weighs).  The pages fix no
attention formulation; this is grouped-query attention with rotary position
embedding (rotate-half pairs (d, d + D/2)) and softmax scaled by 1/sqrt(D),
the formulation of the pages' target models, written out step by step:

  1. rotary embedding of each tree token's q and k at its position id: the
     angle of pair d is the float32 product fl(pos * inv_freq[d]); the pair
     (x_d, x_{d+D/2}) becomes (x_d cos - x_{d+D/2} sin, x_{d+D/2} cos + x_d sin)
     in float64, rounded once to bf16 (round to nearest even);
  2. the rotated k and the v of the tree tokens go into cache slots
     ctx .. ctx+T-1, ctx = ctx_len clamped to [0, Lmax - T];
  3. tree token i attends to cached tokens 0 .. ctx-1 and to tree token j iff
     bit j of its ancestor-mask row is set: softmax over those keys of
     (q . k) / sqrt(D), in float64;
  4. the output of query head h is sum_j p_j v_j, with v from KV head
     h // (Hq / Hkv).
"""
from __future__ import annotations

import numpy as np


def bf16_round(x):
    """float64 -> nearest bf16 value (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    scaled = m * 256.0                 # 8 significant bits
    r = np.round(scaled)               # numpy rounds halves to even
    return np.ldexp(r / 256.0, e)


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rotate(x, pos, inv_freq, round_bf16=True):
    """Rotary embedding of x [..., D] at integer positions pos [...] (step 1)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = np.asarray(inv_freq, dtype=np.float32)
    ang = (np.asarray(pos, dtype=np.float32)[..., None] * inv).astype(np.float64)  # fl32 product
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    y = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return bf16_round(y) if round_bf16 else y


def tree_attention(qkv, S, T, Hq, Hkv, D, k_cache, v_cache, ctx_len, position_ids, mask,
                   inv_freq):
    """qkv [S*T, >= (Hq+2Hkv)D] float64 (bf16 values); k_cache [S,Hkv,Lmax,D] and
    v_cache [S,Hkv,D,Lmax] float64 with the cached slots filled.  Returns
    (out [S*T, Hq*D] float64, k_cache, v_cache after the tree tokens are
    appended)."""
    G = Hq // Hkv
    Lmax = k_cache.shape[2]
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    out = np.zeros((S * T, Hq * D), np.float64)
    scale = 1.0 / np.sqrt(D)
    for s in range(S):
        ctx = int(min(max(int(ctx_len[s]), 0), Lmax - T))
        rows = qkv[s * T:(s + 1) * T]
        pos = np.asarray(position_ids[s])
        q = rotate(rows[:, :Hq * D].reshape(T, Hq, D), pos[:, None], inv_freq)
        k = rotate(rows[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D), pos[:, None], inv_freq)
        v = rows[:, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(T, Hkv, D)
        for t in range(T):
            kc[s, :, ctx + t, :] = k[t]
            vc[s, :, :, ctx + t] = v[t]
        for t in range(T):
            # visible keys: every cached slot, then the tree tokens the mask row marks
            tree_vis = [j for j in range(T) if (int(mask[s][t][j // 32]) >> (j % 32)) & 1]
            keys = list(range(ctx)) + [ctx + j for j in tree_vis]
            for hq in range(Hq):
                h = hq // G
                K = kc[s, h, keys, :]             # [n, D]
                V = vc[s, h][:, keys].T           # [n, D]
                sc = (K @ q[t, hq]) * scale
                p = np.exp(sc - sc.max())
                p /= p.sum()
                out[s * T + t, hq * D:(hq + 1) * D] = p @ V
    return out, kc, vc
