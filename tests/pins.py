"""Independent second definitions used to pin the CPU reference.

Nothing here calls the reference or the HIP library.  Each helper computes
the same quantity by a different route: exhaustive enumeration, a sort of the
whole candidate tree with a recursive order, a transitive closure, or a
brute-force search over paths.
"""
from __future__ import annotations

import functools
import itertools

import numpy as np


def f32mul(a, b):
    return np.float32(np.float32(a) * np.float32(b))


def candidate_tree(ids, q, depth_limit=None):
    """All nodes of the full candidate tree of one query.

    ids, q: [b, k].  Returns a list of dicts with path (tuple of ranks),
    tokens (tuple), rho (float32, one rounding per factor), depth.
    """
    b, k = ids.shape
    depth_limit = b if depth_limit is None else depth_limit
    nodes = []
    level = [((), (), np.float32(1.0))]
    for d in range(depth_limit):
        nxt = []
        for path, toks, rho in level:
            for j in range(k):
                r = f32mul(rho, q[d, j])
                node = (path + (j,), toks + (int(ids[d, j]),), r)
                nxt.append(node)
                nodes.append(dict(path=node[0], tokens=node[1], rho=node[2], depth=d + 1))
        level = nxt
    return nodes


def sorted_candidates(ids, q, depth_limit=None):
    """Whole candidate tree sorted by (rho desc, depth asc, token asc,
    then the parents compared by this same order)."""
    nodes = candidate_tree(ids, q, depth_limit)
    by_path = {n["path"]: n for n in nodes}

    def cmp(a, b):
        if a["rho"] != b["rho"]:
            return -1 if a["rho"] > b["rho"] else 1
        if a["depth"] != b["depth"]:
            return -1 if a["depth"] < b["depth"] else 1
        if a["tokens"][-1] != b["tokens"][-1]:
            return -1 if a["tokens"][-1] < b["tokens"][-1] else 1
        pa, pb = a["path"][:-1], b["path"][:-1]
        if pa == pb:
            return 0
        if len(pa) == 0:
            return -1
        if len(pb) == 0:
            return 1
        return cmp(by_path[pa], by_path[pb])

    return sorted(nodes, key=functools.cmp_to_key(cmp))


def max_subtree_sum(ids, q, N):
    """max over prefix-closed subtrees with exactly N non-root nodes of the
    sum of rho (float64 sum of the float32 rho), by exhaustive enumeration.
    Returns (max, number of subtrees enumerated)."""
    b, k = ids.shape
    rho_of = {}

    def children(path):
        d = len(path)
        if d >= b:
            return []
        out = []
        for j in range(k):
            c = path + (j,)
            if c not in rho_of:
                rho_of[c] = f32mul(rho_of[path], q[d, j])
            out.append(c)
        return out

    rho_of[()] = np.float32(1.0)
    best = [-1.0]
    count = [0]

    def rec(total, frontier, remaining):
        if remaining == 0:
            count[0] += 1
            if total > best[0]:
                best[0] = total
            return
        for idx in range(len(frontier)):
            node = frontier[idx]
            rec(total + float(rho_of[node]), frontier[idx + 1:] + children(node),
                remaining - 1)

    rec(1.0, children(()), N)
    return best[0], count[0]


def closure_mask(parent, n):
    """Reflexive-transitive closure of the child->parent relation (Warshall)."""
    m = n + 1
    A = np.eye(m, dtype=bool)
    for i in range(1, m):
        p = int(parent[i])
        A[i, p] = True
    for kk in range(m):
        A = A | (A[:, [kk]] & A[[kk], :])
    return A


def accept_brute(parent, token, n, target, b):
    """Deepest node whose whole root path matches the targets."""
    best = (0, [0])
    for i in range(n + 1):
        path = [i]
        while path[-1] != 0:
            path.append(int(parent[path[-1]]))
        path = path[::-1]
        ok = all(int(token[v]) == int(target[u]) for u, v in zip(path[:-1], path[1:]))
        if ok and len(path) - 1 > best[0]:
            best = (len(path) - 1, path)
    length, path = best
    return length, path, int(target[path[-1]])


def enumerate_sequences(V, b):
    return np.array(list(itertools.product(range(V), repeat=b)), dtype=np.int32)


def fmaf_exact(a, b, c):
    """float32 fused multiply-add: a*b + c rounded once, to nearest even."""
    from fractions import Fraction
    v = Fraction(float(np.float32(a))) * Fraction(float(np.float32(b))) + Fraction(float(np.float32(c)))
    f = np.float32(float(v))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - v)
        even = (int(np.array(cand, np.float32).view(np.uint32)) & 1) == 0
        key = (err, not even)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])
