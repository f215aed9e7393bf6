"""Calibration of the verify-latency roofline on this GPU.

Bastion page (gist.science), Methodology 3: the budget controller stops the
tree where S(N) = A_hat(T_N) * L_AR / C(N) starts to fall, with C(N) the
latency of a step, from a roofline model of the verify pass that is
calibrated on observed runtimes (to absorb kernel fusion and scheduling
overheads); lay section 3: the controller measures how long this machine
takes to verify a tree of a given size.

Model (the latency form of the benchmark's budget sweep):

    T_verify(N) = max(bytes(N) / (eta_bw * BW), flops(N) / (eta_peak * PEAK)) + c0
    C(N)        = T_draft + T_verify(N)

with bytes(N) and flops(N) of the target shape (verifier.TargetShape),
BW = 8.0e12 B/s and PEAK = 2.5e15 bf16 FLOP/s (MI355X's published figures).
`measure` times verifier.VerifyPass graphs for a grid of N and context
lengths on the GPU; `fit` finds (eta_bw, eta_peak, c0) minimising the
squared relative error of the model over the measured points; `cost_table`
turns fitted constants into the C(n) table bastion_build_trees takes.

    python -m block_diffusion_tree_amd.calibrate [--out FILE]   # on a GPU
"""
from __future__ import annotations

import argparse
import json
import os
import time

import numpy as np

BW = 8.0e12          # B/s
PEAK = 2.5e15        # bf16 dense FLOP/s
N_GRID = (0, 1, 3, 7, 15, 31, 63, 127, 255, 511, 1023)
CTX_GRID = (512, 2048, 8192)


def model(eta_bw, eta_peak, c0, nbytes, nflops):
    """T_verify of the roofline model (seconds), elementwise."""
    return np.maximum(np.asarray(nbytes) / (eta_bw * BW), np.asarray(nflops) / (eta_peak * PEAK)) + c0


def _c0_for(eta_bw, eta_peak, nbytes, nflops, t):
    """The c0 >= 0 minimising sum(((roof + c0 - t) / t)^2) for fixed etas."""
    roof = model(eta_bw, eta_peak, 0.0, nbytes, nflops)
    w = 1.0 / np.asarray(t) ** 2
    c0 = float(np.sum(w * (t - roof)) / np.sum(w))
    return max(c0, 0.0)


def fit(nbytes, nflops, t, eta_max=1.0):
    """(eta_bw, eta_peak, c0) minimising the squared relative error of the
    model over measured points (bytes, flops, seconds), with both
    efficiencies in (0, eta_max] and c0 >= 0: a log-spaced grid over the
    efficiencies with c0 in closed form, then a local refinement.

    When the bytes hardly vary between points (a target whose weights
    dominate its KV cache), the memory term and c0 trade off against each
    other: only their sum is determined, and the fit keeps the largest
    efficiency that explains the points.  C(n) is determined either way."""
    nbytes, nflops, t = (np.asarray(a, dtype=np.float64) for a in (nbytes, nflops, t))

    def loss(eb, ep):
        c0 = _c0_for(eb, ep, nbytes, nflops, t)
        r = (model(eb, ep, c0, nbytes, nflops) - t) / t
        return float(np.sum(r * r)), c0

    best = None
    for eb in np.geomspace(0.02, eta_max, 121):
        for ep in np.geomspace(0.005, eta_max, 121):
            v, c0 = loss(eb, ep)
            if best is None or v < best[0]:
                best = (v, eb, ep, c0)
    _, eb, ep, _ = best
    step = 1.04
    for _ in range(200):
        improved = False
        for deb, dep in ((step, 1), (1 / step, 1), (1, step), (1, 1 / step)):
            if eb * deb > eta_max or ep * dep > eta_max:
                continue
            v, c0 = loss(eb * deb, ep * dep)
            if v < best[0] - 1e-15:
                best = (v, eb * deb, ep * dep, c0)
                eb, ep = eb * deb, ep * dep
                improved = True
        if not improved:
            step = step ** 0.5
            if step < 1.0 + 1e-6:
                break
    v, eb, ep, c0 = best
    rel = (model(eb, ep, c0, nbytes, nflops) - t) / t
    return dict(eta_bw=float(eb), eta_peak=float(ep), c0=float(c0),
                rms_rel_err=float(np.sqrt(np.mean(rel ** 2))), max_rel_err=float(np.abs(rel).max()))


def cost_table(shape, ctx, nmax, eta_bw, eta_peak, c0, t_draft=None):
    """C(n), n = 0..nmax, for contexts ctx [B] (seconds, float64 [B, nmax+1]).
    T_draft defaults to a tenth of the weight stream at the calibrated
    bandwidth (no drafter is timed here)."""
    ctx = np.atleast_1d(np.asarray(ctx, dtype=np.float64))
    n = np.arange(nmax + 1, dtype=np.float64)
    nb = np.array([[shape.bytes(int(k), int(c)) for k in n] for c in ctx])
    nf = np.array([[shape.flops(int(k), int(c)) for k in n] for c in ctx])
    if t_draft is None:
        t_draft = 0.1 * shape.weight_bytes() / (eta_bw * BW)
    return np.ascontiguousarray(t_draft + model(eta_bw, eta_peak, c0, nb, nf), dtype=np.float64)


STORED = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data",
                      "verify_calibration_mi355x.json")


def stored_fit(path: str = STORED) -> dict:
    """The constants fitted on an MI355X (eta_bw, eta_peak, c0, and the fit's
    errors), from the committed result of `python -m
    block_diffusion_tree_amd.calibrate`."""
    with open(path) as fh:
        return json.load(fh)["fit"]


def calibrated_cost_table(B: int, nmax: int, seed: int, fit_: dict = None,
                          ctx_lo: int = 512, ctx_hi: int = 8192):
    """C(n) of B queries with contexts drawn as in synth.make_cost_table
    (uniform on [ctx_lo, ctx_hi] from `seed`), from calibrated constants:
    ([B, nmax+1] float64 seconds, contexts)."""
    from block_diffusion_tree_amd.verifier import QWEN3_8B
    f = fit_ or stored_fit()
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=B)
    return cost_table(QWEN3_8B, ctx, nmax, f["eta_bw"], f["eta_peak"], f["c0"]), ctx


def random_tree(n, seed, device):
    """Parent links of a prefix-closed tree of n non-root nodes whose depth
    stays within a block of 16 positions (pop order: parent[i] < i)."""
    import torch
    rng = np.random.default_rng(seed)
    parent = np.full(n + 1, -1, np.int32)
    depth = np.zeros(n + 1, np.int32)
    for i in range(1, n + 1):
        while True:
            p = int(rng.integers(0, i))
            if depth[p] < 16:
                break
        parent[i] = p
        depth[i] = depth[p] + 1
    return torch.from_numpy(parent).to(device)


def measure(n_grid=N_GRID, ctx_grid=CTX_GRID, reps=10, check_replays=3, log=print):
    """Median graph-replay time of the verify pass for every (N, ctx)."""
    import torch
    from block_diffusion_tree_amd import verifier
    dev = torch.device("cuda:0")
    lmax = max(ctx_grid) + max(n_grid) + 1
    t0 = time.perf_counter()
    tgt = verifier.RandomTarget(lmax=lmax, device=dev)
    torch.cuda.synchronize()
    log(f"random target ready in {time.perf_counter() - t0:.1f} s")
    pts = []
    for ctx in ctx_grid:
        for n in n_grid:
            vp = verifier.VerifyPass(tgt, random_tree(n, seed=n + ctx, device=dev), ctx)
            ref = vp.eager().clone()
            vp.capture()
            # every replay (with eager work in between) gives the eager logits
            for _ in range(check_replays):
                got = vp.replay()
                torch.cuda.synchronize()
                if not torch.equal(got, ref):
                    raise RuntimeError(f"graph replay differs from the eager pass (N={n}, ctx={ctx})")
                _ = vp.eager()
                torch.cuda.synchronize()
            stream = torch.cuda.current_stream()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for a, b in ev:
                a.record(stream)
                vp.replay()
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            pts.append(dict(n=n, ctx=ctx, seconds=ms * 1e-3, bytes=tgt.shape.bytes(n, ctx),
                            flops=tgt.shape.flops(n, ctx)))
            log(f"N={n:5d} ctx={ctx:5d}: {ms:.3f} ms")
            del vp
    return tgt.shape, pts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="write the points and the fit as JSON")
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    shape, pts = measure(reps=args.reps, log=lambda s: print(s, flush=True))
    f = fit([p["bytes"] for p in pts], [p["flops"] for p in pts], [p["seconds"] for p in pts])
    res = dict(target="Qwen3-8B shape, random bf16 weights", bw=BW, peak=PEAK, fit=f, points=pts)
    print(json.dumps(f), flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            json.dump(res, fh, indent=1)


if __name__ == "__main__":
    main()
