"""Phase table of one call from the stamped build (per-block timestamps).

    python -m block_diffusion_tree_amd.build --stamps      # once, on the CPU
    python -m block_diffusion_tree_amd.stamps [--workload main] [--reps 5]

Runs the workload's call through libbastion_stamps.so (the same sources
compiled with -DBASTION_STAMPS), with cold inputs (four rotating batches),
and prints where the time of each call goes: when blocks start, when their
stream ends and their row is finished, per XCD and per dispatch quarter, and
for the tree (or mixture) stage of the query that finishes last, each
phase.  Times are microseconds of the GPU's 100 MHz real-time counter, from
the first block's start; the median over the calls is printed.
"""
from __future__ import annotations

import argparse
import ctypes as C
import os
import sys

import numpy as np

SLOTS = 16
TREE_PHASES = [(3, 4, "load rows' top-k and status"), (4, 5, "family bound"),
               (5, 6, "family select"), (6, 7, "rank (or pool / exact build)"),
               (7, 8, "A_hat, online stop"), (8, 9, "emission (tree, mask, positions)")]
# finer stamps inside the family bound, select and rank (slots 10-13; a
# query whose pool leaves the family skips some of them)
SUB_PHASES = [(4, 10, "bound: complete levels"), (10, 11, "bound: paths, histogram"),
              (11, 5, "bound: histogram scan"), (5, 12, "select: masks, path counts"),
              (12, 6, "select: slot writes"), (6, 13, "rank: counts"),
              (13, 7, "rank: parents, records")]


def run(workload: str, reps: int, split: int):
    import torch
    from block_diffusion_tree_amd import binding, build as hipbuild, synth
    if not os.path.exists(hipbuild.STAMPS_LIB):
        raise SystemExit(f"{hipbuild.STAMPS_LIB} is missing: python -m "
                         "block_diffusion_tree_amd.build --stamps")
    binding.use_library(hipbuild.STAMPS_LIB)
    L = binding.lib()
    L.bastion_debug_set_stamps.argtypes = [C.c_void_p]
    L.bastion_debug_set_stamps.restype = None
    binding.set_tuning(0, split)
    wl = synth.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    nbuf = 2 if wl.K > 1 else 4
    bufs = [synth.make_logits(wl, device=dev, seed=wl.seed + i) for i in range(nbuf)]
    cost = None
    if wl.online:
        c, _ = synth.make_cost_table(wl.B, wl.nmax, seed=wl.seed, **synth.LATENCY_A100)
        cost = torch.from_numpy(c).to(dev)
    if wl.K > 1:
        prior = synth.make_prior_logits(wl, device=dev)
        calls = [binding.prepare_mixture_score(x, prior, k=wl.k, nmax=wl.nmax)[2] for x in bufs]
    else:
        calls = [binding.prepare_build_trees(x, k=wl.k, nmax=wl.nmax, nmin=wl.nmin, cost=cost)[1]
                 for x in bufs]
    for i in range(2 * nbuf):
        calls[i % nbuf]()
    stamps = torch.zeros((1 << 17) * SLOTS, dtype=torch.int64, device=dev)
    tables = []
    for r in range(reps):
        stamps.zero_()
        torch.cuda.synchronize()
        L.bastion_debug_set_stamps(C.c_void_p(stamps.data_ptr()))
        calls[r % nbuf]()
        torch.cuda.synchronize()
        L.bastion_debug_set_stamps(None)
        tables.append(stamps.view(-1, SLOTS).cpu().numpy().astype(np.int64))
    binding.set_tuning(0, -1)
    return wl, tables


def analyse(wl, st):
    """Phase numbers (us) of one call's stamps."""
    started = st[:, 0] != 0
    nstream = int(np.argmin(started)) if not started.all() else len(st)
    s = st[:nstream]
    t0 = s[:, 0].min()
    us = lambda v: (v.astype(np.float64) - t0) / 100.0   # 100 MHz counter
    out = {}
    out["blocks"] = nstream
    out["start"] = us(s[:, 0])
    out["stream_end"] = us(s[:, 1])
    # a row split over several blocks is finished by the last of them only
    done = s[:, 2] != 0
    out["row_done"] = us(s[done, 2])
    xcc = (s[:, 14] & 0xF)[done]
    out["xcc_p50"] = {int(x): float(np.median(out["row_done"][xcc == x])) for x in np.unique(xcc)}
    q4 = ((np.arange(nstream) * 4) // nstream)[done]
    out["quarter_p50"] = [float(np.median(out["row_done"][q4 == i])) if (q4 == i).any()
                          else float("nan") for i in range(4)]
    out["last_row_done"] = float(out["row_done"].max())
    out["merge_gap"] = float(out["row_done"].max() - out["stream_end"].max())
    # tree stages: in the stream blocks (slot 3 set there) or in the second launch
    second = st[nstream:]
    second = second[second[:, 3] != 0]
    trees = s[s[:, 3] != 0] if (s[:, 3] != 0).any() else second
    end_slot = 9
    last = trees[np.argmax(trees[:, end_slot])]
    out["kernel_end"] = float(us(trees[:, end_slot]).max())
    out["last_tree"] = {name: float((last[b] - last[a]) / 100.0)
                        for a, b, name in TREE_PHASES + SUB_PHASES if last[a] and last[b]}
    out["last_tree_start"] = float(us(np.array([last[3]]))[0])
    out["tree_total_p50"] = float(np.median((trees[:, end_slot] - trees[:, 3]) / 100.0))
    # per-phase medians over every tree
    out["phase_p50"] = {}
    for a, b, name in TREE_PHASES + SUB_PHASES:
        ok = (trees[:, a] != 0) & (trees[:, b] != 0)
        if ok.any():
            out["phase_p50"][name] = float(np.median((trees[ok, b] - trees[ok, a]) / 100.0))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="main")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--split", type=int, default=-1, help="bastion_set_tuning split_trees")
    args = ap.parse_args()
    wl, tables = run(args.workload, args.reps, args.split)
    res = [analyse(wl, t) for t in tables]
    med = lambda f: float(np.median([f(r) for r in res]))
    pct = lambda key, p: med(lambda r: np.percentile(r[key], p))
    print(f"# stamps: workload {args.workload}, {res[0]['blocks']} stream blocks, "
          f"median of {len(res)} cold calls (us from the first block's start)\n")
    print("| phase | us |\n|---|---|")
    print(f"| block start min / p50 / max | {pct('start', 0):.1f} / {pct('start', 50):.1f} / "
          f"{pct('start', 100):.1f} |")
    print(f"| stream end min / p50 / max | {pct('stream_end', 0):.1f} / "
          f"{pct('stream_end', 50):.1f} / {pct('stream_end', 100):.1f} |")
    print(f"| row finished min / p50 / max | {pct('row_done', 0):.1f} / "
          f"{pct('row_done', 50):.1f} / {pct('row_done', 100):.1f} |")
    xs = sorted(res[0]["xcc_p50"])
    print("| row finished p50 by XCD | " +
          " / ".join(f"{med(lambda r, x=x: r['xcc_p50'].get(x, np.nan)):.1f}" for x in xs) + " |")
    print("| row finished p50 by dispatch quarter | " +
          " / ".join(f"{med(lambda r, i=i: r['quarter_p50'][i]):.1f}" for i in range(4)) + " |")
    print(f"| last row finished after the last stream end | {med(lambda r: r['merge_gap']):.1f} |")
    print(f"| tree stage of the last query: start | {med(lambda r: r['last_tree_start']):.1f} |")
    for _, _, name in TREE_PHASES + SUB_PHASES:
        v = med(lambda r, n=name: r["last_tree"].get(n, np.nan))
        print(f"| ... {name} | {v:.2f} |")
    print(f"| tree stage duration, p50 over queries | {med(lambda r: r['tree_total_p50']):.1f} |")
    for _, _, name in TREE_PHASES + SUB_PHASES:
        v = med(lambda r, n=name: r["phase_p50"].get(n, np.nan))
        print(f"| ... p50 over queries: {name} | {v:.2f} |")

    print(f"| last tree done (kernel end) | {med(lambda r: r['kernel_end']):.1f} |")
    sys.stdout.flush()


if __name__ == "__main__":
    main()
