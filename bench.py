"""Benchmark of the tree-drafting hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload main]

A step is one bastion_build_trees call (softmax + top-k over the vocabulary,
best-first tree with A_hat, mask and position ids) over one batch of
synthetic logits that is already resident in HBM.  Four distinct input
batches rotate so that no step finds its logits in the 256 MB MALL.  With
--workload mixture a step is one bastion_mixture_score call (branch rows,
chains and q_dep, candidate unions, mixture tree with mask) over two
rotating 5 GB batches.

Prints one JSON line.  `value` is trees per second over the timed steps.
`roofline` is the fused kernel's algorithmic bytes per launch (every logit
read once plus every output written once) over its mean launch time: the
span of HIP events recorded on the kernel's stream before and after the K
back-to-back calls of the timed region, over K (a call of the mixture is its
two launches: the stream kernel and the per-query stage).  Single-call
times (mean, p10 / p50 / p90) come from a second pass with events around
each call; those events add the command processor's gap between packets.
`cpu_baseline` times the CPU reference on the same batch (host copy).
`in_flight` is the rate with two batches in flight (consecutive calls on
two streams, each with its own workspace and outputs): a call's last trees
then overlap the next call's stream, which a serving loop with two
independent batches gets; `value` stays the one-call-at-a-time rate.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

WORKLOAD_TEXT = {
    "main": "B=64 queries x b=16 positions x V=151936 bf16 logits, k=8, fixed N=64",
    "sweep": "B=256 x b=16 x V=128256 fp32 logits, k=4, online stop over N<=256",
    "sweep_peaks": "B=256 x b=16 x V=128256 fp32 logits with the main workload's peaked rows "
                   "(row max + U(2,10)), k=4, online stop over N<=256",
    "latency": "B=1 x b=16 x V=151936 bf16 logits, k=16, online stop over N<=128",
    "tiny": "B=1 x b=4 x V=1024 fp32 logits, k=4, fixed N=32",
    "mixture": "B=128 queries x K=8 branches x b=16 x V=151936 bf16 logits, k=8, mixture tree N=64",
    "verify": "one attention layer of the verify pass over the main workload's 64 trees (N=64, "
              "T=65 tree tokens each): 32 query / 8 KV heads of 128, bf16 KV cache, contexts "
              "U[512, 8192]",
}
HBM_PEAK_GBS = 8000.0
N_BUFFERS = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="main", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--cost", default="a100", choices=["a100", "mi355x", "calibrated"],
                    help="verify-latency table of the online workloads: the roofline with the "
                         "pages' GPU's constants (default), MI355X's published ones, or the "
                         "constants fitted to this verifier's measured runtimes")
    ap.add_argument("--candidates", default="union", choices=["union", "marginal"],
                    help="mixture workload: candidates from the union of the branches' top-k "
                         "(bastion_mixture_score) or the top-k of the mixture marginal "
                         "(bastion_mixture_marginal, a second pass over the branch rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the warm-input, accept, streaming-ceiling and two-in-flight timings "
                         "(profiling runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain device-to-device copy of this many MiB "
                         "(the reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "profiles", "traffic.json"))
    return ap.parse_args()


# the sources the tree and mixture launches are built from (kernels, their
# headers and the launch plan); counter readings taken on other versions of
# them are stale
TREE_PATH_SOURCES = ["api.hip", "api_internal.hpp", "build_trees.hip", "build_params.hpp",
                     "device_common.hpp", "mixture.hpp", "tree_family.hpp", "tree_pool.hpp",
                     "tree_rounds.hpp"]


def kernel_source_hash() -> str:
    """Hash of the tree path's HIP sources and its header."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(root, "block_diffusion_tree_amd", "csrc")
    files = [os.path.join(csrc, f) for f in TREE_PATH_SOURCES]
    files.append(os.path.join(root, "include", "bastion.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def out_bytes(out) -> int:
    return int(sum(t.numel() * t.element_size() for t in out.values()))


def _oracle_pass(sample, wl, cost=None):
    from oracle import oracle
    import numpy as np
    rows = oracle.softmax_topk(sample, k=wl.k)
    tree = oracle.best_first(rows["topk_ids"], rows["topk_p"].astype(np.float32),
                             nmax=wl.nmax, nmin=wl.nmin,
                             cost=None if cost is None else cost[:sample.shape[0]],
                             row_status=rows["row_status"])
    oracle.tree_mask(tree["parent"], tree["n_nodes"])
    return rows


def _timed(fn, min_seconds, max_reps):
    import numpy as np
    times, res = [], None
    while len(times) < max_reps and (sum(times) < min_seconds or len(times) < 2):
        t0 = time.perf_counter()
        res = fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times), res


def cpu_baseline(x_host, wl, n_queries, cost=None, min_seconds=2.0, max_reps=10, n_single=4):
    """The CPU reference on the first n_queries queries of the batch with all
    host threads, repeated until at least min_seconds of wall time (the
    median pass is reported), and on the first n_single queries with one
    thread."""
    from oracle import oracle
    n_single = min(n_single, n_queries)
    threads = oracle.num_threads()
    dt, reps, rows = _timed(lambda: _oracle_pass(x_host[:n_queries], wl, cost), min_seconds,
                            max_reps)
    oracle.set_num_threads(1)
    try:
        dt1, reps1, _ = _timed(lambda: _oracle_pass(x_host[:n_single], wl, cost), 0.5, 3)
    finally:
        oracle.set_num_threads(threads)
    return dict(value=n_queries / dt, unit="trees/s", cores=threads, kind="oracle",
                sample=f"first {n_queries} of {wl.B} queries of the timed batch "
                       f"({n_queries * wl.b} rows): float64 softmax + top-k, best-first tree, "
                       f"mask; median of {reps} passes, {dt:.3f} s per pass",
                single_thread_value=n_single / dt1,
                single_thread_sample=f"first {n_single} queries, one thread: median of "
                                     f"{reps1} passes, {dt1:.3f} s per pass"), rows


def cpu_baseline_mixture(x, prior, wl, mout, n_queries, min_seconds=2.0, max_reps=10,
                         n_single=1):
    """The CPU reference of the mixture call on the first n_queries queries
    (all host threads) and on the first n_single (one thread)."""
    from oracle import oracle
    import numpy as np
    xs = oracle.host_logits(x[:n_queries])
    ps = prior[:n_queries].cpu().numpy()

    def one(n):
        m = oracle.mixture(xs[:n], ps[:n], k=wl.k)
        oracle.mixture_tree(m["prior_w"].astype(np.float32), m["cand_count"], m["cand_tokens"],
                            m["cand_p"].astype(np.float32), nmax=wl.nmax,
                            row_status=m["row_status"])
        return m
    threads = oracle.num_threads()
    dt, reps, m = _timed(lambda: one(n_queries), min_seconds, max_reps)
    oracle.set_num_threads(1)
    try:
        dt1, reps1, _ = _timed(lambda: one(n_single), 0.5, 2)
    finally:
        oracle.set_num_threads(threads)
    ok = bool((mout["chain_tokens"][:n_queries].cpu().numpy() == m["chain_tokens"]).all())
    return dict(value=n_queries / dt, unit="trees/s", cores=threads, kind="oracle",
                sample=f"first {n_queries} of {wl.B} queries of the timed batch "
                       f"({n_queries * wl.K * wl.b} branch rows): float64 softmax + top-k, "
                       f"chains and q_dep, candidate unions, mixture tree; median of "
                       f"{reps} passes, {dt:.3f} s per pass",
                single_thread_value=n_single / dt1,
                single_thread_sample=f"first {n_single} queries, one thread: median of "
                                     f"{reps1} passes, {dt1:.3f} s per pass"), ok


def cpu_baseline_marginal(x, prior, wl, n_queries, min_seconds=2.0, max_reps=10):
    """The CPU reference of the marginal rule (candidates and the mixture
    tree) on the first n_queries queries, all host threads."""
    from oracle import oracle
    import numpy as np
    xs = oracle.host_logits(x[:n_queries])
    ps = prior[:n_queries].cpu().numpy()

    def one():
        m = oracle.mixture_marginal(xs, ps, wl.k)
        cnt = np.full((n_queries, wl.b), wl.k, np.int32)
        oracle.mixture_tree(m["prior_w"].astype(np.float32), cnt, m["marg_ids"],
                            m["cand_p"].astype(np.float32), nmax=wl.nmax,
                            row_status=m["row_status"])
    dt, reps, _ = _timed(one, min_seconds, max_reps)
    return dict(value=n_queries / dt, unit="trees/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"first {n_queries} of {wl.B} queries of the timed batch: float64 mixture "
                       f"marginal over every token, its top-k, mixture tree; median of {reps} "
                       f"passes, {dt:.3f} s per pass")


def stream_ceiling(bufs, dev, reps=20):
    """The practical HBM read rate: a plain streaming-read kernel
    (libbastion_probe.so) over the same input buffers, rotating like the
    timed steps, for a few grid sizes; the best rate in GB/s and its grid."""
    import ctypes as C
    import torch
    from block_diffusion_tree_amd import build as hipbuild
    if not os.path.exists(hipbuild.PROBE_LIB):
        return None
    L = C.CDLL(hipbuild.PROBE_LIB)
    L.bastion_probe_stream_read.restype = C.c_int32
    L.bastion_probe_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p,
                                            C.c_void_p]
    nbytes = bufs[0].numel() * bufs[0].element_size()
    nbytes -= nbytes % 16
    stream = torch.cuda.current_stream()
    sp = C.c_void_p(stream.cuda_stream)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        def go(i):
            st = L.bastion_probe_stream_read(C.c_void_p(bufs[i % len(bufs)].data_ptr()), nbytes,
                                             blocks, C.c_void_p(sink.data_ptr()), sp)
            if st != 0:
                raise RuntimeError(f"stream probe failed ({st})")
        for i in range(3):
            go(i)
        # timed like the steps: one pair of events around reps back-to-back launches
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            go(i)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        gbs = nbytes / (us * 1e-6) / 1e9
        if best is None or gbs > best["gbs"]:
            best = dict(gbs=gbs, us=us, blocks=blocks, bytes=nbytes)
    return best


def time_span(fn, n, stream):
    """One pair of HIP events around n back-to-back calls of fn(i) on
    `stream`: the mean time per call in ms."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def time_launches(fn, n, stream):
    """HIP events around each of n calls of fn(i) on `stream`: times in ms."""
    import numpy as np
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def verify_bytes_flops(vw, ctx):
    """Algorithmic bytes and flops of one tree_attention call: every cached
    and tree key's k and v read once, the qkv rows read once, the output and
    the tree tokens' cache slots written once; q.k and p.v over every visible
    or masked key of a sequence's last chunk alike (4 Hq D T (ctx + T))."""
    import numpy as np
    keys = np.minimum(np.maximum(ctx.astype(np.int64), 0), vw.lmax - vw.T) + vw.T
    kv = 2 * vw.Hkv * vw.D * 2                      # bytes of one key's k and v
    rows = vw.S * vw.T
    nbytes = int(kv * keys.sum() + rows * (vw.Hq + 2 * vw.Hkv) * vw.D * 2
                 + rows * vw.Hq * vw.D * 2 + rows * kv)
    flops = float(4 * vw.Hq * vw.D * vw.T * keys.sum())
    return nbytes, flops


def cpu_baseline_verify(qkv, kc, vc, ctx, pos, mask, inv, vw, out, budget_s=10.0, max_seq=16):
    """The CPU reference on a bounded sample (sequences in order of their
    context length, shortest first, until about budget_s seconds of CPU time
    or max_seq sequences), with a parity check of the GPU output on them."""
    import numpy as np
    import torch
    from oracle import verify_oracle as vo
    order = []
    secs, ok, worst = 0.0, True, 0.0
    T, D = vw.T, vw.D
    for s in np.argsort(ctx, kind="stable"):
        if secs >= budget_s or len(order) >= max_seq:
            break
        order.append(int(s))
        s = int(s)
        rows = qkv[s * T:(s + 1) * T].double().cpu().numpy()
        kcs = kc[s:s + 1].double().cpu().numpy()
        vcs = vc[s:s + 1].permute(0, 1, 3, 2, 4).reshape(1, vw.Hkv, D, vw.lmax).double().cpu().numpy()
        t0 = time.perf_counter()
        ref, _, _ = vo.tree_attention(rows, 1, T, vw.Hq, vw.Hkv, D, kcs, vcs, ctx[s:s + 1],
                                      pos[s:s + 1], mask[s:s + 1], inv)
        secs += time.perf_counter() - t0
        got = out[s * T:(s + 1) * T].double().cpu().numpy()
        vmax = max(np.abs(rows[:, (vw.Hq + vw.Hkv) * D:]).max(), np.abs(vcs).max())
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * vmax + 2.0 ** -8 * np.abs(ref)
        ok = ok and bool((err <= bound).all())
        worst = max(worst, float((err / bound).max()))
    threads = torch.get_num_threads()
    n_seq = len(order)
    return ({"value": n_seq / secs, "unit": "sequences/s (one attention layer)",
             "cores": threads, "kind": "oracle",
             "sample": f"{n_seq} of {vw.S} sequences, the shortest contexts "
                       f"({int(ctx[order[0]])}..{int(ctx[order[-1]])} cached tokens, mean "
                       f"{float(np.mean(ctx)):.0f} over all 64), float64 numpy; {secs:.1f} s"},
            {"sequences": [int(i) for i in order], "within_tolerance": ok,
             "max_err_over_bound": worst})


def main_verify(args):
    """--workload verify: a step is one bastion_tree_attention call (cache
    append, attention, split combine) over the 64 trees that
    bastion_build_trees makes of one main-workload batch."""
    import numpy as np
    import torch
    from block_diffusion_tree_amd import binding, synth
    vw = synth.VERIFY_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()
    wl = synth.WORKLOADS["main"]
    assert wl.B == vw.S and wl.nmax + 1 == vw.T
    ctx_np = synth.make_verify_contexts(vw)
    ctx = torch.from_numpy(ctx_np).to(dev)
    x = synth.make_logits(wl, device=dev)
    trees = binding.build_trees(x, k=wl.k, nmax=wl.nmax, pos_base=ctx)
    mask, pos = trees["mask"], trees["position_ids"]
    del x
    qkv, kc, vc = synth.make_verify_tensors(vw, device=dev)
    inv = binding.rope_inv_freq(1.0e6, vw.D, dev)
    out, call = binding.prepare_tree_attention(qkv, vw.S, vw.T, vw.Hq, vw.Hkv, kc, vc, ctx, pos,
                                               mask, inv, max_ctx=vw.ctx_hi)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(args.steps):
        call()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = time_launches(lambda i: call(), args.steps, stream)
    nbytes, flops = verify_bytes_flops(vw, ctx_np)
    mean_ms = e_start.elapsed_time(e_end) / args.steps
    achieved = nbytes / (mean_ms * 1e-3) / 1e9
    line = {
        "metric": "tree-attention layer: verified trees/sec + achieved HBM GB/s, S=64 T=65, 1 MI355X",
        "value": vw.S / (ms_per_step * 1e-3),
        "unit": "trees/s (one attention layer)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}",
                   "lmax": vw.lmax, "mean_ctx": float(ctx_np.mean())},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "append_kernel + attention_kernel + combine_kernel: the launches "
                               "of one bastion_tree_attention call, timed together",
                     "alg_bytes_per_launch": nbytes,
                     "launch_us_mean": mean_ms * 1e3,
                     "launch_timing": "events around the K back-to-back calls of the timed "
                                      "region; single-call figures from a second pass with "
                                      "events around each call",
                     "single_call_us_mean": float(launch_ms.mean()) * 1e3,
                     "single_call_us_p50": float(np.median(launch_ms)) * 1e3,
                     "mfma": {"flops_per_launch": flops,
                              "achieved_tflops": flops / (mean_ms * 1e-3) / 1e12,
                              "peak_tflops": 2500.0,
                              "frac": flops / (mean_ms * 1e-3) / 2.5e15}},
    }
    if not args.no_cpu_baseline:
        base, par = cpu_baseline_verify(qkv, kc, vc, ctx_np, pos.cpu().numpy(),
                                        mask.cpu().numpy().view(np.uint32),
                                        inv.cpu().numpy(), vw, out)
        line["cpu_baseline"] = base
        line["parity_sample"] = par
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the path shards over queries with no exchange, so N GPUs run N copies.",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "verify":
        main_verify(args)
        return
    import numpy as np
    import torch
    from block_diffusion_tree_amd import binding, synth

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()
    mixture = wl.K > 1
    nbuf = 2 if mixture else N_BUFFERS
    bufs = [synth.make_logits(wl, device=dev, seed=wl.seed + i) for i in range(nbuf)]
    cost = None
    if wl.online:
        if args.cost == "calibrated":
            from block_diffusion_tree_amd import calibrate
            c, _ = calibrate.calibrated_cost_table(wl.B, wl.nmax, seed=wl.seed)
        else:
            consts = synth.LATENCY_A100 if args.cost == "a100" else synth.LATENCY_MI355X
            c, _ = synth.make_cost_table(wl.B, wl.nmax, seed=wl.seed, **consts)
        cost = torch.from_numpy(c).to(dev)
    ws = binding.Workspace(dev)
    marginal = mixture and args.candidates == "marginal"
    if mixture:
        prior = synth.make_prior_logits(wl, device=dev)
        alloc = binding.alloc_marginal_out if marginal else binding.alloc_mixture_out
        mouts = [alloc(wl.B, wl.K, wl.b, wl.k, dev) for _ in range(nbuf)]
        outs = [binding.alloc_tree_out(wl.B, wl.b, wl.k, wl.nmax, dev, with_rows=False)
                for _ in range(nbuf)]
    else:
        outs = [binding.alloc_tree_out(wl.B, wl.b, wl.k, wl.nmax, dev) for _ in range(nbuf)]

    # one C call per step, its arguments marshalled once per input buffer (a
    # caller looping over fixed buffers does the same), so that the host keeps
    # ahead of the GPU and the events time the GPU work
    if mixture:
        prep = binding.prepare_mixture_marginal if marginal else binding.prepare_mixture_score
        calls = [prep(bufs[j], prior, k=wl.k, nmax=wl.nmax, out=mouts[j], tree=outs[j], ws=ws)[2]
                 for j in range(nbuf)]
    else:
        calls = [binding.prepare_build_trees(bufs[j], k=wl.k, nmax=wl.nmax, nmin=wl.nmin, cost=cost,
                                             out=outs[j], ws=ws)[1] for j in range(nbuf)]

    def step(i):
        calls[i % nbuf]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed region: K calls back to back, one pair of HIP events on the
    # stream around them (an event record between calls is a packet of its
    # own for the command processor and would add its gap to every step)
    stream = torch.cuda.current_stream()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(i)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span_ms = e_start.elapsed_time(e_end)
    # the spread of single calls: a second pass with events around each call
    launch_ms = time_launches(step, args.steps, stream)

    extras = {}
    if not args.no_extras:
        # warm: the same input batch every call (what the MALL keeps of it)
        nw = max(10, args.steps // 2)
        warm_mean = time_span(lambda i: calls[0](), nw, stream)
        warm_ms = time_launches(lambda i: calls[0](), nw, stream)
        extras["warm"] = {"launch_us_mean": warm_mean * 1e3,
                          "single_call_us_p50": float(np.median(warm_ms)) * 1e3,
                          "single_call_us_p10": float(np.percentile(warm_ms, 10)) * 1e3,
                          "single_call_us_p90": float(np.percentile(warm_ms, 90)) * 1e3}
        if not mixture:
            # bastion_accept on the trees of buffer 0, timed on its own
            o = outs[0]
            top1 = o["topk_ids"][:, :, 0].cpu().numpy()
            tgt = synth.make_targets(o["parent"].cpu().numpy(), o["token"].cpu().numpy(),
                                     o["depth"].cpu().numpy(), o["n_nodes"].cpu().numpy(),
                                     top1, wl.V, seed=wl.seed)
            tgt = torch.from_numpy(tgt).to(dev)
            acc_ms = time_launches(lambda i: binding.accept(o["parent"], o["token"], o["n_nodes"],
                                                            wl.b, tgt), 30, stream)
            alen = binding.accept(o["parent"], o["token"], o["n_nodes"], wl.b, tgt)[0]
            extras["accept"] = {"launch_us_mean": float(acc_ms.mean()) * 1e3,
                                "launch_us_p50": float(np.median(acc_ms)) * 1e3,
                                "mean_accept_len": float(alen.float().mean())}
        extras["ceiling"] = stream_ceiling(bufs, dev)
        # two batches in flight: consecutive calls alternate between two
        # streams, each with its own workspace and outputs, so that one
        # call's tail (its last trees) overlaps the next call's stream
        s2 = torch.cuda.Stream(device=dev)
        ws2 = binding.Workspace(dev)
        with torch.cuda.stream(s2):
            if mixture:
                mouts2 = [alloc(wl.B, wl.K, wl.b, wl.k, dev) for _ in range(nbuf)]
                outs2 = [binding.alloc_tree_out(wl.B, wl.b, wl.k, wl.nmax, dev, with_rows=False)
                         for _ in range(nbuf)]
                calls2 = [prep(bufs[j], prior, k=wl.k, nmax=wl.nmax, out=mouts2[j], tree=outs2[j],
                               ws=ws2)[2] for j in range(nbuf)]
            else:
                outs2 = [binding.alloc_tree_out(wl.B, wl.b, wl.k, wl.nmax, dev) for _ in range(nbuf)]
                calls2 = [binding.prepare_build_trees(bufs[j], k=wl.k, nmax=wl.nmax, nmin=wl.nmin,
                                                      cost=cost, out=outs2[j], ws=ws2)[1]
                          for j in range(nbuf)]
        pair = (calls, calls2)
        for i in range(2 * nbuf):
            pair[i % 2][i % nbuf]()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            pair[i % 2][i % nbuf]()
        torch.cuda.synchronize()
        fl_us = (time.perf_counter() - t1) * 1e6 / args.steps
        # stream 2 ran on the odd buffers: its outputs must equal the serial ones
        same = all(torch.equal(outs2[j][f], outs[j][f]) for j in range(1, nbuf, 2)
                   for f in ("parent", "token", "rho", "n_nodes"))
        extras["in_flight"] = {"batches": 2, "us_per_step": fl_us,
                               "trees_per_s": wl.B / (fl_us * 1e-6),
                               "outputs_match_serial": bool(same)}

    ms_per_step = wall * 1e3 / args.steps
    # the marginal rule reads every branch logit twice: its ranking needs
    # each row's normaliser first
    alg_bytes = wl.logit_bytes * (2 if marginal else 1) + out_bytes(outs[0])
    if mixture:
        alg_bytes += out_bytes(mouts[0]) + prior.numel() * 4
    mean_ms = span_ms / args.steps
    achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        rec = json.load(open(args.traffic_json)).get(args.workload)
        if rec and rec.get("kernel_source_hash") == kernel_source_hash():
            traffic = rec["traffic_bytes"]
    line = {
        "metric": "draft trees/sec + achieved HBM GB/s, B=64 b=16 V=151936 N<=64, 1 MI355X",
        "value": wl.B / (ms_per_step * 1e-3),
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}",
                   "logits_dtype": wl.dtype, "rotating_buffers": nbuf,
                   **({"cost_table": args.cost} if wl.online else {}),
                   **({"candidates": args.candidates} if mixture else {})},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": ("build_trees_kernel (mixture mode) + mixture_kernel: the two launches "
                                "of one call, timed together" if mixture else
                                "build_trees_kernel, plus tree_kernel when the call builds its trees "
                                "in a launch of their own; the call's launches timed together"),
                     "alg_bytes_per_launch": alg_bytes,
                     "launch_us_mean": mean_ms * 1e3,
                     "launch_timing": "events around the K back-to-back calls of the timed "
                                      "region; the single-call figures below from a second "
                                      "pass with events around each call",
                     "single_call_us_mean": float(launch_ms.mean()) * 1e3,
                     "single_call_us_p50": float(np.median(launch_ms)) * 1e3,
                     "single_call_us_p10": float(np.percentile(launch_ms, 10)) * 1e3,
                     "single_call_us_p90": float(np.percentile(launch_ms, 90)) * 1e3},
    }
    if mixture:
        # A_hat of the emitted trees (the rules' expected committed tokens)
        nn = outs[0]["n_nodes"].long()
        ah = outs[0]["ahat"].gather(1, nn.view(-1, 1)).view(-1)
        line["ahat_at_n"] = {"mean": float(ah.mean()), "min": float(ah.min()),
                             "max": float(ah.max())}
    if wl.online:
        nst = outs[0]["n_nodes"].cpu().numpy()
        line["n_star"] = {"min": int(nst.min()), "p50": float(np.median(nst)),
                          "max": int(nst.max()), "mean": float(nst.mean())}
    ceil = extras.get("ceiling")
    if ceil:
        line["roofline"]["ceiling"] = {
            "achieved_read_gbs": ceil["gbs"], "grid_blocks": ceil["blocks"],
            "kernel": "stream_read_chunks (libbastion_probe.so): the same input buffers read "
                      "once with the same 16-byte loads and nothing else",
            "frac_of_ceiling": achieved / ceil["gbs"]}
    if "warm" in extras:
        w = extras["warm"]
        w["achieved_gbs"] = alg_bytes / (w["launch_us_mean"] * 1e-6) / 1e9
        line["warm"] = w
    if "accept" in extras:
        line["accept"] = extras["accept"]
    if "in_flight" in extras:
        f = extras["in_flight"]
        f["achieved_gbs"] = alg_bytes / (f["us_per_step"] * 1e-6) / 1e9
        f["frac_of_peak"] = f["achieved_gbs"] / HBM_PEAK_GBS
        line["in_flight"] = f
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = n
    if not args.no_cpu_baseline:
        from oracle import oracle
        if marginal:
            base = cpu_baseline_marginal(bufs[0], prior, wl, n_queries=2)
            line["cpu_baseline"] = base
        elif mixture:
            base, ok = cpu_baseline_mixture(bufs[0], prior, wl, mouts[0], n_queries=2)
            line["cpu_baseline"] = base
            line["parity_sample"] = {"queries": 2, "chain_tokens_exact": ok}
        else:
            x_host = oracle.host_logits(bufs[0])
            n_q = wl.B
            base, rows = cpu_baseline(x_host, wl, n_q,
                                      cost=None if cost is None else cost.cpu().numpy())
            line["cpu_baseline"] = base
            # the timed GPU outputs of buffer 0 agree with the reference sample
            g_ids = outs[0]["topk_ids"][:n_q].cpu().numpy()
            line["parity_sample"] = {"queries": n_q,
                                     "topk_ids_exact": bool((g_ids == rows["topk_ids"]).all())}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
