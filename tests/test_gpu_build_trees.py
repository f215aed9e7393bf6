"""GPU parity of bastion_build_trees (and the standalone tree kernels) against
the CPU reference: exact top-k ids, trees, masks, positions and accepts;
q and row sums within 1e-5 relative; the tree stage fed the GPU's own q."""
import numpy as np
import pytest
import torch

from block_diffusion_tree_amd import binding, synth
from oracle import oracle
import gpu_common as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gc.require_gpu()
    yield
    binding.set_tuning(0, -1)


def test_tiny_workload_full_parity():
    wl = synth.WORKLOADS["tiny"]
    x = gc.device_logits(wl)
    g, ref = gc.run_and_check(x, wl.k, wl.nmax)
    assert int(g["n_nodes"][0]) == wl.nmax
    # diagnostic: with the reference's own float64 q (rounded to float32) the
    # tree is the same here, and A_hat agrees to 1e-5
    own = oracle.best_first(ref["topk_ids"], ref["topk_p"].astype(np.float32), nmax=wl.nmax)
    assert np.allclose(gc.np_(g["ahat"]), own["ahat"], rtol=1e-5)


@pytest.mark.parametrize("segments", ["1", "3", "17", "64"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_multi_segment(segments, dtype):
    binding.set_tuning(segments=int(segments))
    wl = synth.scaled(synth.WORKLOADS["main"], B=3, b=5, V=50003, dtype=dtype, nmax=40)
    x = gc.device_logits(wl, seed=7)
    gc.run_and_check(x, wl.k, wl.nmax)


def test_main_workload_full_parity():
    """The headline workload, in the launch configuration the benchmark uses."""
    wl = synth.WORKLOADS["main"]
    x = gc.device_logits(wl)
    g, ref = gc.run_and_check(x, wl.k, wl.nmax)
    assert (gc.np_(g["qstatus"]) == 0).all()
    # determinism: a second call is bitwise identical
    g2 = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    torch.cuda.synchronize()
    for f in g:
        assert torch.equal(g[f], g2[f]), f


def cost_table(B, nmax, seed, consts):
    if consts == "calibrated":
        # the verify-latency roofline fitted on an MI355X
        from block_diffusion_tree_amd import calibrate
        c, _ = calibrate.calibrated_cost_table(B, nmax, seed)
    else:
        c, _ = synth.make_cost_table(B, nmax, seed=seed, **consts)
    return torch.from_numpy(c).to("cuda")


@pytest.mark.parametrize("consts", [synth.LATENCY_A100, synth.LATENCY_MI355X, "calibrated"])
def test_online_budget_sweep_slice(consts):
    wl = synth.scaled(synth.WORKLOADS["sweep"], B=16)
    x = gc.device_logits(wl)
    cost = cost_table(wl.B, wl.nmax, wl.seed, consts)
    g, ref = gc.run_and_check(x, wl.k, wl.nmax, nmin=1, cost=cost, l_ar=1.0)
    # the same N* from a fixed-budget build followed by budget_select
    full = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    nstar, s = binding.budget_select(full["ahat"], full["n_nodes"], 1, cost)
    torch.cuda.synchronize()
    assert torch.equal(nstar, g["n_nodes"])
    rn, rs = oracle.budget_select(gc.np_(full["ahat"]), gc.np_(full["n_nodes"]), 1, gc.np_(cost))
    assert (gc.np_(nstar) == rn).all()
    assert np.array_equal(gc.np_(s), rs)


def test_latency_workload_online():
    wl = synth.WORKLOADS["latency"]
    x = gc.device_logits(wl)
    cost = cost_table(wl.B, wl.nmax, wl.seed, synth.LATENCY_A100)
    gc.run_and_check(x, wl.k, wl.nmax, nmin=1, cost=cost)


def test_sweep_logits_with_peaks_online():
    # config-2 style logits at the Llama vocabulary, where N* lands mid-range
    wl = synth.scaled(synth.WORKLOADS["main"], B=8, V=128256, dtype="f32", k=4, nmax=256,
                      seed=1003)
    x = gc.device_logits(wl)
    cost = cost_table(wl.B, wl.nmax, 5, synth.LATENCY_A100)
    g, _ = gc.run_and_check(x, wl.k, wl.nmax, nmin=1, cost=cost)
    n = gc.np_(g["n_nodes"])
    assert n.min() > 4 and n.max() < 256


@pytest.mark.parametrize("launch", ["stream", "own"])
def test_online_stop_around_the_first_stage(launch):
    """Cost tables shaped so that the stop falls before, on and after the
    32-node first stage of a budget-256 online build, or never; half of the
    rows add a small cost step after one node, large enough that the first
    stage cannot be ruled out in advance but too small to stop there.  The
    trees built in the stream launch and in their own launch."""
    binding.set_tuning(split_trees=1 if launch == "own" else 0)
    wl = synth.scaled(synth.WORKLOADS["main"], B=12, V=32000, nmax=256, seed=1011)
    x = gc.device_logits(wl)
    ref = oracle.softmax_topk(oracle.host_logits(x), k=wl.k)
    fixed = oracle.best_first(ref["topk_ids"], ref["topk_p"].astype(np.float32), nmax=wl.nmax)
    plan = [(1, False), (5, False), (30, False), (31, False), (32, False), (33, False),
            (100, False), (None, False), (5, True), (31, True), (33, True), (None, True)]
    cost = np.ones((wl.B, wl.nmax + 1))
    for r, (m, bump) in enumerate(plan):
        if bump:
            rho = fixed["rho"][r].astype(np.float64)
            # (1 + rho_1) * step lies between rho_32 and rho_2: no stop at
            # one node, while the stop test there is not ruled out by rho_32
            cost[r, 2:] += np.sqrt(rho[32] * rho[2]) / (1.0 + rho[1])
        if m is not None:
            cost[r, m + 1:] = 1.0e6
    g, _ = gc.run_and_check(x, wl.k, wl.nmax, nmin=1, cost=torch.from_numpy(cost).to("cuda"))
    want = [wl.nmax if m is None else m for m, _ in plan]
    assert gc.np_(g["n_nodes"]).tolist() == want


@pytest.mark.parametrize("nmin", [2, 31, 32, 33])
def test_online_stop_with_a_floor_near_the_first_stage(nmin):
    """The same stepped cost tables with nmin around the 32-node first stage
    of the trees' own launch, one table shared by every query in a second
    call: stops below nmin move up to the first allowed peak."""
    binding.set_tuning(split_trees=1)
    wl = synth.scaled(synth.WORKLOADS["main"], B=8, V=32000, nmax=256, seed=1012)
    x = gc.device_logits(wl)
    cost = np.ones((wl.B, wl.nmax + 1))
    for r, m in enumerate([1, 16, 30, 31, 32, 33, 60, None]):
        if m is not None:
            cost[r, m + 1:] = 1.0e6
    cost[::2, 2:] += 1.0e-3   # a small step after one node on every other query
    g, _ = gc.run_and_check(x, wl.k, wl.nmax, nmin=nmin, cost=torch.from_numpy(cost).to("cuda"))
    assert (gc.np_(g["n_nodes"]) >= min(nmin, wl.nmax)).all()
    shared = torch.from_numpy(cost[3]).to("cuda")
    gc.run_and_check(x, wl.k, wl.nmax, nmin=nmin, cost=shared)


def test_trees_in_their_own_launch():
    """Stream grids larger than the machine (here 1280 rows) build the trees
    in a launch of their own, with the online budget stop."""
    wl = synth.scaled(synth.WORKLOADS["sweep"], B=80, V=20000)
    x = gc.device_logits(wl)
    cost = cost_table(wl.B, wl.nmax, wl.seed, synth.LATENCY_A100)
    g, _ = gc.run_and_check(x, wl.k, wl.nmax, nmin=1, cost=cost, l_ar=1.0)
    g2 = binding.build_trees(x, k=wl.k, nmax=wl.nmax, cost=cost)
    torch.cuda.synchronize()
    for f in g:
        assert torch.equal(g[f], g2[f]), f


@pytest.mark.parametrize("name", ["sweep", "sweep_peaks"])
def test_sweep_full_workload_full_parity(name):
    """The whole budget-sweep workload in one call, as the benchmark launches
    it (4096 rows, trees in their own launch, online stop): every row against
    the reference's float64 softmax and top-k; every tree, mask and position
    against the reference fed the GPU's own q.  sweep_peaks: the same shape
    with peaked rows, whose stops fall deep in the budget."""
    wl = synth.WORKLOADS[name]
    x = synth.make_logits(wl, device="cuda")
    cost = cost_table(wl.B, wl.nmax, wl.seed, synth.LATENCY_A100)
    g = binding.build_trees(x, k=wl.k, nmax=wl.nmax, nmin=1, cost=cost, l_ar=1.0)
    torch.cuda.synchronize()
    ref = oracle.softmax_topk(oracle.host_logits(x), k=wl.k)
    gc.check_rows(g, ref)
    gc.check_tree(g, wl.b, wl.k, wl.nmax, 1, gc.np_(cost), 1.0, gc.expected_row_status(ref))
    gc.check_mask(g)
    n = gc.np_(g["n_nodes"])
    assert n.min() >= 1 and n.max() <= wl.nmax
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape", [
    dict(B=4, b=16, V=30011, k=8, nmax=64),        # 16 waves per tree
    dict(B=3, b=3, V=4099, k=32, nmax=200),        # widest candidate lists
    dict(B=2, b=32, V=777, k=2, nmax=1023),        # largest list: 8 waves per tree
])
def test_split_and_fused_trees_agree(shape):
    """The trees' own launch (more waves per tree) builds the same trees as
    the last row block of each query."""
    wl = synth.scaled(synth.WORKLOADS["main"], **shape)
    x = gc.device_logits(wl, seed=9)
    fused = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    binding.set_tuning(split_trees=1)
    try:
        split = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    finally:
        binding.set_tuning(0, -1)
    torch.cuda.synchronize()
    for f in fused:
        assert torch.equal(fused[f], split[f]), f


def test_bad_rows_and_padding():
    wl = synth.scaled(synth.WORKLOADS["tiny"], B=5, b=3, V=2000, nmax=12)
    x = synth.make_logits(wl)
    x[0, 1, 17] = float("nan")
    x[1, 2, 5] = float("inf")
    x[2, 0, :] = float("-inf")
    x[3, 1, 9] = 2.0 ** 21     # valid, but beyond the library's float32 range
    x[4, 2, 0] = -(2.0 ** 20)  # a large negative logit in an ordinary row
    g, ref = gc.run_and_check(x.to("cuda"), wl.k, wl.nmax)
    assert ref["row_status"][3, 1] == oracle.OK
    assert gc.np_(g["qstatus"]).tolist() == [1, 1, 1, binding.Q_RANGE, 0]
    assert gc.np_(g["n_nodes"]).tolist()[:4] == [0, 0, 0, 0]
    assert int(gc.np_(g["n_nodes"])[4]) == wl.nmax


def test_one_hot_rows_give_a_chain_then_zero_mass():
    B, b, V, k = 2, 4, 300, 3
    x = torch.full((B, b, V), float("-inf"))
    for q in range(B):
        for p in range(b):
            x[q, p, (7 * q + 11 * p) % V] = 1.5
    g, _ = gc.run_and_check(x.to("cuda"), k, 20)
    # the chain first (rho 1), then zero-rho nodes in (depth, token, parent) order
    assert gc.np_(g["rho"])[:, 1:5].tolist() == [[1.0] * 4] * 2


@pytest.mark.parametrize("shape", [
    dict(b=1, k=6, V=6, nmax=4),             # star, V == k, all in the scalar tail
    dict(b=5, k=1, V=5, nmax=10),            # greedy chain, exhausted
    dict(b=3, k=5, V=300, nmax=200),         # whole tree (155 nodes) below the budget
    dict(b=32, k=2, V=777, nmax=1023),       # deepest block, largest budget
    dict(b=3, k=32, V=4099, nmax=200),       # widest candidate lists
    dict(b=32, k=32, V=4099, nmax=512),      # deepest and widest: tree LDS above 64 KiB
])
def test_shapes_at_the_limits(shape):
    wl = synth.scaled(synth.WORKLOADS["tiny"], B=2, b=shape["b"], V=shape["V"], k=shape["k"],
                      nmax=shape["nmax"])
    x = gc.device_logits(wl, seed=11)
    g, _ = gc.run_and_check(x, wl.k, wl.nmax)


def test_integer_logits_many_ties():
    torch.manual_seed(3)
    x = torch.randint(-4, 5, (4, 6, 3001)).float().to(torch.bfloat16).to("cuda")
    gc.run_and_check(x, 8, 60)


def test_flat_rows_overflow_the_pool():
    """Equal logits: every node of a depth has the same rho, so a budget of
    100 with k = 8 reaches into the 512 depth-3 nodes and the candidate pool
    of the fast path (256 slots at this budget) overflows; the exact
    round-by-round build must produce the same tree."""
    x = torch.zeros((2, 4, 3001), dtype=torch.bfloat16, device="cuda")
    g, _ = gc.run_and_check(x, 8, 100)
    assert (gc.np_(g["depth"])[:, 1:9] == 1).all()


def test_near_flat_rows_fill_the_pool():
    """Small integer logits over few tokens: wide, tie-heavy levels that fit
    the pool (budget 120, 256 slots)."""
    torch.manual_seed(5)
    x = torch.randint(0, 2, (3, 5, 64)).float().to("cuda")
    gc.run_and_check(x, 6, 120)


def _deviations(g, q):
    """per tree node of query q: depth and number of positions on its path
    whose token is not that position's top-1 token"""
    par, tok, dep = (gc.np_(g[f])[q] for f in ("parent", "token", "depth"))
    top = gc.np_(g["topk_ids"])[q, :, 0]
    out = []
    for i in range(1, int(gc.np_(g["n_nodes"])[q]) + 1):
        n, j = 0, i
        while j > 0:
            n += int(tok[j] != top[dep[j] - 1])
            j = par[j]
        out.append((int(dep[i]), n))
    return out


def test_two_uncertain_positions_leave_the_family():
    """Two positions split evenly between two tokens, one inside the complete
    top levels (k = 4: depths 1-4) and one below them: the tree holds nodes
    that leave the top-1 path at both, which the family of one-deviation paths
    does not contain, so the pool comes from the level-by-level enumeration."""
    B, b, V = 2, 8, 512
    x = torch.full((B, b, V), -4.0)
    for p in range(b):
        x[:, p, 10 + p] = 8.0
    x[:, 1, 200] = 8.0
    x[:, 5, 300] = 8.0
    g, _ = gc.run_and_check(x.to("cuda"), 4, 32)
    assert any(d > 4 and n >= 2 for d, n in _deviations(g, 0))


def test_three_way_ties_below_the_top():
    """Three equal logits under a clear top token at two positions: the
    one-deviation paths through them tie at every later depth (same rho and
    token), and best-first orders them by the tokens where they split."""
    B, b, V = 3, 12, 1024
    torch.manual_seed(8)
    x = torch.randn((B, b, V)) * 0.3
    for p in range(b):
        x[:, p, 5 * p + 1] = 9.0
    for p in (3, 7):
        x[:, p, [700, 40, 333]] = 7.0
    g, _ = gc.run_and_check(x.to(torch.bfloat16).to("cuda"), 8, 64)
    par, rho, dep, tok = (gc.np_(g[f])[0] for f in ("parent", "rho", "depth", "token"))
    # the tree does contain nodes of equal (rho, depth, token) under different parents
    keys = {}
    for i in range(1, int(gc.np_(g["n_nodes"])[0]) + 1):
        keys.setdefault((float(rho[i]), int(dep[i]), int(tok[i])), set()).add(int(par[i]))
    assert max(len(v) for v in keys.values()) >= 3


def test_row_stride_padding_and_pos_base():
    wl = synth.scaled(synth.WORKLOADS["main"], B=2, b=4, V=1000, nmax=20)
    base = synth.make_logits(wl)
    padded = torch.zeros((2, 4, 1024), dtype=base.dtype)
    padded[:, :, :1000] = base
    xp = padded.to("cuda")[:, :, :1000]
    pos_base = torch.tensor([100, 7], dtype=torch.int32, device="cuda")
    g = binding.build_trees(xp, k=wl.k, nmax=wl.nmax, pos_base=pos_base)
    torch.cuda.synchronize()
    ref = oracle.softmax_topk(oracle.host_logits(base), k=wl.k)
    gc.check_rows(g, ref)
    gc.check_tree(g, 4, wl.k, wl.nmax, row_status=ref["row_status"])
    gc.check_mask(g, pos_base)


def test_calls_on_two_streams_match_the_serial_calls():
    """Two batches in flight: calls alternate between two streams, each with
    its own workspace and outputs (the benchmark's two-in-flight rate runs
    this); every output equals the one-call-at-a-time result."""
    wl = synth.scaled(synth.WORKLOADS["main"], B=16, V=32768)
    xs = [synth.make_logits(wl, device="cuda", seed=wl.seed + i) for i in range(4)]
    serial = [binding.build_trees(x, k=wl.k, nmax=wl.nmax) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [binding.Workspace(torch.device("cuda:0")) for _ in streams]
    outs, calls = [], []
    for i in range(8):
        with torch.cuda.stream(streams[i % 2]):
            o, c = binding.prepare_build_trees(xs[i % 4], k=wl.k, nmax=wl.nmax, ws=wss[i % 2])
        outs.append(o)
        calls.append(c)
    for c in calls:
        c()
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        ref = serial[i % 4]
        for f in ("topk_ids", "topk_q", "row_max", "row_sum", "parent", "depth", "token", "rho",
                  "ahat", "n_nodes", "qstatus", "mask", "position_ids"):
            assert torch.equal(o[f], ref[f]), (i, f)


def test_workspace_reuse_across_shapes():
    ws = binding.Workspace()
    a = synth.scaled(synth.WORKLOADS["main"], B=4, b=16, V=40000, nmax=30)
    bb = synth.scaled(synth.WORKLOADS["tiny"], B=9, b=4, V=3000, nmax=25)
    xa, xb = gc.device_logits(a), gc.device_logits(bb)
    ra = binding.build_trees(xa, k=a.k, nmax=a.nmax, ws=ws)
    rb = binding.build_trees(xb, k=bb.k, nmax=bb.nmax, ws=ws)
    ra2 = binding.build_trees(xa, k=a.k, nmax=a.nmax, ws=ws)
    torch.cuda.synchronize()
    for f in ra:
        assert torch.equal(ra[f], ra2[f]), f
    ref = oracle.softmax_topk(oracle.host_logits(xb), k=bb.k)
    gc.check_rows(rb, ref)
    gc.check_tree(rb, 4, bb.k, bb.nmax, row_status=ref["row_status"])


def test_standalone_mask_and_accept():
    wl = synth.scaled(synth.WORKLOADS["main"], B=16, nmax=64)
    x = gc.device_logits(wl)
    g = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    pos_base = torch.arange(16, dtype=torch.int32, device="cuda") * 3
    mask, pos = binding.tree_mask(g["parent"], g["n_nodes"], pos_base)
    torch.cuda.synchronize()
    rm, rp = oracle.tree_mask(gc.np_(g["parent"]), gc.np_(g["n_nodes"]), gc.np_(pos_base))
    assert (gc.np_(mask).view(np.uint32) == rm).all()
    assert (gc.np_(pos) == rp).all()
    top1 = gc.np_(g["topk_ids"])[:, :, 0]
    tgt = synth.make_targets(gc.np_(g["parent"]), gc.np_(g["token"]), gc.np_(g["depth"]),
                             gc.np_(g["n_nodes"]), top1, wl.V, seed=99)
    alen, anodes, bonus = binding.accept(g["parent"], g["token"], g["n_nodes"], wl.b,
                                         torch.from_numpy(tgt).to("cuda"))
    torch.cuda.synchronize()
    ra, rn, rb = oracle.accept(gc.np_(g["parent"]), gc.np_(g["token"]), gc.np_(g["n_nodes"]),
                               wl.b, tgt)
    assert (gc.np_(alen) == ra).all() and (gc.np_(anodes) == rn).all()
    assert (gc.np_(bonus) == rb).all()
    assert ra.max() >= 2


def test_malformed_tree_mask_matches_reference():
    parent = torch.tensor([[-1, 0, 5, 1, 7, 0, 0, 0]], dtype=torch.int32, device="cuda")
    n = torch.tensor([4], dtype=torch.int32, device="cuda")
    mask, pos = binding.tree_mask(parent, n)
    torch.cuda.synchronize()
    rm, rp = oracle.tree_mask(gc.np_(parent), gc.np_(n))
    assert (gc.np_(mask).view(np.uint32) == rm).all() and (gc.np_(pos) == rp).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_largest_vocabulary(dtype):
    """V = 2^19, the largest the 19-bit token field of the pop keys holds, with
    the leaders among the last token ids (and ties between them in bf16)."""
    V = 1 << 19
    g = torch.Generator().manual_seed(21)
    x = torch.randn(2, 3, V, generator=g) * 2.0
    for q in range(2):
        for p in range(3):
            x[q, p, V - 1 - (q + p)] = 9.0
            x[q, p, V - 5 - p] = 8.5
            x[q, p, V - 9] = 8.5
    gc.run_and_check(x.to(dtype).to("cuda"), 6, 30)
