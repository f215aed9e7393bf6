"""Every output of every call is written inside its own bounds: outputs are
views into larger buffers whose margins hold a canary pattern, and after the
call every margin byte must still hold it."""
import pytest
import torch

from block_diffusion_tree_amd import binding, synth
import gpu_common as gc

pytestmark = pytest.mark.gpu

PAD = 4096          # elements of canary before and after each output
CANARY = {torch.int32: -0x2A2A2A2B, torch.float32: -1.2345678e-19,
          torch.float64: -9.87654321e-301}


class Canaried:
    """Outputs allocated as the interiors of canary-filled buffers."""

    def __init__(self, spec, device="cuda"):
        self.bufs, self.views = {}, {}
        for name, (dt, shape) in spec.items():
            n = 1
            for d in shape:
                n *= d
            buf = torch.full((PAD + n + PAD,), CANARY[dt], dtype=dt, device=device)
            self.bufs[name] = (buf, n)
            self.views[name] = buf[PAD:PAD + n].view(shape)

    def check(self):
        torch.cuda.synchronize()
        for name, (buf, n) in self.bufs.items():
            c = CANARY[buf.dtype]
            head, tail = buf[:PAD], buf[PAD + n:]
            assert bool((head == c).all()), f"{name}: a write before the array"
            assert bool((tail == c).all()), f"{name}: a write after the array"


def tree_spec(B, b, k, nmax, rows=True):
    W1 = nmax + 1
    W = (W1 + 31) // 32
    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    spec = dict(parent=(i32, (B, W1)), depth=(i32, (B, W1)), token=(i32, (B, W1)),
                rho=(f32, (B, W1)), ahat=(f64, (B, W1)), n_nodes=(i32, (B,)),
                qstatus=(i32, (B,)), mask=(i32, (B, W1, W)), position_ids=(i32, (B, W1)))
    if rows:
        spec.update(topk_ids=(i32, (B, b, k)), topk_q=(f32, (B, b, k)), row_max=(f32, (B, b)),
                    row_sum=(f32, (B, b)))
    return spec


@pytest.mark.parametrize("name,split", [("main", -1), ("latency", -1), ("tiny", -1),
                                        ("tiny", 1)])
def test_build_trees_writes_inside_its_outputs(name, split):
    gc.require_gpu()
    wl = synth.WORKLOADS[name]
    x = gc.device_logits(wl)
    out = Canaried(tree_spec(wl.B, wl.b, wl.k, wl.nmax))
    cost = None
    if wl.online:
        c, _ = synth.make_cost_table(wl.B, wl.nmax, seed=wl.seed, **synth.LATENCY_A100)
        cost = torch.from_numpy(c).to("cuda")
    binding.set_tuning(split_trees=split)
    try:
        binding.build_trees(x, k=wl.k, nmax=wl.nmax, nmin=wl.nmin, cost=cost, out=out.views)
    finally:
        binding.set_tuning(0, -1)
    out.check()
    # the interiors are the call's real outputs
    ref = binding.build_trees(x, k=wl.k, nmax=wl.nmax, nmin=wl.nmin, cost=cost)
    torch.cuda.synchronize()
    for f in ref:
        assert torch.equal(ref[f], out.views[f]), f


def test_tree_ops_write_inside_their_outputs():
    gc.require_gpu()
    wl = synth.scaled(synth.WORKLOADS["main"], B=6, V=20000, nmax=40)
    x = gc.device_logits(wl)
    g = binding.build_trees(x, k=wl.k, nmax=wl.nmax)
    W1 = wl.nmax + 1
    W = (W1 + 31) // 32
    o = Canaried(dict(mask=(torch.int32, (wl.B, W1, W)), pos=(torch.int32, (wl.B, W1)),
                      alen=(torch.int32, (wl.B,)), anodes=(torch.int32, (wl.B, wl.b + 1)),
                      bonus=(torch.int32, (wl.B,)), nstar=(torch.int32, (wl.B,)),
                      s=(torch.float64, (wl.B, W1))))
    L = binding.lib()
    st = binding._stream()
    p = binding._ptr
    assert L.bastion_tree_mask(p(g["parent"]), p(g["n_nodes"]), wl.B, wl.nmax, None,
                               p(o.views["mask"]), p(o.views["pos"]), st) == 0
    tgt = torch.randint(0, wl.V, (wl.B, W1), dtype=torch.int32, device="cuda")
    assert L.bastion_accept(p(g["parent"]), p(g["token"]), p(g["n_nodes"]), wl.B, wl.b, wl.nmax,
                            p(tgt), p(o.views["alen"]), p(o.views["anodes"]),
                            p(o.views["bonus"]), st) == 0
    cost = torch.linspace(1.0, 2.0, W1, dtype=torch.float64, device="cuda")
    assert L.bastion_budget_select(p(g["ahat"]), p(g["n_nodes"]), wl.B, wl.nmax, 1, p(cost), 0,
                                   1.0, p(o.views["nstar"]), p(o.views["s"]), st) == 0
    o.check()


def test_mixture_writes_inside_its_outputs():
    gc.require_gpu()
    wl = synth.scaled(synth.WORKLOADS["mixture"], B=3, K=4, b=6, V=5003, k=6, nmax=30)
    x = gc.device_logits(wl, seed=3)
    prior = synth.make_prior_logits(wl).to("cuda")
    B, K, b, k = wl.B, wl.K, wl.b, wl.k
    C_ = K * k
    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    mo = Canaried(dict(prior_q=(f32, (B, K)), chain_tokens=(i32, (B, K, b)),
                       qdep_chain=(f64, (B, K)), cand_count=(i32, (B, b)),
                       cand_tokens=(i32, (B, b, C_)), cand_q=(f32, (B, b, C_, K)),
                       row_max=(f32, (B, K, b)), row_sum=(f32, (B, K, b))))
    tr = Canaried(tree_spec(B, b, k, wl.nmax, rows=False))
    binding.mixture_score(x, prior, k=k, nmax=wl.nmax, out=mo.views, tree=tr.views)
    mo.check()
    tr.check()
