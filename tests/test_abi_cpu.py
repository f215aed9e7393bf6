"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bastion.h")


@pytest.fixture(scope="module")
def L():
    from block_diffusion_tree_amd import binding
    return binding.lib()


def declared():
    txt = open(HEADER).read()
    return re.findall(r"^\s*(?:int32_t|size_t|void|const char \*)\s*\**(bastion_\w+)\s*\(", txt, re.M)


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert L.bastion_abi_version() == 1


def test_status_strings(L):
    assert L.bastion_status_string(0) == b"ok"
    assert L.bastion_status_string(1) == b"invalid argument"
    assert L.bastion_status_string(4).startswith(b"workspace")


FAKE = C.c_void_p(1 << 20)   # never dereferenced: validation fails first


def full_out(**nulls):
    from block_diffusion_tree_amd.binding import TreeOut
    vals = {n: FAKE for n, _ in TreeOut._fields_}
    vals.update(nulls)
    return TreeOut(**vals)


def call_build(L, logits=FAKE, dtype=1, B=2, b=4, V=1000, stride=1000, k=8, nmax=16, nmin=1,
               cost=None, cstride=0, l_ar=1.0, out=None, ws=FAKE, ws_bytes=1 << 30):
    out = full_out() if out is None else out
    return L.bastion_build_trees(logits, dtype, B, b, V, stride, k, nmax, nmin, cost, cstride,
                                 l_ar, None, C.byref(out), ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(logits=None), dict(dtype=2), dict(B=0), dict(B=16385), dict(b=0), dict(b=33),
    dict(k=0), dict(k=33), dict(V=7, stride=7, k=8), dict(V=524289, stride=524289),
    dict(nmax=0), dict(nmax=1024), dict(nmin=-1), dict(nmin=17), dict(stride=999),
    dict(logits=C.c_void_p((1 << 20) + 1)), dict(cost=FAKE, l_ar=0.0),
    dict(cost=FAKE, l_ar=float("nan")), dict(cost=FAKE, cstride=-1),
])
def test_build_rejects_bad_arguments(L, kw):
    assert call_build(L, **kw) == 1


def test_build_rejects_incomplete_outputs(L):
    assert call_build(L, out=full_out(parent=None)) == 1
    assert call_build(L, out=full_out(topk_q=None)) == 1
    assert call_build(L, out=full_out(position_ids=None)) == 1   # mask without positions


def test_build_rejects_small_workspace(L):
    need = L.bastion_workspace_bytes(2, 1, 4, 1000, 8, 16, 1)
    assert need >= 1 << 18
    assert call_build(L, ws=None) == 4
    assert call_build(L, ws_bytes=need - 1) == 4
    assert call_build(L, ws=C.c_void_p((1 << 20) + 8)) == 4


def test_workspace_sizes(L):
    assert L.bastion_workspace_bytes(0, 1, 4, 1000, 8, 16, 1) == 0
    assert L.bastion_workspace_bytes(64, 1, 16, 151936, 8, 64, 1) >= (1 << 18) + 64 * 16 * 4
    assert L.bastion_workspace_init(None, 1 << 20, None) == 1
    assert L.bastion_workspace_init(FAKE, 1024, None) == 4


def test_small_kernels_reject_bad_arguments(L):
    assert L.bastion_budget_select(None, FAKE, 2, 8, 1, FAKE, 0, 1.0, FAKE, None, None) == 1
    assert L.bastion_budget_select(FAKE, FAKE, 2, 8, 9, FAKE, 0, 1.0, FAKE, None, None) == 1
    assert L.bastion_budget_select(FAKE, FAKE, 2, 1024, 1, FAKE, 0, 1.0, FAKE, None, None) == 1
    assert L.bastion_budget_select(FAKE, FAKE, 2, 8, 1, FAKE, 0, -1.0, FAKE, None, None) == 1
    assert L.bastion_tree_mask(FAKE, FAKE, 0, 8, None, FAKE, FAKE, None) == 1
    assert L.bastion_tree_mask(FAKE, FAKE, 2, 8, None, None, FAKE, None) == 1
    assert L.bastion_accept(FAKE, FAKE, FAKE, 2, 33, 8, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.bastion_accept(FAKE, FAKE, FAKE, 2, 4, 8, None, FAKE, FAKE, FAKE, None) == 1


def full_mix(**nulls):
    from block_diffusion_tree_amd.binding import MixOut
    vals = {n: FAKE for n, _ in MixOut._fields_}
    vals.update(nulls)
    return MixOut(**vals)


def call_mix(L, logits=FAKE, dtype=1, prior=FAKE, B=2, K=4, b=4, V=1000, stride=1000, k=8,
             nmax=16, mix=None, tree="full", ws=FAKE, ws_bytes=1 << 30):
    mix = full_mix() if mix is None else mix
    t = full_out() if tree == "full" else tree
    return L.bastion_mixture_score(logits, dtype, prior, B, K, b, V, stride, k, nmax,
                                   C.byref(mix), None if t is None else C.byref(t), ws,
                                   ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(logits=None), dict(prior=None), dict(dtype=2), dict(K=0), dict(K=17), dict(B=0),
    dict(b=33), dict(k=0), dict(k=33), dict(nmax=0), dict(nmax=1024), dict(stride=999),
    dict(mix=None, tree=None, logits=None),
])
def test_mixture_rejects_bad_arguments(L, kw):
    assert call_mix(L, **kw) == 1


def test_mixture_rejects_incomplete_outputs_and_workspace(L):
    assert call_mix(L, mix=full_mix(cand_q=None)) == 1
    assert call_mix(L, mix=full_mix(qdep_chain=None)) == 1
    assert call_mix(L, tree=full_out(rho=None)) == 1
    need = L.bastion_workspace_bytes(2, 4, 4, 1000, 8, 16, 1)
    assert call_mix(L, ws_bytes=need - 1) == 4
    assert call_mix(L, tree=None, ws=None) == 4
    # the mixture tree keeps one position's candidates in LDS: K = 16, k = 32
    # and a large budget do not fit
    assert call_mix(L, K=16, k=32, nmax=1000, V=1000) == 2


def test_no_shared_code_between_library_and_reference():
    pkg = os.path.join(ROOT, "block_diffusion_tree_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle|liboracle|bastion_oracle", txt, re.M), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            txt = open(os.path.join(ROOT, "oracle", f)).read()
            assert "block_diffusion_tree_amd" not in txt, f
            assert "bastion.h" not in txt and "libbastion" not in txt, f


def test_binding_rejects_bad_cost_tables():
    """The binding checks a cost table's shape before anything reaches the
    library: a [B, nmax] table (one column short) would shift every C(n)."""
    import torch
    from block_diffusion_tree_amd import binding
    B, nmax = 4, 16
    for bad, what in ((torch.zeros(B, nmax, dtype=torch.float64), "columns"),
                      (torch.zeros(3, nmax + 1, dtype=torch.float64), "rows"),
                      (torch.zeros(B, 2, nmax + 1, dtype=torch.float64), "cost must be")):
        with pytest.raises(ValueError, match=what):
            binding._cost_stride(bad, B, nmax, None)
    with pytest.raises(TypeError):
        binding._cost_stride(torch.zeros(B, nmax + 1, dtype=torch.float32), B, nmax, None)
    with pytest.raises(ValueError, match="GPU"):   # right shape, but on the host
        binding._cost_stride(torch.zeros(B, nmax + 1, dtype=torch.float64), B, nmax, None)


def test_tuning_hook_is_exported(L):
    L.bastion_set_tuning(3, 1)
    L.bastion_set_tuning(0, -1)
