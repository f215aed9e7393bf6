"""ctypes front end of the CPU reference (bastion_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark.  The HIP library and its Python binding never
import this module, and this module imports nothing from them.

Every function takes and returns numpy arrays.  The compiled library is
oracle/liboracle.so; build() compiles it with gcc (fp64, no fast-math, no FMA
contraction, OpenMP over rows and queries).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bastion_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OK, BAD_LOGITS, EXHAUSTED = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so (always when force, else only if missing)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = C.CDLL(LIB)
        _declare(_lib)
    return _lib


P = C.c_void_p
I32, I64, F64 = C.c_int, C.c_int64, C.c_double


def _declare(L):
    L.oracle_abi_version.restype = I32
    L.oracle_num_threads.restype = I32
    L.oracle_set_num_threads.argtypes = [I32]
    L.oracle_set_num_threads.restype = None
    L.oracle_softmax_topk.argtypes = [P, I32, I64, I32, I64, I32, P, P, P, P, P]
    L.oracle_best_first.argtypes = [P, P, P, I32, I32, I32, I32, I32, P, I64, F64,
                                    P, P, P, P, P, P, P]
    L.oracle_budget_select.argtypes = [P, P, I32, I32, I32, P, I64, F64, P, P]
    L.oracle_tree_mask.argtypes = [P, P, I32, I32, P, P, P]
    L.oracle_accept.argtypes = [P, P, P, I32, I32, I32, P, P, P, P]
    L.oracle_mixture.argtypes = [P, I32, P, I32, I32, I32, I32, I64, I32,
                                 P, P, P, P, P, P, P]
    L.oracle_qdep_sequences.argtypes = [P, I32, P, I32, I32, I32, I32, I64, P, I32, P]
    L.oracle_mixture_marginal.argtypes = [P, I32, P, I32, I32, I32, I32, I64, I32, P, P, P, P, P]
    L.oracle_sample_nodes.argtypes = [P, I32, I32, I32, I32, I64, P, F64, C.c_uint32, P, P]
    L.oracle_uniform_at.argtypes = [C.c_uint32] * 4
    L.oracle_uniform_at.restype = F64
    L.oracle_mixture_sample.argtypes = [P, I32, I32, F64, P, P, I32, P, P]
    L.oracle_mixture_tree.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32,
                                      P, P, P, P, P, P, P]
    for f in ("oracle_softmax_topk", "oracle_best_first", "oracle_budget_select",
              "oracle_tree_mask", "oracle_accept", "oracle_mixture",
              "oracle_qdep_sequences", "oracle_mixture_tree", "oracle_mixture_marginal",
              "oracle_sample_nodes", "oracle_mixture_sample"):
        getattr(L, f).restype = None


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the following calls (timing the reference only)."""
    lib().oracle_set_num_threads(int(n))


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _raw_logits(logits):
    """(array, dtype code): float32 as is; bf16 given as uint16 bit patterns."""
    a = np.ascontiguousarray(logits)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    raise TypeError("logits must be float32 or bf16 bits as uint16")


def softmax_topk(logits, k: int):
    """logits [..., V] -> dict of row_max, row_sum, topk_ids, topk_p, row_status."""
    a, dt = _raw_logits(logits)
    lead, V = a.shape[:-1], a.shape[-1]
    nrows = int(np.prod(lead)) if lead else 1
    rm = np.empty(nrows, np.float64)
    rs = np.empty(nrows, np.float64)
    ids = np.empty((nrows, k), np.int32)
    p = np.empty((nrows, k), np.float64)
    st = np.empty(nrows, np.int32)
    lib().oracle_softmax_topk(_p(a), dt, nrows, V, V, k, _p(rm), _p(rs), _p(ids), _p(p), _p(st))
    return dict(row_max=rm.reshape(lead), row_sum=rs.reshape(lead),
                topk_ids=ids.reshape(lead + (k,)), topk_p=p.reshape(lead + (k,)),
                row_status=st.reshape(lead))


def best_first(topk_ids, topk_q, nmax: int, nmin: int = 1, cost=None, l_ar: float = 1.0,
               row_status=None):
    """topk_ids [B,b,k] int32, topk_q [B,b,k] float32 -> tree dict."""
    ids = _c(topk_ids, np.int32)
    qv = _c(topk_q, np.float32)
    B, b, k = ids.shape
    st = None if row_status is None else _c(row_status, np.int32)
    cost_a, cstride = None, 0
    if cost is not None:
        cost_a = _c(cost, np.float64)
        cstride = 0 if cost_a.ndim == 1 or cost_a.shape[0] == 1 else nmax + 1
    W = nmax + 1
    out = dict(parent=np.empty((B, W), np.int32), depth=np.empty((B, W), np.int32),
               token=np.empty((B, W), np.int32), rho=np.empty((B, W), np.float32),
               ahat=np.empty((B, W), np.float64), n_nodes=np.empty(B, np.int32),
               qstatus=np.empty(B, np.int32))
    lib().oracle_best_first(_p(ids), _p(qv), _p(st), B, b, k, nmax, nmin, _p(cost_a),
                            cstride, l_ar, _p(out["parent"]), _p(out["depth"]),
                            _p(out["token"]), _p(out["rho"]), _p(out["ahat"]),
                            _p(out["n_nodes"]), _p(out["qstatus"]))
    return out


def budget_select(ahat, n_avail, nmin: int, cost, l_ar: float = 1.0):
    ah = _c(ahat, np.float64)
    B, W = ah.shape
    nmax = W - 1
    na = _c(n_avail, np.int32)
    cost_a = _c(cost, np.float64)
    cstride = 0 if cost_a.ndim == 1 or cost_a.shape[0] == 1 else nmax + 1
    nstar = np.empty(B, np.int32)
    s = np.empty((B, W), np.float64)
    lib().oracle_budget_select(_p(ah), _p(na), B, nmax, nmin, _p(cost_a), cstride, l_ar,
                               _p(nstar), _p(s))
    return nstar, s


def tree_mask(parent, n_nodes, pos_base=None):
    par = _c(parent, np.int32)
    B, W1 = par.shape
    nmax = W1 - 1
    W = (nmax + 1 + 31) // 32
    nn = _c(n_nodes, np.int32)
    pb = None if pos_base is None else _c(pos_base, np.int32)
    mask = np.empty((B, W1, W), np.uint32)
    pos = np.empty((B, W1), np.int32)
    lib().oracle_tree_mask(_p(par), _p(nn), B, nmax, _p(pb), _p(mask), _p(pos))
    return mask, pos


def accept(parent, token, n_nodes, b: int, target):
    par = _c(parent, np.int32)
    tok = _c(token, np.int32)
    B, W1 = par.shape
    nn = _c(n_nodes, np.int32)
    tg = _c(target, np.int32)
    alen = np.empty(B, np.int32)
    anodes = np.empty((B, b + 1), np.int32)
    bonus = np.empty(B, np.int32)
    lib().oracle_accept(_p(par), _p(tok), _p(nn), B, W1 - 1, b, _p(tg), _p(alen),
                        _p(anodes), _p(bonus))
    return alen, anodes, bonus


def mixture(branch_logits, prior_logits, k: int):
    """branch_logits [B,K,b,V] (float32 or bf16 bits), prior [B,K] float32."""
    a, dt = _raw_logits(branch_logits)
    B, K, b, V = a.shape
    pr = _c(prior_logits, np.float32)
    Cn = K * k
    out = dict(prior_w=np.empty((B, K), np.float64),
               chain_tokens=np.empty((B, K, b), np.int32),
               qdep_chain=np.empty((B, K), np.float64),
               cand_count=np.empty((B, b), np.int32),
               cand_tokens=np.empty((B, b, Cn), np.int32),
               cand_p=np.empty((B, b, Cn, K), np.float64),
               row_status=np.empty((B, K, b), np.int32))
    lib().oracle_mixture(_p(a), dt, _p(pr), B, K, b, V, V, k, _p(out["prior_w"]),
                         _p(out["chain_tokens"]), _p(out["qdep_chain"]),
                         _p(out["cand_count"]), _p(out["cand_tokens"]), _p(out["cand_p"]),
                         _p(out["row_status"]))
    return out


def mixture_marginal(branch_logits, prior_logits, k: int):
    """Candidates by the mixture marginal: branch_logits [B,K,b,V] (float32 or
    bf16 bits), prior [B,K] -> prior_w, marg_ids [B,b,k], marg_p [B,b,k],
    cand_p [B,b,k,K], row_status [B,K,b]."""
    a, dt = _raw_logits(branch_logits)
    B, K, b, V = a.shape
    pr = _c(prior_logits, np.float32)
    out = dict(prior_w=np.empty((B, K), np.float64), marg_ids=np.empty((B, b, k), np.int32),
               marg_p=np.empty((B, b, k), np.float64), cand_p=np.empty((B, b, k, K), np.float64),
               row_status=np.empty((B, K, b), np.int32))
    lib().oracle_mixture_marginal(_p(a), dt, _p(pr), B, K, b, V, V, k, _p(out["prior_w"]),
                                  _p(out["marg_ids"]), _p(out["marg_p"]), _p(out["cand_p"]),
                                  _p(out["row_status"]))
    return out


def sample_nodes(logits, n_nodes, temperature: float, seed: int):
    """One draw per tree node from softmax(logits / T) (Gumbel-max with the
    counter-based uniforms): logits [B, nmax+1, V] (float32 or bf16 bits) ->
    (sampled [B, nmax+1] int32, score [B, nmax+1] float64)."""
    a, dt = _raw_logits(logits)
    B, W1, V = a.shape
    nn = _c(n_nodes, np.int32)
    sampled = np.empty((B, W1), np.int32)
    score = np.empty((B, W1), np.float64)
    lib().oracle_sample_nodes(_p(a), dt, B, W1 - 1, V, V, _p(nn), float(temperature),
                              int(seed) & 0xFFFFFFFF, _p(sampled), _p(score))
    return sampled, score


def uniform_at(seed: int, q: int, node: int, token: int) -> float:
    return float(lib().oracle_uniform_at(seed & 0xFFFFFFFF, q, node, token))


def mixture_sample(prior_logits, temperature: float, u, chain_tokens):
    """Branch draw z ~ softmax(prior / T) by inverse CDF at u [B], and the
    drafted chain of that branch: (z [B], draft [B, b])."""
    pr = _c(prior_logits, np.float32)
    B, K = pr.shape
    ch = _c(chain_tokens, np.int32)
    b = ch.shape[2]
    uu = _c(u, np.float64)
    z = np.empty(B, np.int32)
    draft = np.empty((B, b), np.int32)
    lib().oracle_mixture_sample(_p(pr), B, K, float(temperature), _p(uu), _p(ch), b, _p(z),
                                _p(draft))
    return z, draft


def qdep_sequences(branch_logits, prior_logits, seqs):
    a, dt = _raw_logits(branch_logits)
    B, K, b, V = a.shape
    pr = _c(prior_logits, np.float32)
    sq = _c(seqs, np.int32)
    n = sq.shape[1]
    out = np.empty((B, n), np.float64)
    lib().oracle_qdep_sequences(_p(a), dt, _p(pr), B, K, b, V, V, _p(sq), n, _p(out))
    return out


def mixture_tree(w, cand_count, cand_tokens, cand_q, nmax: int, row_status=None):
    """w [B,K] f32, cand_count [B,b], cand_tokens [B,b,C], cand_q [B,b,C,K] f32."""
    wa = _c(w, np.float32)
    cc = _c(cand_count, np.int32)
    ct = _c(cand_tokens, np.int32)
    cq = _c(cand_q, np.float32)
    B, b, Cn = ct.shape
    K = wa.shape[1]
    st = None if row_status is None else _c(row_status, np.int32)
    W = nmax + 1
    out = dict(parent=np.empty((B, W), np.int32), depth=np.empty((B, W), np.int32),
               token=np.empty((B, W), np.int32), rho=np.empty((B, W), np.float32),
               ahat=np.empty((B, W), np.float64), n_nodes=np.empty(B, np.int32),
               qstatus=np.empty(B, np.int32))
    lib().oracle_mixture_tree(_p(wa), _p(cc), _p(ct), _p(cq), _p(st), B, K, b, Cn, nmax,
                              _p(out["parent"]), _p(out["depth"]), _p(out["token"]),
                              _p(out["rho"]), _p(out["ahat"]), _p(out["n_nodes"]),
                              _p(out["qstatus"]))
    return out


def bf16_bits(t) -> np.ndarray:
    """A torch bfloat16 tensor's bit patterns as a uint16 numpy array."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_logits(t):
    """numpy view of a torch logits tensor in the form the oracle takes."""
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().contiguous().numpy().astype(np.float32, copy=False)
