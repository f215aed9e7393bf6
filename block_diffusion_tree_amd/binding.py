"""Python binding of libbastion.so: argument marshalling only.

Every function takes torch tensors that live on the GPU, allocates the output
tensors with torch (device memory is PyTorch's job here), passes raw device
pointers and the current HIP stream to the C ABI, and returns the outputs.
No step of the computation happens in Python.  If the shared library is
missing or fails to load, every entry raises: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbastion.so")

OK, EINVAL, EUNSUPPORTED, EHIP, EWORKSPACE = 0, 1, 2, 3, 4
Q_OK, Q_BAD_LOGITS, Q_EXHAUSTED, Q_RANGE = 0, 1, 2, 3
F32, BF16 = 0, 1

_lib = None


class BastionError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} (status {status})")


P = C.c_void_p
I32, I64, F64, SZ = C.c_int32, C.c_int64, C.c_double, C.c_size_t


class TreeOut(C.Structure):
    _fields_ = [(n, P) for n in ("topk_ids", "topk_q", "row_max", "row_sum", "parent", "depth",
                                 "token", "rho", "ahat", "n_nodes", "qstatus", "mask",
                                 "position_ids")]


class MixOut(C.Structure):
    _fields_ = [(n, P) for n in ("prior_q", "chain_tokens", "qdep_chain", "cand_count",
                                 "cand_tokens", "cand_q", "row_max", "row_sum")]


class MargOut(C.Structure):
    _fields_ = [(n, P) for n in ("prior_q", "row_max", "row_sum", "marg_ids", "marg_q", "cand_q")]


def use_library(path: str):
    """Load `path` instead of libbastion.so (the stamped build of the same
    sources); must come before the first call."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    LIB_PATH = path


def lib():
    """The loaded library (torch's HIP runtime is loaded first, so both share it)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_diffusion_tree_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.bastion_abi_version.restype = I32
        L.bastion_status_string.restype = C.c_char_p
        L.bastion_status_string.argtypes = [I32]
        L.bastion_workspace_bytes.restype = SZ
        L.bastion_workspace_bytes.argtypes = [I32] * 7
        L.bastion_workspace_init.restype = I32
        L.bastion_workspace_init.argtypes = [P, SZ, P]
        L.bastion_build_trees.restype = I32
        L.bastion_build_trees.argtypes = [P, I32, I32, I32, I32, I64, I32, I32, I32, P, I64, F64,
                                          P, C.POINTER(TreeOut), P, SZ, P]
        L.bastion_budget_select.restype = I32
        L.bastion_budget_select.argtypes = [P, P, I32, I32, I32, P, I64, F64, P, P, P]
        L.bastion_tree_mask.restype = I32
        L.bastion_tree_mask.argtypes = [P, P, I32, I32, P, P, P, P]
        L.bastion_accept.restype = I32
        L.bastion_accept.argtypes = [P, P, P, I32, I32, I32, P, P, P, P, P]
        L.bastion_mixture_marginal.restype = I32
        L.bastion_mixture_marginal.argtypes = [P, I32, P, I32, I32, I32, I32, I64, I32, I32,
                                               C.POINTER(MargOut), C.POINTER(TreeOut), P, SZ, P]
        L.bastion_sample_nodes.restype = I32
        L.bastion_sample_nodes.argtypes = [P, I32, I32, I32, I32, I64, P, C.c_float, C.c_uint32,
                                           P, P]
        L.bastion_mixture_sample.restype = I32
        L.bastion_mixture_sample.argtypes = [P, I32, I32, F64, P, P, I32, P, P, P]
        L.bastion_set_tuning.restype = None
        L.bastion_set_tuning.argtypes = [I32, I32]
        L.bastion_mixture_score.restype = I32
        L.bastion_mixture_score.argtypes = [P, I32, P, I32, I32, I32, I32, I64, I32, I32,
                                            C.POINTER(MixOut), C.POINTER(TreeOut), P, SZ, P]
        _lib = L
    return _lib


def _status_string(s: int) -> str:
    try:
        return lib().bastion_status_string(s).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "?"


def _check(status: int, what: str):
    if status != OK:
        raise BastionError(status, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("logits must be float32 or bfloat16")


class Workspace:
    """Device scratch for the fused calls (grows on demand, zeroed once).

    Calls that share a workspace must not overlap in time: its arrival
    counters belong to one call at a time.  A workspace used on a stream
    other than the one it was allocated on is recorded on that stream, so
    that torch does not hand its memory to someone else while such a call
    may still run (when it grows, or when it is dropped)."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None
        self._alloc_stream = None

    def get(self, nbytes: int):
        cur = torch.cuda.current_stream(self.device)
        if self.buf is None or self.buf.numel() < nbytes:
            old = self.buf
            self.buf = torch.empty(max(nbytes, 1 << 18), dtype=torch.uint8,
                                   device=self.device or "cuda")
            self._alloc_stream = cur
            _check(lib().bastion_workspace_init(_ptr(self.buf), self.buf.numel(), _stream()),
                   "bastion_workspace_init")
            del old   # recorded on every other stream that used it
        elif cur != self._alloc_stream:
            self.buf.record_stream(cur)
        return self.buf


_default_ws = {}


def _workspace(ws, device):
    """The caller's workspace, else one per (device, stream): calls on
    different streams never share arrival counters."""
    if ws is not None:
        return ws
    stream = torch.cuda.current_stream(device)
    key = (str(device), stream.cuda_stream)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def set_tuning(segments: int = 0, split_trees: int = -1):
    """bastion_set_tuning: launch-plan overrides (0 / -1: the library's plan)."""
    lib().bastion_set_tuning(int(segments), int(split_trees))


def _need(t, name, dtype, shape=None, device=None):
    """t must be a contiguous GPU tensor of `dtype` (and `shape`, `device`)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _cost_stride(cost, B, nmax, device):
    """Checks a cost table [1 or B, >= nmax+1] (or [>= nmax+1]) float64 and
    returns its per-query stride (0 when shared)."""
    if cost.dim() == 1:
        rows, cols = 1, cost.size(0)
    elif cost.dim() == 2:
        rows, cols = cost.size(0), cost.size(1)
    else:
        raise ValueError("cost must be [nmax+1], [1, nmax+1] or [B, nmax+1]")
    if cols < nmax + 1:
        raise ValueError(f"cost needs at least nmax+1 = {nmax + 1} columns, got {cols}")
    if rows not in (1, B):
        raise ValueError(f"cost needs 1 or B = {B} rows, got {rows}")
    _need(cost, "cost", torch.float64, device=device)
    return 0 if rows == 1 else cols


def alloc_tree_out(B, b, k, nmax, device, with_rows=True, with_mask=True):
    W1 = nmax + 1
    W = (W1 + 31) // 32
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    out = {}
    if with_rows:
        out.update(topk_ids=torch.empty((B, b, k), **i32), topk_q=torch.empty((B, b, k), **f32),
                   row_max=torch.empty((B, b), **f32), row_sum=torch.empty((B, b), **f32))
    out.update(parent=torch.empty((B, W1), **i32), depth=torch.empty((B, W1), **i32),
               token=torch.empty((B, W1), **i32), rho=torch.empty((B, W1), **f32),
               ahat=torch.empty((B, W1), dtype=torch.float64, device=device),
               n_nodes=torch.empty((B,), **i32), qstatus=torch.empty((B,), **i32))
    if with_mask:
        out.update(mask=torch.empty((B, W1, W), **i32),   # uint32 bit rows, stored as int32
                   position_ids=torch.empty((B, W1), **i32))
    return out


def _check_tree_out(out, B, b, k, nmax, device, with_rows):
    """Caller-supplied outputs must have the shapes and types the call writes."""
    W1 = nmax + 1
    W = (W1 + 31) // 32
    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    spec = dict(parent=(i32, (B, W1)), depth=(i32, (B, W1)), token=(i32, (B, W1)),
                rho=(f32, (B, W1)), ahat=(f64, (B, W1)), n_nodes=(i32, (B,)),
                qstatus=(i32, (B,)))
    if with_rows:
        spec.update(topk_ids=(i32, (B, b, k)), topk_q=(f32, (B, b, k)), row_max=(f32, (B, b)),
                    row_sum=(f32, (B, b)))
    if "mask" in out:
        spec.update(mask=(i32, (B, W1, W)), position_ids=(i32, (B, W1)))
    for name, (dt, shape) in spec.items():
        if name not in out:
            raise ValueError(f"output {name!r} is missing")
        _need(out[name], name, dt, shape, device)


def _tree_struct(out):
    return TreeOut(*[(_ptr(out[n]) if n in out else None) for n, _ in TreeOut._fields_])


def _build_trees_call(logits, k, nmax, nmin, cost, l_ar, pos_base, with_mask, out, ws):
    """Checked arguments of one bastion_build_trees call: (out, call) where
    call() makes the C call (the ctypes objects it needs stay alive with it)."""
    _dev(logits, "logits")
    if logits.dim() != 3 or logits.stride(2) != 1 or logits.stride(0) != logits.size(1) * logits.stride(1):
        raise ValueError("logits must be [B, b, V] with unit stride over V and rows packed")
    B, b, V = logits.shape
    dt = _dtype_code(logits)
    if out is None:
        out = alloc_tree_out(B, b, k, nmax, logits.device, with_mask=with_mask)
    cost_ptr, cstride = None, 0
    if cost is not None:
        cstride = _cost_stride(cost, B, nmax, logits.device)
        cost_ptr = _ptr(cost)
    if pos_base is not None:
        _need(pos_base, "pos_base", torch.int32, (B,), logits.device)
    _check_tree_out(out, B, b, k, nmax, logits.device, with_rows=True)
    L = lib()
    w = _workspace(ws, logits.device)
    need = L.bastion_workspace_bytes(B, 1, b, V, k, nmax, dt)
    buf = w.get(need)
    st = _tree_struct(out)
    args = (_ptr(logits), dt, B, b, V, logits.stride(1), k, nmax, nmin, cost_ptr, cstride, l_ar,
            _ptr(pos_base), C.byref(st), _ptr(buf), buf.numel(), _stream())
    fn = L.bastion_build_trees

    def call(_keep=(st, buf, logits, cost, pos_base, out)):
        _check(fn(*args), "bastion_build_trees")
    return out, call


def build_trees(logits, k: int, nmax: int, nmin: int = 1, cost=None, l_ar: float = 1.0,
                pos_base=None, with_mask: bool = True, out=None, ws=None):
    """bastion_build_trees on logits [B, b, V] (float32 or bfloat16, on GPU)."""
    out, call = _build_trees_call(logits, k, nmax, nmin, cost, l_ar, pos_base, with_mask, out, ws)
    call()
    return out


def prepare_build_trees(logits, k: int, nmax: int, nmin: int = 1, cost=None, l_ar: float = 1.0,
                        pos_base=None, with_mask: bool = True, out=None, ws=None):
    """The same call with its arguments checked and marshalled once, on the
    current stream: returns (out, call), and every call() repeats it on the
    same tensors (what a caller that loops over fixed buffers does)."""
    return _build_trees_call(logits, k, nmax, nmin, cost, l_ar, pos_base, with_mask, out, ws)


def build_trees_noalloc(logits, k: int, nmax: int, nmin: int = 1, cost=None, l_ar: float = 1.0,
                        pos_base=None, with_mask: bool = True, out=None):
    """bastion_build_trees_noalloc: the same call on the library's own per-GPU
    scratch (no workspace; the C call allocates nothing).  Calls that overlap
    on one GPU race on that scratch."""
    _dev(logits, "logits")
    if logits.dim() != 3 or logits.stride(2) != 1 or logits.stride(0) != logits.size(1) * logits.stride(1):
        raise ValueError("logits must be [B, b, V] with unit stride over V and rows packed")
    B, b, V = logits.shape
    dt = _dtype_code(logits)
    if out is None:
        out = alloc_tree_out(B, b, k, nmax, logits.device, with_mask=with_mask)
    cost_ptr, cstride = None, 0
    if cost is not None:
        cstride = _cost_stride(cost, B, nmax, logits.device)
        cost_ptr = _ptr(cost)
    if pos_base is not None:
        _need(pos_base, "pos_base", torch.int32, (B,), logits.device)
    _check_tree_out(out, B, b, k, nmax, logits.device, with_rows=True)
    fn = lib().bastion_build_trees_noalloc
    fn.restype = I32
    fn.argtypes = [P, I32, I32, I32, I32, I64, I32, I32, I32, P, I64, F64, P,
                   C.POINTER(TreeOut), P]
    st = _tree_struct(out)
    _check(fn(_ptr(logits), dt, B, b, V, logits.stride(1), k, nmax, nmin, cost_ptr, cstride, l_ar,
              _ptr(pos_base), C.byref(st), _stream()), "bastion_build_trees_noalloc")
    return out


def budget_select(ahat, n_avail, nmin: int, cost, l_ar: float = 1.0, with_curve: bool = True):
    if ahat.dim() != 2:
        raise ValueError("ahat must be [B, nmax+1]")
    B, W1 = ahat.shape
    _need(ahat, "ahat", torch.float64)
    _need(n_avail, "n_avail", torch.int32, (B,), ahat.device)
    cstride = _cost_stride(cost, B, W1 - 1, ahat.device)
    nstar = torch.empty((B,), dtype=torch.int32, device=ahat.device)
    s = torch.empty((B, W1), dtype=torch.float64, device=ahat.device) if with_curve else None
    _check(lib().bastion_budget_select(_ptr(ahat), _ptr(n_avail), B, W1 - 1, nmin, _ptr(cost),
                                       cstride, l_ar, _ptr(nstar), _ptr(s), _stream()),
           "bastion_budget_select")
    return nstar, s


def tree_mask(parent, n_nodes, pos_base=None):
    if parent.dim() != 2:
        raise ValueError("parent must be [B, nmax+1]")
    B, W1 = parent.shape
    _need(parent, "parent", torch.int32)
    _need(n_nodes, "n_nodes", torch.int32, (B,), parent.device)
    if pos_base is not None:
        _need(pos_base, "pos_base", torch.int32, (B,), parent.device)
    W = (W1 + 31) // 32
    mask = torch.empty((B, W1, W), dtype=torch.int32, device=parent.device)
    pos = torch.empty((B, W1), dtype=torch.int32, device=parent.device)
    _check(lib().bastion_tree_mask(_ptr(parent), _ptr(n_nodes), B, W1 - 1, _ptr(pos_base),
                                   _ptr(mask), _ptr(pos), _stream()), "bastion_tree_mask")
    return mask, pos


def accept(parent, token, n_nodes, b: int, target):
    if parent.dim() != 2:
        raise ValueError("parent must be [B, nmax+1]")
    B, W1 = parent.shape
    dev = parent.device
    _need(parent, "parent", torch.int32)
    _need(token, "token", torch.int32, (B, W1), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    _need(target, "target", torch.int32, (B, W1), dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    anodes = torch.empty((B, b + 1), dtype=torch.int32, device=dev)
    bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(lib().bastion_accept(_ptr(parent), _ptr(token), _ptr(n_nodes), B, b, W1 - 1,
                                _ptr(target), _ptr(alen), _ptr(anodes), _ptr(bonus), _stream()),
           "bastion_accept")
    return alen, anodes, bonus


_verify_lib = None


def _vlib():
    """The tree-attention entry points (bastion_verify.h) of the same library."""
    global _verify_lib
    if _verify_lib is None:
        L = lib()
        L.bastion_tree_attention_workspace_bytes.restype = SZ
        L.bastion_tree_attention_workspace_bytes.argtypes = [I32] * 5
        L.bastion_tree_attention.restype = I32
        L.bastion_tree_attention.argtypes = [P, I64, I32, I32, I32, I32, I32, P, P, I32, P, I32, P,
                                             P, I32, P, P, P, SZ, P]
        _verify_lib = L
    return _verify_lib


_attn_ws = {}


def rope_inv_freq(theta: float = 1.0e6, head_dim: int = 128, device="cuda"):
    """Rotary frequencies theta^(-2d/D), d < D/2, computed in float64 and
    stored as float32 (the table bastion_tree_attention takes)."""
    import numpy as np
    d = np.arange(head_dim // 2, dtype=np.float64)
    return torch.from_numpy((theta ** (-2.0 * d / head_dim)).astype(np.float32)).to(device)


def tree_attention(qkv, S: int, T: int, Hq: int, Hkv: int, k_cache, v_cache, ctx_len,
                   position_ids, mask, inv_freq, out=None, ws=None, max_ctx: int = -1):
    out, call = prepare_tree_attention(qkv, S, T, Hq, Hkv, k_cache, v_cache, ctx_len,
                                       position_ids, mask, inv_freq, out, ws, max_ctx)
    call()
    return out


def prepare_tree_attention(qkv, S: int, T: int, Hq: int, Hkv: int, k_cache, v_cache, ctx_len,
                           position_ids, mask, inv_freq, out=None, ws=None, max_ctx: int = -1):
    """bastion_tree_attention: qkv [S*T, >= (Hq+2Hkv)*128] bf16 rows (unit
    stride over columns), k_cache [S, Hkv, Lmax, 128] and v_cache
    [S, Hkv, Lmax/32, 128, 32] bf16 (32-slot tiles; the tree tokens are
    written into both),
    ctx_len [S] int32, position_ids [S, T] int32, mask [S, T, W] 32-bit words,
    inv_freq [64] float32; max_ctx a host bound of ctx_len (-1: the cache's).
    Returns out [S*T, Hq*128] bf16."""
    D = 128
    dev = qkv.device
    if qkv.dim() != 2 or qkv.stride(1) != 1 or qkv.size(0) != S * T:
        raise ValueError("qkv must be [S*T, C] with unit column stride")
    if qkv.dtype != torch.bfloat16 or not qkv.is_cuda:
        raise TypeError("qkv must be a bfloat16 GPU tensor")
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [S, Hkv, Lmax, 128]")
    Lmax = k_cache.size(2)
    W = (T + 31) // 32
    _need(k_cache, "k_cache", torch.bfloat16, (S, Hkv, Lmax, D), dev)
    _need(v_cache, "v_cache", torch.bfloat16, (S, Hkv, Lmax // 32, D, 32), dev)
    _need(ctx_len, "ctx_len", torch.int32, (S,), dev)
    _need(position_ids, "position_ids", torch.int32, (S, T), dev)
    if mask.dtype not in (torch.int32, torch.uint32):
        raise TypeError("mask must hold 32-bit words")
    _need(mask, "mask", mask.dtype, (S, T, W), dev)
    _need(inv_freq, "inv_freq", torch.float32, (D // 2,), dev)
    if out is None:
        out = torch.empty((S * T, Hq * D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (S * T, Hq * D), dev)
    L = _vlib()
    need = L.bastion_tree_attention_workspace_bytes(S, T, Hq, Hkv, Lmax)
    if need == 0:
        raise ValueError("invalid tree-attention sizes")
    if ws is None:
        key = (str(dev), torch.cuda.current_stream(dev).cuda_stream)
        buf = _attn_ws.get(key)
        if buf is None or buf.numel() < need:
            buf = torch.empty(need, dtype=torch.uint8, device=dev)
            _attn_ws[key] = buf
        ws = buf
    if ws.numel() < need:
        raise ValueError(f"workspace needs {need} bytes")
    args = (_ptr(qkv), qkv.stride(0), S, T, Hq, Hkv, D, _ptr(k_cache), _ptr(v_cache), Lmax,
            _ptr(ctx_len), int(max_ctx), _ptr(position_ids), _ptr(mask), W, _ptr(inv_freq),
            _ptr(out), _ptr(ws), ws.numel(), _stream())
    fn = L.bastion_tree_attention

    def call():
        _check(fn(*args), "bastion_tree_attention")

    return out, call


def alloc_mixture_out(B, K, b, k, device):
    C_ = K * k
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    return dict(prior_q=torch.empty((B, K), **f32),
                chain_tokens=torch.empty((B, K, b), **i32),
                qdep_chain=torch.empty((B, K), dtype=torch.float64, device=device),
                cand_count=torch.empty((B, b), **i32),
                cand_tokens=torch.empty((B, b, C_), **i32),
                cand_q=torch.empty((B, b, C_, K), **f32),
                row_max=torch.empty((B, K, b), **f32),
                row_sum=torch.empty((B, K, b), **f32))


def _mixture_call(branch_logits, prior_logits, k, nmax, with_tree, with_mask, out, tree, ws):
    _dev(branch_logits, "branch_logits")
    _dev(prior_logits, "prior_logits")
    x = branch_logits
    if x.dim() != 4 or x.stride(3) != 1 or x.stride(1) != x.size(2) * x.stride(2) \
            or x.stride(0) != x.size(1) * x.stride(1):
        raise ValueError("branch_logits must be [B, K, b, V] with unit stride over V and rows packed")
    if prior_logits.dtype != torch.float32 or not prior_logits.is_contiguous():
        raise TypeError("prior_logits must be a contiguous float32 GPU tensor")
    B, K, b, V = x.shape
    dt = _dtype_code(x)
    if out is None:
        out = alloc_mixture_out(B, K, b, k, x.device)
    if with_tree and tree is None:
        tree = alloc_tree_out(B, b, k, nmax, x.device, with_rows=False, with_mask=with_mask)
    if not with_tree:
        tree = None
    _need(prior_logits, "prior_logits", torch.float32, (B, K), x.device)
    C_ = K * k
    mspec = dict(prior_q=(torch.float32, (B, K)), chain_tokens=(torch.int32, (B, K, b)),
                 qdep_chain=(torch.float64, (B, K)), cand_count=(torch.int32, (B, b)),
                 cand_tokens=(torch.int32, (B, b, C_)), cand_q=(torch.float32, (B, b, C_, K)),
                 row_max=(torch.float32, (B, K, b)), row_sum=(torch.float32, (B, K, b)))
    for name, (tdt, shape) in mspec.items():
        _need(out[name], name, tdt, shape, x.device)
    if tree is not None:
        _check_tree_out(tree, B, b, k, nmax, x.device, with_rows=False)
    L = lib()
    w = _workspace(ws, x.device)
    buf = w.get(L.bastion_workspace_bytes(B, K, b, V, k, nmax, dt))
    mo = MixOut(*[_ptr(out[n]) for n, _ in MixOut._fields_])
    tst = None if tree is None else _tree_struct(tree)
    ts = None if tst is None else C.byref(tst)
    args = (_ptr(x), dt, _ptr(prior_logits), B, K, b, V, x.stride(2), k, nmax, C.byref(mo), ts,
            _ptr(buf), buf.numel(), _stream())
    fn = L.bastion_mixture_score

    def call(_keep=(mo, tst, buf, x, prior_logits, out, tree)):
        _check(fn(*args), "bastion_mixture_score")
    return out, tree, call


def mixture_score(branch_logits, prior_logits, k: int, nmax: int, with_tree: bool = True,
                  with_mask: bool = True, out=None, tree=None, ws=None):
    """bastion_mixture_score on branch logits [B, K, b, V] (float32 or bfloat16)
    and prior logits [B, K] float32, on GPU.  Returns (mixture outputs, tree
    outputs or None)."""
    out, tree, call = _mixture_call(branch_logits, prior_logits, k, nmax, with_tree, with_mask,
                                    out, tree, ws)
    call()
    return out, tree


def prepare_mixture_score(branch_logits, prior_logits, k: int, nmax: int, with_tree: bool = True,
                          with_mask: bool = True, out=None, tree=None, ws=None):
    """mixture_score with its arguments checked and marshalled once: returns
    (out, tree, call)."""
    return _mixture_call(branch_logits, prior_logits, k, nmax, with_tree, with_mask, out, tree, ws)


def alloc_marginal_out(B, K, b, k, device):
    f32 = dict(dtype=torch.float32, device=device)
    return dict(prior_q=torch.empty((B, K), **f32), row_max=torch.empty((B, K, b), **f32),
                row_sum=torch.empty((B, K, b), **f32),
                marg_ids=torch.empty((B, b, k), dtype=torch.int32, device=device),
                marg_q=torch.empty((B, b, k), **f32), cand_q=torch.empty((B, b, k, K), **f32))


def _marginal_call(branch_logits, prior_logits, k, nmax, with_tree, with_mask, out, tree, ws):
    _dev(branch_logits, "branch_logits")
    x = branch_logits
    if x.dim() != 4 or x.stride(3) != 1 or x.stride(1) != x.size(2) * x.stride(2) \
            or x.stride(0) != x.size(1) * x.stride(1):
        raise ValueError("branch_logits must be [B, K, b, V] with unit stride over V and rows packed")
    B, K, b, V = x.shape
    dt = _dtype_code(x)
    _need(prior_logits, "prior_logits", torch.float32, (B, K), x.device)
    if out is None:
        out = alloc_marginal_out(B, K, b, k, x.device)
    spec = dict(prior_q=(torch.float32, (B, K)), row_max=(torch.float32, (B, K, b)),
                row_sum=(torch.float32, (B, K, b)), marg_ids=(torch.int32, (B, b, k)),
                marg_q=(torch.float32, (B, b, k)), cand_q=(torch.float32, (B, b, k, K)))
    for name, (tdt, shape) in spec.items():
        _need(out[name], name, tdt, shape, x.device)
    if with_tree and tree is None:
        tree = alloc_tree_out(B, b, k, nmax, x.device, with_rows=False, with_mask=with_mask)
    if not with_tree:
        tree = None
    if tree is not None:
        _check_tree_out(tree, B, b, k, nmax, x.device, with_rows=False)
    L = lib()
    w = _workspace(ws, x.device)
    buf = w.get(L.bastion_workspace_bytes(B, K, b, V, k, nmax, dt))
    mo = MargOut(*[_ptr(out[n]) for n, _ in MargOut._fields_])
    tst = None if tree is None else _tree_struct(tree)
    ts = None if tst is None else C.byref(tst)
    args = (_ptr(x), dt, _ptr(prior_logits), B, K, b, V, x.stride(2), k, nmax, C.byref(mo), ts,
            _ptr(buf), buf.numel(), _stream())
    fn = L.bastion_mixture_marginal

    def call(_keep=(mo, tst, buf, x, prior_logits, out, tree)):
        _check(fn(*args), "bastion_mixture_marginal")
    return out, tree, call


def mixture_marginal(branch_logits, prior_logits, k: int, nmax: int, with_tree: bool = True,
                     with_mask: bool = True, out=None, tree=None, ws=None):
    """bastion_mixture_marginal on branch logits [B, K, b, V] and prior logits
    [B, K] float32: candidates from the mixture marginal and, optionally, the
    mixture tree over them.  Returns (outputs, tree outputs or None)."""
    out, tree, call = _marginal_call(branch_logits, prior_logits, k, nmax, with_tree, with_mask,
                                     out, tree, ws)
    call()
    return out, tree


def prepare_mixture_marginal(branch_logits, prior_logits, k: int, nmax: int, with_tree: bool = True,
                             with_mask: bool = True, out=None, tree=None, ws=None):
    """mixture_marginal with its arguments checked and marshalled once:
    returns (out, tree, call)."""
    return _marginal_call(branch_logits, prior_logits, k, nmax, with_tree, with_mask, out, tree, ws)


def sample_nodes(logits, n_nodes, temperature: float, seed: int, out=None):
    """bastion_sample_nodes: logits [B, nmax+1, V] (float32 or bfloat16, the
    target's logits at every tree node), n_nodes [B] int32 -> one draw per
    node, int32 [B, nmax+1] (-1 after n_nodes)."""
    _dev(logits, "logits")
    if logits.dim() != 3 or logits.stride(2) != 1 or logits.stride(0) != logits.size(1) * logits.stride(1):
        raise ValueError("logits must be [B, nmax+1, V] with unit stride over V and rows packed")
    B, W1, V = logits.shape
    _need(n_nodes, "n_nodes", torch.int32, (B,), logits.device)
    if out is None:
        out = torch.empty((B, W1), dtype=torch.int32, device=logits.device)
    _need(out, "sampled", torch.int32, (B, W1), logits.device)
    _check(lib().bastion_sample_nodes(_ptr(logits), _dtype_code(logits), B, W1 - 1, V,
                                      logits.stride(1), _ptr(n_nodes), float(temperature),
                                      int(seed) & 0xFFFFFFFF, _ptr(out), _stream()),
           "bastion_sample_nodes")
    return out


def mixture_sample(prior_logits, temperature: float, u, chain_tokens):
    """bastion_mixture_sample: prior [B, K] float32, u [B] float64, chains
    [B, K, b] int32 -> (z [B], draft [B, b])."""
    if prior_logits.dim() != 2:
        raise ValueError("prior_logits must be [B, K]")
    B, K = prior_logits.shape
    dev = prior_logits.device
    _need(prior_logits, "prior_logits", torch.float32, (B, K), dev)
    _need(u, "u", torch.float64, (B,), dev)
    if chain_tokens.dim() != 3:
        raise ValueError("chain_tokens must be [B, K, b]")
    b = chain_tokens.size(2)
    _need(chain_tokens, "chain_tokens", torch.int32, (B, K, b), dev)
    z = torch.empty((B,), dtype=torch.int32, device=dev)
    draft = torch.empty((B, b), dtype=torch.int32, device=dev)
    _check(lib().bastion_mixture_sample(_ptr(prior_logits), B, K, float(temperature), _ptr(u),
                                        _ptr(chain_tokens), b, _ptr(z), _ptr(draft), _stream()),
           "bastion_mixture_sample")
    return z, draft
