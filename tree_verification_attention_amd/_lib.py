"""ctypes binding of ``libtreeattn.so`` (the C ABI declared in ``include/treeattn.h``).

Argument marshalling only: torch tensors supply device pointers, strides and the current HIP
stream; every step of the computation runs in the library's HIP kernels. There is no CPU path:
calls raise if the library is not built or if an operand is not a GPU tensor.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtreeattn.so")

TA_OK, TA_EINVAL, TA_EUNSUPPORTED, TA_EWORKSPACE, TA_EHIP, TA_ESCRATCH = range(6)
TA_NOALLOC_SCRATCH_BYTES = 96 << 20
TA_BF16, TA_F32 = 0, 1
TA_DEV_BAD_PARENT, TA_DEV_BAD_LEN, TA_DEV_BAD_PAGE, TA_DEV_BAD_COMMIT, TA_DEV_BAD_TOKEN = 1, 2, 4, 8, 16
TA_MAX_TREE = 256

# Functions the header declares (checked against the shared object by the test suite).
EXPORTS = ("tree_mask_build", "tree_attn_workspace_size", "tree_attn_num_splits",
           "tree_attn_prefix", "tree_attn_tree", "tree_attn_merge", "tree_attn_forward",
           "tree_attn_partials", "tree_attn_combine", "tree_attn_workspace_lse_offset",
           "tree_attn_status_string", "tree_attn_abi_version", "tree_greedy_accept",
           "tree_greedy_accept_workspace_size", "tree_spec_sample",
           "tree_spec_sample_workspace_size", "tree_gdn_verify", "tree_gdn_commit",
           "tree_kv_commit", "tree_attn_forward_noalloc")


class TreeAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class TaProblem(ctypes.Structure):
    """Mirror of ``ta_problem`` (same field order, natural C alignment)."""

    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("num_splits", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_sb", ctypes.c_int64), ("q_st", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("kv_s0", ctypes.c_int64), ("kv_s1", ctypes.c_int64), ("kv_s2", ctypes.c_int64),
        ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("Lmax", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("k_tree", ctypes.c_void_p), ("v_tree", ctypes.c_void_p),
        ("kt_sb", ctypes.c_int64), ("kt_st", ctypes.c_int64), ("kt_sh", ctypes.c_int64),
        ("parent", ctypes.c_void_p),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(python tree_verification_attention_amd/build.py)")
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    PP = ctypes.POINTER(TaProblem)
    lib.tree_mask_build.argtypes = [P, I, I, P, P, P]
    lib.tree_attn_workspace_size.argtypes = [PP, ctypes.POINTER(S)]
    lib.tree_attn_num_splits.argtypes = [PP, ctypes.POINTER(I)]
    lib.tree_attn_prefix.argtypes = [PP, P, P, P, S, P, P]
    lib.tree_attn_tree.argtypes = [PP, P, P, P, P]
    lib.tree_attn_merge.argtypes = [I, I, I, I, P, P, P, P, P, I, P, P]
    lib.tree_attn_forward.argtypes = [PP, P, P, P, S, P, P]
    lib.tree_attn_forward_noalloc.argtypes = [PP, P, P, P, P]
    lib.tree_attn_partials.argtypes = [PP, P, S, P, P]
    lib.tree_attn_combine.argtypes = [PP, P, S, P, P, P]
    lib.tree_attn_workspace_lse_offset.argtypes = [PP, ctypes.POINTER(S)]
    lib.tree_attn_status_string.argtypes = [I]
    lib.tree_attn_status_string.restype = ctypes.c_char_p
    lib.tree_attn_abi_version.argtypes = []
    lib.tree_greedy_accept.argtypes = [P, I, ctypes.c_int64, I, I, I, P, P, P, S, P, P, P, P, P, P]
    lib.tree_greedy_accept_workspace_size.argtypes = [I, I, I, I, ctypes.POINTER(S)]
    lib.tree_spec_sample.argtypes = [P, P, ctypes.c_int64, I, I, I, P, P, P, P, P, S, P, P, P, P, P]
    lib.tree_spec_sample_workspace_size.argtypes = [I, I, I, ctypes.POINTER(S)]
    lib.tree_gdn_verify.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, ctypes.c_float, P, P, P]
    lib.tree_gdn_commit.argtypes = [P, P, P, P, I, I, I, I, I, I, P, P, P, P, P]
    lib.tree_kv_commit.argtypes = [PP, P, P, P, P, P, P, P]
    for fn in EXPORTS:
        if fn not in ("tree_attn_status_string",):
            getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().tree_attn_status_string(int(status)).decode()


def _check(fn: str, rc: int):
    if rc != TA_OK:
        raise TreeAttnError(fn, rc, status_string(rc))


def _gpu(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (no CPU path exists)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


_DT = {torch.bfloat16: TA_BF16, torch.float32: TA_F32}


def make_problem(q, k_cache, v_cache, seq_lens, k_tree, v_tree, parent, *, block_table=None,
                 page_size: Optional[int] = None, scale: Optional[float] = None,
                 num_splits: int = 0) -> TaProblem:
    """Describe one layer. Shapes: q [B,T,Hq,D]; k/v_cache [B,Lmax,Hkv,D] or, with a block
    table [B,max_blocks], a page pool [pages,page,Hkv,D]; k/v_tree [B,T,Hkv,D]; parent [B,T];
    seq_lens [B]. Every last dimension must be contiguous."""
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, T, Hq, D = q.shape
    Hkv = k_tree.shape[2] if k_tree is not None else k_cache.shape[2]
    p = TaProblem()
    p.B, p.T, p.Hq, p.Hkv, p.D = B, T, Hq, Hkv, D
    p.dtype = _DT[q.dtype]
    p.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    p.num_splits = int(num_splits)
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_tree", k_tree),
                    ("v_tree", v_tree)):
        if t is not None and (t.dtype != q.dtype or t.stride(-1) != 1):
            raise TypeError(f"{name} must be {q.dtype} with a contiguous last dimension")
    p.q = _gpu(q, "q")
    p.q_sb, p.q_st, p.q_sh = q.stride(0), q.stride(1), q.stride(2)
    if k_cache is not None:
        if tuple(k_cache.stride()) != tuple(v_cache.stride()) or k_cache.shape != v_cache.shape:
            raise ValueError("k_cache and v_cache must share shape and strides")
        p.k_cache = _gpu(k_cache, "k_cache")
        p.v_cache = _gpu(v_cache, "v_cache")
        p.kv_s0, p.kv_s1, p.kv_s2 = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
        p.seq_lens = _gpu(seq_lens, "seq_lens", torch.int32)
        if block_table is not None:
            p.block_table = _gpu(block_table, "block_table", torch.int32)
            p.page_size = int(page_size if page_size is not None else k_cache.shape[1])
            p.max_blocks = block_table.shape[1]
            p.num_pages = k_cache.shape[0]
            p.Lmax = 0
        else:
            p.Lmax = k_cache.shape[1]
    if k_tree is not None:
        if tuple(k_tree.stride()) != tuple(v_tree.stride()) or k_tree.shape != v_tree.shape:
            raise ValueError("k_tree and v_tree must share shape and strides")
        p.k_tree = _gpu(k_tree, "k_tree")
        p.v_tree = _gpu(v_tree, "v_tree")
        p.kt_sb, p.kt_st, p.kt_sh = k_tree.stride(0), k_tree.stride(1), k_tree.stride(2)
        p.parent = _gpu(parent, "parent", torch.int32)
    return p


def workspace_size(p: TaProblem) -> int:
    n = ctypes.c_size_t(0)
    _check("tree_attn_workspace_size", load().tree_attn_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def num_splits(p: TaProblem) -> int:
    n = ctypes.c_int(0)
    _check("tree_attn_num_splits", load().tree_attn_num_splits(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def _workspace(p: TaProblem, ws, device):
    need = workspace_size(p)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def forward(q, k_cache, v_cache, seq_lens, k_tree, v_tree, parent, *, block_table=None,
            page_size=None, scale=None, num_splits: int = 0, out=None, lse=None, workspace=None,
            err=None):
    """Hybrid tree attention of one layer -> (out [B,T,Hq,D] of q's dtype, lse fp32 [B,T,Hq])."""
    p = make_problem(q, k_cache, v_cache, seq_lens, k_tree, v_tree, parent,
                     block_table=block_table, page_size=page_size, scale=scale,
                     num_splits=num_splits)
    B, T, Hq, D = q.shape
    out = torch.empty((B, T, Hq, D), dtype=q.dtype, device=q.device) if out is None else out
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    ws, nbytes = _workspace(p, workspace, q.device)
    _check("tree_attn_forward", load().tree_attn_forward(
        ctypes.byref(p), _gpu(out, "out", q.dtype), _gpu(lse, "lse", torch.float32),
        _gpu(ws, "workspace"), nbytes, _gpu(err, "err", torch.int32), _stream()))
    return out, lse


def forward_noalloc(q, k_cache, v_cache, seq_lens, k_tree, v_tree, parent, *, out, lse,
                    block_table=None, page_size=None, scale=None, num_splits: int = 0, err=None):
    """tree_attn_forward_noalloc: the forward with its partials in the library's fixed device
    array (no workspace); the caller passes the outputs, so nothing is allocated here either."""
    p = make_problem(q, k_cache, v_cache, seq_lens, k_tree, v_tree, parent,
                     block_table=block_table, page_size=page_size, scale=scale,
                     num_splits=num_splits)
    _check("tree_attn_forward_noalloc", load().tree_attn_forward_noalloc(
        ctypes.byref(p), _gpu(out, "out", q.dtype), _gpu(lse, "lse", torch.float32),
        _gpu(err, "err", torch.int32), _stream()))
    return out, lse


def partials(p: TaProblem, workspace, err=None):
    """Launch the divide step (all prefix splits and the tree part) of problem ``p`` into
    ``workspace``; see tree_attn_partials for the workspace layout."""
    _check("tree_attn_partials", load().tree_attn_partials(
        ctypes.byref(p), _gpu(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _gpu(err, "err", torch.int32), _stream()))


def combine(p: TaProblem, workspace, out, lse):
    """Launch the aggregation of the parts in ``workspace`` into ``out`` / ``lse``."""
    _check("tree_attn_combine", load().tree_attn_combine(
        ctypes.byref(p), _gpu(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _gpu(out, "out"), _gpu(lse, "lse", torch.float32), _stream()))


def workspace_lse_offset(p: TaProblem) -> int:
    n = ctypes.c_size_t(0)
    _check("tree_attn_workspace_lse_offset",
           load().tree_attn_workspace_lse_offset(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def prefix(q, k_cache, v_cache, seq_lens, *, block_table=None, page_size=None, scale=None,
           num_splits: int = 0, workspace=None, err=None):
    """Unmasked attention over the committed prefix -> (o_c fp32, lse_c fp32)."""
    p = make_problem(q, k_cache, v_cache, seq_lens, None, None, None,
                     block_table=block_table, page_size=page_size, scale=scale,
                     num_splits=num_splits)
    B, T, Hq, D = q.shape
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    ws, nbytes = _workspace(p, workspace, q.device)
    _check("tree_attn_prefix", load().tree_attn_prefix(
        ctypes.byref(p), o.data_ptr(), lse.data_ptr(), _gpu(ws, "workspace"), nbytes,
        _gpu(err, "err", torch.int32), _stream()))
    return o, lse


def tree(q, k_tree, v_tree, parent, *, scale=None, err=None):
    """Masked attention over the tree's own keys -> (o_s fp32, lse_s fp32)."""
    p = make_problem(q, None, None, None, k_tree, v_tree, parent, scale=scale)
    B, T, Hq, D = q.shape
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    _check("tree_attn_tree", load().tree_attn_tree(
        ctypes.byref(p), o.data_ptr(), lse.data_ptr(), _gpu(err, "err", torch.int32), _stream()))
    return o, lse


def merge(o_a, lse_a, o_b, lse_b, out_dtype=torch.float32):
    """Log-sum-exp merge of two partial results ([B,T,Hq,D] fp32 + [B,T,Hq] fp32 each)."""
    B, T, Hq, D = o_a.shape
    for name, t in (("o_a", o_a), ("lse_a", lse_a), ("o_b", o_b), ("lse_b", lse_b)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        _gpu(t, name, torch.float32)
    o = torch.empty((B, T, Hq, D), dtype=out_dtype, device=o_a.device)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=o_a.device)
    _check("tree_attn_merge", load().tree_attn_merge(
        B, T, Hq, D, o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
        o.data_ptr(), _DT[out_dtype], lse.data_ptr(), _stream()))
    return o, lse


def mask_build(parent, err=None):
    """Ancestor-or-self masks of [B,T] int32 parents -> int64 tensor [B,T,ceil(T/64)] holding
    the uint64 words' bit patterns."""
    B, T = parent.shape
    W = (T + 63) // 64
    mask = torch.empty((B, T, W), dtype=torch.int64, device=parent.device)
    _check("tree_mask_build", load().tree_mask_build(
        _gpu(parent, "parent", torch.int32), B, T, mask.data_ptr(), _gpu(err, "err", torch.int32),
        _stream()))
    return mask


def greedy_accept_workspace_size(dtype, B: int, T: int, V: int) -> int:
    """Workspace bytes (at least 256) that greedy_accept needs for these sizes."""
    if dtype not in _DT:
        raise TypeError(f"unsupported logits dtype {dtype}")
    need = ctypes.c_size_t(0)
    _check("tree_greedy_accept_workspace_size", load().tree_greedy_accept_workspace_size(
        _DT[dtype], B, T, V, ctypes.byref(need)))
    return max(need.value, 256)


def greedy_accept(logits, draft, parent, *, ws=None, err=None):
    """Greedy tree acceptance. logits [B, T + 1, V] (bf16 or fp32; row 0 = the last committed
    token, row i + 1 = tree node i), draft / parent int32 [B, T]; ``ws`` (optional) is a device
    buffer of greedy_accept_workspace_size() bytes, allocated per call when omitted
    -> (greedy [B, T + 1], accept_len [B], path [B, T], next_token [B]), all int32."""
    if logits.dtype not in _DT:
        raise TypeError(f"unsupported logits dtype {logits.dtype}")
    if logits.stride(-1) != 1 or logits.stride(0) != logits.shape[1] * logits.stride(1):
        raise ValueError("logits rows must be evenly strided with a contiguous last dimension")
    B, T1, V = logits.shape
    T = T1 - 1
    dev = logits.device
    greedy = torch.empty((B, T + 1), dtype=torch.int32, device=dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, T), dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(greedy_accept_workspace_size(logits.dtype, B, T, V), dtype=torch.uint8,
                         device=dev)
    _check("tree_greedy_accept", load().tree_greedy_accept(
        _gpu(logits, "logits"), _DT[logits.dtype], logits.stride(1), B, T, V,
        _gpu(draft, "draft", torch.int32), _gpu(parent, "parent", torch.int32), _gpu(ws, "ws"),
        ws.numel() * ws.element_size(), greedy.data_ptr(), n.data_ptr(), path.data_ptr(),
        nxt.data_ptr(), _gpu(err, "err", torch.int32), _stream()))
    return greedy, n, path, nxt


def spec_sample_workspace_size(B: int, T: int, V: int) -> int:
    """Workspace bytes (at least 256) that spec_sample needs for these sizes."""
    need = ctypes.c_size_t(0)
    _check("tree_spec_sample_workspace_size",
           load().tree_spec_sample_workspace_size(B, T, V, ctypes.byref(need)))
    return max(need.value, 256)


def spec_sample(p, q, draft, parent, u_accept, u_sample, *, ws=None, err=None):
    """Tree speculative sampling. p, q float32 [B, T + 1, V] (same row stride, contiguous last
    dimension); draft / parent int32 [B, T]; u_accept float64 [B, T]; u_sample float64 [B]
    -> (accept_len [B], path [B, T], next_token [B]), all int32."""
    for name, t in (("p", p), ("q", q)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
        if t.stride(-1) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{name} rows must be evenly strided with a contiguous last dimension")
    if p.shape != q.shape or p.stride() != q.stride():
        raise ValueError("p and q must have the same shape and strides")
    B, T1, V = p.shape
    T = T1 - 1
    dev = p.device
    if ws is None:
        ws = torch.empty(spec_sample_workspace_size(B, T, V), dtype=torch.uint8, device=dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, T), dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    _check("tree_spec_sample", load().tree_spec_sample(
        _gpu(p, "p"), _gpu(q, "q"), p.stride(1), B, T, V, _gpu(draft, "draft", torch.int32),
        _gpu(parent, "parent", torch.int32), _gpu(u_accept, "u_accept", torch.float64),
        _gpu(u_sample, "u_sample", torch.float64), _gpu(ws, "ws"), ws.numel() * ws.element_size(),
        n.data_ptr(), path.data_ptr(), nxt.data_ptr(), _gpu(err, "err", torch.int32), _stream()))
    return n, path, nxt


def _contig(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d {dtype} tensor")
    return t.data_ptr()


def gdn_verify(q, k, v, g, beta, parent, S0, scale, *, err=None):
    """Tree verification of a gated-delta-net layer. q, k bf16 [B, T, Hk, dk]; v bf16
    [B, T, Hv, dv]; g, beta float32 [B, T, Hv]; parent int32 [B, T]; S0 float32
    [B, Hv, dk, dv] -> o float32 [B, T, Hv, dv]."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=q.device)
    _check("tree_gdn_verify", load().tree_gdn_verify(
        _contig(q, "q", torch.bfloat16, 4), _contig(k, "k", torch.bfloat16, 4),
        _contig(v, "v", torch.bfloat16, 4), _contig(g, "g", torch.float32, 3),
        _contig(beta, "beta", torch.float32, 3), _contig(parent, "parent", torch.int32, 2),
        _contig(S0, "S0", torch.float32, 4), B, T, Hk, Hv, dk, dv, float(scale), o.data_ptr(),
        _gpu(err, "err", torch.int32), _stream()))
    return o


def gdn_commit(k, v, g, beta, path, accept_len, S, *, err=None):
    """Deferred GDN state commit: S (float32 [B, Hv, dk, dv]) becomes, in place, the state after
    the updates of each sequence's accepted path (int32 [B, T], root first; accept_len int32 [B])."""
    B, T, Hk, dk = k.shape
    Hv, dv = v.shape[2], v.shape[3]
    _check("tree_gdn_commit", load().tree_gdn_commit(
        _contig(k, "k", torch.bfloat16, 4), _contig(v, "v", torch.bfloat16, 4),
        _contig(g, "g", torch.float32, 3), _contig(beta, "beta", torch.float32, 3), B, T, Hk, Hv,
        dk, dv, _contig(path, "path", torch.int32, 2), _contig(accept_len, "accept_len",
                                                              torch.int32, 1),
        _contig(S, "S", torch.float32, 4), _gpu(err, "err", torch.int32), _stream()))
    return S


def kv_commit(k_cache, v_cache, seq_lens, k_tree, v_tree, path, accept_len, *, block_table=None,
              page_size=None, new_seq_lens=None, err=None):
    """Accepted-path KV commit: writes the path's tree K/V rows into k_cache / v_cache (in place)
    at positions seq_lens[b] + j and returns the new lengths (``new_seq_lens`` may be
    ``seq_lens`` itself)."""
    # the commit reads neither queries nor parents: k_tree and path stand in for their shapes
    p = make_problem(k_tree, k_cache, v_cache, seq_lens, k_tree, v_tree, path,
                     block_table=block_table, page_size=page_size)
    out = new_seq_lens if new_seq_lens is not None else torch.empty_like(seq_lens)
    _check("tree_kv_commit", load().tree_kv_commit(
        ctypes.byref(p), _gpu(k_cache, "k_cache"), _gpu(v_cache, "v_cache"),
        _gpu(path, "path", torch.int32), _gpu(accept_len, "accept_len", torch.int32),
        _gpu(out, "new_seq_lens", torch.int32), _gpu(err, "err", torch.int32), _stream()))
    return out
