"""CPU oracle for tree-verification attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import this
package. It wraps ``oracle.c`` (plain C, fp64, two-pass softmax; see that file's header for the
definition it computes and the passages it follows) through ctypes and numpy. It imports nothing
from the HIP package and the HIP package imports nothing from here.

Inputs are the exact arrays the GPU receives: bf16 as uint16 bit patterns, fp32 as float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FULL, PREFIX, TREE = 0, 1, 2
_WHICH = {"full": FULL, "prefix": PREFIX, "tree": TREE}
_ERRORS = {1: "parent out of range (need -1 <= parent[i] < i)",
           2: "prefix length or block table out of range",
           3: "bad argument", 4: "out of memory"}


class OracleError(ValueError):
    pass


def build() -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-pthread", _SRC,
           "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_tree_mask.argtypes = [P, I, I, P]
        lib.oracle_tree_mask.restype = I
        lib.oracle_attend.argtypes = [I, I, I, I, I, I, ctypes.c_double, P, P, P, I, P, P, I, I, I,
                                      P, P, P, I, P, I, P, P, I]
        lib.oracle_attend.restype = I
        lib.oracle_merge.argtypes = [I, I, P, P, P, P, P, P]
        lib.oracle_merge.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def tree_mask(parent: np.ndarray) -> np.ndarray:
    """Ancestor-or-self bit mask ``uint64[B, T, ceil(T/64)]`` of a ``[B, T]`` parent array."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    if parent.ndim == 1:
        parent = parent[None]
    B, T = parent.shape
    mask = np.zeros((B, T, (T + 63) // 64), dtype=np.uint64)
    rc = _load().oracle_tree_mask(_ptr(parent), B, T, _ptr(mask))
    if rc:
        raise OracleError(_ERRORS.get(rc, rc))
    return mask


def attend(*, q, k_cache, v_cache, seq_lens, k_tree, v_tree, parent, scale, dtype,
           block_table=None, page_size=0, which="full", rows=None, nthreads=None):
    """Attention of selected rows over [prefix || masked tree] (or one of the two parts).

    Layouts: q ``[B,T,Hq,D]``; k/v_cache contiguous ``[B,Lmax,Hkv,D]`` or, with a block table,
    a page pool ``[pages,page_size,Hkv,D]``; k/v_tree ``[B,T,Hkv,D]``; parent ``[B,T]``.
    ``rows`` is an ``int32[n,3]`` list of (b, i, h), or None for all rows in (b, i, h) order.
    Returns ``(o float64[n, D], lse float64[n])``.
    """
    B, T, Hq, D = q.shape
    Hkv = k_tree.shape[2] if k_tree is not None and k_tree.size else k_cache.shape[2]
    dt = {"bf16": 1, "f32": 0}[dtype]
    want = np.uint16 if dtype == "bf16" else np.float32
    arrs = [np.ascontiguousarray(a, dtype=want) for a in (q, k_cache, v_cache, k_tree, v_tree)]
    q_, kc, vc, kt, vt = arrs
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    parent = np.ascontiguousarray(parent, dtype=np.int32).reshape(B, T)
    if block_table is not None:
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        max_blocks = block_table.shape[1]
        num_pages = kc.shape[0]
        Lmax = 0
    else:
        max_blocks = num_pages = 0
        Lmax = kc.shape[1]
    if rows is None:
        n = B * T * Hq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
        n = rows_arr.shape[0]
    o = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0)) or 1   # the cores this process may run on
    rc = _load().oracle_attend(B, T, Hq, Hkv, D, dt, float(scale), _ptr(q_), _ptr(kc), _ptr(vc),
                               Lmax, _ptr(seq_lens), _ptr(block_table), int(page_size),
                               max_blocks, num_pages, _ptr(kt), _ptr(vt), _ptr(parent),
                               _WHICH[which], _ptr(rows_arr), n, _ptr(o), _ptr(lse),
                               int(nthreads))
    if rc:
        raise OracleError(_ERRORS.get(rc, rc))
    return o, lse


def attend_case(case, which="full", rows=None, nthreads=None):
    """``attend`` on a generated case (any object with the operand attributes)."""
    return attend(q=case.q, k_cache=case.k_cache, v_cache=case.v_cache, seq_lens=case.seq_lens,
                  k_tree=case.k_tree, v_tree=case.v_tree, parent=case.parent, scale=case.scale,
                  dtype=case.dtype, block_table=case.block_table, page_size=case.page_size,
                  which=which, rows=rows, nthreads=nthreads)


def merge(o_a, lse_a, o_b, lse_b):
    """Two-part log-sum-exp merge of partial attention results (float64)."""
    o_a = np.ascontiguousarray(o_a, dtype=np.float64)
    o_b = np.ascontiguousarray(o_b, dtype=np.float64)
    lse_a = np.ascontiguousarray(lse_a, dtype=np.float64)
    lse_b = np.ascontiguousarray(lse_b, dtype=np.float64)
    n, D = o_a.shape
    o = np.empty_like(o_a)
    lse = np.empty_like(lse_a)
    _load().oracle_merge(n, D, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse))
    return o, lse
