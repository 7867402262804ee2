"""Seeded synthetic operands for tree-verification attention.

This module draws the operands of one attention layer of a speculative-decoding verify step:
prefix lengths, a topologically ordered draft-tree parent array, and Q / K / V values. It holds
none of the attention arithmetic. Both the HIP path and the CPU oracle receive exactly the arrays
built here: bf16 values travel as raw uint16 bit patterns, fp32 values as float32.

Shapes follow the operands of LongSpec's Hybrid Tree Attention (LongSpec page, "Fast tree
attention" section): Q for the tree nodes, a committed K/V prefix that needs no mask, and the
speculative (tree) K/V. Tree nodes are numbered in topological order (DFlash-TfM summary page,
"Rollback-free tree verification"): parent[i] is in [-1, i-1], and -1 means the node hangs
directly off the committed prefix.

For one seed, numpy PCG64(seed) draws the prefix lengths, then the parent arrays, then the
outlier channels. Values are fp32 N(0, 1), rounded to bf16 with round-to-nearest-even; each
value tensor (Q, K prefix, V prefix, K tree, V tree), sequence and 4096-row chunk draws from its
own PCG64 stream seeded by SeedSequence([seed, tensor, sequence, chunk]). Padding rows beyond a sequence's length are not drawn; they are filled
with NaN ("nan", used by tests to catch out-of-range reads) or zeros ("finite", used for timing).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# stream keys of the value tensors
_Q, _KP, _VP, _KT, _VT = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic layer shape. ``L`` is a fixed prefix length or an inclusive (lo, hi) range."""

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int
    L: object
    dtype: str = "bf16"          # "bf16" or "f32"
    tree: str = "bounded"        # "uniform", "bounded", "chain", "star", "single", "beam"
    depth_cap: int = 8
    branch_cap: int = 4
    outlier_channels: int = 0
    outlier_scale: float = 8.0
    widths: tuple = ()

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The long-context shapes measured on the pages' target families (LongSpec page, experiments),
# sized for one layer. Sweep entries differ only in tree size and shape.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, Hq=4, Hkv=1, D=64, T=8, L=256, dtype="f32",
                         tree="uniform"),
    "mha_7b": Workload("mha_7b", B=1, Hq=32, Hkv=32, D=128, T=64, L=16384),
    "gqa_64k": Workload("gqa_64k", B=4, Hq=32, Hkv=8, D=128, T=64, L=(32768, 65536)),
    "gqa_64k_pinned": Workload("gqa_64k_pinned", B=4, Hq=32, Hkv=8, D=128, T=64, L=65536),
    "sweep_t1": Workload("sweep_t1", B=8, Hq=32, Hkv=8, D=128, T=1, L=32768, tree="single"),
    "sweep_t6": Workload("sweep_t6", B=8, Hq=32, Hkv=8, D=128, T=6, L=32768, tree="chain"),
    "sweep_t16": Workload("sweep_t16", B=8, Hq=32, Hkv=8, D=128, T=16, L=32768),
    "sweep_t32": Workload("sweep_t32", B=8, Hq=32, Hkv=8, D=128, T=32, L=32768),
    "sweep_t64": Workload("sweep_t64", B=8, Hq=32, Hkv=8, D=128, T=64, L=32768),
    "sweep_t128": Workload("sweep_t128", B=8, Hq=32, Hkv=8, D=128, T=128, L=32768),
    "long_reasoning": Workload("long_reasoning", B=1, Hq=40, Hkv=8, D=128, T=128, L=131072,
                               depth_cap=12, outlier_channels=4),
    # Beam-search-shaped tree (LongSpec page, experimental details: beam widths per step),
    # cut to a 64-node budget.
    "gqa_64k_beam": Workload("gqa_64k_beam", B=4, Hq=32, Hkv=8, D=128, T=64, L=65536,
                             tree="beam", widths=(4, 16, 16, 16, 12)),
}


@dataclasses.dataclass
class Case:
    """Operands of one layer. All arrays are host numpy arrays in C order."""

    wl: Workload
    seed: int
    seq_lens: np.ndarray            # int32 [B]
    parent: np.ndarray              # int32 [B, T]
    q: np.ndarray                   # [B, T, Hq, D]
    k_cache: np.ndarray             # contiguous [B, Lcap, Hkv, D] or paged pool [P, page, Hkv, D]
    v_cache: np.ndarray
    k_tree: np.ndarray              # [B, T, Hkv, D]
    v_tree: np.ndarray
    block_table: Optional[np.ndarray] = None   # int32 [B, max_blocks] when paged
    page_size: int = 0
    lcap: int = 0                   # rows per sequence (contiguous) or max_blocks * page_size
    outlier_channels: Optional[np.ndarray] = None

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def dtype(self) -> str:
        return self.wl.dtype

    @property
    def scale(self) -> float:
        return self.wl.scale


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------------------------
# trees


def uniform_tree(rng: np.random.Generator, T: int) -> np.ndarray:
    """parent[i] drawn uniformly from [-1, i-1]."""
    return np.array([rng.integers(-1, i) for i in range(T)], dtype=np.int32)


def bounded_tree(rng: np.random.Generator, T: int, depth_cap: int, branch_cap: int) -> np.ndarray:
    """Random tree with node depth <= depth_cap and at most branch_cap children per node.

    Node i picks its parent uniformly among the eligible ones: the prefix (-1) while it has fewer
    than branch_cap children, and every earlier node j whose depth is below depth_cap and that
    has fewer than branch_cap children. Root-attached nodes have depth 1.
    """
    parent = np.empty(T, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int64)
    children = np.zeros(T, dtype=np.int64)
    root_children = 0
    for i in range(T):
        elig = [-1] if root_children < branch_cap else []
        elig += [j for j in range(i) if depth[j] < depth_cap and children[j] < branch_cap]
        p = elig[int(rng.integers(len(elig)))]
        parent[i] = p
        if p < 0:
            root_children += 1
            depth[i] = 1
        else:
            children[p] += 1
            depth[i] = depth[p] + 1
    return parent


def beam_tree(rng: np.random.Generator, widths, branch_cap: int) -> np.ndarray:
    """Layered tree: layer k has widths[k] nodes whose parents come from layer k-1."""
    parent = []
    prev = [-1]
    for w in widths:
        kids = {p: 0 for p in prev}
        layer = []
        for _ in range(w):
            elig = [p for p in prev if p < 0 or kids[p] < branch_cap]
            p = elig[int(rng.integers(len(elig)))]
            kids[p] += 1
            layer.append(len(parent))
            parent.append(p)
        prev = layer
    return np.array(parent, dtype=np.int32)


def make_tree(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    T = wl.T
    if wl.tree == "uniform":
        return uniform_tree(rng, T)
    if wl.tree == "bounded":
        return bounded_tree(rng, T, wl.depth_cap, wl.branch_cap)
    if wl.tree == "chain":
        return np.arange(-1, T - 1, dtype=np.int32)
    if wl.tree in ("star", "single"):
        return np.full(T, -1, dtype=np.int32)
    if wl.tree == "beam":
        par = beam_tree(rng, wl.widths, wl.branch_cap)
        assert len(par) == T, (len(par), T)
        return par
    raise ValueError(f"unknown tree kind {wl.tree!r}")


# ---------------------------------------------------------------------------------------------
# cases


_CHUNK_ROWS = 1 << 12
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1))
    return _POOL


def _draw_values(seed, key, shape, dtype, scale_channels=None, scale=1.0):
    """N(0,1) fp32 values of ``shape`` converted to ``dtype`` (bf16 bits or float32).

    The leading axis is cut into chunks of 4096 rows; chunk c draws from its own PCG64 stream
    seeded by SeedSequence([seed, *key, c]), so chunks can be drawn concurrently and a value
    never depends on the thread count. ``scale_channels`` multiplies the listed last-axis
    channels by ``scale`` before rounding.
    """
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty(shape, dtype=out_dtype)
    n = shape[0]

    def work(c):
        s, e = c * _CHUNK_ROWS, min(n, (c + 1) * _CHUNK_ROWS)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key, c])))
        x = rng.standard_normal((e - s,) + tuple(shape[1:]), dtype=np.float32)
        if scale_channels is not None and len(scale_channels):
            x[..., scale_channels] *= np.float32(scale)
        out[s:e] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    n_chunks = (n + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    if n_chunks <= 1:
        for c in range(n_chunks):
            work(c)
    else:
        list(_pool().map(work, range(n_chunks)))
    return out


def _pad_value(dtype, pad):
    if pad == "nan":
        return BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    return np.uint16(0) if dtype == "bf16" else np.float32(0.0)


def make_case(wl: Workload, seed: int = 0, *, layout: str = "contiguous", pad: str = "nan",
              page_size: int = 64, lens=None, parent=None, lcap: Optional[int] = None) -> Case:
    """Build the operands of ``wl`` for ``seed``.

    ``lens`` / ``parent`` override the drawn prefix lengths / parent arrays (the draws still
    happen, so the value streams do not shift). ``layout`` is "contiguous" or "paged"; the paged
    pool places each page at a seeded random physical slot, and unused block-table entries point
    at a page filled with the pad value.
    """
    if layout not in ("contiguous", "paged"):
        raise ValueError(layout)
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hq, Hkv, D = wl.B, wl.T, wl.Hq, wl.Hkv, wl.D
    if isinstance(wl.L, tuple):
        drawn = rng.integers(wl.L[0], wl.L[1], size=B, endpoint=True).astype(np.int32)
    else:
        drawn = np.full(B, int(wl.L), dtype=np.int32)
    seq_lens = drawn if lens is None else np.asarray(lens, dtype=np.int32).reshape(B)
    drawn_par = np.stack([make_tree(rng, wl) for _ in range(B)]) if T else np.zeros((B, 0), np.int32)
    par = drawn_par if parent is None else np.asarray(parent, dtype=np.int32).reshape(B, T)
    chans = None
    if wl.outlier_channels:
        chans = np.sort(rng.choice(D, wl.outlier_channels, replace=False)).astype(np.int64)

    dt = wl.dtype
    q = _draw_values(seed, (_Q, 0), (B * T, Hq, D), dt).reshape(B, T, Hq, D)
    padv = _pad_value(dt, pad)
    maxlen = int(seq_lens.max()) if B else 0
    if layout == "contiguous":
        cap = maxlen if lcap is None else int(lcap)
        if cap < maxlen:
            raise ValueError("lcap below the longest prefix")
        kc = np.full((B, cap, Hkv, D), padv)
        vc = np.full((B, cap, Hkv, D), padv)
        for b in range(B):
            kc[b, :seq_lens[b]] = _draw_values(seed, (_KP, b), (int(seq_lens[b]), Hkv, D), dt,
                                               chans, wl.outlier_scale)
        for b in range(B):
            vc[b, :seq_lens[b]] = _draw_values(seed, (_VP, b), (int(seq_lens[b]), Hkv, D), dt)
        block_table = None
        psz = 0
    else:
        psz = int(page_size)
        if psz < 16 or psz & (psz - 1):
            raise ValueError("page_size must be a power of two >= 16")
        npg = [(int(n) + psz - 1) // psz for n in seq_lens]
        max_blocks = max(max(npg) if npg else 0, 1)
        if lcap is not None:
            max_blocks = max(max_blocks, (int(lcap) + psz - 1) // psz)
        cap = max_blocks * psz
        n_pages = sum(npg) + 1                      # the last physical page is the pad page
        perm = np.random.Generator(np.random.PCG64([seed, 1])).permutation(n_pages - 1)
        pad_page = n_pages - 1
        kc = np.full((n_pages, psz, Hkv, D), padv)
        vc = np.full((n_pages, psz, Hkv, D), padv)
        block_table = np.full((B, max_blocks), pad_page, dtype=np.int32)
        nxt = 0
        for b in range(B):
            for blk in range(npg[b]):
                block_table[b, blk] = perm[nxt]
                nxt += 1

        def scatter(dst, b, vals):
            n = int(seq_lens[b])
            for blk in range(npg[b]):
                rows = vals[blk * psz:min(n, (blk + 1) * psz)]
                dst[block_table[b, blk], :len(rows)] = rows

        for b in range(B):
            scatter(kc, b, _draw_values(seed, (_KP, b), (int(seq_lens[b]), Hkv, D), dt, chans,
                                        wl.outlier_scale))
        for b in range(B):
            scatter(vc, b, _draw_values(seed, (_VP, b), (int(seq_lens[b]), Hkv, D), dt))
    kt = _draw_values(seed, (_KT, 0), (B * T, Hkv, D), dt, chans,
                      wl.outlier_scale).reshape(B, T, Hkv, D)
    vt = _draw_values(seed, (_VT, 0), (B * T, Hkv, D), dt).reshape(B, T, Hkv, D)
    return Case(wl=wl, seed=seed, seq_lens=seq_lens, parent=par, q=q, k_cache=kc, v_cache=vc,
                k_tree=kt, v_tree=vt, block_table=block_table, page_size=psz, lcap=cap,
                outlier_channels=chans)


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of every node of one parent array (root-attached nodes have depth 1)."""
    d = np.zeros(len(parent), dtype=np.int64)
    for i, p in enumerate(parent):
        d[i] = 1 if p < 0 else d[p] + 1
    return d


# ---------------------------------------------------------------------------------------------
# greedy acceptance and commit operands

@dataclasses.dataclass
class AcceptCase:
    """Operands of greedy tree acceptance: target logits [B, T + 1, V] (row 0 = the position of
    the last committed token, row i + 1 = tree node i; bf16 bits or float32), draft tokens and
    parent arrays [B, T]."""

    logits: np.ndarray
    draft: np.ndarray
    parent: np.ndarray
    dtype: str

    @property
    def V(self) -> int:
        return self.logits.shape[-1]


def make_accept_case(B: int, T: int, V: int, seed: int = 0, *, tree: str = "bounded",
                     dtype: str = "bf16", plant: float = 0.8, ties: float = 0.15,
                     blocks: float = 0.05, depth_cap: int = 8, branch_cap: int = 4) -> AcceptCase:
    """Logits N(0, 1) clipped to [-6, 6]; draft tokens uniform in [0, V). In every row, with
    probability ``plant``, one child of that row's node (row 0: a root-attached node) gets its
    draft token's logit set to 7 -- the row's unique maximum by construction, so the child agrees
    with the target; with probability ``ties`` a second random index of that row is also set to
    7 (equal maxima: the first index wins); with probability ``blocks`` two random indices are set
    to 7.5 instead (a maximum no draft token is likely to hit). Nothing here computes an argmax."""
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    wl = Workload("accept", B=B, Hq=1, Hkv=1, D=64, T=T, L=0, tree=tree, depth_cap=depth_cap,
                  branch_cap=branch_cap)
    parent = np.stack([make_tree(rng, wl) for _ in range(B)]).astype(np.int32)
    draft = rng.integers(0, V, size=(B, T), dtype=np.int32)
    x = rng.standard_normal((B, T + 1, V), dtype=np.float32)
    np.clip(x, -6.0, 6.0, out=x)
    for b in range(B):
        kids = [[] for _ in range(T + 1)]
        for i in range(T):
            kids[int(parent[b, i]) + 1].append(i)
        for r in range(T + 1):
            if kids[r] and rng.random() < plant:
                c = kids[r][int(rng.integers(len(kids[r])))]
                x[b, r, draft[b, c]] = 7.0
                if rng.random() < ties:
                    x[b, r, int(rng.integers(V))] = 7.0
            if rng.random() < blocks:
                x[b, r, rng.integers(V, size=2)] = 7.5
    logits = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return AcceptCase(logits=logits, draft=draft, parent=parent, dtype=dtype)


def random_paths(parent: np.ndarray, rng: np.random.Generator, max_len=None):
    """One root path per sequence (root first) ending at a random node, or empty: the shape of
    what greedy acceptance commits. Returns (path [B, T] padded with -1, accept_len [B])."""
    B, T = parent.shape
    path = np.full((B, T), -1, np.int32)
    n = np.zeros(B, np.int32)
    for b in range(B):
        end = int(rng.integers(-1, T))
        chain = []
        while end >= 0:
            chain.append(end)
            end = int(parent[b, end])
        chain.reverse()
        if max_len is not None:
            chain = chain[:max_len]
        path[b, :len(chain)] = chain
        n[b] = len(chain)
    return path, n


@dataclasses.dataclass
class SpecCase:
    """Operands of tree speculative sampling: target and candidate distributions p, q float32
    [B, T + 1, V] (row 0 = the position after the last committed token, row i + 1 = after tree
    node i), draft tokens and parent arrays int32 [B, T], uniforms u_accept float64 [B, T] and
    u_sample float64 [B]."""

    p: np.ndarray
    q: np.ndarray
    draft: np.ndarray
    parent: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z, dtype=np.float64)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def make_spec_case(B: int, T: int, V: int, seed: int = 0, *, tree: str = "bounded",
                   mode: str = "overlap", sharp: float = 2.5, noise: float = 1.0,
                   depth_cap: int = 8, branch_cap: int = 4) -> SpecCase:
    """Target rows p = softmax(N(0, sharp^2) logits); candidate rows q = softmax of the same
    logits plus N(0, noise^2) (partial overlap). ``mode`` "same": q = p; "disjoint": p keeps only
    the odd tokens and q only the even ones (renormalised). The children of every position are
    drawn independently from that position's q row (inverse CDF of a seeded uniform), as a
    drafter sampling them would. Uniforms are seeded float64 in [0, 1)."""
    rng = np.random.Generator(np.random.PCG64([seed, 11]))
    wl = Workload("spec", B=B, Hq=1, Hkv=1, D=64, T=T, L=0, tree=tree, depth_cap=depth_cap,
                  branch_cap=branch_cap)
    parent = np.stack([make_tree(rng, wl) for _ in range(B)]).astype(np.int32)
    p = np.empty((B, T + 1, V), np.float32)
    q = np.empty((B, T + 1, V), np.float32)
    for b in range(B):
        z = rng.standard_normal((T + 1, V), dtype=np.float32) * np.float32(sharp)
        p[b] = _softmax_rows(z)
        if mode == "same":
            q[b] = p[b]
        elif mode == "disjoint":
            mask = (np.arange(V) % 2).astype(np.float32)
            pp = p[b] * mask
            qq = _softmax_rows(z) * (1.0 - mask)
            p[b] = (pp / pp.sum(axis=-1, keepdims=True)).astype(np.float32)
            q[b] = (qq / qq.sum(axis=-1, keepdims=True)).astype(np.float32)
        else:
            q[b] = _softmax_rows(z + rng.standard_normal((T + 1, V), dtype=np.float32)
                                 * np.float32(noise))
    draft = np.zeros((B, T), np.int32)
    for b in range(B):
        for i in range(T):
            row = q[b, int(parent[b, i]) + 1].astype(np.float64)
            c = np.cumsum(row)
            draft[b, i] = min(int(np.searchsorted(c, rng.random() * c[-1], side="right")), V - 1)
    u_accept = rng.random((B, T))
    u_sample = rng.random(B)
    return SpecCase(p=p, q=q, draft=draft, parent=parent, u_accept=u_accept, u_sample=u_sample)


@dataclasses.dataclass
class GdnCase:
    """Operands of one gated-delta-net layer's tree verification: q, k [B, T, H_k, d_k] and v
    [B, T, H_v, d_v] (bf16 bits), log-decays g and write strengths beta fp32 [B, T, H_v], parent
    int32 [B, T], committed states S0 fp32 [B, H_v, d_k, d_v], output scale."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    parent: np.ndarray
    S0: np.ndarray
    scale: float


def make_gdn_case(B: int, T: int, Hk: int = 16, Hv: int = 32, dk: int = 128, dv: int = 128,
                  seed: int = 0, *, tree: str = "bounded", depth_cap: int = 8,
                  branch_cap: int = 4) -> GdnCase:
    """q and k N(0, 1) rows scaled to unit length (as the layer's L2 normalisation does) and
    rounded to bf16; v N(0, 1) in bf16; g uniform in [-0.2, -0.01] (alpha = e^g in about
    [0.82, 0.99]); beta uniform in [0.05, 0.95]; S0 N(0, 0.05^2); scale 1 / sqrt(d_k)."""
    rng = np.random.Generator(np.random.PCG64([seed, 13]))
    wl = Workload("gdn", B=B, Hq=1, Hkv=1, D=64, T=T, L=0, tree=tree, depth_cap=depth_cap,
                  branch_cap=branch_cap)
    parent = np.stack([make_tree(rng, wl) for _ in range(B)]).astype(np.int32)

    def unit(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        x /= np.linalg.norm(x, axis=-1, keepdims=True)
        return f32_to_bf16_bits(x)

    q = unit((B, T, Hk, dk))
    k = unit((B, T, Hk, dk))
    v = f32_to_bf16_bits(rng.standard_normal((B, T, Hv, dv), dtype=np.float32))
    g = rng.uniform(-0.2, -0.01, (B, T, Hv)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (B, T, Hv)).astype(np.float32)
    S0 = (rng.standard_normal((B, Hv, dk, dv), dtype=np.float32) * np.float32(0.05))
    return GdnCase(q=q, k=k, v=v, g=g, beta=beta, parent=parent, S0=S0, scale=float(dk) ** -0.5)
