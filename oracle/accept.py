"""CPU oracle for greedy tree acceptance and accepted-path KV commit -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import this
module. It imports nothing from the HIP package.

Greedy verification (textbook page, "Faster decoding", the greedy verification contract): the
target model's greedy token at every position is the argmax of its logits; the longest draft
prefix that agrees with those greedy tokens is accepted, and the target's greedy token after the
last accepted position is emitted as the correction (or bonus) token. On a draft tree (nodes in
topological order, parent[i] in [-1, i-1], -1 = hanging off the committed prefix):

  * logits row 0 of a sequence is the position of its last committed token, row i + 1 is tree
    node i; g[r] = argmax of row r, the first index holding the maximum of the row's non-NaN
    entries (a row of NaN only gives 0);
  * node i agrees iff draft[i] == g[0] (root-attached) or draft[i] == g[parent[i] + 1];
  * node i is accepted iff it agrees and its parent is accepted (or it is root-attached);
  * the committed path runs from the root to the deepest accepted node (smallest node index among
    equally deep ones); the correction token is g at that node's row, or g[0] if none is accepted.

Commit (textbook page, "Faster decoding", reserve / execute / commit: after verification only the
target KV of the accepted draft prefix is committed; rejected branches are released, and the
correction token's KV is produced by the next round): the K/V rows of the path's nodes are copied,
in path order, to cache positions L_b, L_b + 1, ... of their sequence, and the length becomes
L_b + accept_len. A commit past the cache capacity writes nothing for that sequence and keeps its
length.
"""
from __future__ import annotations

import numpy as np


def _widen(logits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        a = np.asarray(logits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return a.view(np.float32).astype(np.float64)
    return np.asarray(logits, dtype=np.float32).astype(np.float64)


def greedy_tokens(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Argmax of every logits row (last axis): the first index holding the row's maximum over its
    non-NaN entries (so -inf can win a row of -inf and NaN); a row of NaN only gives 0."""
    x = _widen(logits, dtype)
    nan = np.isnan(x)
    m = np.where(nan, -np.inf, x).max(axis=-1, keepdims=True)
    return np.argmax((x == m) & ~nan, axis=-1).astype(np.int32)


def greedy_accept(logits: np.ndarray, draft: np.ndarray, parent: np.ndarray, dtype: str):
    """logits [B, T + 1, V] (bf16 bits or fp32), draft / parent int32 [B, T].

    Returns (greedy [B, T + 1], accept_len [B], path [B, T] (root first, -1 past the end),
    next_token [B])."""
    B, T = draft.shape
    g = greedy_tokens(logits, dtype)
    acc_len = np.zeros(B, np.int32)
    path = np.full((B, T), -1, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        accepted = [False] * T
        depth = [0] * T
        best = -1
        for i in range(T):
            p = int(parent[b, i])
            if p < -1 or p >= i:
                raise ValueError(f"parent[{b}][{i}] = {p} is not in [-1, {i - 1}]")
            want = g[b, 0] if p < 0 else g[b, p + 1]
            if draft[b, i] == want and (p < 0 or accepted[p]):
                accepted[i] = True
                depth[i] = 1 if p < 0 else depth[p] + 1
                if best < 0 or depth[i] > depth[best]:
                    best = i
        if best < 0:
            nxt[b] = g[b, 0]
            continue
        chain = []
        j = best
        while j >= 0:
            chain.append(j)
            j = int(parent[b, j])
        chain.reverse()
        acc_len[b] = len(chain)
        path[b, :len(chain)] = chain
        nxt[b] = g[b, best + 1]
    return g, acc_len, path, nxt


def commit_kv(k_cache, v_cache, seq_lens, k_tree, v_tree, path, accept_len, *, block_table=None,
              page_size=None):
    """Returns copies of (k_cache, v_cache) with the accepted rows written, and the new lengths.

    Contiguous caches are [B, Lmax, Hkv, D]; paged pools are [P, page_size, Hkv, D] with
    block_table [B, max_blocks]. Tree K/V are [B, T, Hkv, D]."""
    kc, vc = k_cache.copy(), v_cache.copy()
    new_lens = np.asarray(seq_lens, np.int32).copy()
    B = len(new_lens)
    cap = block_table.shape[1] * page_size if block_table is not None else kc.shape[1]
    for b in range(B):
        L, n = int(seq_lens[b]), int(accept_len[b])
        if n <= 0:
            continue
        if L + n > cap:
            continue
        for j in range(n):
            node, pos = int(path[b, j]), L + j
            if block_table is None:
                kc[b, pos] = k_tree[b, node]
                vc[b, pos] = v_tree[b, node]
            else:
                pg = int(block_table[b, pos // page_size])
                kc[pg, pos % page_size] = k_tree[b, node]
                vc[pg, pos % page_size] = v_tree[b, node]
        new_lens[b] = L + n
    return kc, vc, new_lens
