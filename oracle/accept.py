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

Tree speculative sampling (textbook page, "Faster decoding", section on modified rejection sampling
keeping the target distribution): at one position a candidate X drawn from the candidate
distribution q is accepted with probability a(v) = min(1, p(v) / q(v)); on rejection the emitted
token is drawn from the residual r = [p - q]_+ / Z, Z = sum_u [p - q]_+ (the rejection
probability; Z = 0 means nothing is ever rejected). The pages apply this left to right along a
chain, stop at the first rejection with a correction token, and draw a bonus token from the
target's next distribution when every candidate is accepted. Tree reading (the pages give no
tree rule): the children of a position are candidates drawn independently from that position's
q and are tried in index order; after a rejection the residual takes the place of p for the next
child (the same identity applied again), so a chain is exactly the pages' rule. All children
rejected: the correction token is drawn from the last residual; an accepted node without
children ends the path with a bonus token drawn from its row's p. Randomness comes in as
uniforms in [0, 1): u_accept per node, u_sample per sequence; accept iff u < a, and a token is
drawn from weights w as the smallest index whose running sum of w exceeds u * sum(w).

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


def sample_index(w: np.ndarray, u: float) -> int:
    """The smallest index whose running sum of the non-negative weights w exceeds u * sum(w); if
    rounding leaves none, the last index with positive weight (0 if there is none)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    hit = np.nonzero(c > u * c[-1])[0]
    if hit.size:
        return int(hit[0])
    pos = np.nonzero(w > 0)[0]
    return int(pos[-1]) if pos.size else 0


def spec_sample(p: np.ndarray, q: np.ndarray, draft: np.ndarray, parent: np.ndarray,
                u_accept: np.ndarray, u_sample: np.ndarray):
    """p, q: float32 [B, T + 1, V] target and candidate distributions (row 0 at the last
    committed token, row i + 1 at tree node i: the distributions of the next token there);
    draft / parent int32 [B, T]; u_accept float64 [B, T]; u_sample float64 [B].

    Returns (accept_len [B], path [B, T] (root first, -1 past the end), next_token [B])."""
    B, T = draft.shape
    acc_len = np.zeros(B, np.int32)
    path = np.full((B, T), -1, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        kids = [[] for _ in range(T + 1)]          # kids[pos + 1]: children of pos, index order
        for i in range(T):
            pa = int(parent[b, i])
            if pa < -1 or pa >= i:
                raise ValueError(f"parent[{b}][{i}] = {pa} is not in [-1, {i - 1}]")
            kids[pa + 1].append(i)
            if not 0 <= int(draft[b, i]) < p.shape[2]:
                raise ValueError(f"draft[{b}][{i}] = {int(draft[b, i])} is outside the vocabulary")
        chain, pos = [], -1
        while True:
            row = pos + 1
            target = p[b, row].astype(np.float64)  # the pages' p at this position
            cand = q[b, row].astype(np.float64)    # the pages' q
            taken = None
            for c in kids[row]:
                x = int(draft[b, c])
                excess = np.maximum(target - cand, 0.0)
                Z = excess.sum()
                if Z == 0.0:
                    a = 1.0                        # no rejection is possible
                elif cand[x] > 0.0:
                    a = min(1.0, target[x] / cand[x])
                else:
                    a = 1.0 if target[x] > 0.0 else 0.0
                if u_accept[b, c] < a:
                    taken = c
                    break
                target = excess / Z                # the residual r replaces p for the next child
            if taken is None:
                # every child rejected: correction from the last residual; no child: bonus from p
                nxt[b] = sample_index(target, float(u_sample[b]))
                break
            chain.append(taken)
            pos = taken
        acc_len[b] = len(chain)
        path[b, :len(chain)] = chain
    return acc_len, path, nxt


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
