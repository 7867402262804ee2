"""Pins of the greedy-acceptance and KV-commit oracle (CPU only).

The greedy contract (textbook page, "Faster decoding": accept the longest prefix that agrees with
the target's greedy tokens, then emit the target's token at the first disagreement) is checked
against independent restatements: linear speculation on a chain, brute-force enumeration of every
root path on small trees, and direct constructions of the tie and NaN rules. The commit is checked
for layout independence and for leaving everything outside the committed rows untouched.
"""
import itertools

import numpy as np
import pytest

import oracle.accept as A
from tree_verification_attention_amd import inputs


def py_argmax(row):
    """First maximal index among the non-NaN entries by a plain scan; all NaN gives 0."""
    best, idx, found = 0.0, 0, False
    for j, v in enumerate(row):
        if v == v and (not found or v > best):
            best, idx, found = v, j, True
    return idx


def widen(case):
    if case.dtype == "bf16":
        return inputs.bf16_bits_to_f32(case.logits).astype(np.float64)
    return case.logits.astype(np.float64)


def brute(case, b):
    """Every root path whose nodes all agree with their parent row's greedy token; the longest
    wins, ties to the path ending at the smallest node index."""
    x = widen(case)[b]
    T = case.draft.shape[1]
    g = [py_argmax(list(x[r])) for r in range(T + 1)]
    par = case.parent[b]
    best = []
    for end in range(T):
        chain, j = [], end
        while j >= 0:
            chain.append(j)
            j = int(par[j])
        chain.reverse()
        ok = all(case.draft[b, n] == g[int(par[n]) + 1] for n in chain)
        if ok and (len(chain) > len(best) or (len(chain) == len(best) and chain[-1] < best[-1])):
            best = chain
    nxt = g[best[-1] + 1] if best else g[0]
    return best, nxt, g


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chain_equals_linear_speculation(dtype):
    for seed in range(6):
        c = inputs.make_accept_case(3, 7, 40, seed, tree="chain", dtype=dtype, plant=0.85,
                                    ties=0.2, blocks=0.0)
        g, n, path, nxt = A.greedy_accept(c.logits, c.draft, c.parent, c.dtype)
        x = widen(c)
        for b in range(3):
            gl = [py_argmax(list(x[b, r])) for r in range(8)]
            k = 0
            while k < 7 and c.draft[b, k] == gl[k]:
                k += 1
            assert n[b] == k
            assert list(path[b, :k]) == list(range(k)) and np.all(path[b, k:] == -1)
            assert nxt[b] == gl[k]
            assert list(g[b]) == gl


def test_brute_force_every_small_tree():
    checked = 0
    for T in range(1, 5):
        for par in itertools.product(*[range(-1, i) for i in range(T)]):
            for seed in range(2):
                c = inputs.make_accept_case(1, T, 12, seed + 10 * T, tree="uniform", plant=0.9,
                                            ties=0.3, blocks=0.1)
                c.parent[0] = np.array(par, np.int32)
                # re-plant against this parent array: agreement follows the rows of its parents
                rng = np.random.default_rng(seed)
                x = widen(c)[0]
                for i in range(T):
                    if rng.random() < 0.8:
                        x[par[i] + 1, c.draft[0, i]] = 7.0
                c.logits[0] = inputs.f32_to_bf16_bits(x.astype(np.float32))
                g, n, path, nxt = A.greedy_accept(c.logits, c.draft, c.parent, c.dtype)
                best, bnxt, bg = brute(c, 0)
                assert n[0] == len(best) and list(path[0, :n[0]]) == best, (par, seed)
                assert nxt[0] == bnxt and list(g[0]) == bg
                checked += 1
    assert checked > 60


def test_random_trees_invariants():
    c = inputs.make_accept_case(6, 64, 500, 3, plant=0.95, ties=0.1, blocks=0.02)
    g, n, path, nxt = A.greedy_accept(c.logits, c.draft, c.parent, c.dtype)
    assert n.max() >= 3
    for b in range(6):
        best, bnxt, _ = brute(c, b)
        assert n[b] == len(best) and list(path[b, :n[b]]) == best and nxt[b] == bnxt
        p = list(path[b, :n[b]])
        if p:
            assert c.parent[b, p[0]] == -1
            assert all(c.parent[b, p[k]] == p[k - 1] for k in range(1, len(p)))
            assert all(c.draft[b, v] == g[b, c.parent[b, v] + 1] for v in p)
            # maximality: no child of the last node agrees with the last node's greedy token
            kids = [i for i in range(64) if c.parent[b, i] == p[-1]]
            assert all(c.draft[b, i] != g[b, p[-1] + 1] for i in kids)


def test_tie_and_nan_rules():
    x = np.zeros((1, 2, 10), np.float32)
    x[0, 0, [7, 3]] = 5.0           # equal maxima: the first index wins
    x[0, 1, 0] = np.nan
    x[0, 1, 4] = 2.0                # NaN never wins
    g = A.greedy_tokens(x, "f32")
    assert g[0, 0] == 3 and g[0, 1] == 4
    y = np.full((1, 1, 5), np.nan, np.float32)
    assert A.greedy_tokens(y, "f32")[0, 0] == 0
    z = np.full((1, 1, 5), -np.inf, np.float32)
    assert A.greedy_tokens(z, "f32")[0, 0] == 0
    w = np.array([[[np.nan, -np.inf, -np.inf]]], np.float32)   # -inf is the non-NaN maximum
    assert A.greedy_tokens(w, "f32")[0, 0] == 1 == py_argmax(list(w[0, 0]))


def test_star_accepts_at_most_one_node():
    c = inputs.make_accept_case(4, 20, 64, 5, tree="star", plant=1.0, ties=0.0, blocks=0.0)
    _, n, path, _ = A.greedy_accept(c.logits, c.draft, c.parent, c.dtype)
    assert np.all(n == 1)


def test_commit_contiguous_equals_paged_and_touches_only_the_path():
    wl = inputs.Workload("c", B=3, Hq=4, Hkv=2, D=64, T=12, L=(5, 130))
    rng = np.random.default_rng(0)
    cc = inputs.make_case(wl, 1, layout="contiguous", pad="finite", lcap=160)
    cp = inputs.make_case(wl, 1, layout="paged", pad="finite", page_size=16, lcap=160)
    path, n = inputs.random_paths(cc.parent, rng)
    kc, vc, lens = A.commit_kv(cc.k_cache, cc.v_cache, cc.seq_lens, cc.k_tree, cc.v_tree, path, n)
    kp, vp, lensp = A.commit_kv(cp.k_cache, cp.v_cache, cp.seq_lens, cp.k_tree, cp.v_tree, path, n,
                                block_table=cp.block_table, page_size=cp.page_size)
    assert np.array_equal(lens, cc.seq_lens + n) and np.array_equal(lens, lensp)
    for b in range(3):
        L = int(cc.seq_lens[b])
        for pos in range(int(lens[b])):
            pg, r = cp.block_table[b, pos // 16], pos % 16
            assert np.array_equal(kc[b, pos], kp[pg, r]) and np.array_equal(vc[b, pos], vp[pg, r])
        for j in range(n[b]):
            assert np.array_equal(kc[b, L + j], cc.k_tree[b, path[b, j]])
        # rows before L and after the new length are untouched
        assert np.array_equal(kc[b, :L], cc.k_cache[b, :L])
        assert np.array_equal(kc[b, lens[b]:], cc.k_cache[b, lens[b]:])


def test_commit_past_capacity_writes_nothing():
    wl = inputs.Workload("c", B=2, Hq=2, Hkv=1, D=64, T=8, L=62, tree="chain")
    c = inputs.make_case(wl, 0, pad="finite", lcap=64)
    path = np.tile(np.arange(8, dtype=np.int32), (2, 1))
    n = np.array([2, 3], np.int32)          # 62 + 2 fits, 62 + 3 does not
    kc, vc, lens = A.commit_kv(c.k_cache, c.v_cache, c.seq_lens, c.k_tree, c.v_tree, path, n)
    assert list(lens) == [64, 62]
    assert np.array_equal(kc[1], c.k_cache[1]) and np.array_equal(vc[1], c.v_cache[1])
