"""Pins of the tree speculative-sampling oracle (CPU only).

The property the pages build the method on (textbook page, "Faster decoding", section on modified
rejection sampling keeping the target distribution) is that the emitted tokens follow the target
distribution p whatever the candidate distribution q is. Following the pages' own test advice
(same page, correctness tests: a tiny vocabulary with p = q, partial overlap and disjoint supports;
forced first rejection, late rejection and full acceptance), these pins check the oracle's output
frequencies against p by seeded Monte Carlo on tiny vocabularies, and check closed forms of the
degenerate cases. None of them restates the oracle's acceptance formula.
"""
import numpy as np
import pytest

import oracle.accept as A


def run(p_rows, q_rows, parent, drafts, u_acc, u_smp):
    """Broadcast one tree's rows over N sequences with per-sequence drafts and uniforms."""
    N, T = drafts.shape
    p = np.broadcast_to(np.asarray(p_rows, np.float32), (N,) + np.shape(p_rows))
    q = np.broadcast_to(np.asarray(q_rows, np.float32), (N,) + np.shape(q_rows))
    par = np.broadcast_to(np.asarray(parent, np.int32), (N, T))
    return A.spec_sample(p, q, drafts.astype(np.int32), par, u_acc, u_smp)


def draw(rng, q_row, n):
    c = np.cumsum(np.asarray(q_row, np.float64))
    return np.minimum(np.searchsorted(c, rng.random(n) * c[-1], side="right"), len(c) - 1)


def close_to(freq, target, n, sig=5.0):
    target = np.asarray(target, np.float64)
    tol = sig * np.sqrt(np.maximum(target * (1 - target), 1e-4) / n) + 1e-9
    assert np.all(np.abs(freq - target) <= tol), (freq, target, tol)


P = [0.5, 0.3, 0.2, 0.0]
Q_PARTIAL = [0.1, 0.1, 0.1, 0.7]


@pytest.mark.parametrize("q_row", [P, Q_PARTIAL, [0.0, 0.0, 0.0, 1.0], [0.25, 0.25, 0.25, 0.25]],
                         ids=["p_eq_q", "partial", "disjoint", "flat"])
@pytest.mark.parametrize("K", [1, 2, 3])
def test_first_token_follows_p_with_k_sibling_candidates(q_row, K):
    # K root children drawn independently from q; the first emitted token (the accepted child's
    # token, else the correction) must be distributed as p
    rng = np.random.default_rng(100 + K)
    N = 30000
    parent = [-1] * K
    p_rows = [P] * (K + 1)
    q_rows = [q_row] * (K + 1)
    drafts = np.stack([draw(rng, q_row, N) for _ in range(K)], axis=1)
    n, path, nxt = run(p_rows, q_rows, parent, drafts, rng.random((N, K)), rng.random(N))
    first = np.where(n > 0, drafts[np.arange(N), np.maximum(path[:, 0], 0)], nxt)
    close_to(np.bincount(first, minlength=4) / N, P, N)


def test_every_emitted_token_of_a_chain_follows_its_row():
    # chain of 3 candidates, rows with different p and q: given that a round emits at least k
    # tokens, its k-th token follows row k-1's p
    rng = np.random.default_rng(7)
    N = 40000
    p_rows = [[0.6, 0.3, 0.1], [0.2, 0.2, 0.6], [0.1, 0.8, 0.1], [0.3, 0.3, 0.4]]
    q_rows = [[0.3, 0.3, 0.4], [0.5, 0.4, 0.1], [0.1, 0.6, 0.3], [1 / 3, 1 / 3, 1 / 3]]
    drafts = np.stack([draw(rng, q_rows[k], N) for k in range(3)], axis=1)
    n, path, nxt = run(p_rows, q_rows, [-1, 0, 1], drafts, rng.random((N, 3)), rng.random(N))
    for k in range(4):
        reach = n >= k
        tok = np.where(n[reach] > k, drafts[reach][:, min(k, 2)], nxt[reach])
        close_to(np.bincount(tok, minlength=3) / reach.sum(), p_rows[k], reach.sum())
    # the accepted prefix is a prefix of the chain
    for b in range(200):
        assert list(path[b, :n[b]]) == list(range(n[b]))


def test_tree_with_branching_follows_p_at_depth_two():
    # root with 2 children, each with 2 children; q rows differ per position: the second emitted
    # token (when a round emits two) follows p of the first accepted node's row
    rng = np.random.default_rng(3)
    N = 40000
    parent = [-1, -1, 0, 0, 1, 1]
    p_rows = [[0.4, 0.4, 0.2], [0.1, 0.2, 0.7], [0.5, 0.25, 0.25]] + [[1 / 3] * 3] * 4
    q_rows = [[0.2, 0.2, 0.6], [0.4, 0.4, 0.2], [0.1, 0.1, 0.8]] + [[1 / 3] * 3] * 4
    d0 = draw(rng, q_rows[0], N), draw(rng, q_rows[0], N)
    d1 = draw(rng, q_rows[1], N), draw(rng, q_rows[1], N)
    d2 = draw(rng, q_rows[2], N), draw(rng, q_rows[2], N)
    drafts = np.stack([d0[0], d0[1], d1[0], d1[1], d2[0], d2[1]], axis=1)
    n, path, nxt = run(p_rows, q_rows, parent, drafts, rng.random((N, 6)), rng.random(N))
    first = np.where(n > 0, drafts[np.arange(N), np.maximum(path[:, 0], 0)], nxt)
    close_to(np.bincount(first, minlength=3) / N, p_rows[0], N)
    for node, row in ((0, 1), (1, 2)):
        sel = (n >= 1) & (path[:, 0] == node)
        tok = np.where(n[sel] >= 2, drafts[sel, np.maximum(path[sel, 1], 0)], nxt[sel])
        close_to(np.bincount(tok, minlength=3) / sel.sum(), p_rows[row], sel.sum())


def test_p_equal_q_accepts_the_first_child_chain():
    rng = np.random.default_rng(5)
    V = 16
    row = rng.random(V).astype(np.float32)
    row /= row.sum()
    parent = np.array([[-1, -1, 0, 0, 2, 1, 4]], np.int32)
    rows = np.broadcast_to(row, (1, 8, V)).copy()
    drafts = rng.integers(0, V, (1, 7)).astype(np.int32)
    n, path, nxt = A.spec_sample(rows, rows, drafts, parent, np.full((1, 7), 0.999999),
                                 np.array([0.0]))
    # first children: root -> 0 -> 2 -> 4 -> 6 (a leaf)
    assert n[0] == 4 and list(path[0, :4]) == [0, 2, 4, 6]
    assert nxt[0] == int(np.nonzero(row > 0)[0][0])     # u = 0: the first token with mass


def test_disjoint_supports_reject_everything_and_correct_from_p():
    V = 10
    p = np.zeros(V, np.float32)
    p[1::2] = 0.2                                        # uniform over the odd tokens
    q = np.zeros(V, np.float32)
    q[0::2] = 0.2
    parent = np.array([[-1, -1, -1, 0]], np.int32)
    rows_p = np.broadcast_to(p, (1, 5, V)).copy()
    rows_q = np.broadcast_to(q, (1, 5, V)).copy()
    for u in (0.05, 0.3, 0.55, 0.95):
        n, path, nxt = A.spec_sample(rows_p, rows_q, np.array([[0, 2, 4, 6]], np.int32), parent,
                                     np.zeros((1, 4)), np.array([u]))
        assert n[0] == 0 and np.all(path == -1)
        assert nxt[0] == 2 * int(u * 5) + 1


def test_forced_rejection_depths():
    # drafted tokens carry p >= q (always accepted) down to depth d, then p = 0 (always
    # rejected): the accepted length is d, whatever the uniforms
    V = 6
    T = 5
    parent = np.array([[-1, 0, 1, 2, 3]], np.int32)
    for d in range(T + 1):
        p = np.full((1, T + 1, V), 0.1, np.float32)
        q = np.full((1, T + 1, V), 0.1, np.float32)
        p[0, :, 0] = 0.5
        q[0, :, 0] = 0.5
        drafts = np.zeros((1, T), np.int32)
        if d < T:
            p[0, d, 0] = 0.0
            p[0, d, 1] = 0.6
        n, path, nxt = A.spec_sample(p, q, drafts, parent, np.full((1, T), 0.999),
                                     np.array([0.3]))
        assert n[0] == d and list(path[0, :d]) == list(range(d))
        if d < T:
            assert nxt[0] == 1                           # residual mass sits on token 1 only
        else:
            assert nxt[0] == 0                           # bonus from the leaf's p: 0.5 on token 0


def test_zero_residual_mass_means_no_rejection():
    # p <= q everywhere: Z = 0, so the candidate is accepted even by a uniform above p(x)/q(x)
    V = 5
    p = np.full((1, 2, V), 0.1, np.float32)
    q = np.full((1, 2, V), 0.2, np.float32)
    n, path, _ = A.spec_sample(p, q, np.array([[3]], np.int32), np.array([[-1]], np.int32),
                               np.array([[0.99]]), np.array([0.5]))
    assert n[0] == 1 and path[0, 0] == 0


def test_sample_index_closed_forms():
    for k in range(7):
        w = np.zeros(7)
        w[k] = 3.0
        for u in (0.0, 0.5, 0.999):
            assert A.sample_index(w, u) == k
    for u in np.linspace(0.01, 0.99, 37):
        assert A.sample_index(np.ones(9), u) == int(u * 9)
    assert A.sample_index(np.zeros(4), 0.3) == 0
    # u * sum(w) landing exactly on a running sum belongs to the next index (u = k / n exactly)
    for k in range(4):
        assert A.sample_index(np.ones(4), k / 4) == k
    assert A.sample_index(np.array([0.0, 2.0, 0.0, 2.0]), 0.5) == 3


def test_bad_parent_raises():
    p = np.full((1, 3, 4), 0.25, np.float32)
    with pytest.raises(ValueError):
        A.spec_sample(p, p, np.zeros((1, 2), np.int32), np.array([[-1, 1]], np.int32),
                      np.zeros((1, 2)), np.zeros(1))
