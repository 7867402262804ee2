"""Pins of the gated-delta-net tree-verification oracle (CPU only).

Closed forms of the delta rule (DFlash-TfM summary page, "Rollback-free tree verification for
GDN": S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T): with a unit key and
beta = 1 the state maps that key exactly to the new value; with beta = 0 it only decays; with
orthonormal keys and alpha = 1 it is the sum of the path's outer products; a node reads nothing
off its root path; and the deferred commit continues exactly as the tree did.
"""
import numpy as np
import pytest

import oracle.gdn as G
from tree_verification_attention_amd import inputs


def f32_case(B=2, T=12, Hk=2, Hv=4, dk=16, dv=8, seed=0, tree="bounded"):
    c = inputs.make_gdn_case(B, T, Hk, Hv, dk, dv, seed, tree=tree)
    # fp32 operands: the bf16 bits widened, so closed forms can set exact values
    w = lambda a: (a.astype(np.uint32) << 16).view(np.float32).copy()
    return c, w(c.q), w(c.k), w(c.v)


def path_of(parent, b, i):
    out = []
    while i >= 0:
        out.append(i)
        i = int(parent[b, i])
    return out[::-1]


def run(c, q, k, v, **kw):
    args = dict(g=c.g, beta=c.beta, parent=c.parent, S0=c.S0)
    args.update(kw)
    return G.gdn_tree_verify(q, k, v, args["g"], args["beta"], args["parent"], args["S0"],
                             c.scale, dtype="f32")


def test_unit_key_with_full_write_returns_the_value():
    c, q, k, v = f32_case(seed=1)
    dk = k.shape[-1]
    rng = np.random.default_rng(0)
    k[:] = 0
    idx = rng.integers(0, dk, k.shape[:3])
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)      # basis keys: exactly unit
    q[:] = k
    o = run(c, q, k, v, beta=np.ones_like(c.beta))
    Hv, Hk = v.shape[2], k.shape[2]
    for h in range(Hv):
        np.testing.assert_allclose(o[:, :, h], c.scale * v[:, :, h], rtol=0, atol=1e-12)


def test_partial_write_of_a_root_node():
    # q = k = a unit basis key: o = scale * (alpha (1 - beta) S0^T k + beta v) for root nodes
    c, q, k, v = f32_case(seed=2, tree="star")
    dk = k.shape[-1]
    k[:] = 0
    k[..., 3] = 1.0
    q[:] = k
    o = run(c, q, k, v)
    G_ = v.shape[2] // k.shape[2]
    for b in range(c.parent.shape[0]):
        for i in range(c.parent.shape[1]):
            for h in range(v.shape[2]):
                a = np.exp(np.float64(c.g[b, i, h]))
                bt = np.float64(c.beta[b, i, h])
                want = c.scale * (a * (1 - bt) * c.S0[b, h][3].astype(np.float64) + bt * v[b, i, h])
                np.testing.assert_allclose(o[b, i, h], want, rtol=1e-12, atol=1e-14)


def test_no_write_only_decays_along_the_path():
    c, q, k, v = f32_case(seed=3)
    o = run(c, q, k, v, beta=np.zeros_like(c.beta))
    for b in range(c.parent.shape[0]):
        for i in range(c.parent.shape[1]):
            for h in range(v.shape[2]):
                gam = np.exp(sum(np.float64(c.g[b, j, h]) for j in path_of(c.parent, b, i)))
                hk = h // (v.shape[2] // k.shape[2])
                want = c.scale * gam * (c.S0[b, h].astype(np.float64).T @ q[b, i, hk])
                np.testing.assert_allclose(o[b, i, h], want, rtol=1e-12, atol=1e-15)


def test_orthonormal_keys_sum_the_path_outer_products():
    c, q, k, v = f32_case(T=14, dk=16, seed=4)
    k[:] = 0
    for i in range(14):
        k[:, i, :, i] = 1.0                                    # node i writes basis key e_i
    o = run(c, q, k, v, g=np.zeros_like(c.g), beta=np.ones_like(c.beta),
            S0=np.zeros_like(c.S0))
    Hk = k.shape[2]
    for b in range(c.parent.shape[0]):
        for i in range(14):
            for h in range(v.shape[2]):
                hk = h // (v.shape[2] // Hk)
                want = sum(q[b, i, hk, j] * v[b, j, h].astype(np.float64)
                           for j in path_of(c.parent, b, i))
                np.testing.assert_allclose(o[b, i, h], c.scale * want, rtol=1e-12, atol=1e-14)


def test_nodes_off_the_path_do_not_matter():
    c, q, k, v = f32_case(T=16, seed=5)
    o = run(c, q, k, v)
    rng = np.random.default_rng(1)
    for b in range(c.parent.shape[0]):
        i = 15
        on = set(path_of(c.parent, b, i))
        k2, v2, g2, b2 = k.copy(), v.copy(), c.g.copy(), c.beta.copy()
        for j in range(16):
            if j not in on:
                k2[b, j] = rng.standard_normal(k2[b, j].shape)
                v2[b, j] = rng.standard_normal(v2[b, j].shape)
                g2[b, j] = -1.0
                b2[b, j] = 0.5
        o2 = run(c, q, k2, v2, g=g2, beta=b2)
        np.testing.assert_array_equal(o2[b, i], o[b, i])


def test_topological_relabelling_permutes_outputs():
    c, q, k, v = f32_case(T=10, seed=6)
    o = run(c, q, k, v)
    b = 0
    par = c.parent[b]
    depth = [len(path_of(c.parent, b, i)) for i in range(10)]
    order = sorted(range(10), key=lambda i: (depth[i], -i))    # another topological order
    pos = {old: new for new, old in enumerate(order)}
    par2 = np.array([[pos[int(par[o_])] if par[o_] >= 0 else -1 for o_ in order]], np.int32)
    sl = lambda a: a[b:b + 1, order]
    o2 = G.gdn_tree_verify(sl(q), sl(k), sl(v), sl(c.g), sl(c.beta), par2, c.S0[b:b + 1],
                           c.scale, dtype="f32")
    np.testing.assert_allclose(o2[0], o[b, order], rtol=1e-12, atol=1e-15)


def test_deferred_commit_continues_like_the_tree():
    # committing node n and then verifying n's child c as a one-node tree gives c's output
    c, q, k, v = f32_case(T=16, seed=7, tree="chain")
    o = run(c, q, k, v)
    B = c.parent.shape[0]
    for n in (0, 5, 14):
        S1 = G.gdn_commit(q, k, v, c.g, c.beta, c.parent, c.S0, np.full(B, n), dtype="f32")
        o1 = G.gdn_tree_verify(q[:, n + 1:n + 2], k[:, n + 1:n + 2], v[:, n + 1:n + 2],
                               c.g[:, n + 1:n + 2], c.beta[:, n + 1:n + 2],
                               np.full((B, 1), -1, np.int32), S1.astype(np.float64), c.scale,
                               dtype="f32")
        np.testing.assert_allclose(o1[:, 0], o[:, n + 1], rtol=1e-10, atol=1e-14)
    S_none = G.gdn_commit(q, k, v, c.g, c.beta, c.parent, c.S0, np.full(B, -1), dtype="f32")
    np.testing.assert_array_equal(S_none, c.S0)


def test_bad_parent_raises():
    c, q, k, v = f32_case(T=4)
    par = c.parent.copy()
    par[0, 2] = 3
    with pytest.raises(ValueError):
        run(c, q, k, v, parent=par)
