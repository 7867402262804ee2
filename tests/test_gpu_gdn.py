"""GPU parity of gated-delta-net tree verification and its deferred state commit against the
node-by-node fp64 oracle.

Tolerance (fp32 arithmetic on bf16 inputs): every output is a sum of at most d_k-term dot products
chained through at most T levels of the triangular solve; with unit keys and states of order 1
the rounding error stays below (d_k + T) * 2^-24 * |value| ~ 2.3e-5 for d_k = 128, T = 256, so
outputs and committed states must agree to 5e-5 absolute.
"""
import numpy as np
import pytest
import torch

import oracle.gdn as G
from tree_verification_attention_amd import _lib, inputs

pytestmark = pytest.mark.gpu
TOL = 5e-5


def say(*a):
    print(*a, flush=True)


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def verify(c, err=None):
    o = _lib.gdn_verify(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), dev(c.parent),
                        dev(c.S0), c.scale, err=err)
    torch.cuda.synchronize()
    return o.cpu().numpy()


CASES = [
    ("qwen_like_t128", dict(B=4, T=128, Hk=16, Hv=32, dk=128, dv=128), {}),
    ("chain_256", dict(B=1, T=256, Hk=2, Hv=4, dk=128, dv=128), {"tree": "chain"}),
    ("deep_bounded_256", dict(B=2, T=256, Hk=2, Hv=2, dk=128, dv=64), {"depth_cap": 40}),
    ("dk64_dv96", dict(B=2, T=64, Hk=4, Hv=8, dk=64, dv=96), {}),
    ("star", dict(B=2, T=50, Hk=2, Hv=2, dk=128, dv=32), {"tree": "star"}),
    ("uniform", dict(B=2, T=100, Hk=1, Hv=3, dk=64, dv=128), {"tree": "uniform"}),
    ("one_node", dict(B=3, T=1, Hk=2, Hv=4, dk=128, dv=32), {"tree": "single"}),
    ("dk64_dv256_t200", dict(B=1, T=200, Hk=1, Hv=2, dk=64, dv=256), {"depth_cap": 24}),
    # enough (sequence, head, 32-column) blocks for two per CU: 64-column, 512-thread workgroups
    ("wide_dk64_t128", dict(B=4, T=128, Hk=8, Hv=32, dk=64, dv=128), {}),
    ("wide_chain_128", dict(B=8, T=128, Hk=4, Hv=16, dk=128, dv=128), {"tree": "chain"}),
    ("wide_dv256_t100", dict(B=2, T=100, Hk=4, Hv=32, dk=128, dv=256), {"tree": "uniform"}),
    ("wide_one_node", dict(B=8, T=1, Hk=4, Hv=16, dk=128, dv=128), {"tree": "single"}),
]


@pytest.mark.parametrize("name,shape,kw", CASES, ids=[c[0] for c in CASES])
def test_gdn_verify(name, shape, kw):
    c = inputs.make_gdn_case(shape["B"], shape["T"], shape["Hk"], shape["Hv"], shape["dk"],
                             shape["dv"], 3, **kw)
    o = verify(c)
    ref = G.gdn_tree_verify(c.q, c.k, c.v, c.g, c.beta, c.parent, c.S0, c.scale)
    d = np.abs(o - ref).max()
    say(f"{name}: max|dO| {d:.3e} (max|O| {np.abs(ref).max():.3f})")
    assert d <= TOL


def test_gdn_bad_parent_sets_flag():
    c = inputs.make_gdn_case(2, 8, 1, 2, 64, 32, 1)
    c.parent[1, 3] = 5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    verify(c, err)
    assert int(err.item()) & _lib.TA_DEV_BAD_PARENT


@pytest.mark.parametrize("name,shape,kw", [
    ("qwen_like_t128", dict(B=4, T=128, Hk=16, Hv=32, dk=128, dv=128), {}),
    ("chain_256_full", dict(B=2, T=256, Hk=1, Hv=2, dk=64, dv=64), {"tree": "chain"}),
], ids=["qwen_like_t128", "chain_256_full"])
def test_gdn_commit(name, shape, kw):
    c = inputs.make_gdn_case(shape["B"], shape["T"], shape["Hk"], shape["Hv"], shape["dk"],
                             shape["dv"], 4, **kw)
    rng = np.random.default_rng(2)
    path, n = inputs.random_paths(c.parent, rng)
    if kw.get("tree") == "chain":
        path[0] = np.arange(shape["T"])
        n[0] = shape["T"]                        # the whole 256-node chain accepted
    n[-1] = 0                                    # one sequence accepts nothing
    path[-1] = -1
    S = dev(c.S0)
    _lib.gdn_commit(dev(c.k), dev(c.v), dev(c.g), dev(c.beta), dev(path), dev(n), S)
    torch.cuda.synchronize()
    last = np.array([path[b, n[b] - 1] if n[b] > 0 else -1 for b in range(shape["B"])])
    ref = G.gdn_commit(c.q, c.k, c.v, c.g, c.beta, c.parent, c.S0, last)
    d = np.abs(S.cpu().numpy() - ref).max()
    say(f"{name}: accept_len {n.tolist()} max|dS| {d:.3e}")
    assert d <= TOL
    assert np.array_equal(S.cpu().numpy()[-1], c.S0[-1])


def test_gdn_commit_bad_path_sets_flag():
    c = inputs.make_gdn_case(2, 8, 1, 2, 64, 32, 1)
    path = np.full((2, 8), -1, np.int32)
    path[0, :2] = [0, 9]
    n = np.array([2, 9], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    S = dev(c.S0)
    _lib.gdn_commit(dev(c.k), dev(c.v), dev(c.g), dev(c.beta), dev(path), dev(n), S, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & _lib.TA_DEV_BAD_COMMIT
    np.testing.assert_array_equal(S.cpu().numpy()[1], c.S0[1])   # accept_len 9 > T: unchanged
    # sequence 0 stops at the invalid entry: its state is node 0's
    ref = G.gdn_commit(c.q, c.k, c.v, c.g, c.beta, c.parent, c.S0, np.array([0, -1]))
    assert np.abs(S.cpu().numpy()[0] - ref[0]).max() <= TOL


def test_gdn_commit_stops_mid_path():
    """An invalid entry past the first 32 path steps: the updates before it (across a staging
    boundary) are applied, the rest are not."""
    c = inputs.make_gdn_case(2, 64, 2, 4, 128, 64, 5, tree="chain")
    path = np.tile(np.arange(64, dtype=np.int32), (2, 1))
    path[0, 40] = 99
    n = np.array([64, 37], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    S = dev(c.S0)
    _lib.gdn_commit(dev(c.k), dev(c.v), dev(c.g), dev(c.beta), dev(path), dev(n), S, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & _lib.TA_DEV_BAD_COMMIT
    ref = G.gdn_commit(c.q, c.k, c.v, c.g, c.beta, c.parent, c.S0, np.array([39, 36]))
    d = np.abs(S.cpu().numpy() - ref).max()
    say(f"stops_mid_path: max|dS| {d:.3e}")
    assert d <= TOL
