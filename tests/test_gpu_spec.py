"""GPU parity of tree speculative sampling against the CPU oracle.

Uniforms are inputs, so the GPU and the oracle take every decision on the same numbers; both take
them in fp64 (the GPU sums residual masses in a different order, so a decision could only differ
when a uniform falls within ~1e-15 of a threshold). Accepted lengths, paths and emitted tokens are
compared exactly.
"""
import numpy as np
import pytest
import torch

import oracle.accept as A
from tree_verification_attention_amd import _lib, inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run(case, pad_to=None, err=None):
    p = torch.from_numpy(case.p).cuda()
    q = torch.from_numpy(case.q).cuda()
    if pad_to is not None:   # rows padded to a longer stride: row_stride != V
        B, T1, V = p.shape
        pb = torch.zeros((B, T1, pad_to), dtype=torch.float32, device="cuda")
        qb = torch.zeros_like(pb)
        pb[..., :V] = p
        qb[..., :V] = q
        p, q = pb[..., :V], qb[..., :V]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = _lib.spec_sample(p, q, dev(case.draft), dev(case.parent), dev(case.u_accept),
                           dev(case.u_sample), err=err)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def check(case, name, pad_to=None):
    n, path, nxt = run(case, pad_to)
    rn, rpath, rnxt = A.spec_sample(case.p, case.q, case.draft, case.parent, case.u_accept,
                                    case.u_sample)
    say(f"{name}: accept_len {n.tolist()[:8]} next {nxt.tolist()[:4]}")
    assert np.array_equal(n, rn), (n, rn)
    assert np.array_equal(path, rpath)
    assert np.array_equal(nxt, rnxt), (nxt, rnxt)
    return n


CASES = [
    ("llama_vocab", dict(B=4, T=64, V=128256), {}),
    ("qwen_vocab", dict(B=2, T=64, V=152064), {"noise": 2.0}),
    ("star_low_acceptance", dict(B=3, T=40, V=20000), {"tree": "star", "noise": 3.0}),
    ("chain_256_p_eq_q", dict(B=2, T=256, V=5000), {"tree": "chain", "mode": "same"}),
    ("disjoint_supports", dict(B=3, T=24, V=6000), {"mode": "disjoint"}),
    ("beam_like_uniform", dict(B=2, T=64, V=9000), {"tree": "uniform", "noise": 0.5}),
    ("tiny_vocab", dict(B=4, T=8, V=3), {"noise": 1.0}),
    ("one_node", dict(B=5, T=1, V=4097), {"tree": "single"}),
]


@pytest.mark.parametrize("name,shape,kw", CASES, ids=[c[0] for c in CASES])
def test_spec_sample(name, shape, kw):
    case = inputs.make_spec_case(shape["B"], shape["T"], shape["V"], 5, **kw)
    # rows must start 16-byte aligned: a vocabulary that is not a multiple of 4 gets a padded stride
    V = shape["V"]
    n = check(case, name, pad_to=None if V % 4 == 0 else V + (-V) % 4)
    if kw.get("mode") == "same":
        assert n.min() > 0
    if kw.get("mode") == "disjoint":
        assert n.max() == 0


def test_spec_sample_largest_vocabulary():
    # 2^20 entries per row: 256 chunks, every lane of the chunk search holding four
    case = inputs.make_spec_case(2, 3, 1 << 20, 8, tree="chain", noise=2.0)
    check(case, "vocab 2^20")
    case.u_accept[:] = 0.999                 # rejections: corrections drawn over 256 chunks
    check(case, "vocab 2^20, corrections")


def test_spec_sample_many_seeds_and_ragged_rows():
    for seed in range(8):
        case = inputs.make_spec_case(6, 32, 4099, seed, noise=1.5)
        check(case, f"seed {seed}", pad_to=4100)


def test_spec_sample_forced_trials():
    # uniforms near 1 reject every child whose probability ratio is below 1, so positions with
    # several children take second and later trials (the workgroup's row passes)
    case = inputs.make_spec_case(3, 48, 30000, 2, tree="star", noise=0.7)
    case.u_accept[:] = 0.97
    check(case, "forced later trials")
    case.u_accept[:] = 0.0
    check(case, "always accept")


@pytest.mark.parametrize("fill", [0, 255])
def test_spec_sample_workspace_contents_do_not_matter(fill):
    """Pass slots read as already written (0x00: sums of 0.0) or as NaN (0xFF) must not leak into
    a call: the mass kernel resets every slot before the walk polls it."""
    case = inputs.make_spec_case(3, 48, 30000, 2, tree="star", noise=0.7)
    case.u_accept[:] = 0.97   # several trials per position: the walk's row passes
    B, T1, V = case.p.shape
    ws = torch.full((_lib.spec_sample_workspace_size(B, T1 - 1, V),), fill, dtype=torch.uint8,
                    device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = _lib.spec_sample(dev(case.p), dev(case.q), dev(case.draft), dev(case.parent),
                           dev(case.u_accept), dev(case.u_sample), ws=ws)
    torch.cuda.synchronize()
    n, path, nxt = [o.cpu().numpy() for o in out]
    rn, rpath, rnxt = A.spec_sample(case.p, case.q, case.draft, case.parent, case.u_accept,
                                    case.u_sample)
    assert np.array_equal(n, rn) and np.array_equal(path, rpath) and np.array_equal(nxt, rnxt)


def test_spec_sample_zero_residual_mass_accepts():
    case = inputs.make_spec_case(2, 6, 1000, 1, tree="chain")
    case.q[:] = case.p * np.float32(1.5)    # p <= q everywhere: no rejection is possible
    case.u_accept[:] = 0.999
    n = check(case, "zero residual mass")
    assert np.all(n == 6)


def test_spec_sample_flags():
    case = inputs.make_spec_case(2, 8, 500, 3)
    case.parent[1, 5] = 7
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    run(case, err=err)
    assert int(err.item()) & _lib.TA_DEV_BAD_PARENT
    case = inputs.make_spec_case(2, 8, 500, 3)
    case.draft[0, 2] = 500
    err.zero_()
    run(case, err=err)
    assert int(err.item()) & _lib.TA_DEV_BAD_TOKEN


def test_spec_sample_rejects_a_short_workspace():
    case = inputs.make_spec_case(2, 8, 50000, 3)
    p = torch.from_numpy(case.p).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.TreeAttnError) as ei:
        _lib.spec_sample(p, p, dev(case.draft), dev(case.parent), dev(case.u_accept),
                         dev(case.u_sample), ws=ws)
    assert ei.value.status == _lib.TA_EWORKSPACE
