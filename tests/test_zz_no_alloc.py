"""The allocation-free forward (tree_attn_forward_noalloc, through the C ABI) against the
forward with a caller workspace (tree_attn_forward) on the same inputs.

Both run the same kernels with the same split plan, so their outputs must agree bit for bit (a
stronger bar than the oracle tolerance, which the small case also checks). Calls follow one
another on one device with inputs of different sizes, the second smaller than the first, so the
fixed scratch array holds the larger call's partials when the smaller one runs.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from tree_verification_attention_amd import _lib, inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def both(case):
    """(noalloc out, lse, err) and (forward out, lse, err) of one case."""
    g = dict(q=dev(case.q), k_cache=dev(case.k_cache), v_cache=dev(case.v_cache),
             seq_lens=dev(case.seq_lens), k_tree=dev(case.k_tree), v_tree=dev(case.v_tree),
             parent=dev(case.parent))
    kw = dict(block_table=dev(case.block_table), page_size=case.page_size or None,
              scale=case.scale)
    args = (g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], g["k_tree"], g["v_tree"],
            g["parent"])
    B, T, Hq, D = case.q.shape
    out = torch.full((B, T, Hq, D), float("nan"), dtype=g["q"].dtype, device="cuda")
    lse = torch.full((B, T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    err_n = torch.zeros(1, dtype=torch.int32, device="cuda")
    _lib.forward_noalloc(*args, out=out, lse=lse, err=err_n, **kw)
    err_f = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref_o, ref_l = _lib.forward(*args, err=err_f, **kw)
    torch.cuda.synchronize()
    return out, lse, int(err_n.item()), ref_o, ref_l, int(err_f.item())


def check_equal(case, what):
    out, lse, en, ref_o, ref_l, ef = both(case)
    say(f"{what}: lens={case.seq_lens.tolist()} flags {en}/{ef}")
    assert en == 0 and ef == 0
    assert torch.equal(out, ref_o), f"{what}: O differs from tree_attn_forward"
    assert torch.equal(lse, ref_l), f"{what}: LSE differs from tree_attn_forward"
    return out, lse


def test_noalloc_matches_forward_two_calls_shrinking():
    # 1: the headline layer, 76 MB of partials (every prefix 65536, 8 splits)
    big = inputs.make_case(inputs.WORKLOADS["gqa_64k_pinned"], 0, pad="finite")
    check_equal(big, "headline layer")
    del big
    # 2: a smaller, ragged, paged problem right after it, also checked against the oracle
    w = inputs.Workload("small", B=3, Hq=8, Hkv=2, D=128, T=24, L=(0, 900))
    small = inputs.make_case(w, 2, layout="paged", page_size=32)
    out, lse = check_equal(small, "small paged")
    o_ref, l_ref = oracle.attend_case(small)
    do = float(np.abs(out.float().cpu().numpy().reshape(-1, 128) - o_ref).max())
    dl = float(np.abs(lse.cpu().numpy().reshape(-1) - l_ref).max())
    say(f"small paged vs oracle: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
    assert do <= 2e-2 and dl <= 1e-3


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    """A problem whose partials exceed the array: TA_ESCRATCH, nothing launched, outputs kept."""
    w = inputs.Workload("wide", B=16, Hq=32, Hkv=8, D=128, T=256, L=64)
    case = inputs.make_case(w, 1, pad="finite")
    g = [dev(getattr(case, k)) for k in ("q", "k_cache", "v_cache", "seq_lens", "k_tree",
                                          "v_tree", "parent")]
    out = torch.zeros(case.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(case.q.shape[:3], dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.TreeAttnError) as e:
        _lib.forward_noalloc(*g, out=out, lse=lse, scale=case.scale)
    assert e.value.status == _lib.TA_ESCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == 0)
