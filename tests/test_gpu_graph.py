"""HIP-graph capture of the fused forward and of greedy acceptance.

Serving loops capture a verify step once and replay it. The library's calls allocate nothing and
record no memset, so a captured step must reproduce the eager result on every replay, with
the program's own eager work (buffer clears, input updates, synchronisations) between replays,
and must read the inputs' current contents rather than those seen at capture.
"""
import numpy as np
import pytest
import torch

from tree_verification_attention_amd import _lib, inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def capture(fn):
    """Warm ``fn`` up on a side stream, then capture one call of it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_forward_graph_replays(layout):
    w = inputs.Workload("graph", B=2, Hq=8, Hkv=2, D=128, T=24, L=(100, 900))
    case = inputs.make_case(w, 2, layout=layout, page_size=64)
    say(f"graph forward {layout} lens={case.seq_lens.tolist()}")
    g = dict(q=dev(case.q), kc=dev(case.k_cache), vc=dev(case.v_cache), lens=dev(case.seq_lens),
             kt=dev(case.k_tree), vt=dev(case.v_tree), par=dev(case.parent),
             bt=dev(case.block_table))
    kw = dict(block_table=g["bt"], page_size=case.page_size or None, scale=case.scale)
    p = _lib.make_problem(g["q"], g["kc"], g["vc"], g["lens"], g["kt"], g["vt"], g["par"], **kw)
    out = torch.empty_like(g["q"])
    lse = torch.empty(g["q"].shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.zeros(_lib.workspace_size(p), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step():
        _lib.forward(g["q"], g["kc"], g["vc"], g["lens"], g["kt"], g["vt"], g["par"], **kw,
                     out=out, lse=lse, workspace=ws, err=err)

    graph = capture(step)
    for it in range(4):
        if it == 2:
            # new queries in place: the replay must see them
            g["q"].copy_(torch.roll(g["q"], 1, dims=1))
        ref_o, ref_l = _lib.forward(g["q"], g["kc"], g["vc"], g["lens"], g["kt"], g["vt"],
                                    g["par"], **kw)
        torch.cuda.synchronize()
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(out, ref_o), f"replay {it}: O differs from the eager call"
        assert torch.equal(lse, ref_l), f"replay {it}: LSE differs from the eager call"


def test_greedy_accept_graph_replays():
    case = inputs.make_accept_case(3, 32, 50_000, 9)
    lg, dr, pa = dev(case.logits), dev(case.draft), dev(case.parent)
    B, T = case.draft.shape
    ws = torch.zeros(_lib.greedy_accept_workspace_size(lg.dtype, B, T, lg.shape[2]),
                     dtype=torch.uint8, device="cuda")
    res = {}

    def step():
        res["out"] = _lib.greedy_accept(lg, dr, pa, ws=ws)

    graph = capture(step)
    for it in range(4):
        if it == 2:
            # a different target row 0: the accepted paths change
            lg[:, 0].copy_(torch.roll(lg[:, 0], 7, dims=-1))
        ref = _lib.greedy_accept(lg, dr, pa)
        torch.cuda.synchronize()
        for t in res["out"]:
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, r in zip(("greedy", "accept_len", "path", "next_token"), res["out"], ref):
            assert torch.equal(a, r), f"replay {it}: {name} differs from the eager call"
