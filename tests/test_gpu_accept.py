"""GPU parity of greedy tree acceptance and accepted-path KV commit against the CPU oracle.

Integer and byte work: every output is compared bit for bit (argmax per row, accepted path and
length, correction token; the whole cache after a commit, as raw bit patterns).
"""
import numpy as np
import pytest
import torch

import oracle.accept as A
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


def run_accept(case, pad_to=None):
    lg = dev(case.logits)
    if pad_to is not None:   # rows padded to a longer stride: exercises row_stride != V
        B, T1, V = lg.shape
        big = torch.zeros((B, T1, pad_to), dtype=lg.dtype, device="cuda")
        big[..., :V] = lg
        lg = big[..., :V]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _lib.greedy_accept(lg, dev(case.draft), dev(case.parent), err=err)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out], int(err.item())


def check_accept(case, name, pad_to=None):
    (g, n, path, nxt), err = run_accept(case, pad_to)
    rg, rn, rpath, rnxt = A.greedy_accept(case.logits, case.draft, case.parent, case.dtype)
    say(f"{name}: accept_len {n.tolist()[:8]} max {n.max()}")
    assert err == 0
    assert np.array_equal(g, rg), f"{name}: greedy tokens differ"
    assert np.array_equal(n, rn) and np.array_equal(path, rpath) and np.array_equal(nxt, rnxt)
    return n


ACCEPT = [
    ("llama_vocab_bf16", dict(B=4, T=64, V=128256), {}),
    ("qwen_vocab_f32", dict(B=2, T=64, V=152064), {"dtype": "f32"}),
    ("deep_chain_256", dict(B=2, T=256, V=3000), {"tree": "chain", "plant": 1.0, "ties": 0.0,
                                                  "blocks": 0.0}),
    ("full_accept_bounded", dict(B=3, T=64, V=5000), {"plant": 1.0, "ties": 0.0, "blocks": 0.0}),
    ("ties_everywhere", dict(B=3, T=40, V=64), {"plant": 0.9, "ties": 0.9}),
    ("single_node", dict(B=5, T=1, V=777), {"tree": "single"}),
    ("star", dict(B=2, T=50, V=2048), {"tree": "star", "plant": 1.0}),
    ("beam_tree", dict(B=2, T=64, V=4096), {"tree": "uniform"}),
]


@pytest.mark.parametrize("name,shape,kw", ACCEPT, ids=[a[0] for a in ACCEPT])
def test_greedy_accept(name, shape, kw):
    case = inputs.make_accept_case(shape["B"], shape["T"], shape["V"], 11, **kw)
    es = 4 if kw.get("dtype") == "f32" else 2
    # rows must start 16-byte aligned: a vocabulary that is not a multiple of 16 / es gets a
    # padded row stride
    pad = None if (shape["V"] * es) % 16 == 0 else -(-shape["V"] * es // 16) * 16 // es
    n = check_accept(case, name, pad_to=pad)
    if kw.get("plant") == 1.0 and kw.get("tree") != "star":
        assert n.max() >= 3


def test_greedy_accept_ragged_vocab_strided_rows_nan_and_inf():
    case = inputs.make_accept_case(3, 16, 1001, 5, plant=0.9)
    x = inputs.bf16_bits_to_f32(case.logits)
    x[0, 3, :] = np.nan                      # all NaN: index 0
    x[1, 0, :7] = np.nan                     # NaN never wins
    x[1, 0, 1000] = 9.0                      # maximum in the scalar tail of the row
    x[2, 5, :] = -np.inf
    x[2, 5, 0] = np.nan                      # -inf is the non-NaN maximum, first at index 1
    case.logits = inputs.f32_to_bf16_bits(x)
    check_accept(case, "ragged vocab", pad_to=1008)


def test_greedy_accept_ties_and_nan_spread_over_the_row_chunks():
    # rows of a large vocabulary are scanned in several chunks: equal maxima placed all over the
    # row (the first must win, whichever chunk holds it), rows whose first half is NaN, and
    # maxima at the very first and very last entries
    case = inputs.make_accept_case(4, 64, 128256, 9, plant=0.8)
    x = inputs.bf16_bits_to_f32(case.logits)
    rng = np.random.default_rng(4)
    V = x.shape[-1]
    for b in range(4):
        for r in range(0, 65, 3):
            idx = rng.choice(V, size=int(rng.integers(2, 9)), replace=False)
            x[b, r, idx] = 11.0
    x[0, 1, :V // 2] = np.nan
    x[1, 2, :] = -3.0
    x[1, 2, V - 1] = 12.0
    x[2, 4, 0] = 12.0
    x[3, 7, :] = np.nan
    x[3, 8, 1:] = np.nan
    x[0, 9, :] = -np.abs(x[0, 9, :]) - 0.5      # every entry negative
    x[0, 10, :] = -1.0                           # maximum 0 held by -0 before +0: they tie
    x[0, 10, 70001] = -0.0
    x[0, 10, 90001] = 0.0
    x[0, 11, 5] = np.nan                         # a NaN and a larger value later in the row
    x[0, 11, 100000] = 20.0
    case.logits = inputs.f32_to_bf16_bits(x)
    check_accept(case, "ties over chunks")


def test_greedy_accept_f32_special_rows():
    case = inputs.make_accept_case(2, 12, 40000, 3, dtype="f32", plant=0.9)
    x = case.logits
    x[0, 1, :] = -2.0
    x[0, 1, 30000] = -0.0
    x[0, 1, 35000] = 0.0
    x[0, 2, :] = np.nan
    x[0, 3, :] = -np.inf
    x[0, 3, 39999] = np.nan
    x[1, 4, 100] = np.inf
    x[1, 4, 39000] = np.inf
    x[1, 5, 7] = np.nan
    x[1, 5, 20000] = 50.0
    check_accept(case, "f32 special rows")


def test_greedy_accept_one_workspace_many_sizes():
    """One workspace serves calls of different sizes one after another (larger, smaller, larger
    again, a single node): each call only reads the chunk winners it wrote, so every call matches
    the oracle whatever the previous one left there."""
    sizes = [(4, 64, 128256, "bf16"), (2, 16, 3000, "bf16"), (6, 100, 50000, "f32"),
             (3, 1, 776, "bf16"), (4, 64, 128256, "bf16")]
    need = max(_lib.greedy_accept_workspace_size(torch.bfloat16 if dt == "bf16" else torch.float32,
                                                 B, T, V) for B, T, V, dt in sizes)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for k, (B, T, V, dt) in enumerate(sizes):
        case = inputs.make_accept_case(B, T, V, 20 + k, dtype=dt)
        g, n, path, nxt = _lib.greedy_accept(dev(case.logits), dev(case.draft), dev(case.parent),
                                             ws=ws)
        torch.cuda.synchronize()
        rg, rn, rpath, rnxt = A.greedy_accept(case.logits, case.draft, case.parent, case.dtype)
        say(f"shared workspace call {k}: B={B} T={T} V={V} {dt} accept_len {n.tolist()[:6]}")
        assert np.array_equal(g.cpu().numpy(), rg) and np.array_equal(n.cpu().numpy(), rn)
        assert np.array_equal(path.cpu().numpy(), rpath) and np.array_equal(nxt.cpu().numpy(), rnxt)


def test_greedy_accept_rejects_a_short_workspace():
    case = inputs.make_accept_case(4, 64, 128256, 2)
    lg = dev(case.logits)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.TreeAttnError) as ei:
        _lib.greedy_accept(lg, dev(case.draft), dev(case.parent), ws=ws)
    assert ei.value.status == _lib.TA_EWORKSPACE


def test_greedy_accept_bad_parent_sets_flag():
    case = inputs.make_accept_case(2, 8, 128, 1)
    case.parent[1, 4] = 6
    _, err = run_accept(case)
    assert err & _lib.TA_DEV_BAD_PARENT


def commit_case(D, dtype, layout, seed):
    wl = inputs.Workload("commit", B=3, Hq=4, Hkv=2, D=D, T=24, L=(1, 200), dtype=dtype)
    case = inputs.make_case(wl, seed, layout=layout, page_size=16, lcap=240)
    path, n = inputs.random_paths(case.parent, np.random.default_rng(seed))
    return case, path, n


def run_commit(case, path, n, alias=False):
    k, v = dev(case.k_cache), dev(case.v_cache)
    lens = dev(case.seq_lens)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _lib.kv_commit(k, v, lens, dev(case.k_tree), dev(case.v_tree), dev(path), dev(n),
                         block_table=dev(case.block_table), page_size=case.page_size or None,
                         new_seq_lens=lens if alias else None, err=err)
    torch.cuda.synchronize()
    bits = np.uint16 if case.dtype == "bf16" else np.uint32
    kk = k.cpu().view(torch.int16 if bits is np.uint16 else torch.int32).numpy().view(bits)
    vv = v.cpu().view(torch.int16 if bits is np.uint16 else torch.int32).numpy().view(bits)
    return kk, vv, out.cpu().numpy(), int(err.item())


@pytest.mark.parametrize("D,dtype,layout", [(128, "bf16", "contiguous"), (128, "bf16", "paged"),
                                            (64, "bf16", "paged"), (64, "f32", "contiguous"),
                                            (128, "f32", "paged")])
def test_kv_commit(D, dtype, layout):
    case, path, n = commit_case(D, dtype, layout, D + len(layout))
    say(f"commit D={D} {dtype} {layout} lens={case.seq_lens.tolist()} n={n.tolist()}")
    kk, vv, lens, err = run_commit(case, path, n, alias=(layout == "paged"))
    rk, rv, rlens = A.commit_kv(case.k_cache, case.v_cache, case.seq_lens, case.k_tree, case.v_tree,
                                path, n, block_table=case.block_table, page_size=case.page_size)
    bits = np.uint16 if dtype == "bf16" else np.uint32
    assert err == 0
    assert np.array_equal(lens, rlens)
    assert np.array_equal(kk, rk.view(bits)) and np.array_equal(vv, rv.view(bits))


def test_kv_commit_overflow_and_bad_path():
    case, path, n = commit_case(128, "bf16", "contiguous", 3)
    cap = case.k_cache.shape[1]
    case.seq_lens[0] = cap - 1
    n[0] = 2                                   # past the capacity: nothing written
    path[0, :2] = [0, 1]
    kk, vv, lens, err = run_commit(case, path, n)
    assert err & _lib.TA_DEV_BAD_COMMIT
    assert lens[0] == cap - 1
    assert np.array_equal(kk[0], case.k_cache[0]) and np.array_equal(vv[0], case.v_cache[0])
