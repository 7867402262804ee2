"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars: ancestor masks bit-exact; bf16 inputs max |dO| <= 2e-2 and max |dLSE| <= 1e-3; fp32
inputs max |dO| <= 1e-4 and max |dLSE| <= 1e-4 (fp32 accumulation over at most a few thousand
terms per lane, errors ~1e-6). Inputs are the generator's seeded cases; padding rows are NaN so
that any read past a sequence's length shows up as a NaN in the output.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from tree_verification_attention_amd import _lib, inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-4, 1e-4)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_gpu(case):
    return dict(q=dev(case.q), k_cache=dev(case.k_cache), v_cache=dev(case.v_cache),
                seq_lens=dev(case.seq_lens), k_tree=dev(case.k_tree), v_tree=dev(case.v_tree),
                parent=dev(case.parent), block_table=dev(case.block_table),
                page_size=case.page_size or None)


def run_forward(case, **kw):
    g = to_gpu(case)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = _lib.forward(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], g["k_tree"],
                            g["v_tree"], g["parent"], block_table=g["block_table"],
                            page_size=g["page_size"], scale=case.scale, err=err, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), int(err.item())


def check(case, o_gpu, lse_gpu, o_ref, lse_ref, what, rows=None):
    """Bars of the module docstring over the given rows; prints the worst row of each."""
    atol_o, atol_l = TOL[case.dtype]
    o_gpu = o_gpu.reshape(o_ref.shape)
    lse_gpu = lse_gpu.reshape(lse_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: -inf pattern differs"
    B, T, Hq = case.q.shape[:3]

    def name(k):
        if rows is not None:
            return tuple(int(x) for x in rows[k])
        return (int(k // (T * Hq)), int(k // Hq % T), int(k % Hq))

    do = dl = 0.0
    wo = wl_ = "-"
    if o_ref.size:
        e = np.abs(o_gpu - o_ref).reshape(len(lse_ref), -1).max(axis=1)
        k = int(np.argmax(e))
        do, wo = float(e[k]), name(k)
    if fin.any():
        e = np.where(fin, np.abs(np.where(fin, lse_gpu, 0) - np.where(fin, lse_ref, 0)), 0)
        k = int(np.argmax(e))
        dl, wl_ = float(e[k]), name(k)
    say(f"{what}: {len(lse_ref)} rows, max|dO|={do:.3e} at (b,i,h)={wo}, "
        f"max|dLSE|={dl:.3e} at {wl_}")
    assert do <= atol_o, f"{what}: max|dO| {do} > {atol_o}"
    assert dl <= atol_l, f"{what}: max|dLSE| {dl} > {atol_l}"


def wl(name="p", B=2, Hq=8, Hkv=2, D=128, T=16, L=(1, 700), dtype="bf16", tree="bounded", **kw):
    return inputs.Workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, L=L, dtype=dtype, tree=tree, **kw)


# ------------------------------------------------------------------------------------------------
# mask


def mask_gpu(parent):
    m = _lib.mask_build(dev(parent))
    torch.cuda.synchronize()
    return m.cpu().numpy().view(np.uint64)


def test_mask_example_chain_star():
    par = np.array([[-1, 0, -1, 2, 2]], dtype=np.int32)
    got = mask_gpu(par)
    assert [int(x) for x in got[0, :, 0]] == [0x01, 0x03, 0x04, 0x0C, 0x14]
    for T in (1, 63, 64, 65, 200, 256):
        for par in (np.arange(-1, T - 1, dtype=np.int32)[None], np.full((1, T), -1, np.int32)):
            assert np.array_equal(mask_gpu(par), oracle.tree_mask(par)), T


@pytest.mark.parametrize("T", [2, 7, 16, 64, 100, 128, 255, 256])
def test_mask_random_trees_bit_exact(T):
    rng = np.random.default_rng(T)
    par = np.stack([inputs.uniform_tree(rng, T) for _ in range(3)] +
                   [inputs.bounded_tree(rng, T, 12, 4) for _ in range(3)])
    assert np.array_equal(mask_gpu(par), oracle.tree_mask(par))


def test_mask_bad_parent_sets_flag():
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _lib.mask_build(dev(np.array([[-1, 5, 0]], dtype=np.int32)), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & _lib.TA_DEV_BAD_PARENT


# ------------------------------------------------------------------------------------------------
# fused forward, small sizes (every row checked)

SMALL = [
    ("tiny_f32", inputs.WORKLOADS["tiny_f32"], {}),
    ("gqa_d128_ragged", wl(), {}),
    ("gqa_d64_ragged", wl(D=64, L=(0, 300), T=12), {}),
    ("mha_g1", wl(Hq=4, Hkv=4, T=64, L=(200, 333)), {}),
    ("g5_two_rowblocks", wl(B=1, Hq=10, Hkv=2, T=128, L=(60, 200), depth_cap=12), {}),
    ("g4_t128_rowblocks", wl(B=2, Hq=8, Hkv=2, T=128, L=(1, 130)), {}),
    ("chain_t256", wl(B=1, Hq=2, Hkv=1, T=256, L=70, tree="chain"), {}),
    ("d64_t200_masked_ring", wl(B=2, Hq=4, Hkv=2, D=64, T=200, L=(65, 300), depth_cap=30), {}),
    ("single_node", wl(B=3, T=1, tree="single", L=(0, 129)), {}),
    ("star", wl(B=2, T=20, tree="star", L=(64, 64)), {}),
    ("uniform_f32_d128", wl(D=128, T=9, dtype="f32", tree="uniform", L=(1, 300)), {}),
    # fp32, one split (the single-launch forward): prefixes of 2, 1, 1 and 0 keys, a 256-node chain
    ("f32_one_split_short_prefixes", wl(B=4, Hq=4, Hkv=1, D=64, T=12, dtype="f32", L=(0, 2)), {}),
    ("f32_chain_t256", wl(B=1, Hq=2, Hkv=1, D=64, T=256, dtype="f32", tree="chain", L=(100, 100)),
     {}),
    ("f32_forced_splits_3", wl(B=2, Hq=4, Hkv=2, D=128, T=16, dtype="f32", L=(0, 500)),
     {"num_splits": 3}),
    # a last row block of at most 128 packed rows (half its wavefronts idle or fewer), with
    # several parts per sequence dealt by length
    ("short_last_block_g5_t128", wl(B=3, Hq=10, Hkv=2, T=128, L=(300, 2000), depth_cap=12), {}),
    ("short_last_block_g5_t110", wl(B=2, Hq=10, Hkv=2, T=110, L=(700, 3000), depth_cap=12), {}),
    ("short_last_block_d64_t80", wl(B=1, Hq=16, Hkv=4, D=64, T=80, L=(2000, 2000)), {}),
    # exactly 64 sequences, the most whose parts are still dealt by length
    ("batch64_dealt", wl(B=64, Hq=4, Hkv=2, T=4, L=(0, 700)), {}),
    # 256 nodes x 4 query heads: four 256-row blocks per KV head
    ("t256_g4_four_rowblocks", wl(B=1, Hq=8, Hkv=2, T=256, L=(500, 1000), depth_cap=16), {}),
    # every prefix a multiple of 64 keys: no tail tile in the masked part
    ("lengths_multiple_of_64", wl(B=3, L=(640, 640)), {}),
    ("forced_splits_1", wl(L=(300, 700)), {"num_splits": 1}),
    ("forced_splits_7", wl(L=(300, 700)), {"num_splits": 7}),
    # more than 64 sequences: every sequence takes S parts of a chunk sized from the longest
    ("batch80_undealt", wl(B=80, Hq=2, Hkv=1, T=4, L=(0, 600)), {}),
    ("batch70_forced_splits_3", wl(B=70, Hq=4, Hkv=2, T=8, L=(0, 400)), {"num_splits": 3}),
]


@pytest.mark.parametrize("name,w,kw", SMALL, ids=[s[0] for s in SMALL])
def test_forward_small(name, w, kw):
    for layout in ("contiguous", "paged"):
        case = inputs.make_case(w, 0, layout=layout, page_size=16 if w.D == 64 else 64)
        say(f"case {name} {layout} lens={case.seq_lens.tolist()}")
        o, lse, err = run_forward(case, **kw)
        assert err == 0
        o_ref, lse_ref = oracle.attend_case(case)
        check(case, o, lse, o_ref, lse_ref, f"{name}/{layout}")


@pytest.mark.parametrize("psz", [16, 32, 128, 256, 1024, 4096])
def test_forward_paged_page_sizes(psz):
    """Page sizes other than the small cases' 64 (D = 128): pages of 128 to 4096 keys hold several
    tiles (a tile can start mid-page; at 4096 a whole sequence sits in one page), 16 and 32 split a
    tile over several pages."""
    w = wl(B=3, Hq=8, Hkv=2, D=128, T=20, L=(1, 1500))
    case = inputs.make_case(w, 4, layout="paged", page_size=psz)
    say(f"paged page_size {psz} lens={case.seq_lens.tolist()}")
    o, lse, err = run_forward(case)
    assert err == 0
    o_ref, lse_ref = oracle.attend_case(case)
    check(case, o, lse, o_ref, lse_ref, f"paged/{psz}")


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_forward_capacity_beyond_lengths(layout):
    """A cache allocated three times longer than the longest prefix: the splits are sized from the
    lengths on the device, all of them still cover the prefix exactly once."""
    w = wl(B=3, Hq=8, Hkv=2, D=128, T=24, L=(300, 2000))
    case = inputs.make_case(w, 8, layout=layout, page_size=32 if layout == "paged" else 64,
                            lcap=6000)
    g = to_gpu(case)
    p = _lib.make_problem(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], g["k_tree"],
                          g["v_tree"], g["parent"], block_table=g["block_table"],
                          page_size=g["page_size"], scale=case.scale)
    say(f"capacity 6000 {layout}: lens={case.seq_lens.tolist()} splits={_lib.num_splits(p)}")
    for splits in (0, 5):
        o, lse, err = run_forward(case, num_splits=splits)
        assert err == 0
        o_ref, lse_ref = oracle.attend_case(case)
        check(case, o, lse, o_ref, lse_ref, f"capacity/{layout}/splits={splits}")


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_forward_very_ragged_batch(layout):
    """Lengths 0, 70 and 40 000 in one batch: the parts are dealt by length (the long sequence
    takes nearly all of them); with 16-key pages and two splits the long one needs two parts for
    its block-table entries to fit the LDS cache."""
    w = wl(B=3, Hq=4, Hkv=2, D=128, T=8, L=(0, 40000))
    case = inputs.make_case(w, 9, layout=layout, page_size=16, lens=[0, 70, 40000])
    for splits in (0, 2):
        say(f"ragged {layout} splits={splits} lens={case.seq_lens.tolist()}")
        o, lse, err = run_forward(case, num_splits=splits)
        assert err == 0
        o_ref, lse_ref = oracle.attend_case(case)
        check(case, o, lse, o_ref, lse_ref, f"ragged/{layout}/splits={splits}")


def test_forward_cache_rows_far_apart():
    """A contiguous cache whose key rows are 2 MiB apart: the prefix spans more than 2^31 bytes,
    so every tile is addressed from a 64-bit base (only offsets inside a 64-row tile are 32-bit)."""
    w = wl(B=1, Hq=8, Hkv=1, D=128, T=16, L=1100)
    case = inputs.make_case(w, 6)
    g = to_gpu(case)
    Lc = case.k_cache.shape[1]
    row = 1 << 20   # elements between consecutive key rows
    views = []
    for name in ("k_cache", "v_cache"):
        big = torch.empty(Lc * row, dtype=torch.bfloat16, device="cuda")
        v = big.as_strided((1, Lc, 1, 128), (Lc * row, row, 128, 1))
        v.copy_(g[name])
        views.append((big, v))
    say(f"far rows: {Lc} rows x {row * 2} bytes = {Lc * row * 2 / 2**30:.2f} GiB per tensor")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = _lib.forward(g["q"], views[0][1], views[1][1], g["seq_lens"], g["k_tree"],
                            g["v_tree"], g["parent"], scale=case.scale, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o_ref, lse_ref = oracle.attend_case(case)
    check(case, out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "far rows")
    del views


def test_unfused_calls_and_merge():
    w = wl(B=2, Hq=8, Hkv=2, D=128, T=24, L=(0, 500), tree="uniform")
    case = inputs.make_case(w, 3)
    g = to_gpu(case)
    o_c, l_c = _lib.prefix(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], scale=case.scale)
    o_s, l_s = _lib.tree(g["q"], g["k_tree"], g["v_tree"], g["parent"], scale=case.scale)
    o_m, l_m = _lib.merge(o_c, l_c, o_s, l_s, out_dtype=torch.float32)
    o_b, l_b = _lib.merge(o_c, l_c, o_s, l_s, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref_c = oracle.attend_case(case, which="prefix")
    ref_s = oracle.attend_case(case, which="tree")
    ref = oracle.attend_case(case)
    check(case, o_c.cpu().numpy(), l_c.cpu().numpy(), *ref_c, "prefix")
    check(case, o_s.cpu().numpy(), l_s.cpu().numpy(), *ref_s, "tree")
    check(case, o_m.cpu().numpy(), l_m.cpu().numpy(), *ref, "merge(prefix, tree) fp32")
    check(case, o_b.float().cpu().numpy(), l_b.cpu().numpy(), *ref, "merge(prefix, tree) bf16")
    # merging the oracle's own parts through the GPU merge reproduces the oracle's whole
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    sh = (2, 24, 8)
    o_x, l_x = _lib.merge(t(ref_c[0]).view(*sh, 128), t(ref_c[1]).view(sh),
                          t(ref_s[0]).view(*sh, 128), t(ref_s[1]).view(sh))
    torch.cuda.synchronize()
    np.testing.assert_allclose(o_x.cpu().numpy().reshape(-1, 128), ref[0], atol=1e-5)
    np.testing.assert_allclose(l_x.cpu().numpy().reshape(-1), ref[1], atol=1e-5)


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_fused_tree_part_matches_tree_call(layout):
    """tree_attn_partials computes the masked part in the prefix launch (the last split's
    workgroups go on with it). With prefix lengths of whole 64-key tiles there is no tail, so
    that part must equal what tree_attn_tree returns, bit for bit: the same per-row arithmetic
    over the same tree tiles. Several row blocks, D = 64 and 128."""
    for D, T, Hq, Hkv in ((128, 64, 8, 2), (64, 40, 4, 4), (128, 100, 10, 2), (64, 200, 4, 2)):
        w = wl(B=3, Hq=Hq, Hkv=Hkv, D=D, T=T, L=(130, 900))
        case = inputs.make_case(w, 5, layout=layout, page_size=16 if D == 64 else 64)
        case.seq_lens[:] = (case.seq_lens // 64) * 64
        case.seq_lens[0] = 0                      # an empty prefix rides along too
        g = to_gpu(case)
        p = _lib.make_problem(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], g["k_tree"],
                              g["v_tree"], g["parent"], block_table=g["block_table"],
                              page_size=g["page_size"], scale=case.scale)
        ws = torch.empty(_lib.workspace_size(p), dtype=torch.uint8, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        _lib.partials(p, ws, err=err)
        o_s, l_s = _lib.tree(g["q"], g["k_tree"], g["v_tree"], g["parent"], scale=case.scale)
        torch.cuda.synchronize()
        n, rows = _lib.num_splits(p), 3 * T * Hq
        slots = 2 * n + 1   # up to 2 n prefix parts per sequence, then the masked part
        o_part = ws[:slots * rows * D * 4].view(torch.float32).view(slots, rows, D)[2 * n]
        off = _lib.workspace_lse_offset(p)
        l_part = ws[off:off + slots * rows * 4].view(torch.float32).view(slots, rows)[2 * n]
        say(f"fused masked part D={D} T={T} {layout}: {n} splits, lens {case.seq_lens.tolist()}")
        assert int(err.item()) == 0
        assert torch.equal(o_part, o_s.view(rows, D)), "O of the masked part differs"
        assert torch.equal(l_part, l_s.view(rows)), "LSE of the masked part differs"


def test_merge_degenerate_parts():
    sh = (1, 3, 2)
    o_a = torch.randn(*sh, 64, device="cuda")
    o_b = torch.randn(*sh, 64, device="cuda")
    l_a = torch.randn(sh, device="cuda")
    ninf = torch.full(sh, -float("inf"), device="cuda")
    o, l = _lib.merge(o_a, l_a, o_b, ninf)
    torch.cuda.synchronize()
    assert torch.allclose(o, o_a, atol=1e-6) and torch.allclose(l, l_a, atol=1e-6)
    o, l = _lib.merge(o_a, ninf, o_b, ninf)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isinf(l))


def test_device_errors_set_the_flag():
    w = wl(B=2, T=8, L=(50, 90), tree="uniform")
    case = inputs.make_case(w, 1)
    case.parent[1, 3] = 5                      # not topological
    case.seq_lens[0] = case.k_cache.shape[1] + 1  # beyond the capacity
    _, _, err = run_forward(case)
    assert err & _lib.TA_DEV_BAD_PARENT and err & _lib.TA_DEV_BAD_LEN


@pytest.mark.parametrize("splits,shape", [(1, "g4"), (2, "g4"), (0, "g4"), (0, "g5_rowblocks")])
def test_rising_logits_take_the_exact_path(splits, shape):
    """Prefix keys from position 256 on are shifted by +48 in every channel, so a row whose query
    sums to more than about one standard deviation scores them ~48 nats above the first tile: their
    exponentials against the first tile's maximum overflow fp32, and only the exact (moving
    maximum) path gives a finite, correct result. "g5_rowblocks": 350 packed rows per KV head in
    two row blocks of 8 wavefronts, the second with 94 rows."""
    if shape == "g4":
        w = wl(B=2, Hq=8, Hkv=2, T=16, L=(600, 900))
    else:
        w = wl(B=2, Hq=10, Hkv=2, T=70, L=(1500, 2500), depth_cap=12)
    case = inputs.make_case(w, 7)
    k = inputs.bf16_bits_to_f32(case.k_cache)
    for b, L in enumerate(case.seq_lens):
        k[b, 256:L] += 48.0
    case.k_cache[...] = inputs.f32_to_bf16_bits(k)
    say(f"rising logits, splits={splits}, lens={case.seq_lens.tolist()}")
    o, lse, err = run_forward(case, num_splits=splits)
    assert err == 0
    o_ref, lse_ref = oracle.attend_case(case)
    assert np.max(lse_ref) > 40.0   # the shifted keys dominate some rows
    check(case, o, lse, o_ref, lse_ref, f"rising logits splits={splits}")


def test_determinism():
    case = inputs.make_case(wl(L=(900, 1500)), 5)
    o1, l1, _ = run_forward(case)
    o2, l2, _ = run_forward(case)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_workspace_contents_do_not_matter(dtype):
    """A workspace full of 0xFF bytes (NaN partials, part counts of -1) gives the same bits as a
    fresh one: every slot the combine reads is written by the same call first."""
    w = wl(L=(900, 1500)) if dtype == "bf16" else wl(D=64, T=9, dtype="f32", L=(1, 300))
    case = inputs.make_case(w, 6)
    o1, l1, _ = run_forward(case, num_splits=3)
    dirty = torch.full((64 << 20,), 255, dtype=torch.uint8, device="cuda")
    o2, l2, err = run_forward(case, num_splits=3, workspace=dirty)
    assert err == 0
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------------------------------------
# full configuration sizes, in the default launch plan (the one bench.py times)
#
# Every output row is compared for the headline layer (every prefix 64k), the drawn-length GQA
# layer, the long-reasoning layer and the MHA layer (each contiguous and paged) and the sweep's
# small trees. The larger sweep trees and the beam tree are compared on at least two rows of every
# 32-row wavefront tile of every (sequence, KV head, row block). The oracle runs on every core this
# process may use; its results are kept for the module, so the layouts and the unfused calls of
# one workload share them.


def oracle_threads():
    return max(1, len(os.sched_getaffinity(0)))


_CASES = {}
_REFS = {}


def full_case(name, layout="contiguous"):
    key = (name, layout)
    if key not in _CASES:
        _CASES.clear()   # one full-size case on the host at a time
        _CASES[key] = inputs.make_case(inputs.WORKLOADS[name], 0, layout=layout, page_size=64)
    return _CASES[key]


def oracle_ref(name, which="full", rows=None):
    """The oracle on the contiguous case of ``name`` (seed 0): every row, or ``rows``. The paged
    case of the same seed holds the same values (tests/test_oracle_pins.py pins paged = contiguous
    for the oracle), so one result checks both layouts."""
    key = (name, which, None if rows is None else rows.tobytes())
    if key not in _REFS:
        case = full_case(name)
        t0 = time.perf_counter()
        _REFS[key] = oracle.attend_case(case, which=which, rows=rows, nthreads=oracle_threads())
        n = len(_REFS[key][1])
        say(f"oracle {name}/{which}: {n} rows in {time.perf_counter() - t0:.1f} s on "
            f"{oracle_threads()} threads")
    return _REFS[key]


def tile_rows(case, seed=0):
    """At least two rows of every 32-row wavefront tile of every (sequence, KV head, row block).
    Packed row r = node * G + member of KV head g is query head g * G + member of that node; the
    first pick walks the lane position across tiles, the second is drawn."""
    B, T, Hq, Hkv = case.wl.B, case.wl.T, case.wl.Hq, case.wl.Hkv
    G, R = Hq // Hkv, T * (Hq // Hkv)
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        for g in range(Hkv):
            for w0 in range(0, R, 32):
                n = min(32, R - w0)
                for r in (w0 + (7 * b + 5 * g + 3 * (w0 // 32)) % n, w0 + int(rng.integers(n))):
                    node, m = divmod(r, G)
                    rows.add((b, node, g * G + m))
    return np.array(sorted(rows), dtype=np.int32)


def compare_rows(case, o, lse, rows, ref, what):
    B, T, Hq, D = case.q.shape
    if rows is None:
        check(case, o.reshape(-1, D), lse.reshape(-1), ref[0], ref[1], what)
    else:
        idx = (rows[:, 0] * T + rows[:, 1]) * Hq + rows[:, 2]
        check(case, o.reshape(-1, D)[idx], lse.reshape(-1)[idx], ref[0], ref[1], what,
              rows=rows)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite rows"


ALL_ROWS = ["gqa_64k_pinned", "gqa_64k", "long_reasoning", "mha_7b", "sweep_t1", "sweep_t6",
            "sweep_t16"]
TILE_ROWS = ["sweep_t32", "sweep_t64", "sweep_t128", "gqa_64k_beam"]


@pytest.mark.parametrize("name", ALL_ROWS)
def test_forward_full_size_every_row(name):
    case = full_case(name)
    say(f"full {name}: lens={case.seq_lens.tolist()}, all {case.q.shape[0] * case.q.shape[1] * case.q.shape[2]} rows")
    o, lse, err = run_forward(case)
    assert err == 0
    compare_rows(case, o, lse, None, oracle_ref(name), f"full {name}")


@pytest.mark.parametrize("name", ["gqa_64k", "gqa_64k_pinned", "long_reasoning", "mha_7b"])
def test_forward_full_size_paged_every_row(name):
    """The same layers with their prefixes in a pool of 64-key pages in random order."""
    case = full_case(name, "paged")
    say(f"full {name} paged: lens={case.seq_lens.tolist()}")
    o, lse, err = run_forward(case)
    assert err == 0
    compare_rows(case, o, lse, None, oracle_ref(name), f"full {name} paged")


@pytest.mark.parametrize("name", TILE_ROWS)
def test_forward_full_size_every_tile(name):
    case = full_case(name)
    rows = tile_rows(case)
    say(f"full {name}: lens={case.seq_lens.tolist()}, {len(rows)} rows over every wavefront tile")
    o, lse, err = run_forward(case)
    assert err == 0
    compare_rows(case, o, lse, rows, oracle_ref(name, rows=rows), f"full {name}")


def test_unfused_calls_full_size():
    """tree_attn_prefix, tree_attn_tree and tree_attn_merge on the headline layer, every row,
    against the oracle's prefix-only, tree-only and whole results."""
    name = "gqa_64k_pinned"
    case = full_case(name)
    g = to_gpu(case)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_c, l_c = _lib.prefix(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], scale=case.scale,
                           err=err)
    o_s, l_s = _lib.tree(g["q"], g["k_tree"], g["v_tree"], g["parent"], scale=case.scale,
                         err=err)
    o_m, l_m = _lib.merge(o_c, l_c, o_s, l_s, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    del g
    for o, l, which in ((o_c, l_c, "prefix"), (o_s, l_s, "tree"), (o_m, l_m, "full")):
        compare_rows(case, o.float().cpu().numpy(), l.cpu().numpy(), None,
                     oracle_ref(name, which), f"unfused {which} {name}")
