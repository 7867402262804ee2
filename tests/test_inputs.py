"""The seeded input generators: determinism, tree constraints, bf16 rounding, layouts."""
import numpy as np
import pytest
import torch

from tree_verification_attention_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38,
                                  1e-40, np.inf, -np.inf], dtype=np.float32)])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", ["tiny_f32", "mha_7b"])
def test_same_seed_same_case(name):
    wl = inputs.WORKLOADS[name]
    if name == "mha_7b":
        wl = wl.replace(L=300)
    a = inputs.make_case(wl, 3)
    b = inputs.make_case(wl, 3)
    c = inputs.make_case(wl, 4)
    for f in ("seq_lens", "parent", "q", "k_cache", "v_cache", "k_tree", "v_tree"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=True)
    assert not np.array_equal(a.q, c.q)


def test_tree_constraints():
    rng = np.random.default_rng(0)
    for T in (1, 6, 16, 64, 128, 256):
        for cap in (8, 12):
            par = inputs.bounded_tree(rng, T, cap, 4)
            assert np.all(par < np.arange(T)) and np.all(par >= -1)
            assert inputs.tree_depths(par).max() <= cap
            kids = np.bincount(par[par >= 0], minlength=T)
            assert kids.max(initial=0) <= 4 and np.sum(par < 0) <= 4
        u = inputs.uniform_tree(rng, T)
        assert np.all(u < np.arange(T)) and np.all(u >= -1)
    beam = inputs.make_tree(rng, inputs.WORKLOADS["gqa_64k_beam"])
    assert len(beam) == 64 and np.all(beam < np.arange(64))
    d = inputs.tree_depths(beam)
    assert [int(np.sum(d == k)) for k in range(1, 6)] == [4, 16, 16, 16, 12]


def test_sweep_and_named_trees():
    assert inputs.make_case(inputs.WORKLOADS["sweep_t6"].replace(B=1, L=8), 0).parent.tolist() == \
        [[-1, 0, 1, 2, 3, 4]]
    assert inputs.make_case(inputs.WORKLOADS["sweep_t1"].replace(B=1, L=8), 0).parent.tolist() == [[-1]]


def test_ragged_lengths_and_nan_padding():
    wl = inputs.Workload("r", B=5, Hq=4, Hkv=2, D=16, T=4, L=(3, 40))
    c = inputs.make_case(wl, 1)
    assert c.seq_lens.min() >= 3 and c.seq_lens.max() <= 40
    assert c.k_cache.shape[1] == c.seq_lens.max()
    for b in range(5):
        L = c.seq_lens[b]
        assert np.all(c.k_cache[b, L:] == inputs.BF16_NAN)
        assert not np.any(c.k_cache[b, :L] == inputs.BF16_NAN)
    f = inputs.make_case(wl, 1, pad="finite", lcap=64)
    assert f.k_cache.shape[1] == 64 and np.all(f.k_cache[0, f.seq_lens[0]:] == 0)
    # values do not depend on the padding choice
    assert np.array_equal(f.q, c.q)
    assert np.array_equal(f.k_cache[2, :c.seq_lens[2]], c.k_cache[2, :c.seq_lens[2]])


def test_paged_layout_holds_the_same_rows():
    wl = inputs.Workload("p", B=3, Hq=4, Hkv=2, D=16, T=3, L=(1, 200))
    c = inputs.make_case(wl, 2)
    p = inputs.make_case(wl, 2, layout="paged", page_size=32)
    ps = p.page_size
    used = set()
    for b in range(3):
        L = int(c.seq_lens[b])
        nblk = (L + ps - 1) // ps
        pages = p.block_table[b, :nblk]
        used.update(int(x) for x in pages)
        rows = p.k_cache[pages].reshape(-1, 2, 16)[:L]
        assert np.array_equal(rows, c.k_cache[b, :L])
        assert np.all(p.block_table[b, nblk:] == p.k_cache.shape[0] - 1)
    assert len(used) == sum((int(n) + ps - 1) // ps for n in c.seq_lens)
    assert np.all(p.k_cache[-1] == inputs.BF16_NAN)


def test_outlier_channels():
    wl = inputs.WORKLOADS["long_reasoning"].replace(L=64, T=8)
    c = inputs.make_case(wl, 0)
    ch = c.outlier_channels
    assert len(ch) == 4 and len(set(ch.tolist())) == 4
    k = inputs.bf16_bits_to_f32(c.k_cache).astype(np.float64)
    v = inputs.bf16_bits_to_f32(c.v_cache).astype(np.float64)
    others = np.setdiff1d(np.arange(128), ch)
    assert 6 < k[..., ch].std() < 10 and 0.8 < k[..., others].std() < 1.2
    assert 0.8 < v[..., ch].std() < 1.2
