"""C-ABI library checks that need no GPU: exports, status strings, argument validation.

Nothing here enqueues GPU work: every call below is rejected (or answered) on the host before
any launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "treeattn.h")

from tree_verification_attention_amd import _lib  # noqa: E402


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtreeattn.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_every_declared_function_is_exported(lib):
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.tree_attn_abi_version() == 100
    for code in range(6):
        assert _lib.status_string(code) != "unknown status"
    assert _lib.status_string(99) == "unknown status"


def problem(**kw):
    p = _lib.TaProblem()
    p.B, p.T, p.Hq, p.Hkv, p.D = 2, 8, 8, 2, 128
    p.dtype = _lib.TA_BF16
    p.scale = 128 ** -0.5
    fake = 1 << 20  # a 16-byte aligned non-null placeholder; never dereferenced on the host
    p.q = p.k_cache = p.v_cache = p.k_tree = p.v_tree = fake
    p.seq_lens = p.parent = fake
    p.q_sb, p.q_st, p.q_sh = 8 * 8 * 128, 8 * 128, 128
    p.kv_s0, p.kv_s1, p.kv_s2 = 1000 * 2 * 128, 2 * 128, 128
    p.kt_sb, p.kt_st, p.kt_sh = 8 * 2 * 128, 2 * 128, 128
    p.Lmax = 1000
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def ws_size(lib, p):
    n = ctypes.c_size_t(0)
    rc = lib.tree_attn_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return rc, n.value


def test_workspace_size_is_host_only_and_sane(lib):
    rc, n = ws_size(lib, problem())
    assert rc == _lib.TA_OK
    k = ctypes.c_int(0)
    assert lib.tree_attn_num_splits(ctypes.byref(problem()), ctypes.byref(k)) == 0
    rows = 2 * 8 * 8
    assert n >= k.value * rows * (128 + 1) * 4
    # forced split count
    k2 = ctypes.c_int(0)
    assert lib.tree_attn_num_splits(ctypes.byref(problem(num_splits=3)), ctypes.byref(k2)) == 0
    assert k2.value == 3


def test_bf16_split_plan_fills_one_round_of_workgroups(lib):
    """The planner's split count keeps the bf16 launch within one workgroup per CU (256 on a
    host without a device, as on MI355X): 640 packed rows per KV head need three row blocks,
    so 1 * 8 * 3 = 24 workgroups per split and 10 splits (11 would leave 8 waiting)."""
    T, Hq, Hkv, L = 128, 40, 8, 131072
    p = problem(B=1, T=T, Hq=Hq, Hkv=Hkv, Lmax=L, q_sb=T * Hq * 128, q_st=Hq * 128,
                kv_s0=L * Hkv * 128, kv_s1=Hkv * 128, kt_sb=T * Hkv * 128, kt_st=Hkv * 128)
    k = ctypes.c_int(0)
    assert lib.tree_attn_num_splits(ctypes.byref(p), ctypes.byref(k)) == _lib.TA_OK
    assert k.value == 10
    # 32 workgroups per split divide the CUs exactly: 8 splits
    p = problem(B=4, T=64, Hq=32, Hkv=8, Lmax=65536, q_sb=64 * 32 * 128, q_st=32 * 128,
                kv_s0=65536 * 8 * 128, kv_s1=8 * 128, kt_sb=64 * 8 * 128, kt_st=8 * 128)
    assert lib.tree_attn_num_splits(ctypes.byref(p), ctypes.byref(k)) == _lib.TA_OK
    assert k.value == 8


@pytest.mark.parametrize("field,value,status", [
    ("D", 96, _lib.TA_EUNSUPPORTED), ("dtype", 7, _lib.TA_EUNSUPPORTED),
    ("T", 0, _lib.TA_EINVAL), ("T", 257, _lib.TA_EINVAL), ("Hq", 7, _lib.TA_EINVAL),
    ("scale", 0.0, _lib.TA_EINVAL), ("scale", float("nan"), _lib.TA_EINVAL),
    ("q", 0, _lib.TA_EINVAL), ("q", (1 << 20) + 8, _lib.TA_EINVAL),
    ("q_st", 1001, _lib.TA_EINVAL), ("num_splits", -1, _lib.TA_EINVAL),
])
def test_invalid_problems_are_rejected_before_launch(lib, field, value, status):
    p = problem(**{field: value})
    rc, _ = ws_size(lib, p)
    assert rc == status
    o = ctypes.c_void_p(1 << 20)
    assert lib.tree_attn_forward(ctypes.byref(p), o, o, o, 1 << 30, None, None) == status


def test_forward_argument_errors(lib):
    o = ctypes.c_void_p(1 << 20)
    rc, need = ws_size(lib, problem())
    for bad in (dict(seq_lens=0), dict(k_cache=0), dict(parent=0), dict(v_tree=0),
                dict(kv_s1=100), dict(block_table=1 << 20, page_size=24, max_blocks=4,
                                       num_pages=4),
                dict(block_table=1 << 20, page_size=64, max_blocks=0, num_pages=4)):
        assert lib.tree_attn_forward(ctypes.byref(problem(**bad)), o, o, o, need, None,
                                     None) == _lib.TA_EINVAL, bad
    # workspace checks
    assert lib.tree_attn_forward(ctypes.byref(problem()), o, o, o, need - 1, None,
                                 None) == _lib.TA_EWORKSPACE
    assert lib.tree_attn_forward(ctypes.byref(problem()), o, o, None, need, None,
                                 None) == _lib.TA_EWORKSPACE
    assert lib.tree_attn_forward(ctypes.byref(problem()), o, o, ctypes.c_void_p((1 << 20) + 16),
                                 need, None, None) == _lib.TA_EWORKSPACE
    assert lib.tree_attn_prefix(ctypes.byref(problem()), o, None, o, need, None,
                                None) == _lib.TA_EINVAL


@pytest.mark.parametrize("page_size,max_blocks", [
    (24, 4),            # not a power of two
    (8, 4),             # below 16 keys
    (-(1 << 31), 4),    # negative
    ((1 << 30) + 1, 1),  # above 2^30 (the page shift's range)
    (1 << 16, 1 << 16),  # capacity max_blocks * page_size past INT32_MAX
    (64, 0),            # no block-table entries
])
def test_paged_parameters_rejected_by_every_entry_point(lib, page_size, max_blocks):
    """A block table with bad paging parameters is refused on the host by every entry point that
    plans the split -- the tree-only call, the workspace / split queries and the combine included,
    none of which reads the prefix -- before any capacity or page shift is computed from it."""
    p = problem(block_table=FAKE, page_size=page_size, max_blocks=max_blocks, num_pages=4)
    o = ctypes.c_void_p(FAKE)
    n = ctypes.c_size_t(0)
    k = ctypes.c_int(0)
    assert lib.tree_attn_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.TA_EINVAL
    assert lib.tree_attn_num_splits(ctypes.byref(p), ctypes.byref(k)) == _lib.TA_EINVAL
    assert lib.tree_attn_tree(ctypes.byref(p), o, o, None, None) == _lib.TA_EINVAL
    assert lib.tree_attn_combine(ctypes.byref(p), o, 1 << 30, o, o, None) == _lib.TA_EINVAL
    assert lib.tree_attn_forward(ctypes.byref(p), o, o, o, 1 << 30, None, None) == _lib.TA_EINVAL
    assert lib.tree_attn_partials(ctypes.byref(p), o, 1 << 30, None, None) == _lib.TA_EINVAL
    assert lib.tree_kv_commit(ctypes.byref(p), o, o, o, o, o, None, None) == _lib.TA_EINVAL
    # B = 0 plans nothing but is still refused with such parameters
    p0 = problem(B=0, block_table=FAKE, page_size=page_size, max_blocks=max_blocks, num_pages=4)
    assert lib.tree_attn_workspace_size(ctypes.byref(p0), ctypes.byref(n)) == _lib.TA_EINVAL


def test_largest_page_size_plans(lib):
    """Pages of 2^30 keys are admitted (one block-table entry) and plan without overflow."""
    p = problem(block_table=FAKE, page_size=1 << 30, max_blocks=1, num_pages=1)
    k = ctypes.c_int(0)
    assert lib.tree_attn_num_splits(ctypes.byref(p), ctypes.byref(k)) == _lib.TA_OK
    assert k.value >= 1


def test_noalloc_forward_rejects_problems_beyond_its_scratch(lib):
    """The allocation-free forward refuses, on the host and before any launch, a problem whose
    split partials need more than its fixed device array; argument errors come first."""
    T, Hq, Hkv, L = 256, 32, 8, 16384
    big = problem(B=16, T=T, Hq=Hq, Hkv=Hkv, Lmax=L, q_sb=T * Hq * 128, q_st=Hq * 128,
                  kv_s0=L * Hkv * 128, kv_s1=Hkv * 128, kt_sb=T * Hkv * 128, kt_st=Hkv * 128)
    rc, need = ws_size(lib, big)
    assert rc == _lib.TA_OK and need > _lib.TA_NOALLOC_SCRATCH_BYTES
    o = ctypes.c_void_p(FAKE)
    assert lib.tree_attn_forward_noalloc(ctypes.byref(big), o, o, None, None) == _lib.TA_ESCRATCH
    assert "TA_NOALLOC_SCRATCH_BYTES" in _lib.status_string(_lib.TA_ESCRATCH)
    assert lib.tree_attn_forward_noalloc(ctypes.byref(problem(D=96)), o, o, None,
                                         None) == _lib.TA_EUNSUPPORTED
    assert lib.tree_attn_forward_noalloc(ctypes.byref(problem(B=0)), o, o, None, None) == 0
    # the headline layer (4 x 64 nodes x 32 heads, 8 splits) fits
    hl = problem(B=4, T=64, Hq=32, Hkv=8, Lmax=65536, q_sb=64 * 32 * 128, q_st=32 * 128,
                 kv_s0=65536 * 8 * 128, kv_s1=8 * 128, kt_sb=64 * 8 * 128, kt_st=8 * 128)
    rc, need = ws_size(lib, hl)
    assert rc == _lib.TA_OK and need <= _lib.TA_NOALLOC_SCRATCH_BYTES


def test_merge_and_mask_argument_errors(lib):
    o = ctypes.c_void_p(1 << 20)
    assert lib.tree_attn_merge(1, 2, 3, 96, o, o, o, o, o, 0, o, None) == _lib.TA_EUNSUPPORTED
    assert lib.tree_attn_merge(1, 2, 3, 64, o, o, o, o, o, 5, o, None) == _lib.TA_EUNSUPPORTED
    assert lib.tree_attn_merge(1, 2, 3, 64, None, o, o, o, o, 0, o, None) == _lib.TA_EINVAL
    assert lib.tree_attn_merge(0, 2, 3, 64, None, None, None, None, None, 0, None, None) == 0
    assert lib.tree_mask_build(o, 1, 0, o, None, None) == _lib.TA_EINVAL
    assert lib.tree_mask_build(o, 1, 257, o, None, None) == _lib.TA_EINVAL
    assert lib.tree_mask_build(None, 1, 8, o, None, None) == _lib.TA_EINVAL
    assert lib.tree_mask_build(None, 0, 8, None, None, None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        _lib.forward(q, q, q, torch.zeros(1, dtype=torch.int32), q[:, :, :1], q[:, :, :1],
                     torch.zeros(1, 2, dtype=torch.int32))


FAKE = 1 << 20   # aligned non-null placeholder, never dereferenced: every call below is rejected


def test_greedy_accept_rejects_bad_arguments_on_the_host(lib):
    S = ctypes.c_size_t
    n = S(0)
    assert lib.tree_greedy_accept_workspace_size(_lib.TA_BF16, 4, 64, 128256, ctypes.byref(n)) == 0
    assert n.value >= 4 * 65 * 8 and n.value % 256 == 0
    assert lib.tree_greedy_accept_workspace_size(7, 4, 64, 100, ctypes.byref(n)) == _lib.TA_EUNSUPPORTED
    assert lib.tree_greedy_accept_workspace_size(_lib.TA_BF16, 4, 257, 100, ctypes.byref(n)) == _lib.TA_EINVAL
    args = lambda **kw: [kw.get("logits", FAKE), kw.get("dtype", _lib.TA_BF16),
                         kw.get("stride", 128), 2, kw.get("T", 8), kw.get("V", 128), FAKE, FAKE,
                         FAKE, kw.get("ws_bytes", 1 << 20), FAKE, FAKE, FAKE, FAKE, None, None]
    assert lib.tree_greedy_accept(*args(stride=100)) == _lib.TA_EINVAL       # stride < V
    assert lib.tree_greedy_accept(*args(V=124, stride=124)) == _lib.TA_EINVAL  # rows not 16-B apart
    assert lib.tree_greedy_accept(*args(logits=FAKE + 2)) == _lib.TA_EINVAL   # misaligned base
    assert lib.tree_greedy_accept(*args(ws_bytes=8)) == _lib.TA_EWORKSPACE
    assert lib.tree_greedy_accept(*args(T=0)) == _lib.TA_EINVAL


def test_spec_sample_rejects_bad_arguments_on_the_host(lib):
    S = ctypes.c_size_t
    n = S(0)
    assert lib.tree_spec_sample_workspace_size(4, 64, 128256, ctypes.byref(n)) == 0
    assert n.value >= 2 * 4 * 65 * 32 * 8
    assert lib.tree_spec_sample_workspace_size(1, 8, (1 << 20) + 1, ctypes.byref(n)) == _lib.TA_EINVAL
    args = lambda **kw: [kw.get("p", FAKE), FAKE, kw.get("stride", 1024), 2, 8,
                         kw.get("V", 1024), FAKE, FAKE, FAKE, FAKE, FAKE,
                         kw.get("ws_bytes", 1 << 20), FAKE, FAKE, FAKE, None, None]
    assert lib.tree_spec_sample(*args(stride=1000)) == _lib.TA_EINVAL      # stride < V
    assert lib.tree_spec_sample(*args(stride=1026, V=1025)) == _lib.TA_EINVAL  # rows misaligned
    assert lib.tree_spec_sample(*args(p=FAKE + 4)) == _lib.TA_EINVAL
    assert lib.tree_spec_sample(*args(ws_bytes=64)) == _lib.TA_EWORKSPACE


def test_gdn_calls_reject_bad_arguments_on_the_host(lib):
    f = ctypes.c_float(0.088)
    base = dict(B=2, T=16, Hk=2, Hv=4, dk=128, dv=64)

    def verify(**kw):
        a = dict(base, **kw)
        return lib.tree_gdn_verify(kw.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"],
                                   a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"], f, FAKE, None, None)

    assert verify(dk=96) == _lib.TA_EUNSUPPORTED
    assert verify(dv=48) == _lib.TA_EUNSUPPORTED
    assert verify(dv=288) == _lib.TA_EUNSUPPORTED
    assert verify(Hv=6, Hk=4) == _lib.TA_EINVAL
    assert verify(T=257) == _lib.TA_EINVAL
    assert verify(q=FAKE + 2) == _lib.TA_EINVAL
    assert verify(q=0) == _lib.TA_EINVAL
    assert verify(B=0) == _lib.TA_OK
    assert lib.tree_gdn_commit(FAKE, FAKE, FAKE, FAKE, 2, 16, 2, 4, 64, 64, FAKE, FAKE, 0,
                               None, None) == _lib.TA_EINVAL


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c11"), ("g++", "-std=c++17")])
def test_header_compiles_as_c_and_cxx(tmp_path, compiler, std):
    """The public header is plain C: it compiles on its own as C11 and as C++17 (the HIP
    runtime API header supplies hipStream_t), with every declaration usable from C."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / "use_header.c"
    src.write_text('#include "treeattn.h"\n'
                   "int use(const ta_problem *p, size_t *n) {\n"
                   "    int k = 0;\n"
                   "    return tree_attn_workspace_size(p, n) | tree_attn_num_splits(p, &k);\n"
                   "}\n")
    lang = ["-x", "c++"] if compiler == "g++" else []
    cmd = [compiler, std, "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
           "-I/opt/rocm/include", *lang, "-c", str(src), "-o", str(tmp_path / "use_header.o")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
