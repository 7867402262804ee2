"""Host logic of bench.py (no GPU): the work model, the roofline classification, the counter
summaries it writes under profiles/ and reads back, and the one-GPU guard."""
import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def fake_case(B, T, Hq, Hkv, D, lens, parent, dtype="bf16", block_table=None, page_size=0):
    wl = types.SimpleNamespace(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    return types.SimpleNamespace(wl=wl, seq_lens=np.array(lens, dtype=np.int32),
                                 parent=np.array(parent, dtype=np.int32).reshape(B, T),
                                 block_table=block_table, page_size=page_size)


def test_work_model_by_hand():
    # one sequence, 10 prefix keys, a 2-node chain, 2 query heads on 1 KV head, D = 64, bf16
    w = bench.work_of(fake_case(1, 2, 2, 1, 64, [10], [-1, 0]))
    kv = 2 * 2 * 1 * 64 * 10          # K and V of every prefix key
    q = 2 * 1 * 2 * 2 * 64
    tree = 2 * 2 * 1 * 2 * 1 * 64
    meta = 4 * 2 + 4                  # parents, lengths
    out = 2 * 1 * 2 * 2 * 64 + 4 * 1 * 2 * 2
    assert w["kernel_bytes"] == kv + q + tree + meta
    assert w["step_bytes"] == kv + q + tree + meta + out
    # every (row, visible key) pair costs 4 D flops; node 0 sees itself, node 1 sees 0 and 1
    assert w["flops"] == 4 * 64 * 2 * (2 * 10 + 1 + 2)


def test_work_model_paged_counts_block_table_entries():
    bt = np.zeros((2, 4), dtype=np.int32)
    w = bench.work_of(fake_case(2, 1, 1, 1, 64, [100, 17], [-1, -1], block_table=bt,
                                page_size=64))
    w0 = bench.work_of(fake_case(2, 1, 1, 1, 64, [100, 17], [-1, -1]))
    assert w["kernel_bytes"] - w0["kernel_bytes"] == 4 * (2 + 1)


def test_bound_classification():
    # the headline layer: 275 GFLOP take 110 us at the bf16 peak, 1.08 GB take 135 us at 8 TB/s
    assert bench.bound_of(274_895_323_136, 1_079_018_512) == "hbm"
    # the long-reasoning layer: 344 GFLOP (137 us) against 0.54 GB (67 us)
    assert bench.bound_of(343_597_383_680, 537_000_000) == "mfma"
    # plain decode: next to no flops
    assert bench.bound_of(1e9, 1e9) == "hbm"


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for k, c, v in rows:
            f.write(f"\"{k}\",{c},{v}\n")


KNAME = "void ta::attn_prefix_kernel<128, 8, false>(ta::AttnArgs)"


def test_traffic_summary_round_trip(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    fetch, write = tmp_path / "fetch", tmp_path / "write"
    # two kernel dispatches, 1 GiB copies reading 524288 KiB (factor 2) and writing 1 GiB, plus a
    # small upload copy the calibration ignores
    write_csv(str(fetch / "a" / "run_counter_collection.csv"),
              [(KNAME, "FETCH_SIZE", 500000), (KNAME, "FETCH_SIZE", 510000),
               ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288),
               ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288),
               ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 10)])
    write_csv(str(write / "a" / "run_counter_collection.csv"),
              [(KNAME, "WRITE_SIZE", 30000), (KNAME, "WRITE_SIZE", 30000),
               ("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576)])
    bench.parse_pmc(str(fetch), str(write), "wl")
    t = bench.traffic_entry("wl")
    assert t is not None
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes"] == pytest.approx(505000 * 1024 * 2.0)
    assert t["traffic_bytes"] == pytest.approx(505000 * 2048 + 30000 * 1024)
    with open(bench.traffic_path("wl")) as f:
        head = f.read()
    assert "--no-configs" in head and "FETCH_SIZE" in head
    # a summary taken before the kernel sources changed is not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.traffic_entry("wl") is None


def test_util_summary_round_trip(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    util, issue = tmp_path / "util", tmp_path / "issue"
    write_csv(str(util / "run_counter_collection.csv"),
              [(KNAME, "MfmaUtil", 50.0), (KNAME, "SQ_INSTS_VALU", 4e7), (KNAME, "SQ_WAVES", 2048)])
    cyc = 500_000
    write_csv(str(issue / "run_counter_collection.csv"),
              [(KNAME, "GRBM_GUI_ACTIVE", 8 * cyc),
               (KNAME, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * cyc),
               (KNAME, "SQ_ACTIVE_INST_VALU", 0.25 * 1024 * cyc),   # quad-cycles: share 1.0
               (KNAME, "SQ_ACTIVE_INST_LDS", 0.025 * 1024 * cyc),
               (KNAME, "SQ_INSTS_VALU_TRANS_F32", 8e6)])
    bench.parse_util([str(util), str(issue)], "wl")
    u = bench.util_entry("wl")
    assert u["mfma_util_pct"] == pytest.approx(50.0)
    assert u["mfma_busy_share"] == pytest.approx(0.5, rel=1e-3)
    assert u["valu_issue_share"] == pytest.approx(1.0, rel=1e-3)
    assert u["lds_issue_share"] == pytest.approx(0.1, rel=1e-3)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.util_entry("wl") is None


def test_power_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    trace = {"t0_unix": 100.0, "bucket_s": 0.05, "first_steps_us": [300.0] * 5 + [400.0] * 20,
             "buckets": [{"t_s": 0.0, "steps": 25, "median_us": 380.0, "min_us": 300.0,
                          "max_us": 400.0}]}
    tp = tmp_path / "trace.json"
    tp.write_text(json.dumps(trace))
    sample = {"gpu_data": [{"power": {"socket_power": {"value": 1400}},
                            "clock": {"gfx_0": {"clk": {"value": 1700}}}}]}
    sp = tmp_path / "smi.txt"
    sp.write_text(f"T 99.5\n{json.dumps(sample)}\nT 100.5\nnot json\n")
    bench.power_summary(str(tp), str(sp), 1.0)
    text = (tmp_path / "profiles" / f"{bench.KERNEL_NAME}_gqa_64k_pinned_power.txt").read_text()
    assert "mean 400.0 us" in text          # steps 5..24
    assert "1400" in text and "1700" in text


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
