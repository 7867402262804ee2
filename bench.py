#!/usr/bin/env python3
"""Tree-verification attention benchmark on one MI355X.

Headline workload: one GQA bf16 attention layer of a speculative-decoding verify step -- B = 4
sequences, 32 query heads over 8 KV heads, head_dim 128, a 64-node draft tree per sequence
(depth <= 8, at most 4 children per node) and a 65536-token committed prefix per sequence.
Inputs are seeded synthetic values (see tree_verification_attention_amd.inputs), copied to HBM
before the timed region.

A step is one call of tree_attn_forward: all prefix splits plus the masked tree part, then the
log-sum-exp combine. ``value`` is the achieved algorithmic HBM bandwidth of a step (prefix K/V,
Q, tree K/V and parents read once; O and LSE written once) in TB/s; ``us_per_layer`` is the
same step's time. The roofline entry is for the split step that carries all the HBM traffic:
one tree_attn_partials call (one prefix-kernel launch; its last split also takes the masked
part, the tree keys and the prefix tail), launched alone and timed with HIP events on its
stream.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --parse-pmc FETCH_DIR WRITE_DIR   (writes the traffic summary)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tree-verify attention µs/layer + achieved HBM TB/s, 64-node tree @64k ctx"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFS = 157.3        # MI355X fp32 vector
KERNEL_NAME = "attn_prefix_kernel"
COPY_BYTES = 1 << 30
FLUSH_BYTES = 1 << 29
CSRC = os.path.join(ROOT, "tree_verification_attention_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# the sources of the two kernels the traffic counters cover
TRAFFIC_SOURCES = ("attn_prefix.hip", "lds_dma.h", "ancestors.h", "launch.h", "abi.cpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in sorted(os.path.join(CSRC, n) for n in TRAFFIC_SOURCES):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def work_of(case):
    """Algorithmic bytes and flops of one layer (and of its dominant kernel)."""
    wl = case.wl
    es = 2 if wl.dtype == "bf16" else 4
    B, T, Hq, Hkv, D = wl.B, wl.T, wl.Hq, wl.Hkv, wl.D
    sum_l = int(case.seq_lens.astype("int64").sum())
    kv = 2 * es * Hkv * D * sum_l
    q = es * B * T * Hq * D
    tree = 2 * es * B * T * Hkv * D
    meta = 4 * B * T + 4 * B
    if case.block_table is not None:
        ps = case.page_size
        meta += 4 * int(sum((int(n) + ps - 1) // ps for n in case.seq_lens))
    out = es * B * T * Hq * D + 4 * B * T * Hq
    from tree_verification_attention_amd.inputs import tree_depths
    visible_tree = int(sum(tree_depths(case.parent[b]).sum() for b in range(B)))
    flops = 4 * D * Hq * (T * sum_l + visible_tree)
    return {"kernel_bytes": kv + q + tree + meta, "step_bytes": kv + q + tree + meta + out,
            "flops": flops, "sum_len": sum_l}


def bound_of(flops, nbytes):
    """The resource whose peak takes longer for this much work: "mfma" (bf16 dense) or "hbm"."""
    return "mfma" if flops / (MFMA_BF16_PEAK_TFS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9) else "hbm"


def to_device(case):
    import numpy as np
    import torch

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    return {k: dev(getattr(case, k)) for k in ("q", "k_cache", "v_cache", "seq_lens", "k_tree",
                                                "v_tree", "parent", "block_table")}


class Launch:
    """Device operands, outputs and workspace of one case, and its two timed calls: the fused
    forward (tree_attn_forward) and the split step alone (tree_attn_partials)."""

    def __init__(self, case):
        import ctypes

        import torch

        from tree_verification_attention_amd import _lib

        g = to_device(case)
        self.g = g
        self.p = _lib.make_problem(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], g["k_tree"],
                                   g["v_tree"], g["parent"], block_table=g["block_table"],
                                   page_size=case.page_size or None, scale=case.scale)
        self.lib = _lib.load()
        B, T, Hq, D = case.q.shape
        self.out = torch.empty((B, T, Hq, D), dtype=g["q"].dtype, device="cuda")
        self.lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
        self.ws_bytes = _lib.workspace_size(self.p)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.stream = torch.cuda.current_stream()
        sh = self.stream.cuda_stream
        pp = ctypes.byref(self.p)
        self.args_fwd = (pp, self.out.data_ptr(), self.lse.data_ptr(), self.ws.data_ptr(),
                         self.ws_bytes, self.err.data_ptr(), sh)
        self.args_part = (pp, self.ws.data_ptr(), self.ws_bytes, self.err.data_ptr(), sh)
        self.n_splits = _lib.num_splits(self.p)
        self._status = _lib.status_string

    def fwd(self):
        rc = self.lib.tree_attn_forward(*self.args_fwd)
        if rc:
            raise RuntimeError(f"tree_attn_forward: {self._status(rc)}")

    def part(self):
        rc = self.lib.tree_attn_partials(*self.args_part)
        if rc:
            raise RuntimeError(f"tree_attn_partials: {self._status(rc)}")

    def check_flag(self):
        flag = int(self.err.item())
        if flag:
            raise RuntimeError(f"device error flag {flag}")


def events_around(fn, stream, steps, before=None):
    """HIP events recorded on ``stream`` around each of ``steps`` calls of ``fn`` (``before``, if
    given, runs ahead of each call outside the events); returns the durations in us."""
    import torch

    evs = []
    for _ in range(steps):
        if before is not None:
            before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def time_case(case, steps, warmup, label):
    """Time ``steps`` fused forwards back to back and ``steps`` dominant-kernel launches of
    ``case``, each of the latter after an evicting read."""
    import torch

    L = Launch(case)
    print(f"[bench] {label}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        L.fwd()
    torch.cuda.synchronize()
    # timed region: exactly `steps` fused steps, nothing between them
    t0 = time.perf_counter()
    for _ in range(steps):
        L.fwd()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the per-step spread, from a second pass of `steps` forwards right after the timed one: an
    # event pair around every step costs the step about 6 us, so the timed pass records none
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(L.stream)
        L.fwd()
        ev[i][1].record(L.stream)
    torch.cuda.synchronize()
    step_us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    # the dominant kernel alone, same stream, same events; before each launch a 512 MiB read
    # (outside the events) evicts the 256 MB last-level cache and the L2s
    evict = make_evict()
    for _ in range(warmup):
        L.part()
    torch.cuda.synchronize()
    kern_us = events_around(L.part, L.stream, steps, evict)
    L.check_flag()
    print(f"[bench] {label}: done ({wall * 1e6 / steps:.1f} us/step wall)", file=sys.stderr,
          flush=True)
    return {"wall_s": wall, "step_us": step_us, "kernel_us": kern_us,
            "n_splits": L.n_splits, "ws_bytes": L.ws_bytes}


def time_evicted(case, steps, warmup, label):
    """The fused forward and the split step of ``case``, each call timed with HIP events after a
    512 MiB evicting read (every step starts from cold caches, as a layer of a decode step whose
    KV was last touched one step earlier). The two calls alternate, so that both meet the same
    state of the part's power management (a loop of one after a loop of the other would time
    the first in the clock dip that follows the warm-up)."""
    import torch

    L = Launch(case)
    evict = make_evict()
    print(f"[bench] {label}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        L.fwd()
        L.part()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        pair = []
        for fn in (L.fwd, L.part):
            evict()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(L.stream)
            fn()
            e1.record(L.stream)
            pair.append((e0, e1))
        evs.append(pair)
    torch.cuda.synchronize()
    fwd_us = [a.elapsed_time(b) * 1e3 for (a, b), _ in evs]
    part_us = [a.elapsed_time(b) * 1e3 for _, (a, b) in evs]
    L.check_flag()
    return {"fwd_us": fwd_us, "part_us": part_us, "n_splits": L.n_splits}


def make_evict():
    """A function that reads FLUSH_BYTES of device memory. A read, not a fill: it leaves the caches
    holding clean lines of another buffer, so the timed kernel pays for no write-back of them."""
    import torch

    buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((), dtype=torch.float32, device="cuda")
    return lambda: torch.sum(buf, dim=0, out=out)


# One entry per configuration the benchmark covers (the pages' workload families, all on seeded
# synthetic inputs): (key, workload, layout, description).
CONFIGS = [
    ("tiny_f32", "tiny_f32", "contiguous",
     "Tiny fp32: B=1, 4 q / 1 KV heads, D=64, prefix 256, 8-node tree (parent uniform in [-1, i-1])"),
    ("mha_7b", "mha_7b", "contiguous",
     "MHA 7B-layer bf16: B=1, 32/32 heads, D=128, prefix 16384, 64-node tree (depth<=8, <=4 children)"),
    ("gqa_64k", "gqa_64k", "contiguous",
     "GQA bf16: B=4, 32/8 heads, D=128, prefix lengths drawn in [32768, 65536], 64-node trees"),
    ("gqa_64k_pinned", "gqa_64k_pinned", "contiguous",
     "GQA bf16, every prefix 65536 (the headline layer), cold caches"),
    ("gqa_64k_pinned_paged", "gqa_64k_pinned", "paged",
     "the headline layer with its prefix in a pool of 64-key pages in random order"),
    ("sweep_t1", "sweep_t1", "contiguous",
     "tree-size sweep: B=8, 32/8 heads, D=128, prefix 32768, one node (plain decode)"),
    ("sweep_t6", "sweep_t6", "contiguous", "tree-size sweep, 6-node chain"),
    ("sweep_t16", "sweep_t16", "contiguous", "tree-size sweep, 16-node tree"),
    ("sweep_t32", "sweep_t32", "contiguous", "tree-size sweep, 32-node tree"),
    ("sweep_t64", "sweep_t64", "contiguous", "tree-size sweep, 64-node tree"),
    ("sweep_t128", "sweep_t128", "contiguous", "tree-size sweep, 128-node tree"),
    ("long_reasoning", "long_reasoning", "contiguous",
     "Long-reasoning bf16: B=1, 40/8 heads, D=128, prefix 131072, 128-node tree (depth<=12), "
     "K x8 on 4 channels"),
    ("gqa_64k_beam", "gqa_64k_beam", "contiguous",
     "GQA bf16 64k with a beam-search tree (layer widths 4, 16, 16, 16, 12)"),
]


def time_configs(steps, warmup, seed):
    """Every configuration of CONFIGS: median / p10 / p90 of the fused forward and of the split
    step (HIP events, evicting read before each call), bytes and flops against the HBM and bf16
    MFMA peaks, and the node x q-head throughput."""
    import gc

    import torch

    from tree_verification_attention_amd import inputs

    out = {}
    for key, name, layout, desc in CONFIGS:
        wl = inputs.WORKLOADS[name]
        case = inputs.make_case(wl, seed, layout=layout, page_size=64, pad="finite")
        w = work_of(case)
        r = time_evicted(case, steps, warmup, key)
        f, k = statistics.median(r["fwd_us"]), statistics.median(r["part_us"])
        lens = case.seq_lens
        e = {"workload": desc, "B": wl.B, "T": wl.T, "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D,
             "dtype": wl.dtype, "prefix": [int(lens.min()), int(lens.max())],
             "layout": layout, "splits": r["n_splits"],
             "us_per_layer": round(f, 2), "us_p10": round(pct(r["fwd_us"], 0.1), 2),
             "us_p90": round(pct(r["fwd_us"], 0.9), 2),
             "split_step_us": round(k, 2),
             "tb_per_s": round(w["step_bytes"] / (f * 1e-6) / 1e12, 4),
             "frac_hbm": round(w["step_bytes"] / (f * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "split_frac_hbm": round(w["kernel_bytes"] / (k * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "node_qheads_per_s": round(wl.B * wl.T * wl.Hq / (f * 1e-6), 1),
             "algorithmic_bytes": w["step_bytes"], "flops": w["flops"]}
        if wl.dtype == "bf16":
            e["tflops"] = round(w["flops"] / (f * 1e-6) / 1e12, 1)
            e["frac_mfma"] = round(w["flops"] / (f * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
            e["split_frac_mfma"] = round(w["flops"] / (k * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
            e["bound"] = bound_of(w["flops"], w["step_bytes"])
        else:
            e["bound"] = "latency (fp32 path, 0.15 MB)"
        if layout == "contiguous":
            # HBM traffic and counter shares of the split step, where profiles/ holds them for
            # the kernel as it stands
            t, u = traffic_entry(name), util_entry(name)
            if t:
                e["split_traffic_bytes"] = round(t["traffic_bytes"])
            if u:
                e["split_counters"] = u
        out[key] = e
        print(f"[bench] {key}: {f:.1f} us/layer (split {k:.1f} us), "
              f"{e['tb_per_s']:.2f} TB/s", file=sys.stderr, flush=True)
        del case, r
        gc.collect()
        torch.cuda.empty_cache()
    return out


def copy_ceiling(steps=10):
    """A plain 1 GiB device-to-device copy (torch copy_, HIP events): 2 GiB of HBM traffic per
    copy, the practical bandwidth ceiling to set beside the 8 TB/s peak."""
    import torch

    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    us = events_around(lambda: dst.copy_(src), torch.cuda.current_stream(), steps)
    m = statistics.median(us)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_per_copy": 2 * COPY_BYTES, "us": round(m, 2),
            "gbs": round(2 * COPY_BYTES / (m * 1e-6) / 1e9, 1),
            "frac": round(2 * COPY_BYTES / (m * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "1 GiB read + 1 GiB written per copy, median of HIP-event timings"}


def host_cpu():
    """Host cores and CPU model for the CPU-baseline record."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "model": model}


def time_breakdown(case, steps, warmup):
    """The unfused entry points on the same layer, each call timed alone with HIP events after an
    evicting read: mask build, prefix part (its splits merged), tree part, two-way merge."""
    import torch

    from tree_verification_attention_amd import _lib

    g = to_device(case)
    evict = make_evict()
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(steps):
            evict()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return round(statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs), 2)

    kw = dict(scale=case.scale)
    oc, lc = _lib.prefix(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"], **kw)
    os_, ls = _lib.tree(g["q"], g["k_tree"], g["v_tree"], g["parent"], **kw)
    out = {
        "mask_build_us": timed(lambda: _lib.mask_build(g["parent"])),
        "prefix_us": timed(lambda: _lib.prefix(g["q"], g["k_cache"], g["v_cache"], g["seq_lens"],
                                               **kw)),
        "tree_us": timed(lambda: _lib.tree(g["q"], g["k_tree"], g["v_tree"], g["parent"], **kw)),
        "merge_us": timed(lambda: _lib.merge(oc, lc, os_, ls, out_dtype=torch.bfloat16)),
        "note": "unfused entry points, each call timed alone (median) after an evicting read; "
                "the prefix call includes the merge of its own splits",
    }
    del g, oc, lc, os_, ls
    torch.cuda.empty_cache()
    return out


def time_next_rows(steps, warmup, seed):
    """Greedy tree acceptance over a Llama-3-size vocabulary and the accepted-path KV commit, at
    the headline batch / tree / head shape; each call timed with HIP events after a cache-evicting read."""
    import numpy as np
    import torch

    import oracle.accept as oacc
    from tree_verification_attention_amd import _lib, inputs

    B, T, V = 4, 64, 128256
    ac = inputs.make_accept_case(B, T, V, seed)
    lg = torch.from_numpy(ac.logits.view(np.int16)).view(torch.bfloat16).cuda()
    draft, parent = torch.from_numpy(ac.draft).cuda(), torch.from_numpy(ac.parent).cuda()
    evict = make_evict()
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(steps):
            evict()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(b) * 1e3 for a, b in evs)

    print("[bench] greedy acceptance", file=sys.stderr, flush=True)
    acc_ws = torch.zeros(_lib.greedy_accept_workspace_size(lg.dtype, B, T, V), dtype=torch.uint8,
                         device="cuda")
    acc_us = timed(lambda: _lib.greedy_accept(lg, draft, parent, ws=acc_ws))
    _, n_gpu, path_gpu, _ = _lib.greedy_accept(lg, draft, parent)
    acc_bytes = B * (T + 1) * V * 2 + 8 * B * T + 4 * B * (T + 1) + 12 * B + 4 * B * T
    t0 = time.perf_counter()
    oacc.greedy_accept(ac.logits, ac.draft, ac.parent, "bf16")
    cpu_s = time.perf_counter() - t0
    del lg
    torch.cuda.empty_cache()

    print("[bench] tree speculative sampling", file=sys.stderr, flush=True)
    sc = inputs.make_spec_case(B, T, V, seed)
    sp, sq = torch.from_numpy(sc.p).cuda(), torch.from_numpy(sc.q).cuda()
    sd, spa = torch.from_numpy(sc.draft).cuda(), torch.from_numpy(sc.parent).cuda()
    sua, sus = torch.from_numpy(sc.u_accept).cuda(), torch.from_numpy(sc.u_sample).cuda()
    sws = torch.empty(_lib.spec_sample_workspace_size(B, T, V), dtype=torch.uint8, device="cuda")
    spec_us = timed(lambda: _lib.spec_sample(sp, sq, sd, spa, sua, sus, ws=sws))
    s_n, _, _ = _lib.spec_sample(sp, sq, sd, spa, sua, sus, ws=sws)
    # the mass kernel reads p and q of every row whose position has children
    internal = sum(len(set(int(x) for x in sc.parent[b])) for b in range(B))
    spec_bytes = 4 * V * 2 * internal
    t0 = time.perf_counter()
    oacc.spec_sample(sc.p, sc.q, sc.draft, sc.parent, sc.u_accept, sc.u_sample)
    spec_cpu_s = time.perf_counter() - t0
    del sp, sq
    torch.cuda.empty_cache()

    print("[bench] GDN tree verification", file=sys.stderr, flush=True)
    import oracle.gdn as ogdn
    GT, GHk, GHv, Gd = 128, 16, 32, 128
    gc = inputs.make_gdn_case(B, GT, GHk, GHv, Gd, Gd, seed)
    bt = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    gq, gk, gv = bt(gc.q), bt(gc.k), bt(gc.v)
    gg, gb = torch.from_numpy(gc.g).cuda(), torch.from_numpy(gc.beta).cuda()
    gp, gs0 = torch.from_numpy(gc.parent).cuda(), torch.from_numpy(gc.S0).cuda()
    gdn_us = timed(lambda: _lib.gdn_verify(gq, gk, gv, gg, gb, gp, gs0, gc.scale))
    # algorithmic work: K S0 and Q S0 (2 T dk dv each), and per node and ancestor-or-self pair
    # the two key dot products (2 dk each) and the rank-1 terms (2 dv each)
    pairs = 0
    for b in range(B):
        for t in range(GT):
            j = t
            while j >= 0:
                pairs += 1
                j = int(gc.parent[b, j])
    gdn_mfma_flops = GHv * B * 4 * GT * Gd * Gd           # K S0 and Q S0: bf16 MFMA
    gdn_valu_flops = GHv * pairs * (4 * Gd + 4 * Gd)       # path coefficients and terms: fp32
    gdn_flops = gdn_mfma_flops + gdn_valu_flops
    gdn_bytes = (gc.q.nbytes + gc.k.nbytes + gc.v.nbytes + gc.g.nbytes + gc.beta.nbytes
                 + gc.parent.nbytes + gc.S0.nbytes + B * GT * GHv * Gd * 4)
    t0 = time.perf_counter()
    ogdn.gdn_tree_verify(gc.q, gc.k, gc.v, gc.g, gc.beta, gc.parent, gc.S0, gc.scale)
    gdn_cpu_s = time.perf_counter() - t0
    # the deferred commit: the committed states take the accepted path's updates (in place; a
    # repeated call keeps applying them, which changes the values, not the work)
    gpath, gn = inputs.random_paths(gc.parent, np.random.default_rng(seed + 1))
    gpath_d, gn_d = torch.from_numpy(gpath).cuda(), torch.from_numpy(gn).cuda()
    gS = gs0.clone()
    print("[bench] GDN deferred commit", file=sys.stderr, flush=True)
    gcom_us = timed(lambda: _lib.gdn_commit(gk, gv, gg, gb, gpath_d, gn_d, gS))
    # states read and written once, plus each accepted node's key, value, decay and beta
    gcom_bytes = 2 * gc.S0.nbytes + int(gn.sum()) * (GHk * Gd * 2 + GHv * Gd * 2 + GHv * 8) + 4 * B

    wl = inputs.Workload("commit", B=B, Hq=32, Hkv=8, D=128, T=T, L=4096)
    cc = inputs.make_case(wl, seed, pad="finite", lcap=4096 + T)
    dv = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
                    if a.dtype == np.uint16 else torch.from_numpy(a).cuda())
    kc, vc, kt, vt = dv(cc.k_cache), dv(cc.v_cache), dv(cc.k_tree), dv(cc.v_tree)
    lens = dv(cc.seq_lens)
    path, n = inputs.random_paths(cc.parent, np.random.default_rng(seed))
    path_d, n_d = dv(path), dv(n)
    out = torch.empty_like(lens)
    print("[bench] kv commit", file=sys.stderr, flush=True)
    com_us = timed(lambda: _lib.kv_commit(kc, vc, lens, kt, vt, path_d, n_d, new_seq_lens=out))
    com_bytes = int(n.sum()) * 8 * 128 * 2 * 2 * 2 + 12 * B + 4 * B * T
    return {
        "greedy_accept": {
            "workload": f"B={B}, T={T} bounded tree, vocab {V}, bf16 logits",
            "us": round(acc_us, 2), "algorithmic_bytes": acc_bytes,
            "achieved_gbs": round(acc_bytes / (acc_us * 1e-6) / 1e9, 1), "peak_gbs": HBM_PEAK_GBS,
            "frac": round(acc_bytes / (acc_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mean_accept_len": float(n_gpu.float().mean().item()),
            "cpu_oracle_s": round(cpu_s, 3)},
        "spec_sample": {
            "workload": f"B={B}, T={T} bounded tree, vocab {V}, fp32 p and q",
            "us": round(spec_us, 2), "mass_kernel_bytes": spec_bytes,
            "achieved_gbs": round(spec_bytes / (spec_us * 1e-6) / 1e9, 1),
            "peak_gbs": HBM_PEAK_GBS,
            "frac": round(spec_bytes / (spec_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mean_accept_len": float(s_n.float().mean().item()),
            "cpu_oracle_s": round(spec_cpu_s, 3)},
        "gdn_verify": {
            "workload": f"B={B}, T={GT} bounded tree, H_k={GHk}, H_v={GHv}, d_k=d_v={Gd}, "
                        "bf16 q/k/v, fp32 states",
            "us": round(gdn_us, 2), "algorithmic_flops": gdn_flops,
            **gdn_roofline(gdn_us, gdn_mfma_flops, gdn_valu_flops, gdn_bytes),
            "bytes": gdn_bytes, "cpu_oracle_s": round(gdn_cpu_s, 3)},
        "gdn_commit": {
            "workload": f"B={B}, H_v={GHv}, d_k=d_v={Gd} fp32 states, {int(gn.sum())} accepted "
                        "nodes in all",
            "us": round(gcom_us, 2), "algorithmic_bytes": gcom_bytes,
            "achieved_gbs": round(gcom_bytes / (gcom_us * 1e-6) / 1e9, 1),
            "peak_gbs": HBM_PEAK_GBS,
            "frac": round(gcom_bytes / (gcom_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "kv_commit": {
            "workload": f"B={B}, Hkv=8, D=128 bf16, contiguous cache, {int(n.sum())} rows committed",
            "us": round(com_us, 2), "algorithmic_bytes": com_bytes,
            "achieved_gbs": round(com_bytes / (com_us * 1e-6) / 1e9, 1), "peak_gbs": HBM_PEAK_GBS,
            "frac": round(com_bytes / (com_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
            "note": "latency-bound: a few hundred KB move per call"},
    }


def gdn_roofline(us, mfma_flops, valu_flops, nbytes):
    """Each resource of the GDN verify kernel against its own peak: the K S0 / Q S0 products
    (counted once, though the kernel runs each as two bf16 MFMAs for the high and low halves of
    S0) against the dense bf16 MFMA peak, the fp32 path terms against the fp32 vector peak, the
    bytes against HBM; ``frac`` is the largest, ``bound`` names it."""
    t = us * 1e-6
    parts = {"mfma_bf16": mfma_flops / t / 1e12 / MFMA_BF16_PEAK_TFS,
             "valu_fp32": valu_flops / t / 1e12 / FP32_PEAK_TFS,
             "hbm": nbytes / t / 1e9 / HBM_PEAK_GBS}
    bound = max(parts, key=parts.get)
    return {"mfma_tflops": round(mfma_flops / t / 1e12, 2), "mfma_peak_tflops": MFMA_BF16_PEAK_TFS,
            "valu_tflops": round(valu_flops / t / 1e12, 2), "valu_peak_tflops": FP32_PEAK_TFS,
            "achieved_gbs": round(nbytes / t / 1e9, 1), "peak_gbs": HBM_PEAK_GBS,
            "fracs": {k: round(v, 4) for k, v in parts.items()}, "bound": bound,
            "frac": round(parts[bound], 4),
            "note": "latency-bound: every resource well below its peak"}


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]


def cpu_baseline(case, threads, budget_s=10.0):
    """The oracle on a bounded sample: whole sequences (every node and head over its prefix and
    tree), one after another, until about ``budget_s`` seconds of CPU work are done."""
    import numpy as np

    import oracle

    wl = case.wl
    es = 2 if wl.dtype == "bf16" else 4
    done_bytes, dt, seqs, rows_done = 0, 0.0, 0, 0
    for b in range(wl.B):
        rows = np.array([(b, i, h) for i in range(wl.T) for h in range(wl.Hq)], dtype=np.int32)
        print(f"[bench] cpu baseline: sequence {b}, {len(rows)} rows on {threads} threads",
              file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        oracle.attend_case(case, rows=rows, nthreads=threads)
        dt += time.perf_counter() - t0
        L = int(case.seq_lens[b])
        done_bytes += (2 * es * wl.Hkv * wl.D * L + es * wl.T * wl.Hq * wl.D
                       + 2 * es * wl.T * wl.Hkv * wl.D + 4 * wl.T + es * wl.T * wl.Hq * wl.D
                       + 4 * wl.T * wl.Hq)
        seqs += 1
        rows_done += len(rows)
        if dt >= budget_s:
            break
    lens = [int(x) for x in case.seq_lens[:seqs]]
    return {"value": done_bytes / dt / 1e12, "unit": "TB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"sequences 0..{seqs - 1} of {wl.B} (prefix lengths {lens}): every node x "
                      f"q-head over its prefix and tree ({rows_done} rows), fp64 two-pass softmax",
            "seconds": round(dt, 3),
            "us_per_layer_extrapolated": round(dt * 1e6 * int(case.seq_lens.sum()) / max(sum(lens), 1), 1)}


def traffic_path(workload):
    return os.path.join(PROFILES, f"{KERNEL_NAME}_{workload}_traffic.txt")


def traffic_entry(workload):
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.loads("".join(ln for ln in f if not ln.startswith("#")))
    if t.get("kernel_src_sha256") != kernel_source_hash():
        return None   # the kernel changed since the counters were taken
    return t


UTIL_COUNTERS = ("MfmaUtil", "LdsBankConflict", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                 "SQ_WAVES")
# where the cycles go: MFMA busy, VALU / LDS issue, waits, per SIMD (a second pass)
ISSUE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                  "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY",
                  "SQ_INSTS_VALU_TRANS_F32", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
N_XCD, N_SIMD = 8, 1024


def pmc_command(counters, out_dir, workload):
    return (f"rocprofv3 --pmc {' '.join(counters)} -d {out_dir} -o run --output-format csv -- "
            f"python3 bench.py --workload {workload} --steps 4 --warmup 1 --no-secondary "
            f"--no-configs --no-cpu-baseline --no-next-rows")


def util_path(workload):
    return os.path.join(PROFILES, f"{KERNEL_NAME}_{workload}_util.txt")


def parse_util(util_dirs, workload):
    """Per-dispatch averages of the dominant kernel's counters from the utilisation pass
    (UTIL_COUNTERS) and the issue pass (ISSUE_COUNTERS), with the per-SIMD cycle shares derived
    from them, into a text summary under profiles/."""
    vals = {}
    for d in util_dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if KERNEL_NAME in row["Kernel_Name"]:
                        vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {KERNEL_NAME} dispatches under {' '.join(util_dirs)}")
    m = {k: statistics.mean(v) for k, v in vals.items()}
    os.makedirs(PROFILES, exist_ok=True)
    lines = [
        f"# rocprofv3 counters of {KERNEL_NAME} (one tree_attn_partials call), workload {workload}, "
        f"mean per dispatch",
        f"# utilisation pass: {pmc_command(UTIL_COUNTERS, 'UTIL_DIR', workload)}",
        f"# issue pass:       {pmc_command(ISSUE_COUNTERS, 'ISSUE_DIR', workload)}",
        f"# summary: python3 bench.py --workload {workload} --parse-util UTIL_DIR ISSUE_DIR",
        f"# kernel sources sha256: {kernel_source_hash()}",
        "",
    ]
    for k in sorted(vals):
        lines.append(f"{k}: {m[k]:.6g} ({len(vals[k])} dispatches)")
    derived = {}
    if "GRBM_GUI_ACTIVE" in m:
        cyc = m["GRBM_GUI_ACTIVE"] / N_XCD          # counted once per XCD
        derived["cycles per dispatch (GRBM_GUI_ACTIVE / 8 XCDs)"] = cyc
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            derived["MFMA busy share per SIMD"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cyc
        if "SQ_ACTIVE_INST_VALU" in m:               # quad-cycles, summed over waves
            derived["VALU issue share per SIMD"] = 4 * m["SQ_ACTIVE_INST_VALU"] / N_SIMD / cyc
        if "SQ_ACTIVE_INST_LDS" in m:
            derived["LDS issue share per SIMD"] = 4 * m["SQ_ACTIVE_INST_LDS"] / N_SIMD / cyc
        if "SQ_WAVE_CYCLES" in m and "SQ_WAVES" in m:
            derived["wave lifetime share (wave-cycles / waves / cycles)"] = (
                4 * m["SQ_WAVE_CYCLES"] / m["SQ_WAVES"] / cyc)
    if "SQ_WAIT_INST_ANY" in m and "SQ_WAVE_CYCLES" in m:
        derived["wave-cycles waiting to issue (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)"] = (
            m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"])
    if "SQ_INSTS_VALU_TRANS_F32" in m and "SQ_INSTS_VALU" in m:
        derived["transcendental share of VALU instructions"] = (
            m["SQ_INSTS_VALU_TRANS_F32"] / m["SQ_INSTS_VALU"])
    if derived:
        lines += ["", "derived:"] + [f"  {k}: {v:.4g}" for k, v in derived.items()]
    lines += ["", "MfmaUtil: percent of the cycles the MFMA units were busy; LdsBankConflict: percent of",
              "LDS active cycles lost to bank conflicts (rocprofv3 derived metrics). SQ_ACTIVE_INST_*",
              "and SQ_WAVE_CYCLES count quad-cycles summed over waves; SQ_VALU_MFMA_BUSY_CYCLES counts",
              "cycles summed over the 1024 SIMDs; GRBM_GUI_ACTIVE counts cycles summed over the 8 XCDs."]
    with open(util_path(workload), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def util_entry(workload):
    """MFMA utilisation and the derived shares of a util summary, or None (absent or taken
    before the kernel sources last changed)."""
    path = util_path(workload)
    if not os.path.exists(path):
        return None
    out, sha = {}, None
    with open(path) as f:
        for ln in f:
            if ln.startswith("# kernel sources sha256:"):
                sha = ln.split(":", 1)[1].strip()
            elif ln.startswith("MfmaUtil:") and ln.rstrip().endswith("dispatches)"):
                out["mfma_util_pct"] = float(ln.split()[1])
            elif ln.strip().startswith(("MFMA busy share", "VALU issue share", "LDS issue share")):
                k, v = ln.strip().rsplit(":", 1)
                out[k.split(" share")[0].lower().replace(" ", "_") + "_share"] = float(v)
    return out if sha == kernel_source_hash() else None


def parse_pmc(fetch_dir, write_dir, workload):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the attention and copy kernels, scaled by
    what the counters read for a plain copy of known size."""

    def read(d, counter):
        out = []   # (kernel name, value) per dispatch
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") == counter:
                        out.append((row["Kernel_Name"], float(row["Counter_Value"])))
        return out

    def kernel(vals):
        # one tree_attn_partials call = one prefix-kernel dispatch (the masked part rides on
        # its last split)
        xs = [v for k, v in vals if KERNEL_NAME in k]
        if not xs:
            raise SystemExit(f"no dispatches of {KERNEL_NAME} in the counters")
        return statistics.mean(xs), len(xs), next(k for k, _ in vals if KERNEL_NAME in k)

    def copy(vals):
        # the 1 GiB calibration copies: the largest copy dispatches (input uploads are tiny)
        xs = [(k, v) for k, v in vals if "copy" in k.lower()]
        if not xs:
            raise SystemExit("no copy dispatches in the counters (bench.py's copy-ceiling leg "
                             "makes them)")
        top = max(v for _, v in xs)
        big = [v for _, v in xs if v >= 0.9 * top]
        return statistics.mean(big), len(big), xs[0][0]

    fetch = read(fetch_dir, "FETCH_SIZE")
    write = read(write_dir, "WRITE_SIZE")
    kf, nkf, kname = kernel(fetch)
    kw, _, _ = kernel(write)
    cf, ncf, cname = copy(fetch)
    cw, _, _ = copy(write)
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    entry = {"workload": workload, "kernel": kname, "dispatches": nkf,
             "fetch_kib": kf, "write_kib": kw, "copy_kernel": cname, "copy_dispatches": ncf, "copy_fetch_kib": cf,
             "copy_write_kib": cw, "fetch_scale": f_scale, "write_scale": w_scale,
             "fetch_bytes": kf * 1024.0 * f_scale, "write_bytes": kw * 1024.0 * w_scale,
             "kernel_src_sha256": kernel_source_hash()}
    entry["traffic_bytes"] = entry["fetch_bytes"] + entry["write_bytes"]
    os.makedirs(PROFILES, exist_ok=True)
    out = traffic_path(workload)
    with open(out, "w") as f:
        f.write(f"# HBM traffic of one tree_attn_partials call (one {KERNEL_NAME} dispatch: the "
                f"prefix splits and the masked part) on workload {workload}.\n"
                f"# FETCH pass: {pmc_command(['FETCH_SIZE'], 'FETCH_DIR', workload)}\n"
                f"# WRITE pass: {pmc_command(['WRITE_SIZE'], 'WRITE_DIR', workload)}\n"
                f"# summary:    python3 bench.py --workload {workload} --parse-pmc FETCH_DIR WRITE_DIR\n"
                f"# Counter KiB are scaled by bytes / KiB-read of the plain 1 GiB copies in the same "
                f"runs (the copy-ceiling leg).\n")
        json.dump(entry, f, indent=1)
        f.write("\n")
    print(json.dumps(entry, indent=1))


ACCEPT_BYTES = 4 * 65 * 128256 * 2   # the bf16 logits rows one greedy-acceptance call reads


def accept_stats_summary(stats_dir, steps):
    """Text summary of a rocprofv3 --kernel-trace --stats run of --next-rows-only."""
    import re

    paths = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel stats under {stats_dir}")
    with open(paths[0]) as f:
        stats = list(csv.DictReader(f))
    names = ("argmax_kernel", "accept_kernel", "spec_mass_kernel", "spec_walk_kernel",
             "gdn_verify_kernel", "gdn_commit_kernel", "commit_kernel")
    rows = [r for r in stats if any(n in r["Name"] for n in names)]
    bench = None
    logs = glob.glob(stats_dir.rstrip("/") + ".log")
    if logs:
        m = re.search(r'^\{.*\}$', open(logs[0]).read(), re.M)
        bench = json.loads(m.group(0)) if m else None
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "next_rows_accept_sampling_gdn_commit_stats.txt")
    lines = [
        "# rocprofv3 kernel statistics, greedy tree acceptance (B=4, T=64, vocab 128256, bf16 "
        "logits), tree speculative sampling (same tree and vocabulary, fp32 p and q), GDN tree "
        "verification (B=4, T=128, H_k=16, H_v=32, d_k=d_v=128) with its deferred state commit, and "
        "accepted-path KV commit "
        "(B=4, Hkv=8, D=128 bf16)",
        f"# command: rocprofv3 --kernel-trace --stats -d STATS_DIR -o run --output-format csv -- "
        f"python3 bench.py --next-rows-only --steps {steps} --warmup 5",
        f"# summary: python3 bench.py --steps {steps} --accept-stats-summary STATS_DIR",
        "",
        "kernel | calls | average us | min us | max us",
    ]
    for r in rows:
        lines.append(f"{r['Name'][:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f}")
    arg = [r for r in rows if "argmax_kernel" in r["Name"]]
    if arg:
        us = float(arg[0]["AverageNs"]) / 1e3
        lines += ["", f"argmax_kernel: {ACCEPT_BYTES} logits bytes per call / {us:.2f} us = "
                      f"{ACCEPT_BYTES / us / 1e3:.1f} GB/s ({ACCEPT_BYTES / us / 1e3 / HBM_PEAK_GBS:.3f} "
                      f"of {HBM_PEAK_GBS:.0f} GB/s); every call follows a 512 MiB evicting read"]
    if bench:
        lines.append(f"bench.py next-row timings of the same run, under the tracer (HIP events "
                     f"around each call): {json.dumps(bench)}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_summary(stats_dir, workload, steps, warmup):
    """Text summary of a rocprofv3 --kernel-trace --stats run of this script's default JSON run:
    the kernel statistics, then the headline layer's loops taken apart by position in the trace
    (W warm-up forwards, the S timed forwards, S forwards with per-step events, W warm-up split
    steps, the S timed split steps, as time_case issues them), with every forward step of the
    fresh process listed on its own."""
    import re

    def one(pattern):
        paths = glob.glob(os.path.join(stats_dir, "**", pattern), recursive=True)
        if not paths:
            raise SystemExit(f"no {pattern} under {stats_dir}")
        return paths[0]

    with open(one("*kernel_stats.csv")) as f:
        stats = list(csv.DictReader(f))
    with open(one("*kernel_trace.csv")) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    spans = [(r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace]
    prefix_idx = [i for i, (n, _, _) in enumerate(spans) if KERNEL_NAME in n]
    W, S = warmup, steps
    fwd_idx = prefix_idx[:W + S]                      # forwards: prefix kernel then merge kernel
    fused = [(spans[i][2] - spans[i][1]) / 1e3 for i in prefix_idx[W:W + S]]
    alone = [(spans[i][2] - spans[i][1]) / 1e3 for i in prefix_idx[2 * W + 2 * S:2 * W + 3 * S]]
    step_rows = []
    for k, i in enumerate(fwd_idx):
        j = i + 1                                     # the combine launch follows on the stream
        merge_us = (spans[j][2] - spans[j][1]) / 1e3 if "merge_kernel" in spans[j][0] else None
        nxt = fwd_idx[k + 1] if k + 1 < len(fwd_idx) else None
        step_us = (spans[nxt][1] - spans[i][1]) / 1e3 if nxt is not None else None
        step_rows.append((k, (spans[i][2] - spans[i][1]) / 1e3, merge_us, step_us))
    bench = {}
    logs = glob.glob(os.path.join(os.path.dirname(stats_dir.rstrip("/")),
                                  os.path.basename(stats_dir.rstrip("/")) + ".log"))
    if logs:
        txt = open(logs[0]).read()
        for key in ("kernel_avg_us", "us_per_layer"):
            m = re.search(rf'"{key}": ([0-9.]+)', txt)
            bench[key] = float(m.group(1)) if m else None
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{KERNEL_NAME}_{workload}_stats.txt")
    lines = [
        f"# rocprofv3 kernel statistics, workload {workload}",
        f"# command: rocprofv3 --kernel-trace --stats -d STATS_DIR -o run --output-format csv -- "
        f"python3 bench.py --gpus 1 --steps {steps} --warmup {warmup} > STATS_DIR.log",
        f"# summary: python3 bench.py --workload {workload} --steps {steps} --warmup {warmup} "
        f"--stats-summary STATS_DIR",
        "",
        "kernel | calls | average us | min us | max us",
    ]
    for r in stats:
        lines.append(f"{r['Name'][:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f}")
    lines += [
        "",
        f"headline layer, {KERNEL_NAME}, timed fused-forward loop ({len(fused)} launches, back to "
        f"back, no cache flush): average {statistics.mean(fused):.2f} us, median "
        f"{statistics.median(fused):.2f} us",
        f"headline layer, {KERNEL_NAME}, kernel-alone loop ({len(alone)} launches, 512 MiB "
        f"evicting read before each): average {statistics.mean(alone):.2f} us, median "
        f"{statistics.median(alone):.2f} us",
        f"bench.py in the same run: kernel_avg_us {bench.get('kernel_avg_us')} (HIP events around "
        f"the kernel-alone calls), us_per_layer {bench.get('us_per_layer')} (wall, timed forwards)",
        "",
        "every forward step of the fresh process (first W warm-up, then the S timed): prefix "
        "kernel us | combine (merge kernel) us | start-to-start step us",
    ]
    for k, a, m, st in step_rows:
        tag = "warm-up" if k < W else "timed"
        lines.append(f"step {k:3d} ({tag}): {a:8.2f} | {m if m is None else round(m, 2)} | "
                     f"{st if st is None else round(st, 2)}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def power_trace(seconds, seed):
    """The headline forward back to back for ``seconds`` from a fresh process: per-step HIP
    event times, the first 400 one by one and all of them in 50 ms buckets of wall-clock time
    since the first step (printed as one JSON object). Run beside a power / clock sampler to see how the part's power management
    paces the kernel."""
    import torch

    from tree_verification_attention_amd import inputs

    case = inputs.make_case(inputs.WORKLOADS["gqa_64k_pinned"], seed, pad="finite")
    L = Launch(case)
    torch.cuda.synchronize()
    batch = 20
    t_start = time.time()
    buckets, first = {}, []
    while time.time() - t_start < seconds:
        evs = []
        for _ in range(batch):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(L.stream)
            L.fwd()
            e1.record(L.stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = time.time() - t_start
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        if len(first) < 400:
            first.extend(round(x, 1) for x in us)
        buckets.setdefault(int(t / 0.05), []).extend(us)
    L.check_flag()
    return {"t0_unix": t_start, "bucket_s": 0.05, "first_steps_us": first,
            "buckets": [{"t_s": round(k * 0.05, 3), "steps": len(v),
                         "median_us": round(statistics.median(v), 1),
                         "min_us": round(min(v), 1), "max_us": round(max(v), 1)}
                        for k, v in sorted(buckets.items())]}


def power_summary(trace_path, smi_path, seconds):
    """Text summary of a --power-trace run and of the amd-smi samples taken beside it."""
    import re

    with open(trace_path) as f:
        d = json.load(f)
    first = d["first_steps_us"]
    smi = []
    with open(smi_path) as f:
        parts = re.split(r"^T (\S+)\n", f.read(), flags=re.M)
    for i in range(1, len(parts), 2):
        try:
            j = json.loads(parts[i + 1])
            g = j["gpu_data"][0] if isinstance(j, dict) else j[0]
            smi.append((float(parts[i]) - d["t0_unix"], g["power"]["socket_power"]["value"],
                        g["clock"]["gfx_0"]["clk"]["value"]))
        except (ValueError, KeyError, IndexError, TypeError):
            continue
    lines = [
        "# the headline forward (tree_attn_forward, workload gqa_64k_pinned) back to back from a "
        "fresh process, with the part's socket power and shader clock sampled beside it",
        f"# trace:   python3 bench.py --power-trace {seconds:g} > TRACE_JSON",
        "# sampler, started just before the trace: for i in $(seq 1 100); do echo \"T $(date "
        "+%s.%N)\"; amd-smi metric -p -c --json; done > SMI_SAMPLES",
        f"# summary: python3 bench.py --power-summary TRACE_JSON SMI_SAMPLES {seconds:g}",
        "",
        "step times (HIP events on the launch stream), us, steps 0.. in order:",
    ]
    for i in range(0, min(len(first), 120), 10):
        lines.append(f"  {i:3d}: " + " ".join(f"{x:6.1f}" for x in first[i:i + 10]))
    w = first[5:25]
    lines += ["", f"steps 5..24 (what a run with 5 warm-up and 20 timed steps times): mean "
              f"{statistics.mean(w):.1f} us, median {statistics.median(w):.1f} us",
              "", "median step time per second of the trace:"]
    per_s = {}
    for bk in d["buckets"]:
        per_s.setdefault(int(bk["t_s"]), []).append(bk["median_us"])
    for k in sorted(per_s):
        lines.append(f"  second {k}: {statistics.median(per_s[k]):.1f} us")
    lines += ["", "amd-smi samples (time since the first step, s | socket power W | gfx clock MHz; "
              "the values refresh about once a second):"]
    prev = None
    for t, pw, clk in smi:
        if (pw, clk) != prev:
            lines.append(f"  {t:6.2f} | {pw:5} | {clk:5}")
        prev = (pw, clk)
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"{KERNEL_NAME}_gqa_64k_pinned_power.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def clock_summary(clk_dir, workload, steps, warmup):
    """Shader clock of every headline dispatch from a rocprofv3 --pmc GRBM_COUNT GRBM_GUI_ACTIVE
    pass. GRBM_COUNT ticks once per shader clock on each of the eight XCDs, over a window that is
    the dispatch's duration plus a fixed profiler overhead. The overhead and the clock of light
    kernels come from the two lightly loaded kernels of the run -- the 512 MiB evicting read (a
    memory-bound torch reduction, ~140 us) and the merge (~11 us) -- taken at one clock f:
    count = overhead + 8 f duration. Each prefix dispatch then runs at (GRBM_COUNT - overhead) /
    8 / duration."""
    paths = glob.glob(os.path.join(clk_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter collection under {clk_dir}")
    by = {}
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            d = by.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                                 "s": int(r["Start_Timestamp"]),
                                                 "e": int(r["End_Timestamp"])})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    ds = sorted(by.values(), key=lambda d: d["s"])
    red = [d for d in ds if "reduce_kernel" in d["name"]]
    if not red:
        raise SystemExit("no evicting reads (reduce_kernel) to calibrate against")
    mrg = [d for d in ds if "merge_kernel" in d["name"]]
    if not mrg:
        raise SystemExit("no merge dispatches to calibrate against")
    # two light kernels of very different lengths at one clock f: count = over + 8 f t
    tr_, cr = (statistics.median(d["e"] - d["s"] for d in red),
               statistics.median(d["GRBM_COUNT"] for d in red))
    tm, cm = (statistics.median(d["e"] - d["s"] for d in mrg),
              statistics.median(d["GRBM_COUNT"] for d in mrg))
    f_light = (cr - cm) / 8 / (tr_ - tm)
    over = cm - 8 * f_light * tm

    def ghz(d):
        return (d["GRBM_COUNT"] - over) / 8 / (d["e"] - d["s"])

    pre = [d for d in ds if KERNEL_NAME in d["name"]]
    W, S = warmup, steps
    fused, alone = pre[:W + S], pre[2 * W + S:2 * W + 2 * S]
    lines = [
        f"# shader clock of the headline prefix-kernel dispatches, workload {workload}",
        f"# command: rocprofv3 --pmc GRBM_COUNT GRBM_GUI_ACTIVE --kernel-trace -d CLK_DIR -o run "
        f"--output-format csv -- python3 bench.py --gpus 1 --steps {steps} --warmup {warmup} "
        f"--no-configs --no-next-rows --no-cpu-baseline --no-secondary",
        f"# summary: python3 bench.py --workload {workload} --steps {steps} --warmup {warmup} "
        f"--clock-summary CLK_DIR",
        f"# counter dispatches run one at a time with idle gaps between them, so the clocks here "
        f"are those of a lightly loaded part; fitted over the evicting reads and the merges: "
        f"light-kernel clock {f_light:.3f} GHz, GRBM_COUNT overhead per dispatch {over:.0f}",
        "",
        "dispatch | duration us | shader cycles per XCD | clock GHz",
    ]
    for k, d in enumerate(fused + alone):
        tag = ("forward warm-up" if k < W else "forward timed" if k < W + S else
               "kernel alone")
        cyc = (d["GRBM_COUNT"] - over) / 8
        lines.append(f"{tag} {k:2d} | {(d['e'] - d['s']) / 1e3:8.2f} | {cyc:9.0f} | {ghz(d):.3f}")
    cyc = [(d["GRBM_COUNT"] - over) / 8 for d in fused + alone]
    lines += ["", f"median shader cycles per dispatch: {statistics.median(cyc):.0f} "
                  f"(= {statistics.median(cyc) / 2.4e3:.1f} us at the 2.4 GHz top clock)",
              f"median clock: {statistics.median(ghz(d) for d in fused + alone):.3f} GHz",
              "evicting reads (torch reduction over 512 MiB): median "
              f"{statistics.median((d['e'] - d['s']) / 1e3 for d in red):.1f} us"]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{KERNEL_NAME}_{workload}_clock.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def workload_table(steps, warmup, seed):
    """One row per bf16 workload: fused forward (wall, back to back) and the split step (HIP
    events after an evicting read), against the HBM and bf16 MFMA peaks."""
    import gc

    import torch

    from tree_verification_attention_amd import inputs

    print("| workload | B | T | Hq/Hkv | prefix | splits | forward us | TB/s | split step us | "
          "frac HBM | TFLOP/s | frac MFMA |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for name, wl in inputs.WORKLOADS.items():
        if wl.dtype != "bf16":
            continue
        case = inputs.make_case(wl, seed, pad="finite")
        w = work_of(case)
        r = time_case(case, steps, warmup, name)
        fwd_us = r["wall_s"] * 1e6 / steps
        k = statistics.mean(r["kernel_us"])
        gbs = w["kernel_bytes"] / (k * 1e-6) / 1e9
        tf = w["flops"] / (k * 1e-6) / 1e12
        lens = case.seq_lens
        pre = str(int(lens[0])) if lens.min() == lens.max() else f"{int(lens.min())}-{int(lens.max())}"
        print(f"| {name} | {wl.B} | {wl.T} | {wl.Hq}/{wl.Hkv} | {pre} | {r['n_splits']} | "
              f"{fwd_us:.1f} | {w['step_bytes'] / (fwd_us * 1e-6) / 1e12:.2f} | {k:.1f} | "
              f"{gbs / HBM_PEAK_GBS:.3f} | {tf:.0f} | {tf / MFMA_BF16_PEAK_TFS:.3f} |", flush=True)
        del case, r
        gc.collect()
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_64k_pinned")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the unfused breakdown of the headline layer")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing every configuration (the configs entry)")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip timing greedy acceptance and the KV commit")
    ap.add_argument("--parse-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--parse-util", nargs="+", metavar="DIR",
                    help="summarise the rocprofv3 --pmc passes of the utilisation and issue "
                         "counters")
    ap.add_argument("--next-rows-only", action="store_true",
                    help="time only greedy acceptance and the KV commit; print their JSON")
    ap.add_argument("--accept-stats-summary", metavar="STATS_DIR",
                    help="summarise a rocprofv3 --stats run of --next-rows-only into profiles/")
    ap.add_argument("--stats-summary", metavar="STATS_DIR",
                    help="write the text summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--power-trace", type=float, metavar="SECONDS",
                    help="run the headline forward back to back for SECONDS, print step times")
    ap.add_argument("--power-summary", nargs=3, metavar=("TRACE_JSON", "SMI_SAMPLES", "SECONDS"),
                    help="summarise a --power-trace run and its amd-smi samples")
    ap.add_argument("--clock-summary", metavar="CLK_DIR",
                    help="summarise a rocprofv3 --pmc GRBM_COUNT GRBM_GUI_ACTIVE pass")
    ap.add_argument("--table", action="store_true",
                    help="time every bf16 workload (fused forward and split step) and print a "
                         "table row for each instead of the JSON line")
    args = ap.parse_args()

    if args.stats_summary:
        stats_summary(args.stats_summary, args.workload, args.steps, args.warmup)
        return

    if args.power_summary:
        power_summary(args.power_summary[0], args.power_summary[1], float(args.power_summary[2]))
        return
    if args.clock_summary:
        clock_summary(args.clock_summary, args.workload, args.steps, args.warmup)
        return
    if args.accept_stats_summary:
        accept_stats_summary(args.accept_stats_summary, args.steps)
        return
    if args.parse_util:
        parse_util(args.parse_util, args.workload)
        return
    if args.parse_pmc:
        parse_pmc(args.parse_pmc[0], args.parse_pmc[1], args.workload)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the tree-attention path here is single-device "
              "(its sharding across GPUs is a design note, not built); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from tree_verification_attention_amd import _lib, inputs

    _lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.next_rows_only:
        print(json.dumps(time_next_rows(args.steps, args.warmup, args.seed)), flush=True)
        return
    if args.power_trace:
        print(json.dumps(power_trace(args.power_trace, args.seed)), flush=True)
        return
    if args.table:
        workload_table(args.steps, args.warmup, args.seed)
        return
    wl = inputs.WORKLOADS[args.workload]
    print(f"[bench] generating {wl.name} (seed {args.seed})", file=sys.stderr, flush=True)
    case = inputs.make_case(wl, args.seed, pad="finite")
    work = work_of(case)
    res = time_case(case, args.steps, args.warmup, wl.name)

    ms_per_step = res["wall_s"] * 1e3 / args.steps
    value = work["step_bytes"] / (ms_per_step * 1e-3) / 1e12
    kern_avg_us = statistics.mean(res["kernel_us"])
    achieved = work["kernel_bytes"] / (kern_avg_us * 1e-6) / 1e9
    traffic = traffic_entry(wl.name)
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) values rounded to bf16, bounded-random trees)",
        "config": {"workload": "GQA bf16, 64-node tree, every prefix 64k tokens", "name": wl.name,
                   "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.D,
                   "tree_nodes": wl.T, "prefix_lens": case.seq_lens.tolist(),
                   "tree": f"{wl.tree}, depth<={wl.depth_cap}, children<={wl.branch_cap}",
                   "layout": "contiguous [B, L, Hkv, D]", "kv_splits": res["n_splits"]},
        "us_per_layer": round(ms_per_step * 1e3, 2),
        "us_per_layer_events": {"p10": round(pct(res["step_us"], 0.1), 2),
                                "median": round(pct(res["step_us"], 0.5), 2),
                                "p90": round(pct(res["step_us"], 0.9), 2)},
        "node_qheads_per_s": wl.B * wl.T * wl.Hq / (ms_per_step * 1e-3),
        "prefix_token_kvheads_per_s": work["sum_len"] * wl.Hkv / (ms_per_step * 1e-3),
        "algorithmic_bytes_per_step": work["step_bytes"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "kernel": f"{KERNEL_NAME} (tree_attn_partials: the prefix splits and, on "
                               f"the last split, the masked part)",
                     "kernel_avg_us": round(kern_avg_us, 2),
                     "kernel_bytes": work["kernel_bytes"]},
        "mfma": {"achieved_tflops": round(work["flops"] / (kern_avg_us * 1e-6) / 1e12, 1),
                 "peak_tflops": MFMA_BF16_PEAK_TFS,
                 "frac": round(work["flops"] / (kern_avg_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                 "flops_per_step": work["flops"]},
    }
    torch.cuda.empty_cache()
    if not args.no_secondary and wl.name == "gqa_64k_pinned":
        print("[bench] unfused breakdown", file=sys.stderr, flush=True)
        line["breakdown"] = time_breakdown(case, max(5, args.steps // 5), 3)
    if not args.no_configs:
        line["configs"] = time_configs(args.steps, args.warmup, args.seed)
    if not args.no_next_rows and wl.name == "gqa_64k_pinned":
        line["next_rows"] = time_next_rows(args.steps, args.warmup, args.seed)
        torch.cuda.empty_cache()
    line["copy_ceiling"] = copy_ceiling()
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        line["cpu_baseline"] = cpu_baseline(case, threads)
        line["cpu_baseline"].update(host_cpu())
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
