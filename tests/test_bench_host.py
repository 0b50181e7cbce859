"""Host-side pieces of bench.py: the algorithmic work counts and the oracle
baseline leg, run on CPU tensors of a small workload."""
import math
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402


def test_tile_flops_counts_visible_pairs():
    """4*d flops per visible pair and query head: a causal 4x4 rotated tile
    (2,2) has 9 FULL blocks, 1 DIAG block and 6 SKIP blocks."""
    blocks = oracle.block_list_ref(4, 4, 2, 2, True, True)
    L, hq, d = 8, 3, 16
    want = 4 * d * hq * (9 * L * L + L * (L + 1) // 2)
    assert bench.tile_flops(blocks, L, hq, d) == want
    # brute force over token positions gives the same pair count
    q_parts = [b[2] for b in blocks if b[1] == 0]
    kv_parts = [b[3] for b in blocks if b[0] == 0]
    qp = oracle.tile_positions_ref(q_parts, L)
    kp = oracle.tile_positions_ref(kv_parts, L)
    assert 4 * d * hq * int((kp[None, :] <= qp[:, None]).sum()) == want


def test_merge_bytes():
    # n partial rows of d bf16 values and one fp32 lse each, plus the output row
    assert bench.merge_bytes(8, 10, 128, 2) == 8 * 10 * 260 + 10 * 260


@pytest.mark.parametrize("wid,want_live,want_all", [
    (4, 9_814_671_360, 9_814_671_360),    # every sibling partial row is live
    (5, 10_485_760_000, 18_538_823_680),  # 7.5 of the 16 per-KV partials dead
])
def test_merge_bytes_follow_the_rows_the_kernel_reads(wid, want_live, want_all):
    """The merge's rate is priced on the bytes the kernel moves: every lse,
    the output rows of partials with a finite lse, and the merged row.  On
    the 16-partial workload that is 10.49 GB, not the 18.54 GB of reading
    every partial row, so a rate near the HBM peak stays below it."""
    w = workloads.WORKLOADS[wid]
    blocks = oracle.block_list_ref(w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col,
                                   w.causal, w.kv_rotate)
    q_parts = [b[2] for b in blocks if b[1] == 0]
    peer_kv, _ = bench.peer_kv_sets(w, oracle.block_list_ref)
    rows = len(q_parts) * w.part_len * w.heads_q
    live = bench.live_partial_rows(w, q_parts, peer_kv)
    assert bench.merge_bytes(len(peer_kv), rows, w.head_dim, 2) == want_all
    got = bench.merge_live_bytes(len(peer_kv), rows, w.head_dim, 2, live)
    assert got == want_live
    # The fastest merge measured on this path (1.83 ms on the 16-partial
    # workload) priced on live bytes stays under the 8 TB/s peak; priced on
    # all rows it would not.
    assert got / 1.83e-3 / 1e9 <= bench.PEAK_HBM_GBS
    if wid == 5:
        assert want_all / 1.83e-3 / 1e9 > bench.PEAK_HBM_GBS


def test_cpu_baseline_leg_reports_all_runs():
    w = workloads.WORKLOADS[1]
    blocks = oracle.block_list_ref(w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col,
                                   w.causal, w.kv_rotate)
    q_parts = [b[2] for b in blocks if b[1] == 0]
    kv_parts = [b[3] for b in blocks if b[0] == 0]
    q = workloads.gather(w, "q", q_parts, "cpu")
    k = workloads.gather(w, "k", kv_parts, "cpu")
    v = workloads.gather(w, "v", kv_parts, "cpu")
    rows = q.shape[0] * w.heads_q
    o_parts = torch.randn((2, rows, w.head_dim))
    l_parts = torch.randn((2, rows))
    flops = bench.tile_flops(blocks, w.part_len, w.heads_q, w.head_dim)
    res = bench.cpu_baseline(w, q, k, v, q_parts, kv_parts, flops, o_parts, l_parts, budget_s=0.5)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s" and res["cores"] >= 1
    assert res["value"] > 0 and res["single_core"]["value"] > 0 and res["single_core"]["cores"] == 1
    assert math.isclose(res["full_tile_s_extrapolated"], flops / (res["value"] * 1e12), rel_tol=1e-9)
    assert res["merge"]["unit"] == "GB/s" and res["merge"]["value"] > 0
    assert np.isfinite(res["merge"]["value"])


def test_source_key_ignores_comments_only():
    """The key that ties counter summaries to a kernel's code: equal for a
    comment or whitespace edit, different for a code edit."""
    base = "int f(int x) {\n    return x + 1;  // one more\n}\n/* block\n comment */\n"
    assert bench.code_only(base) == bench.code_only(base.replace("one more", "plus one"))
    assert bench.code_only(base) == bench.code_only(base.replace("    return", "  return"))
    assert bench.code_only(base) != bench.code_only(base.replace("x + 1", "x + 2"))
    files = {"a.hip": base, "b.h": "#define N 4\n"}
    k0 = bench.source_sha256("tile_fwd_bf16_d128", lambda n: files.get(n, base))
    k1 = bench.source_sha256("tile_fwd_bf16_d128", lambda n: files.get(n, base).replace("// one", "// 1"))
    k2 = bench.source_sha256("tile_fwd_bf16_d128", lambda n: files.get(n, base).replace("+ 1", "+ 3"))
    assert k0 == k1 != k2


def test_profile_summaries_are_well_formed():
    """Every summary in profiles/ lists commands that run committed files only
    (bench.py under rocprofv3); every counter summary (one with a `- kernel:`
    header) also names a kernel bench.py knows, keys the code it measured
    with a sha256, gives positive traffic and was taken with the copy
    calibration its traffic is scaled by."""
    import glob
    import re
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    counter_kernels = set()
    for path in paths:
        text = open(path).read()
        cmds = [ln.strip() for ln in text.splitlines() if ln.strip().startswith("rocprofv3 ")]
        assert cmds and all(" -- python bench.py " in c and "--no-cpu-baseline" in c for c in cmds), path
        assert "_work" not in text, path
        m = re.search(r"^- kernel: `([^`]+)`", text, re.M)
        if m is None:
            continue
        kernel = m.group(1)
        counter_kernels.add(kernel)
        assert kernel in bench.KERNEL_SOURCES, path
        assert re.search(r"^- source_sha256: `[0-9a-f]{64}`", text, re.M), path
        assert float(re.search(r"^- hbm_bytes_per_launch: `([^`]+)`", text, re.M).group(1)) > 0
        assert all("--copy-calibration 1024" in c for c in cmds), path
    assert set(bench.KERNEL_SOURCES) <= counter_kernels


def test_plan_costs_of_the_1m_token_tile():
    """Transfer sizes of the 8x8 mesh tile (L=16384, GQA 32/8, d=128, bf16):
    a Q partition 128 MiB, a KV partition 64 MiB, a partial output 130 MiB
    (with its lse); block times share the tile time over visible pairs."""
    w = workloads.WORKLOADS[4]
    blocks = oracle.block_list_ref(8, 8, 4, 4, True, True)
    c = bench.plan_costs(w, blocks, 100.0, link_gbs=100.0)
    assert c["recv_q_s"] == 16384 * 32 * 128 * 2 / 100e9
    assert c["recv_kv_s"] == 2 * 16384 * 8 * 128 * 2 / 100e9
    assert c["send_o_s"] == 16384 * 32 * (128 * 2 + 4) / 100e9
    assert math.isclose(35 * c["full_block_s"] + c["diag_block_s"], 0.1, rel_tol=1e-12)
    res = bench.plan_leg(w, blocks, 100.0)
    assert res["lower_bound_ms"] <= res["makespan_ms"] <= res["eager_makespan_ms"] + 1e-9
    assert math.isclose(res["compute_ms"], 100.0, rel_tol=1e-9)
