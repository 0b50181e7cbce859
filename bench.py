"""Benchmark of the Mesh-Attention tile hot path on one MI355X.

A step is one pass of the whole hot path over one synthetic tile: the host
block list (tile geometry, KV-rotation order, causal classes), the tile
forward (QK^T, mask, online softmax, PV, epilogue) and the LSE merge of the
partial results of the query rows.  Inputs are resident in HBM before the
timed region.  The merge combines this GPU's fresh partial with the partials
its mesh-row peers would return; those are synthetic (random outputs, finite
log-sum-exp, and -inf exactly where the peer's tile has no visible key for the
row), since the merge's cost depends only on their sizes and on which rows
are dead.  Their correctness against real sibling tiles is what the parity
tests check.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..5]
                    [--backward-steps N] [--no-cpu-baseline] [--copy-calibration MIB]
                    [--others none|all|1,2,...]

After the forward steps, --backward-steps N (default 3, 0 = off; bf16 tiles)
times the tile backward on the same tile: the row-term kernel D = rowsum(dO*O)
and the dQ and dK/dV kernels, reported in "tile_bwd" (not part of "value").
The rows' lse and O are this tile's own forward results, which have the shapes
and value ranges of the final ones; dO is synthetic.

--others (default "all") then measures the other workloads the same way, each
with fewer steps and a shorter oracle sample, under "per_workload" (the
headline workload is repeated there, so the table holds all five).  The
headline "value" is always the --workload tile.

The merge's byte count follows what the kernel reads: every partial's lse,
the output rows of the partials whose lse is finite (a partial that saw no
key for a row is not read), and the merged row it writes.  "gbs" and
"frac_hbm" use that count; "bytes_all_rows" is the count if every partial
row were read.

--copy-calibration runs one plain device copy of MIB MiB after the steps, so
that a hardware-counter run can scale FETCH_SIZE / WRITE_SIZE by what they
read for a copy of known size.

--gemm-ceiling MS (default 130; 0 skips it) runs the vendor bf16 GEMM
(torch.mm, 8192^3, contiguous operands) back to back for about MS
milliseconds after the headline's steps and reports
its rate under "gemm_ceiling": a dense matrix-core load of the tile's
duration, run at the clock the GPU holds under such a load, as a ceiling to
read the tile kernel's fraction of the spec peak against.  It is a reference
measurement, not part of the hot path.

The vendor attention reference (on by default; --no-sdpa-reference skips it)
times torch scaled_dot_product_attention with its flash backend forced on the
headline tile's block shapes, one FULL
block without a mask and one DIAG block with the causal mask (K/V heads
repeated to the query heads), and reports under "sdpa_reference" the time a
tile of the same block counts would take, n_full * t_full + n_diag * t_diag,
with the rate on the tile's algorithmic flops and the tile kernel's speedup
over it.  Also a reference measurement.  Either reference that fails is
reported with its error instead of its figures.

Prints one JSON line on stdout (everything else goes to stderr).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tile-forward TFLOP/s (% bf16 MFMA peak) + LSE-merge GB/s, 1M-token tile"
PEAK_BF16_TFLOPS = 2516.6   # 4096 flop/clk/CU x 256 CUs x 2.4 GHz, dense
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


# Kernel sources whose hash keys the counter-derived traffic in profiles/.
KERNEL_SOURCES = {
    "tile_fwd_bf16_d128": ["tile_fwd_bf16.hip", "tile_common.hpp", "kernels.h"],
    "tile_bwd_dq_bf16_d128": ["tile_bwd_bf16.hip", "tile_common.hpp", "kernels.h"],
    "tile_bwd_dkdv_bf16_d128": ["tile_bwd_bf16.hip", "tile_common.hpp", "kernels.h"],
    "tile_fwd_f32": ["tile_fwd_f32.hip", "tile_common.hpp", "kernels.h"],
    "lse_merge_kernel": ["lse_merge.hip", "kernels.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed, so
    that a key built from it changes when the code changes and not when only
    a comment does.  (The sources hold no comment markers inside strings.)"""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha256(kernel, read=None):
    """Key of the code a kernel is built from: sha256 over its source files'
    code (comments and whitespace runs ignored).  read(name) -> text defaults
    to the files in csrc/."""
    import hashlib
    if read is None:
        def read(name):
            with open(os.path.join(ROOT, "long_context_distributed_amd", "csrc", name)) as f:
                return f.read()
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(code_only(read(name)).encode())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3 counter
    summaries in profiles/ (FETCH_SIZE and WRITE_SIZE scaled by a copy of
    known size), or None when no summary matches the current kernel source."""
    import glob
    want = source_sha256(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and line.startswith("- "):
                    key, val = line[2:].split(":", 1)
                    fields[key.strip()] = val.strip().strip("`")
        if (fields.get("kernel") == kernel and fields.get("workload") == str(workload)
                and fields.get("source_sha256") == want and "hbm_bytes_per_launch" in fields):
            return float(fields["hbm_bytes_per_launch"])
    return None


def tile_flops(blocks, part_len, heads_q, head_dim):
    """Algorithmic flops: 4*d per visible (query, key) pair per query head;
    FULL blocks L*L pairs, DIAG blocks L*(L+1)/2, SKIP none."""
    pairs = 0
    for b in blocks:
        if b[4] == 0:
            pairs += part_len * part_len
        elif b[4] == 1:
            pairs += part_len * (part_len + 1) // 2
    return 4.0 * head_dim * heads_q * pairs


def merge_bytes(n, rows, d, elt):
    """Algorithmic bytes of one merge if every partial row is read: n partial
    rows (O and lse) read, one written."""
    return n * rows * (d * elt + 4) + rows * (d * elt + 4)


def merge_live_bytes(n, rows, d, elt, live):
    """Bytes the merge moves when the output rows of dead partials (lse =
    -inf, `live` of the n*rows are finite) are not read: every lse, the live
    output rows, and the merged row with its lse."""
    return n * rows * 4 + live * d * elt + rows * (d * elt + 4)


def _oracle_rows_rate(w, qh, kh, vh, qpos, kpos, rows_all, budget_s):
    """Times oracle.attention_ref on batches of sampled rows for about
    budget_s seconds; returns (flops per second, rows done, seconds used)."""
    import numpy as np
    import oracle
    scale = 1.0 / math.sqrt(w.head_dim)
    done, flops, t_used, batch = 0, 0.0, 0.0, 16
    while t_used < budget_s and done < len(rows_all):
        rows = rows_all[done:done + batch]
        t0 = time.perf_counter()
        oracle.attention_ref(qh, kh, vh, qpos, kpos, w.causal, scale, rows=rows)
        dt = time.perf_counter() - t0
        vis = (kpos[None, :] <= qpos[rows[:, 0]][:, None]).sum(axis=1) if w.causal else \
            np.full(len(rows), len(kpos))
        flops += float(4.0 * w.head_dim * vis.sum())
        t_used += dt
        done += len(rows)
        batch = min(4 * batch, max(16, int(len(rows) * (budget_s - t_used) / max(dt, 1e-3))))
    return flops / max(t_used, 1e-9), done, t_used


def cpu_baseline(w, q, k, v, q_parts, kv_parts, tile_flops_total, o_parts, l_parts, budget_s=12.0):
    """The oracle, as it stands, on bounded samples of the same workload:
    sampled query rows of the tile on every host core (the reported value),
    the same on one core, and the merge oracle on sampled rows of the merge's
    partials."""
    import numpy as np
    import oracle
    import workloads
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    qh = q.detach().cpu().double().numpy()
    kh = k.detach().cpu().double().numpy()
    vh = v.detach().cpu().double().numpy()
    qpos = oracle.tile_positions_ref(q_parts, w.part_len)
    kpos = oracle.tile_positions_ref(kv_parts, w.part_len)
    rows_all = workloads.sample_rows(q.shape[0], w.heads_q, w.heads_kv, w.part_len,
                                     n_sample=200000, seed=3)
    rows_all = rows_all[np.random.default_rng(7).permutation(len(rows_all))]
    rate, done, t_used = _oracle_rows_rate(w, qh, kh, vh, qpos, kpos, rows_all, 0.6 * budget_s)
    rest = rows_all[done:] if done < len(rows_all) else rows_all  # a small tile is timed again
    with threadpool_limits(limits=1):
        rate1, done1, t1 = _oracle_rows_rate(w, qh, kh, vh, qpos, kpos, rest, 0.25 * budget_s)
    # Merge oracle: contiguous blocks of rows of the partials, all n parts.
    n_parts, rows, d = o_parts.shape
    gen = np.random.default_rng(8)
    m_rows, m_bytes, m_t = 0, 0.0, 0.0
    while m_t < 0.15 * budget_s and m_rows < rows:
        r0 = int(gen.integers(0, max(rows - 4096, 1)))
        op = o_parts[:, r0:r0 + 4096].float().cpu().numpy()
        lp = l_parts[:, r0:r0 + 4096].cpu().numpy()
        t0 = time.perf_counter()
        oracle.lse_merge_ref(op, lp)
        m_t += time.perf_counter() - t0
        m_rows += op.shape[1]
        m_bytes += merge_bytes(n_parts, op.shape[1], d, o_parts.element_size())
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} (token, head) rows of the same tile, exact float64 two-pass "
                      f"softmax over their visible keys, {t_used:.1f} s",
            "full_tile_s_extrapolated": tile_flops_total / rate,
            "single_core": {"value": rate1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                            "sample": f"{done1} rows of the same tile on one core, {t1:.1f} s"},
            "merge": {"value": m_bytes / max(m_t, 1e-9) / 1e9, "unit": "GB/s",
                      "cores": int(threads),
                      "sample": f"{m_rows} merged rows of the {n_parts} partials, float64, "
                                f"{m_t:.1f} s"}}


def backward_leg(steps, wid, w, q, k, v, o, lse, q_parts, blocks, fwd_flops, dev):
    """Times the tile backward: D = rowsum(dO * O), then dQ and dK/dV."""
    import torch
    import long_context_distributed_amd as mat
    import workloads
    do = workloads.gather(w, "do", q_parts, dev)
    delta = torch.empty_like(lse)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(w.head_dim)

    def run(ev):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if ev is not None else None
        if e:
            e[0].record()
        mat.bwd_delta(o, do, out=delta)
        if e:
            e[1].record()
        mat.tile_bwd(q, k, v, do, lse, delta, blocks, w.part_len, scale, dq=dq, dk=dk, dv=dv)
        if e:
            e[2].record()
            ev.append(e)

    run(None)
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        run(ev)
    torch.cuda.synchronize()
    t_delta = sum(e[0].elapsed_time(e[1]) for e in ev) / len(ev)
    t_bwd = sum(e[1].elapsed_time(e[2]) for e in ev) / len(ev)
    bwd_flops = 2.5 * fwd_flops        # five products of 2*d flops per visible pair and head
    exec_flops = 3.5 * fwd_flops       # seven: S and dP are formed in both kernels
    tflops = bwd_flops / (t_bwd * 1e-3) / 1e12
    dbytes = 2 * o.numel() * o.element_size() + delta.numel() * 4
    log(f"[bench] backward {t_bwd:.3f} ms = {tflops:.1f} TFLOP/s algorithmic "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of peak), "
        f"{exec_flops / (t_bwd * 1e-3) / 1e12:.1f} TFLOP/s executed; row terms {t_delta:.3f} ms")
    return {"ms": t_bwd, "tflops": tflops, "frac_peak": tflops / PEAK_BF16_TFLOPS,
            "flops": bwd_flops, "executed_flops": exec_flops,
            "executed_tflops": exec_flops / (t_bwd * 1e-3) / 1e12, "steps": steps,
            "kernels": ["tile_bwd_dq_bf16_d128", "tile_bwd_dkdv_bf16_d128"],
            "traffic": {kn: measured_traffic(kn, wid) for kn in
                        ("tile_bwd_dq_bf16_d128", "tile_bwd_dkdv_bf16_d128")},
            "row_terms": {"ms": t_delta, "bytes": dbytes,
                          "gbs": dbytes / (t_delta * 1e-3) / 1e9}}


def peer_kv_sets(w, block_list):
    """KV partitions behind each partial the merge combines: the mesh-row
    sibling tiles' KV sets, or (the per-KV-partition merge) one partition
    each.  block_list(R, C, r, c, causal, rotate) gives a tile's blocks."""
    R, C, r, c = w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col
    if w.merge == "per_kv_part":
        kv = [b[3] for b in block_list(R, C, r, c, w.causal, w.kv_rotate) if b[0] == 0]
        return [[kp] for kp in kv], None
    sets = []
    for i in range(C):
        sb = block_list(R, C, r, i, w.causal, w.kv_rotate)
        sets.append([b[3] for b in sb if b[0] == 0])
    return sets, c


def dead_partials(w, q_parts, peer_kv):
    """dead[i][s]: partial i holds no key visible to Q slot s (lse = -inf on
    all of the slot's rows), i.e. none of its KV partitions is at or before
    the slot's partition (causal only)."""
    return [[w.causal and not any(kp <= qp for kp in kvp) for qp in q_parts] for kvp in peer_kv]


def live_partial_rows(w, q_parts, peer_kv):
    """Partial rows with a finite lse: the rows the merge reads outputs of."""
    dead = dead_partials(w, q_parts, peer_kv)
    return sum(w.part_len * w.heads_q for row in dead for x in row if not x)


def _peer_partials(w, mat, q_parts, n_tok, rows, d, dtype, dev):
    """Partials the peers would return: same shapes, random outputs, finite
    lse, and -inf where the peer's tile holds no KV partition at or before
    the row's partition.  Returns (o_parts, l_parts, own index or None)."""
    import torch
    peer_kv, own = peer_kv_sets(w, mat.block_list)
    n_parts = len(peer_kv)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    o_parts = (0.05 * torch.randn((n_parts, rows, d), generator=gen, device=dev)).to(dtype)
    l_parts = 10.0 + torch.randn((n_parts, rows), generator=gen, device=dev)
    for i, row in enumerate(dead_partials(w, q_parts, peer_kv)):
        for s_, dead in enumerate(row):
            if dead:
                l_parts[i].view(n_tok, w.heads_q)[s_ * w.part_len:(s_ + 1) * w.part_len] = -math.inf
    return o_parts, l_parts, own


def measure_workload(wid, steps, warmup, backward_steps, cpu_budget, copy_calibration, dev,
                     after_forward=None):
    """Times whole steps (block list + tile forward + merge) of one workload,
    with per-kernel HIP events on the launch stream, then the backward, then
    the oracle on host cores.  after_forward(result) -> dict, if given, runs
    right after the forward steps (the GPU still at the clock it holds under
    that load) and its entries join the result.  Returns (result dict, step
    ms)."""
    import torch
    import long_context_distributed_amd as mat
    import workloads

    w = workloads.WORKLOADS[wid]
    scale = 1.0 / math.sqrt(w.head_dim)
    R, C, r, c = w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col

    blocks = mat.block_list(R, C, r, c, w.causal, w.kv_rotate)
    q_parts = [b[2] for b in blocks if b[1] == 0]
    kv_parts = [b[3] for b in blocks if b[0] == 0]
    log(f"[bench] workload {wid}: {w.name}")
    q = workloads.gather(w, "q", q_parts, dev)
    k = workloads.gather(w, "k", kv_parts, dev)
    v = workloads.gather(w, "v", kv_parts, dev)
    n_tok, d = q.shape[0], w.head_dim
    rows = n_tok * w.heads_q
    elt = 2 if w.dtype == "bf16" else 4

    o_parts, l_parts, own = _peer_partials(w, mat, q_parts, n_tok, rows, d, q.dtype, dev)
    n_parts = o_parts.shape[0]
    if own is not None:
        o_own, l_own = o_parts[own].view_as(q), l_parts[own].view(n_tok, w.heads_q)
    else:
        o_own = torch.empty_like(q)
        l_own = torch.empty((n_tok, w.heads_q), dtype=torch.float32, device=dev)
    o_m = torch.empty((rows, d), dtype=q.dtype, device=dev)
    l_m = torch.empty((rows,), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    flops = tile_flops(blocks, w.part_len, w.heads_q, d)
    mbytes_all = merge_bytes(n_parts, rows, d, elt)
    live = int(torch.isfinite(l_parts).sum().item())
    assert live == live_partial_rows(w, q_parts, peer_kv_sets(w, mat.block_list)[0])
    mbytes = merge_live_bytes(n_parts, rows, d, elt, live)

    ev = []

    def step(record):
        bl = mat.block_list(R, C, r, c, w.causal, w.kv_rotate)
        e0 = torch.cuda.Event(enable_timing=True) if record else None
        e1 = torch.cuda.Event(enable_timing=True) if record else None
        e2 = torch.cuda.Event(enable_timing=True) if record else None
        if record:
            e0.record()
        mat.tile_fwd(q, k, v, bl, w.part_len, scale, out=o_own, lse=l_own)
        if record:
            e1.record()
        mat.lse_merge(o_parts, l_parts, out=o_m, lse_out=l_m)
        if record:
            e2.record()
            ev.append((e0, e1, e2))

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / steps
    t_tile = sum(e0.elapsed_time(e1) for e0, e1, _ in ev) / len(ev)   # ms
    t_merge = sum(e1.elapsed_time(e2) for _, e1, e2 in ev) / len(ev)  # ms
    tile_tflops = flops / (t_tile * 1e-3) / 1e12
    merge_gbs = mbytes / (t_merge * 1e-3) / 1e9
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    tile_kernel = "tile_fwd_bf16_d128" if w.dtype == "bf16" else "tile_fwd_f32"
    log(f"[bench] tile {t_tile:.3f} ms = {tile_tflops:.1f} TFLOP/s ({100 * tile_tflops / peak:.1f}% "
        f"of {peak}); merge {t_merge:.3f} ms = {merge_gbs:.0f} GB/s "
        f"({100 * merge_gbs / PEAK_HBM_GBS:.1f}% of HBM, {mbytes / 1e9:.3f} GB read+written); "
        f"step {ms_step:.3f} ms")

    res = {
        "workload": wid,
        "dtype": w.dtype,
        "config": {"workload": w.name, "mesh": f"{R}x{C}", "tile": [r, c],
                   "part_len": w.part_len, "q_tokens": n_tok, "kv_tokens": k.shape[0],
                   "heads_q": w.heads_q, "heads_kv": w.heads_kv, "head_dim": d,
                   "causal": w.causal, "kv_rotate": w.kv_rotate, "merge_partials": n_parts,
                   "parallelism": "one GPU's tile"},
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "step_tflops": flops / (ms_step * 1e-3) / 1e12,
        "tile_fwd": {"ms": t_tile, "tflops": tile_tflops, "frac_peak": tile_tflops / peak,
                     "peak": peak, "flops": flops, "kernel": tile_kernel,
                     "traffic": measured_traffic(tile_kernel, wid)},
        "lse_merge": {"ms": t_merge, "gbs": merge_gbs, "frac_hbm": merge_gbs / PEAK_HBM_GBS,
                      "bytes": mbytes, "bytes_all_rows": mbytes_all,
                      "live_partial_rows": live, "partial_rows": n_parts * rows,
                      "traffic": measured_traffic("lse_merge_kernel", wid)},
    }
    if after_forward is not None:
        res.update(after_forward(res))
    # Row a1 (host): the block list of this tile, library call against the oracle's brute force.
    t0 = time.perf_counter()
    for _ in range(1000):
        mat.block_list(R, C, r, c, w.causal, w.kv_rotate)
    bl_us = (time.perf_counter() - t0) * 1e3
    res["block_list"] = {"us": bl_us, "blocks": len(blocks),
                         "note": "host call through the Python binding, mean of 1000"}
    if cpu_budget > 0:
        import oracle
        t0 = time.perf_counter()
        for _ in range(20):
            ref_bl = oracle.block_list_ref(R, C, r, c, w.causal, w.kv_rotate)
        res["block_list"]["oracle_us"] = (time.perf_counter() - t0) / 20 * 1e6
        res["block_list"]["equal_to_oracle"] = ref_bl == blocks
    res["plan"] = plan_leg(w, blocks, t_tile)
    if backward_steps > 0 and w.dtype == "bf16":
        res["tile_bwd"] = backward_leg(backward_steps, wid, w, q, k, v, o_own, l_own,
                                       q_parts, blocks, flops, dev)
    if copy_calibration > 0:
        src = torch.empty(copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy calibration: {copy_calibration} MiB read + written by one copy kernel")
    if cpu_budget > 0:
        log(f"[bench] timing the oracle on host cores ({cpu_budget:.0f} s budget)")
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, q_parts, kv_parts, flops, o_parts,
                                           l_parts, cpu_budget)
    del q, k, v, o_parts, l_parts, o_own, l_own, o_m, l_m
    torch.cuda.empty_cache()
    return res, ms_step


XGMI_LINK_GBS = 153.0   # one MI355X xGMI link, GB/s per direction (AMD spec figure)


def plan_costs(w, blocks, t_tile_ms, link_gbs=XGMI_LINK_GBS):
    """Costs of the planner's step model for one tile: transfer times of a Q
    partition, a KV partition and a partial output over one link, and the
    time of a FULL and a DIAG block from the measured tile time shared over
    the visible pairs."""
    elt = 2 if w.dtype == "bf16" else 4
    L, d = w.part_len, w.head_dim
    pairs = sum(L * L if b[4] == 0 else L * (L + 1) // 2 if b[4] == 1 else 0 for b in blocks)
    per_pair = t_tile_ms * 1e-3 / pairs
    bw = link_gbs * 1e9
    return {"recv_q_s": L * w.heads_q * d * elt / bw,
            "recv_kv_s": 2 * L * w.heads_kv * d * elt / bw,
            "send_o_s": L * w.heads_q * (d * elt + 4) / bw,
            "full_block_s": per_pair * L * L,
            "diag_block_s": per_pair * (L * (L + 1) // 2)}


def plan_leg(w, blocks, t_tile_ms):
    """Row f2 (host): the greedy plan of this GPU's tile with the measured
    block time and one xGMI link, beside the eager variant and the lower
    bound max(total transfer, total compute)."""
    import long_context_distributed_amd as mat
    costs = plan_costs(w, blocks, t_tile_ms)
    R, C, r, c = w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col
    t0 = time.perf_counter()
    for _ in range(100):
        steps = mat.plan(R, C, r, c, w.causal, w.kv_rotate, costs)
    plan_us = (time.perf_counter() - t0) * 1e4
    eager = mat.plan(R, C, r, c, w.causal, w.kv_rotate, costs, delay=False)
    comm = sum(st["comm_s"] for st in steps)
    comp = sum(st["compute_s"] for st in steps)
    span = steps[-1]["end_s"] if steps else 0.0
    res = {"link_gbs": XGMI_LINK_GBS, "costs_s": costs, "steps": len(steps),
           "makespan_ms": span * 1e3, "eager_makespan_ms": (eager[-1]["end_s"] if eager else 0.0) * 1e3,
           "transfer_ms": comm * 1e3, "compute_ms": comp * 1e3,
           "lower_bound_ms": max(comm, comp) * 1e3,
           "compute_busy": comp / span if span else 1.0, "plan_us": plan_us,
           "note": "host planner (step model), not a multi-GPU run"}
    log(f"[bench] plan: {len(steps)} steps, makespan {span * 1e3:.2f} ms (eager "
        f"{res['eager_makespan_ms']:.2f} ms, bound {res['lower_bound_ms']:.2f} ms), "
        f"compute busy {100 * res['compute_busy']:.1f}%, planner {plan_us:.0f} us")
    return res


def gemm_ceiling(ms, dev):
    """Vendor bf16 GEMM (8192 x 8192 x 8192) run back to back for ~ms
    milliseconds; returns its rate and the duration measured with events."""
    import torch
    n = 8192
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    a = torch.randn((n, n), generator=gen, device=dev).to(torch.bfloat16).contiguous()
    b = torch.randn((n, n), generator=gen, device=dev).to(torch.bfloat16).contiguous()
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    reps = max(1, int(ms / max(e0.elapsed_time(e1), 1e-3)))
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1)
    tflops = 2.0 * n ** 3 * reps / (t * 1e-3) / 1e12
    log(f"[bench] gemm ceiling: {reps} x bf16 {n}^3 in {t:.1f} ms = {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS})")
    return {"kernel": "torch.mm bf16 8192^3 (vendor GEMM)", "reps": reps, "ms": t,
            "tflops": tflops, "frac_peak": tflops / PEAK_BF16_TFLOPS}


def sdpa_reference(wid, dev, reps=5):
    """Vendor attention on one FULL and one DIAG block of the workload (see
    --sdpa-reference); a dict with the block times and the tile-equivalent
    rate, or the reason it could not run."""
    import torch
    import long_context_distributed_amd as mat
    import workloads

    w = workloads.WORKLOADS[wid]
    if w.dtype != "bf16":
        return {"error": "the flash backend takes bf16 / fp16 only"}
    blocks = mat.block_list(w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col, w.causal, w.kv_rotate)
    n_full = sum(1 for b in blocks if b[4] == mat.FULL)
    n_diag = sum(1 for b in blocks if b[4] == mat.DIAG)
    L, hq, d = w.part_len, w.heads_q, w.head_dim
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    q, k, v = (torch.randn((1, hq, L, d), generator=gen, device=dev).to(torch.bfloat16).contiguous()
               for _ in range(3))
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
    except ImportError as e:
        return {"error": f"torch.nn.attention unavailable: {e}"}
    res = {"kernel": "torch scaled_dot_product_attention (flash backend)",
           "shape": f"1 x {hq} heads x {L} x {d}, bf16", "n_full": n_full, "n_diag": n_diag}
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for causal, key in ((False, "full_block_ms"), (True, "diag_block_ms")):
                torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
                e1.record()
                torch.cuda.synchronize()
                res[key] = e0.elapsed_time(e1) / reps
    except RuntimeError as e:
        return {"error": f"flash backend unavailable: {str(e)[:200]}"}
    t = n_full * res["full_block_ms"] + n_diag * res["diag_block_ms"]
    flops = tile_flops(blocks, L, hq, d)
    res.update({"tile_equiv_ms": t, "tflops": flops / (t * 1e-3) / 1e12})
    res["frac_peak"] = res["tflops"] / PEAK_BF16_TFLOPS
    log(f"[bench] sdpa reference: FULL {res['full_block_ms']:.3f} ms, DIAG {res['diag_block_ms']:.3f} ms, "
        f"tile of {n_full}F/{n_diag}D {t:.1f} ms = {res['tflops']:.1f} TFLOP/s")
    return res


def _others(spec):
    if spec == "none":
        return []
    if spec == "all":
        return [1, 2, 3, 4, 5]
    return sorted({int(x) for x in spec.split(",") if x.strip()})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--backward-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--others", default="all",
                    help="other workloads measured after the headline: none, all or a list")
    ap.add_argument("--gemm-ceiling", type=float, default=130.0, metavar="MS")
    ap.add_argument("--sdpa-reference", dest="sdpa_reference", action="store_true", default=True)
    ap.add_argument("--no-sdpa-reference", dest="sdpa_reference", action="store_false")
    ap.add_argument("--others-steps", type=int, default=5)
    ap.add_argument("--others-cpu-budget", type=float, default=5.0)
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's tile only: the hot path is one GPU's share of the "
              "mesh and the library has no multi-GPU path; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cpu_budget = 0.0 if a.no_cpu_baseline else a.cpu_budget

    def references(res):
        """The vendor GEMM and vendor attention references, run right after
        the headline's forward steps."""
        out = {}
        if a.gemm_ceiling > 0:
            try:
                out["gemm_ceiling"] = gemm_ceiling(a.gemm_ceiling, dev)
            except RuntimeError as e:
                out["gemm_ceiling"] = {"error": str(e)[:200]}
        if a.sdpa_reference:
            try:
                ref = sdpa_reference(a.workload, dev)
            except RuntimeError as e:
                ref = {"error": str(e)[:200]}
            if "tile_equiv_ms" in ref:
                ref["tile_fwd_speedup"] = ref["tile_equiv_ms"] / res["tile_fwd"]["ms"]
            out["sdpa_reference"] = ref
        return out

    head, ms_step = measure_workload(a.workload, a.steps, a.warmup, a.backward_steps, cpu_budget,
                                     a.copy_calibration, dev, after_forward=references)
    tf = head["tile_fwd"]
    result = {
        "metric": METRIC,
        "value": head["step_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "tile_fwd": tf,
        "lse_merge": head["lse_merge"],
        "roofline": {"bound": "mfma", "achieved": tf["tflops"], "peak": tf["peak"],
                     "unit": "TFLOP/s", "frac": tf["frac_peak"], "traffic": tf["traffic"],
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE)",
                     "kernel": tf["kernel"]},
        "block_list": head["block_list"],
    }
    for key in ("plan", "tile_bwd", "cpu_baseline"):
        if key in head:
            result[key] = head[key]
    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count,
                        "memory_gib": round(props.total_memory / 2 ** 30, 1)}
    for key in ("gemm_ceiling", "sdpa_reference"):
        if key in head:
            result[key] = head[key]
    others = _others(a.others)
    if others:
        per = {}
        for wid in others:
            if wid == a.workload:
                per[str(wid)] = {k_: v_ for k_, v_ in head.items()
                                 if k_ not in ("gemm_ceiling", "sdpa_reference")}
                continue
            res, _ = measure_workload(wid, a.others_steps, 1, 2 if a.backward_steps > 0 else 0,
                                      0.0 if a.no_cpu_baseline else a.others_cpu_budget, 0, dev)
            per[str(wid)] = res
        result["per_workload"] = per
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
