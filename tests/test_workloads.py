"""The seeded input generators (CPU): the properties the parity tests and the
benchmark rely on.  Each (tensor, partition) has its own stream, so a
partition has the same values in every tile that holds it; the fp32 workload
is numpy's default_rng(seed) drawing Q, K, V in that order; shapes, dtypes
and distributions follow the workload definitions; sampled rows include the
forced edge rows."""
import numpy as np
import pytest
import torch

import workloads


def test_partition_is_the_same_in_every_tile_that_holds_it():
    w = workloads.small("bf16", 40, 3, 3, 1, 1, True, True, 4, 2, 128)
    a = workloads.gather(w, "k", [4, 7, 1], "cpu")
    b = workloads.gather(w, "k", [7, 2], "cpu")
    L = w.part_len
    assert torch.equal(a[L:2 * L], b[:L])                # partition 7 in two tiles
    assert torch.equal(workloads.partition(w, "k", 4), workloads.partition(w, "k", 4))
    assert not torch.equal(a[:L], a[L:2 * L])            # different partitions differ
    assert not torch.equal(workloads.partition(w, "q", 4)[:, :2], workloads.partition(w, "k", 4))


def test_streams_differ_between_tensors_and_seeds():
    w0 = workloads.small("bf16", 16, 2, 2, 0, 0, True, True, 2, 2, 128, seed=0)
    w1 = workloads.small("bf16", 16, 2, 2, 0, 0, True, True, 2, 2, 128, seed=1)
    parts = {t: workloads.partition(w0, t, 1).float() for t in ("q", "k", "v", "do")}
    for a in parts:
        for b in parts:
            if a < b:
                assert not torch.equal(parts[a], parts[b]), (a, b)
    assert not torch.equal(workloads.partition(w1, "q", 1), workloads.partition(w0, "q", 1))
    seeds = {workloads.stream_seed(0, t, p) for t in workloads.TENSORS for p in range(256)}
    assert len(seeds) == len(workloads.TENSORS) * 256


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_shapes_dtypes_and_distributions(wid):
    w = workloads.WORKLOADS[wid]
    assert w.dtype == "bf16" and w.head_dim == 128 and w.heads_q % w.heads_kv == 0
    q = workloads.partition(w, "q", 0)
    k = workloads.partition(w, "k", 0)
    assert q.shape == (w.part_len, w.heads_q, 128) and q.dtype == torch.bfloat16
    assert k.shape == (w.part_len, w.heads_kv, 128) and k.dtype == torch.bfloat16
    qf, kf = q.float(), k.float()
    assert abs(float(qf.mean())) < 0.01 and abs(float(qf.std()) - 1.0) < 0.01
    k_std = 2.0 if wid == 5 else 1.0                     # K ~ N(0, 4) on the 16x4 workload
    assert abs(float(kf.std()) - k_std) < 0.01 * k_std
    # bf16 values are the round-to-nearest-even images of the float32 draws
    gen = torch.Generator().manual_seed(workloads.stream_seed(w.seed, "q", 0))
    x = torch.randn((w.part_len, w.heads_q, 128), generator=gen)
    assert torch.equal(x.to(torch.bfloat16), q)


def test_fp32_workload_is_numpy_default_rng_in_order():
    w = workloads.WORKLOADS[1]
    assert w.dtype == "f32" and w.numpy_whole_sequence and w.seed == 0
    rng = np.random.default_rng(0)
    want = {t: rng.standard_normal((w.seq_len, w.heads_q if t == "q" else w.heads_kv, w.head_dim))
            .astype(np.float32) for t in ("q", "k", "v")}
    for t in ("q", "k", "v"):
        got = workloads.gather(w, t, list(range(w.n_parts)), "cpu").numpy()
        assert np.array_equal(got, want[t]), t


def test_row_terms_ranges():
    w = workloads.small("bf16", 300, 2, 2, 1, 0, True, True, 8, 2, 128)
    lse, delta = workloads.row_terms(w, [2, 3], "cpu")
    assert lse.shape == delta.shape == (600, 8) and lse.dtype == delta.dtype == torch.float32
    assert float(lse.min()) >= 10.0 and float(lse.max()) < 14.0
    assert abs(float(delta.mean())) < 0.05 and abs(float(delta.std()) - 1.0) < 0.05
    lse2, _ = workloads.row_terms(w, [3], "cpu")
    assert torch.equal(lse[300:], lse2)                   # per-partition streams here too


def test_sample_rows_include_the_edge_rows():
    L, hq, hkv, n_tok = 1000, 32, 8, 4000
    rows = workloads.sample_rows(n_tok, hq, hkv, L, n_sample=64, seed=1)
    assert rows.dtype == np.int64 and rows.shape[1] == 2
    assert len({tuple(r) for r in rows.tolist()}) == len(rows)   # no duplicates
    assert rows[:, 0].min() >= 0 and rows[:, 0].max() < n_tok
    assert rows[:, 1].min() >= 0 and rows[:, 1].max() < hq
    have = {tuple(r) for r in rows.tolist()}
    for s in range(n_tok // L):
        for u in (0, 1, L // 2, L - 1):
            for h in (0, 3, 4, 31):                       # 0, G-1, G, H_q-1 with G = 4
                assert (s * L + u, h) in have
    assert np.array_equal(rows, workloads.sample_rows(n_tok, hq, hkv, L, n_sample=64, seed=1))
