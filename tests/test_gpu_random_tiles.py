"""GPU parity of the tile forward on seeded random tile geometries: mesh
shape, tile position, causal or not, rotated or contiguous KV order, ragged
partition lengths, group sizes, dtype and head dim drawn per case, and in
half the cases only a random subset of the tile's KV slots listed (blocks
not listed count as skipped).  Every row is compared with the oracle over
the same KV partitions.  Every call goes through the C ABI."""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available
from tests.parity import compare, run_tile, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]

N_CASES = 40


def random_case(seed):
    """One seeded geometry: (workload, KV slots listed or None for all)."""
    rng = np.random.default_rng(1000 + seed)
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    d = 128 if dtype == "bf16" else int(rng.choice([64, 128]))
    R, C = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    r, c = int(rng.integers(0, R)), int(rng.integers(0, C))
    causal, rot = bool(rng.random() < 0.6), bool(rng.integers(0, 2))
    L = int(rng.integers(1, 17)) if rng.random() < 0.25 else int(rng.integers(17, 258))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.integers(1, 8 if dtype == "bf16" else 5))
    w = workloads.small(dtype, L, R, C, r, c, causal, rot, g * hkv, hkv, d, seed=seed)
    subset = None
    if R > 1 and rng.random() < 0.5:
        k = int(rng.integers(1, R))
        subset = sorted(int(x) for x in rng.choice(R, size=k, replace=False))
    return w, subset


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_tile_matches_oracle_all_rows(seed):
    w, subset = random_case(seed)
    say(f"[case] seed {seed}: {w.name}, KV slots {subset if subset is not None else 'all'}")
    t = run_tile(w)
    if subset is not None:
        blocks = [b for b in t["blocks"] if b[1] in subset]
        t = run_tile(w, blocks=blocks, inputs=(t["q"], t["k"], t["v"]))
    L = w.part_len
    slots = range(len(t["kv_parts"])) if subset is None else subset
    kv_parts = [t["kv_parts"][j] for j in slots]
    k = np.concatenate([t["k"][j * L:(j + 1) * L].float().cpu().numpy() for j in slots])
    v = np.concatenate([t["v"][j * L:(j + 1) * L].float().cpu().numpy() for j in slots])
    ref_o, ref_lse = oracle.tile_rows_ref(t["q"], k, v, t["q_parts"], kv_parts, L, w.causal,
                                          1.0 / math.sqrt(w.head_dim))
    compare(t["o"], t["lse"], ref_o, ref_lse, w.dtype, what=f"seed {seed}: {w.name}")


N_BWD_CASES = 16


def random_bwd_case(seed):
    """One seeded bf16 geometry for the backward (whole tile listed)."""
    rng = np.random.default_rng(5000 + seed)
    R, C = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    r, c = int(rng.integers(0, R)), int(rng.integers(0, C))
    causal, rot = bool(rng.random() < 0.6), bool(rng.integers(0, 2))
    L = int(rng.integers(1, 17)) if rng.random() < 0.25 else int(rng.integers(17, 300))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.integers(1, 8))
    return workloads.small("bf16", L, R, C, r, c, causal, rot, g * hkv, hkv, 128, seed=seed)


@pytest.mark.parametrize("seed", range(N_BWD_CASES))
def test_random_tile_bwd_matches_oracle(seed):
    from tests.test_gpu_backward import _compare, _oracle_row_terms, _run_case
    w = random_bwd_case(seed)
    say(f"[case] backward seed {seed}: {w.name}")
    t = _run_case(w)
    lse_r, delta_r = _oracle_row_terms(w, t["q_parts"], t["q"], t["do"])
    refs = oracle.tile_bwd_ref(t["q"], t["k"], t["v"], t["do"], lse_r, delta_r, t["q_parts"],
                               t["kv_parts"], w.part_len, w.causal, 1.0 / math.sqrt(w.head_dim))
    for name, got, ref in zip(("dq", "dk", "dv"), (t["dq"], t["dk"], t["dv"]), refs):
        _compare(name, got, ref, f"seed {seed}: {w.name}")
