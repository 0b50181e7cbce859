"""Full-size parity of the tile backward on the bf16 workloads, in the launch
configuration the benchmark times (one mesh_attn_tile_bwd call on the whole
tile).

The backward is checked as a function of its inputs: q, k, v, dO come from the
seeded generators and the rows' lse and D are synthetic too (generated with
the same seeded streams for both sides; values in the range of real ones), so
that the oracle can compute sampled outputs one by one:
  * sampled dq rows (token, head), plus forced edge rows: the row against
    every key of the tile;
  * sampled dk / dv rows (key token, KV head), plus the first and last key of
    every KV slot: the key against every query row of the tile and every
    query head of its group.
Tolerance as for the small cases: max |error| <= 2e-2 * max |reference| over
the sampled rows, and relative Frobenius error <= 1e-2.
"""
import gc
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available
from tests.parity import say, tile_geometry

pytestmark = [pytest.mark.gpu, pytest.mark.slow,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]

RTOL_MAX = 2e-2
RTOL_FRO = 1e-2


def _check(name, got, ref, what):
    err = np.abs(got - ref)
    scale_max = float(np.max(np.abs(ref)))
    e_max = float(err.max())
    fro = float(np.linalg.norm(err)) / max(float(np.linalg.norm(ref)), 1e-30)
    say(f"[parity] {what} {name}: {got.shape[0]} sampled rows max|err|={e_max:.3e} "
        f"(max|ref| {scale_max:.3e}) rel fro={fro:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite {name}"
    assert e_max <= RTOL_MAX * scale_max + 1e-6, f"{what}: {name} max error {e_max}"
    assert fro <= RTOL_FRO, f"{what}: {name} relative error {fro}"


def _f64(t):
    return t.detach().cpu().double().numpy()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_backward_workload(wid):
    import torch
    import long_context_distributed_amd as mat
    w = workloads.WORKLOADS[wid]
    say(f"[case] backward workload {wid}: {w.name}")
    L, G = w.part_len, w.heads_q // w.heads_kv
    scale = 1.0 / math.sqrt(w.head_dim)
    blocks = mat.block_list(w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col, w.causal, w.kv_rotate)
    q_parts, kv_parts = tile_geometry(w, blocks)
    q = workloads.gather(w, "q", q_parts, "cuda")
    k = workloads.gather(w, "k", kv_parts, "cuda")
    v = workloads.gather(w, "v", kv_parts, "cuda")
    do = workloads.gather(w, "do", q_parts, "cuda")
    lse, delta = workloads.row_terms(w, q_parts, "cuda")
    dq, dk, dv = mat.tile_bwd(q, k, v, do, lse, delta, blocks, L, scale)
    torch.cuda.synchronize()
    q_pos = oracle.tile_positions_ref(q_parts, L)
    k_pos = oracle.tile_positions_ref(kv_parts, L)

    # dq rows: one query row against all keys of its KV head
    rows = workloads.sample_rows(q.shape[0], w.heads_q, w.heads_kv, L, n_sample=48, seed=5)
    got, ref = [], []
    for hk in range(w.heads_kv):
        sel = rows[rows[:, 1] // G == hk]
        if len(sel) == 0:
            continue
        k_h, v_h = _f64(k[:, hk:hk + 1]), _f64(v[:, hk:hk + 1])
        for i, h in sel:
            r = oracle.attention_bwd_ref(_f64(q[i:i + 1, h:h + 1]), k_h, v_h, _f64(do[i:i + 1, h:h + 1]),
                                         _f64(lse[i:i + 1, h:h + 1]), _f64(delta[i:i + 1, h:h + 1]),
                                         q_pos[i:i + 1], k_pos, w.causal, scale)[0]
            ref.append(r[0, 0])
            got.append(_f64(dq[i, h]))
        del k_h, v_h
        gc.collect()
    _check("dq", np.array(got), np.array(ref), f"workload {wid}")

    # dk / dv rows: one key against all query rows of the tile and the group's heads
    n_kv_tok = k.shape[0]
    rng = np.random.default_rng(6)
    keys = {(int(t), int(hk)) for t, hk in zip(rng.integers(0, n_kv_tok, 12),
                                               rng.integers(0, w.heads_kv, 12))}
    for j in range(len(kv_parts)):
        keys.add((j * L, (j * 3) % w.heads_kv))
        keys.add((j * L + L - 1, (j * 5 + 1) % w.heads_kv))
    keys = sorted(keys, key=lambda x: (x[1], x[0]))
    got_k, ref_k, got_v, ref_v = [], [], [], []
    for hk in sorted({x[1] for x in keys}):
        heads = slice(hk * G, (hk + 1) * G)
        q_g, do_g = _f64(q[:, heads]), _f64(do[:, heads])
        lse_g, delta_g = _f64(lse[:, heads]), _f64(delta[:, heads])
        for j, _ in [x for x in keys if x[1] == hk]:
            _, rk, rv = oracle.attention_bwd_ref(q_g, _f64(k[j:j + 1, hk:hk + 1]), _f64(v[j:j + 1, hk:hk + 1]),
                                                 do_g, lse_g, delta_g, q_pos, k_pos[j:j + 1], w.causal, scale)
            ref_k.append(rk[0, 0])
            ref_v.append(rv[0, 0])
            got_k.append(_f64(dk[j, hk]))
            got_v.append(_f64(dv[j, hk]))
        del q_g, do_g
        gc.collect()
    _check("dk", np.array(got_k), np.array(ref_k), f"workload {wid}")
    _check("dv", np.array(got_v), np.array(ref_v), f"workload {wid}")
    del q, k, v, do, dq, dk, dv
    gc.collect()
    torch.cuda.empty_cache()
