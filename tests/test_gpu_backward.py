"""GPU parity of the tile backward (dQ, dK, dV shares) and of the row terms
D = rowsum(dO * O) against the oracle.

Each side computes its own inputs from the same seeded q, k, v, dO (drawn on
the device; the oracle reads the values back): the
library gets the rows' final lse and O from its own forward over the whole
row (the ring-shaped tile (p, 0) of a P x 1 mesh holds partition p against
every partition) and D from its delta kernel; the oracle computes exact lse,
O and D in float64.  Every call goes through the C ABI.

Tolerance (the pages and the task state none for gradients): per tensor,
max |error| <= 2e-2 * max |reference| and ||error|| <= 1e-2 * ||reference||.
The products use bf16 P and dS (relative rounding 2^-9 each) accumulated in
float32, and the library's lse carries the forward's error (<= 1e-3).
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available
from tests.parity import say, tile_geometry

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]

RTOL_MAX = 2e-2
RTOL_FRO = 1e-2

CASES = [
    # L, mesh, tile, causal, rotate, Hq, Hkv
    (64, (2, 2), (0, 0), True, True, 4, 2),
    (17, (2, 2), (0, 1), True, True, 4, 1),      # ragged; Q slots with no visible key
    (129, (4, 4), (2, 2), True, True, 8, 1),     # G=8, ragged, three kinds
    (128, (4, 4), (1, 3), True, True, 2, 2),     # MHA
    (1, (2, 3), (1, 1), True, True, 4, 4),       # one-token partitions
    (16, (1, 1), (0, 0), True, False, 4, 2),     # diagonal block only
    (96, (3, 2), (1, 0), False, False, 6, 2),    # non-causal, G=3
    (300, (2, 4), (1, 2), True, True, 16, 2),    # G=8, two head groups, two key blocks
    (520, (2, 2), (1, 0), True, True, 4, 1),     # nine 64-key tiles per block, three key blocks
    (100, (2, 2), (1, 0), True, True, 12, 1),    # G=12
    (70, (2, 3), (0, 2), True, True, 10, 2),     # G=5
    (90, (4, 2), (2, 1), True, False, 4, 2),     # causal with contiguous KV order
]


def _wl(case, seed=0):
    L, (R, C), (r, c), causal, rot, hq, hkv = case
    return workloads.small("bf16", L, R, C, r, c, causal, rot, hq, hkv, 128, seed=seed)


def _library_row_terms(w, q_parts, dout):
    """lse and D of the tile's Q rows over the whole row, by the library:
    forward of partition p against all partitions (tile (p, 0) of a P x 1
    mesh), then the delta kernel."""
    import torch
    import long_context_distributed_amd as mat
    P = w.n_parts
    scale = 1.0 / math.sqrt(w.head_dim)
    os, lses = [], []
    for qp in q_parts:
        blocks = mat.block_list(P, 1, qp, 0, w.causal, True)
        _, kv_parts = tile_geometry(w, blocks)
        q = workloads.gather(w, "q", [qp], "cuda")
        k = workloads.gather(w, "k", kv_parts, "cuda")
        v = workloads.gather(w, "v", kv_parts, "cuda")
        o, lse = mat.tile_fwd(q, k, v, blocks, w.part_len, scale)
        os.append(o)
        lses.append(lse)
    o = torch.cat(os).contiguous()
    lse = torch.cat(lses).contiguous()
    return lse, mat.bwd_delta(o, dout)


def _oracle_row_terms(w, q_parts, q, dout):
    P = w.n_parts
    # drawn on the device (the streams are device-specific), read back by the oracle
    k_all = workloads.gather(w, "k", list(range(P)), "cuda")
    v_all = workloads.gather(w, "v", list(range(P)), "cuda")
    q_pos = oracle.tile_positions_ref(q_parts, w.part_len)
    k_pos = np.arange(P * w.part_len)
    o, lse = oracle.attention_ref(q, k_all, v_all, q_pos, k_pos, w.causal, 1.0 / math.sqrt(w.head_dim))
    return lse, oracle.bwd_delta_ref(o, dout)


def _compare(name, got, ref, what):
    got = got.cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite {name}"
    scale_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = np.abs(got - ref)
    e_max = float(err.max()) if err.size else 0.0
    fro = float(np.linalg.norm(err)) / max(float(np.linalg.norm(ref)), 1e-30)
    say(f"[parity] {what} {name}: max|err|={e_max:.3e} (max|ref| {scale_max:.3e}) rel fro={fro:.3e}")
    assert e_max <= RTOL_MAX * scale_max + 1e-6, f"{what}: {name} max error {e_max}"
    assert fro <= RTOL_FRO or scale_max == 0.0, f"{what}: {name} relative error {fro}"


def _run_case(w):
    import long_context_distributed_amd as mat
    blocks = mat.block_list(w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col, w.causal, w.kv_rotate)
    assert blocks == oracle.block_list_ref(w.mesh_rows, w.mesh_cols, w.tile_row, w.tile_col,
                                           w.causal, w.kv_rotate)
    q_parts, kv_parts = tile_geometry(w, blocks)
    q = workloads.gather(w, "q", q_parts, "cuda")
    k = workloads.gather(w, "k", kv_parts, "cuda")
    v = workloads.gather(w, "v", kv_parts, "cuda")
    do = workloads.gather(w, "do", q_parts, "cuda")
    lse, delta = _library_row_terms(w, q_parts, do)
    dq, dk, dv = mat.tile_bwd(q, k, v, do, lse, delta, blocks, w.part_len)
    return dict(blocks=blocks, q_parts=q_parts, kv_parts=kv_parts, q=q, k=k, v=v, do=do,
                dq=dq, dk=dk, dv=dv)


@pytest.mark.parametrize("case", CASES, ids=[f"L{c[0]}-{c[1][0]}x{c[1][1]}-t{c[2]}-c{int(c[3])}"
                                             f"-G{c[5]}/{c[6]}" for c in CASES])
def test_tile_bwd_matches_oracle(case):
    w = _wl(case)
    say(f"[case] backward {w.name}")
    t = _run_case(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    lse_r, delta_r = _oracle_row_terms(w, t["q_parts"], t["q"], t["do"])
    rdq, rdk, rdv = oracle.tile_bwd_ref(t["q"], t["k"], t["v"], t["do"], lse_r, delta_r,
                                        t["q_parts"], t["kv_parts"], w.part_len, w.causal, scale)
    for name, got, ref in (("dq", t["dq"], rdq), ("dk", t["dk"], rdk), ("dv", t["dv"], rdv)):
        _compare(name, got, ref, w.name)
    # Rows that no visible pair of the tile reaches are exactly zero (closed
    # form: a query partition qp sees a key partition kp iff kp <= qp).
    L = w.part_len
    for s, qp in enumerate(t["q_parts"]):
        if w.causal and not any(kp <= qp for kp in t["kv_parts"]):
            assert np.all(t["dq"][s * L:(s + 1) * L].cpu().numpy() == 0), "unreached dq rows not 0"
    for j, kp in enumerate(t["kv_parts"]):
        if w.causal and not any(kp <= qp for qp in t["q_parts"]):
            for g in (t["dk"], t["dv"]):
                assert np.all(g[j * L:(j + 1) * L].cpu().numpy() == 0), "unreached dk/dv rows not 0"


def test_tile_shares_sum_to_full_gradient():
    """All tiles of a 2x3 mesh (causal, rotated): the library's shares, added
    at their partitions, equal the oracle's gradient of full attention."""
    import torch
    R, C, L, hq, hkv = 2, 3, 48, 4, 2
    base = workloads.small("bf16", L, R, C, 0, 0, True, True, hq, hkv, 128, seed=3)
    P = R * C
    N = P * L
    dq = torch.zeros((N, hq, 128), dtype=torch.float64)
    dk = torch.zeros((N, hkv, 128), dtype=torch.float64)
    dv = torch.zeros((N, hkv, 128), dtype=torch.float64)
    for r in range(R):
        for c in range(C):
            w = workloads.small("bf16", L, R, C, r, c, True, True, hq, hkv, 128, seed=3)
            t = _run_case(w)
            qi = torch.from_numpy(oracle.tile_positions_ref(t["q_parts"], L))
            ki = torch.from_numpy(oracle.tile_positions_ref(t["kv_parts"], L))
            dq.index_add_(0, qi, t["dq"].cpu().double())
            dk.index_add_(0, ki, t["dk"].cpu().double())
            dv.index_add_(0, ki, t["dv"].cpu().double())
    q = workloads.gather(base, "q", list(range(P)), "cuda")
    k = workloads.gather(base, "k", list(range(P)), "cuda")
    v = workloads.gather(base, "v", list(range(P)), "cuda")
    do = workloads.gather(base, "do", list(range(P)), "cuda")
    pos = np.arange(N)
    rdq, rdk, rdv, _, _, _ = oracle.full_grads_ref(q, k, v, do, pos, pos, True, 1.0 / math.sqrt(128))
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        _compare(name, got, ref, "2x3 mesh sum")


@pytest.mark.parametrize("dtype,d,rows", [("bf16", 128, 1000), ("bf16", 24, 77), ("bf16", 512, 33),
                                          ("f32", 64, 500), ("f32", 12, 9), ("f32", 512, 40)])
def test_bwd_delta_matches_oracle(dtype, d, rows):
    import torch
    import long_context_distributed_amd as mat
    g = torch.Generator().manual_seed(rows + d)
    tdt = workloads.torch_dtype(dtype)
    o = torch.randn((rows, d), generator=g).to(tdt)
    do = torch.randn((rows, d), generator=g).to(tdt)
    got = mat.bwd_delta(o.cuda(), do.cuda()).cpu().numpy()
    ref = oracle.bwd_delta_ref(o, do)
    tol = 1e-5 * math.sqrt(d) * 4
    err = float(np.max(np.abs(got - ref)))
    say(f"[parity] bwd_delta {dtype} d={d} rows={rows}: max|err|={err:.3e}")
    assert err <= tol


def test_tile_bwd_deterministic_and_in_bounds():
    """Two backward runs are bitwise identical (no atomics, fixed reduction
    order); guard bands around dq, dk, dv and delta stay untouched."""
    import torch
    import long_context_distributed_amd as mat
    w = _wl((130, (4, 4), (2, 2), True, True, 8, 2))
    t = _run_case(w)
    pad = 4096

    def guarded(shape, fill):
        n = int(np.prod(shape))
        big = torch.full((n + 2 * pad,), fill, dtype=torch.float32, device="cuda")
        return big, big[pad:pad + n].view(shape)

    bq, dq2 = guarded(t["dq"].shape, -7.0)
    bk, dk2 = guarded(t["dk"].shape, 3.5)
    bv, dv2 = guarded(t["dv"].shape, 9.25)
    lse, delta = _library_row_terms(w, t["q_parts"], t["do"])
    bd, delta2 = guarded(delta.shape, 1.5)
    mat.bwd_delta(_library_row_terms_o(w, t["q_parts"]), t["do"], out=delta2)
    mat.tile_bwd(t["q"], t["k"], t["v"], t["do"], lse, delta2, t["blocks"], w.part_len,
                 dq=dq2, dk=dk2, dv=dv2)
    torch.cuda.synchronize()
    assert torch.equal(delta2, delta), "row terms not deterministic"
    for name, a, b in (("dq", dq2, t["dq"]), ("dk", dk2, t["dk"]), ("dv", dv2, t["dv"])):
        assert torch.equal(a, b), f"{name} not deterministic"
    for big, fill, name in ((bq, -7.0, "dq"), (bk, 3.5, "dk"), (bv, 9.25, "dv"), (bd, 1.5, "delta")):
        assert torch.all(big[:pad] == fill) and torch.all(big[-pad:] == fill), f"{name} canary hit"


def _library_row_terms_o(w, q_parts):
    """The rows' final O by the library (as in _library_row_terms)."""
    import torch
    import long_context_distributed_amd as mat
    outs = []
    for qp in q_parts:
        blocks = mat.block_list(w.n_parts, 1, qp, 0, w.causal, True)
        _, kv_parts = tile_geometry(w, blocks)
        o, _ = mat.tile_fwd(workloads.gather(w, "q", [qp], "cuda"), workloads.gather(w, "k", kv_parts, "cuda"),
                            workloads.gather(w, "v", kv_parts, "cuda"), blocks, w.part_len,
                            1.0 / math.sqrt(w.head_dim))
        outs.append(o)
    return torch.cat(outs).contiguous()
