"""GPU parity at the edges: score magnitudes that move the softmax shift
often, and tiles at the library's maximum slot and block counts (forward and
backward).  Every call goes through the C ABI.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available
from tests.parity import compare, run_tile, say, tile_geometry

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_large_scores(dtype, d):
    """Q and K with standard deviation 8: scaled scores spread over about
    +-250, so rows see new maxima far above the current shift."""
    w = workloads.small(dtype, 160, 2, 2, 1, 0, True, True, 4, 2, d, std=(8.0, 8.0, 1.0))
    t = run_tile(w)
    ref_o, ref_lse = oracle.tile_rows_ref(t["q"], t["k"], t["v"], t["q_parts"], t["kv_parts"],
                                          w.part_len, w.causal, 1.0 / math.sqrt(d))
    compare(t["o"], t["lse"], ref_o, ref_lse, dtype, what=f"large scores {dtype}",
            tol=_tol(dtype, ref_lse))


def _tol(dtype, ref_lse):
    """The per-dtype bounds, widened for float32 to its resolution at these
    scores: with scaled scores of magnitude M, lse and the exponents carry
    rounding of a few ulp(M) ~ M 2^-23 (about 3e-5 at M = 250), which a fixed
    1e-5 cannot hold.  bf16 keeps its bounds."""
    import tests.parity as par
    to, tl = par.TOL[dtype]
    if dtype != "f32":
        return to, tl
    fin = np.isfinite(ref_lse)
    m = float(np.max(np.abs(ref_lse[fin]))) if fin.any() else 0.0
    extra = 4.0 * m * 2.0 ** -23
    return to + extra, tl + extra


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128)])
def test_rising_scores(dtype, d):
    """Scores that grow along the keys (a new row maximum in every 32-key
    step, by up to ~30 in base e per step): the shift moves again and again."""
    import torch
    import long_context_distributed_amd as mat
    L, hq, hkv = 256, 2, 1
    g = torch.Generator(device="cuda").manual_seed(9)
    tdt = workloads.torch_dtype(dtype)
    # q = ones and k_j = ramp_j * ones / sqrt(d): the scaled score of key j is ramp_j
    q = torch.ones((L, hq, d), device="cuda", dtype=torch.float32)
    ramp = torch.linspace(0.0, 60.0, L, device="cuda").view(L, 1, 1)
    k = (ramp * torch.ones((L, hkv, d), device="cuda") / math.sqrt(d)
         + 0.01 * torch.randn((L, hkv, d), generator=g, device="cuda"))
    v = torch.randn((L, hkv, d), generator=g, device="cuda")
    q, k, v = (x.to(tdt).contiguous() for x in (q, k, v))
    blocks = [(0, 0, 0, 0, mat.DIAG)]
    o, lse = mat.tile_fwd(q, k, v, blocks, L, 1.0 / math.sqrt(d))
    ref_o, ref_lse = oracle.tile_rows_ref(q, k, v, [0], [0], L, True, 1.0 / math.sqrt(d))
    say(f"[edge] rising scores: lse range {float(np.min(ref_lse)):.1f} .. {float(np.max(ref_lse)):.1f}")
    compare(o, lse, ref_o, ref_lse, dtype, what=f"rising scores {dtype}", tol=_tol(dtype, ref_lse))


MAX_MESHES = [(64, 1, 40, 0), (1, 64, 0, 33), (32, 32, 17, 9)]


@pytest.mark.parametrize("R,C,r,c", MAX_MESHES, ids=[f"{m[0]}x{m[1]}" for m in MAX_MESHES])
def test_max_slots_forward(R, C, r, c):
    """64 KV slots (64x1), 64 Q slots (1x64) and 32x32 = 1024 blocks."""
    w = workloads.small("bf16", 8, R, C, r, c, True, True, 4, 2, 128)
    t = run_tile(w)
    assert len(t["blocks"]) == R * C
    ref_o, ref_lse = oracle.tile_rows_ref(t["q"], t["k"], t["v"], t["q_parts"], t["kv_parts"],
                                          w.part_len, w.causal, 1.0 / math.sqrt(128))
    compare(t["o"], t["lse"], ref_o, ref_lse, "bf16", what=f"{R}x{C} tile ({r},{c})")


@pytest.mark.parametrize("R,C,r,c", MAX_MESHES, ids=[f"{m[0]}x{m[1]}" for m in MAX_MESHES])
def test_max_slots_backward(R, C, r, c):
    """The backward on the same tiles, as a function of synthetic row terms."""
    import long_context_distributed_amd as mat
    w = workloads.small("bf16", 8, R, C, r, c, True, True, 4, 2, 128)
    blocks = mat.block_list(R, C, r, c, True, True)
    q_parts, kv_parts = tile_geometry(w, blocks)
    q = workloads.gather(w, "q", q_parts, "cuda")
    k = workloads.gather(w, "k", kv_parts, "cuda")
    v = workloads.gather(w, "v", kv_parts, "cuda")
    do = workloads.gather(w, "do", q_parts, "cuda")
    lse, delta = workloads.row_terms(w, q_parts, "cuda")
    lse = lse - 8.0  # short rows: lse near ln(visible count)
    scale = 1.0 / math.sqrt(128)
    dq, dk, dv = mat.tile_bwd(q, k, v, do, lse, delta, blocks, w.part_len, scale)
    refs = oracle.tile_bwd_ref(q, k, v, do, lse, delta, q_parts, kv_parts, w.part_len, True, scale)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g = got.cpu().numpy()
        err = float(np.max(np.abs(g - ref)))
        top = float(np.max(np.abs(ref)))
        fro = float(np.linalg.norm(g - ref)) / max(float(np.linalg.norm(ref)), 1e-30)
        say(f"[edge] {R}x{C} backward {name}: max|err|={err:.3e} (max|ref| {top:.3e}) fro={fro:.2e}")
        assert err <= 2e-2 * top + 1e-6 and fro <= 1e-2, name


def test_empty_block_list():
    """No listed block (every pair SKIP): the forward writes (0, -inf) for every
    row and the backward writes zero gradients, over buffers pre-filled with
    garbage."""
    import torch
    import long_context_distributed_amd as mat
    w = workloads.small("bf16", 70, 2, 2, 0, 0, True, True, 4, 2, 128)
    q = workloads.gather(w, "q", [0, 1], "cuda")
    k = workloads.gather(w, "k", [0, 2], "cuda")
    v = workloads.gather(w, "v", [0, 2], "cuda")
    do = workloads.gather(w, "do", [0, 1], "cuda")
    o = torch.full_like(q, 3.0)
    lse = torch.full((q.shape[0], 4), 5.0, device="cuda")
    mat.tile_fwd(q, k, v, [], w.part_len, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    lse_r, delta = workloads.row_terms(w, [0, 1], "cuda")
    dq = torch.full(q.shape, 7.0, device="cuda")
    dk = torch.full(k.shape, 7.0, device="cuda")
    dv = torch.full(v.shape, 7.0, device="cuda")
    mat.tile_bwd(q, k, v, do, lse_r, delta, [], w.part_len, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.timeout(600)
def test_byte_ranges_past_32_bits():
    """A partition whose token rows span more than 4 GiB of each tensor (1024
    heads, L = 16449): every load's buffer range is clamped to the rows it
    serves, so none wraps around 2^32.  Unclamped, the range of the tile that
    starts at row 64 (2^14 + 1 rows left, 2^18 bytes each) would wrap to 256
    bytes and rows 65..127 of Q, K and V would read as zero.  Forward and
    backward, checked on rows and keys of the first tiles and at the end."""
    import torch
    import long_context_distributed_amd as mat
    L, H, d = 16449, 1024, 128
    say(f"[case] byte ranges past 32 bits: L={L}, {H} heads, d={d}")
    scale = 1.0 / math.sqrt(d)
    g = torch.Generator(device="cuda").manual_seed(21)
    q, k, v, do = (torch.randn((L, H, d), generator=g, device="cuda", dtype=torch.bfloat16)
                   for _ in range(4))
    assert L * H * d * 2 > 2 ** 32
    blocks = [(0, 0, 0, 0, mat.DIAG)]
    o, lse = mat.tile_fwd(q, k, v, blocks, L, scale)
    torch.cuda.synchronize()
    pos = np.arange(L)
    toks = np.array([0, 1, 63, 64, 65, 66, 95, 96, 127, 128, 200, L // 2, L - 2, L - 1])
    heads = [0, 517, H - 1]
    for h in heads:
        sl = slice(h, h + 1)
        rows = np.stack([toks, np.zeros_like(toks)], axis=1)
        ref_o, ref_l = oracle.attention_ref(q[:, sl], k[:, sl], v[:, sl], pos, pos, True, scale,
                                            rows=rows)
        got_o = o[toks, h].float().cpu().numpy()
        got_l = lse[toks, h].cpu().numpy()
        e_o = float(np.max(np.abs(got_o - ref_o)))
        e_l = float(np.max(np.abs(got_l - ref_l)))
        say(f"[edge] >4 GiB rows, head {h}: max|dO|={e_o:.2e} max|dlse|={e_l:.2e}")
        assert e_o <= 2e-2 and e_l <= 1e-3, (h, e_o, e_l)

    # backward with the tile's own lse and D = rowsum(dO * O)
    delta = mat.bwd_delta(o, do)
    dq, dk, dv = mat.tile_bwd(q, k, v, do, lse, delta, blocks, L, scale)
    torch.cuda.synchronize()
    del o
    keys = toks
    for h in heads:
        sl = slice(h, h + 1)
        f64 = lambda t: t[:, sl].double().cpu().numpy()  # noqa: E731
        qh, kh, vh, doh = f64(q), f64(k), f64(v), f64(do)
        lh, dh = f64(lse), f64(delta)
        ref_dq = oracle.attention_bwd_ref(qh[toks], kh, vh, doh[toks], lh[toks], dh[toks],
                                          pos[toks], pos, True, scale)[0]
        _, ref_dk, ref_dv = oracle.attention_bwd_ref(qh, kh[keys], vh[keys], doh, lh, dh, pos,
                                                     pos[keys], True, scale)
        for name, got, ref in (("dq", dq[toks, h], ref_dq[:, 0]), ("dk", dk[keys, h], ref_dk[:, 0]),
                               ("dv", dv[keys, h], ref_dv[:, 0])):
            got = got.cpu().numpy()
            err = float(np.max(np.abs(got - ref)))
            top = float(np.max(np.abs(ref)))
            say(f"[edge] >4 GiB rows, head {h}: {name} max|err|={err:.2e} (max|ref| {top:.2e})")
            assert err <= 2e-2 * top + 1e-6, (h, name, err, top)


@pytest.mark.parametrize("dtype,d,scale", [("bf16", 128, 0.02), ("bf16", 128, 0.5), ("f32", 64, 0.3)])
def test_non_default_scale(dtype, d, scale):
    """Softmax scales other than 1/sqrt(d): near-uniform attention (0.02) and
    sharp attention (0.5, scaled scores of standard deviation ~5.7); the
    backward (bf16) from the tile's own lse and D = rowsum(dO * O)."""
    import torch
    import long_context_distributed_amd as mat
    w = workloads.small(dtype, 80, 2, 2, 1, 0, True, True, 4, 2, d)
    blocks = mat.block_list(2, 2, 1, 0, True, True)
    q_parts, kv_parts = tile_geometry(w, blocks)
    q = workloads.gather(w, "q", q_parts, "cuda")
    k = workloads.gather(w, "k", kv_parts, "cuda")
    v = workloads.gather(w, "v", kv_parts, "cuda")
    o, lse = mat.tile_fwd(q, k, v, blocks, w.part_len, scale)
    ref_o, ref_l = oracle.tile_rows_ref(q, k, v, q_parts, kv_parts, w.part_len, True, scale)
    compare(o, lse, ref_o, ref_l, dtype, what=f"scale {scale} {dtype}", tol=_tol(dtype, ref_l))
    if dtype != "bf16":
        return
    do = workloads.gather(w, "do", q_parts, "cuda")
    delta = mat.bwd_delta(o, do)
    dq, dk, dv = mat.tile_bwd(q, k, v, do, lse, delta, blocks, w.part_len, scale)
    torch.cuda.synchronize()
    refs = oracle.tile_bwd_ref(q, k, v, do, lse.cpu().double().numpy(), delta.cpu().double().numpy(),
                               q_parts, kv_parts, w.part_len, True, scale)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g = got.cpu().numpy()
        err = float(np.max(np.abs(g - ref)))
        top = float(np.max(np.abs(ref)))
        fro = float(np.linalg.norm(g - ref)) / max(float(np.linalg.norm(ref)), 1e-30)
        say(f"[edge] scale {scale} backward {name}: max|err|={err:.3e} (max|ref| {top:.3e}) fro={fro:.2e}")
        assert err <= 2e-2 * top + 1e-6 and fro <= 1e-2, name
