"""The hot path captured in a HIP graph: the library allocates nothing and
launches only on the caller's stream, so one step (tile forward + LSE merge)
and the backward (row terms + dQ and dK/dV kernels) can be captured and
replayed.  Every replay, with eager work and synchronisations between
replays, must equal the eager result bit for bit (the kernels are
deterministic)."""
import math

import pytest

import workloads
from tests.conftest import gpu_available
from tests.parity import say, tile_geometry

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]


def _tile(L=96):
    import long_context_distributed_amd as mat
    w = workloads.small("bf16", L, 2, 2, 1, 0, True, True, 4, 2, 128)
    blocks = mat.block_list(2, 2, 1, 0, True, True)
    q_parts, kv_parts = tile_geometry(w, blocks)
    q = workloads.gather(w, "q", q_parts, "cuda")
    k = workloads.gather(w, "k", kv_parts, "cuda")
    v = workloads.gather(w, "v", kv_parts, "cuda")
    do = workloads.gather(w, "do", q_parts, "cuda")
    return w, blocks, q, k, v, do


def test_forward_and_merge_replay_in_a_graph():
    import torch
    import long_context_distributed_amd as mat
    say("[case] graph: tile forward + merge")
    w, blocks, q, k, v, _ = _tile()
    scale = 1.0 / math.sqrt(128)
    rows = q.shape[0] * q.shape[1]
    # the tile writes its partial straight into slot 0 of the merge's inputs
    parts = torch.randn((3, rows, 128), device="cuda").to(torch.bfloat16)
    lparts = torch.randn((3, rows), device="cuda")
    o = parts[0].view(q.shape)
    lse = lparts[0].view(q.shape[0], q.shape[1])
    om = torch.empty((rows, 128), device="cuda", dtype=torch.bfloat16)
    lm = torch.empty((rows,), device="cuda")

    def step():
        mat.tile_fwd(q, k, v, blocks, w.part_len, scale, out=o, lse=lse)
        mat.lse_merge(parts, lparts, out=om, lse_out=lm)

    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, om, lm)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (o, lse, om, lm):
            t.fill_(7.0)            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "merged o", "merged lse"), (o, lse, om, lm), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"


def test_backward_replays_in_a_graph():
    import torch
    import long_context_distributed_amd as mat
    say("[case] graph: row terms + tile backward")
    w, blocks, q, k, v, do = _tile(80)
    scale = 1.0 / math.sqrt(128)
    o, lse = mat.tile_fwd(q, k, v, blocks, w.part_len, scale)
    delta = torch.empty_like(lse)
    dq = torch.empty(q.shape, device="cuda")
    dk = torch.empty(k.shape, device="cuda")
    dv = torch.empty(v.shape, device="cuda")

    def step():
        mat.bwd_delta(o, do, out=delta)
        mat.tile_bwd(q, k, v, do, lse, delta, blocks, w.part_len, scale, dq=dq, dk=dk, dv=dv)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (delta, dq, dk, dv)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (delta, dq, dk, dv):
            t.fill_(-3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("delta", "dq", "dk", "dv"), (delta, dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
