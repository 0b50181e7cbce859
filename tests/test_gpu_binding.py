"""The Python binding with device tensors: bad output buffers, overlapping
buffers and bad sizes are refused before any launch, and a call on an explicit
stream gives the same result as on the current stream."""
import math

import pytest

import workloads
from tests.conftest import gpu_available
from tests.parity import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]


def _inputs():
    w = workloads.small("bf16", 64, 2, 2, 1, 0, True, True, 4, 2, 128)
    import long_context_distributed_amd as mat
    blocks = mat.block_list(2, 2, 1, 0, True, True)
    q_parts = [b[2] for b in blocks if b[1] == 0]
    kv_parts = [b[3] for b in blocks if b[0] == 0]
    q = workloads.gather(w, "q", q_parts, "cuda")
    k = workloads.gather(w, "k", kv_parts, "cuda")
    v = workloads.gather(w, "v", kv_parts, "cuda")
    return w, blocks, q, k, v


def test_bad_calls_are_refused():
    import torch
    import long_context_distributed_amd as mat
    say("[case] binding: refused calls")
    w, blocks, q, k, v = _inputs()
    L = w.part_len
    with pytest.raises(ValueError, match="part_len"):
        mat.tile_fwd(q, k, v, blocks, 0)
    with pytest.raises(ValueError, match="contiguous"):
        mat.tile_fwd(q.transpose(0, 1), k, v, blocks, L)
    with pytest.raises(ValueError, match="overlap"):
        mat.tile_fwd(q, k, v, blocks, L, out=q)
    with pytest.raises(ValueError, match="wrong shape"):
        mat.tile_fwd(q, k, v, blocks, L, lse=torch.empty(7, device="cuda"))
    o, lse = mat.tile_fwd(q, k, v, blocks, L)
    rows = q.shape[0] * q.shape[1]
    parts = torch.stack([o.reshape(rows, 128)] * 2)
    lparts = torch.stack([lse.reshape(rows)] * 2)
    with pytest.raises(ValueError, match="lse_out"):
        mat.lse_merge(parts, lparts, lse_out=torch.empty(rows - 1, device="cuda"))
    with pytest.raises(ValueError, match="lse_out"):
        mat.lse_merge(parts, lparts, lse_out=torch.empty(rows, device="cuda", dtype=torch.float64))
    with pytest.raises(ValueError, match="overlap"):
        mat.lse_merge(parts, lparts, out=parts[0])
    # a float32 [T, H] output placed inside the bf16 input o
    t_, h_ = o.shape[0], o.shape[1]
    inside = o.view(-1)[: 2 * t_ * h_].view(torch.float32).view(t_, h_)
    with pytest.raises(ValueError, match="overlap"):
        mat.bwd_delta(o, o, out=inside)
    torch.cuda.synchronize()


def test_explicit_stream_matches_current_stream():
    import torch
    import long_context_distributed_amd as mat
    say("[case] binding: explicit stream")
    w, blocks, q, k, v = _inputs()
    scale = 1.0 / math.sqrt(128)
    o0, l0 = mat.tile_fwd(q, k, v, blocks, w.part_len, scale)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o1 = torch.empty_like(q)
        l1 = torch.empty_like(l0)
    o1, l1 = mat.tile_fwd(q, k, v, blocks, w.part_len, scale, out=o1, lse=l1, stream=s)
    s.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
