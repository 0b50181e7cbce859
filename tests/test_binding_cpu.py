"""The Python binding on the CPU: it refuses host tensors (the library has no
CPU path and the binding never computes anything itself), and its argument
checks (one device, contiguity, no overlap of outputs with inputs) reject bad
calls before the library is reached."""
import types

import pytest
import torch

import long_context_distributed_amd as mat


def _cpu(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_every_entry_point_refuses_host_tensors():
    q = _cpu(64, 4, 128)
    k = _cpu(64, 2, 128)
    blocks = [(0, 0, 0, 0, mat.DIAG)]
    lse = _cpu(64, 4, dtype=torch.float32)
    calls = [
        lambda: mat.tile_fwd(q, k, k, blocks, 64),
        lambda: mat.lse_merge(_cpu(2, 16, 128), _cpu(2, 16, dtype=torch.float32)),
        lambda: mat.bwd_delta(q, q),
        lambda: mat.tile_bwd(q, k, k, q, lse, lse, blocks, 64),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="no CPU path"):
            call()


def _fake(device, contiguous=True):
    return types.SimpleNamespace(is_cuda=True, device=torch.device(device),
                                 is_contiguous=lambda: contiguous)


def test_one_device_and_contiguity():
    mat._require_device(_fake("cuda:0"), _fake("cuda:0"))
    with pytest.raises(ValueError, match="one device"):
        mat._require_device(_fake("cuda:0"), _fake("cuda:1"))
    with pytest.raises(ValueError, match="contiguous"):
        mat._require_device(_fake("cuda:0"), _fake("cuda:0", contiguous=False))


def test_outputs_must_not_overlap():
    base = torch.zeros(1024)
    a, b, c = base[:256], base[256:512], base[200:300]
    mat._no_overlap([a], [b])                 # adjacent, disjoint
    with pytest.raises(ValueError, match="overlap"):
        mat._no_overlap([c], [a])             # output over an input
    with pytest.raises(ValueError, match="overlap"):
        mat._no_overlap([a, c], [b])          # two outputs over each other
    mat._no_overlap([base[:0]], [a])          # empty output


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    """Without the built library the binding raises; nothing computes on the host."""
    from long_context_distributed_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libmeshattn.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _lib.load()
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        mat.block_list(2, 2, 0, 0, True, True)
