"""Mesh-Attention tile hot path for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libmeshattn.so`` (include/mesh_attn.h):
argument marshalling only.  PyTorch supplies device memory and the stream;
every step of the computation runs in the library's HIP kernels.

    block_list(mesh_rows, mesh_cols, row, col, causal, kv_rotate) -> [Block tuples]
    tile_fwd(q, k, v, blocks, part_len, softmax_scale=None) -> (o, lse)
    lse_merge(o_parts, lse_parts) -> (o, lse)
    bwd_delta(o, dout) -> delta
    tile_bwd(q, k, v, dout, lse, delta, blocks, part_len, softmax_scale=None) -> (dq, dk, dv)
    plan(mesh_rows, mesh_cols, row, col, causal, kv_rotate, costs, delay=True) -> [steps]
"""
import ctypes
import math

from . import _lib
from ._lib import (BF16, COMM_NONE, COMM_RECV_KV, COMM_RECV_Q, COMM_SEND_O, DIAG, F32,  # noqa: F401
                   FULL, SKIP)

__all__ = ["MeshAttnError", "block_list", "tile_fwd", "lse_merge", "bwd_delta", "tile_bwd", "plan",
           "FULL", "DIAG", "SKIP", "COMM_NONE", "COMM_RECV_Q", "COMM_RECV_KV", "COMM_SEND_O",
           "library_path"]


class MeshAttnError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def library_path():
    return _lib.LIB_PATH


def _check(lib, status):
    if status != _lib.OK:
        msg = lib.mesh_attn_last_error().decode() or lib.mesh_attn_status_string(status).decode()
        raise MeshAttnError(status, msg)


def block_list(mesh_rows, mesh_cols, row, col, causal, kv_rotate):
    """Blocks (q_slot, kv_slot, q_part, kv_part, kind) of tile (row, col)."""
    lib = _lib.load()
    n = ctypes.c_int32(0)
    st = lib.mesh_attn_block_list(mesh_rows, mesh_cols, row, col, int(bool(causal)),
                                  int(bool(kv_rotate)), None, 0, ctypes.byref(n))
    if st != _lib.ERR_CAPACITY:
        _check(lib, st)
    arr = (_lib.Block * n.value)()
    _check(lib, lib.mesh_attn_block_list(mesh_rows, mesh_cols, row, col, int(bool(causal)),
                                         int(bool(kv_rotate)), arr, n.value, ctypes.byref(n)))
    return [(b.q_slot, b.kv_slot, b.q_part, b.kv_part, b.kind) for b in arr]


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream, device):
    import torch
    if stream is not None and stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _require_device(*ts):
    """Every tensor contiguous and on one HIP device (there is no CPU path)."""
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device (no CPU path)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors must be on one device ({dev} and {t.device})")


def _no_overlap(outs, ins):
    """Outputs may overlap neither the inputs nor each other (the kernels
    read inputs while writing outputs)."""
    def span(t):
        a = t.data_ptr()
        return a, a + t.numel() * t.element_size()
    for i, o in enumerate(outs):
        a0, a1 = span(o)
        for x in list(ins) + list(outs[i + 1:]):
            b0, b1 = span(x)
            if a0 < b1 and b0 < a1:
                raise ValueError("output buffers must not overlap the inputs or each other")


def _tile_desc(q, k, v, blocks, part_len, softmax_scale):
    _require_device(q, k, v)
    if int(part_len) < 1:
        raise ValueError("part_len must be >= 1")
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("expected q [Tq, Hq, d] and k, v [Tk, Hkv, d]")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k and v must share a dtype")
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if dk != d:
        raise ValueError("head_dim of q and k differ")
    if tq % part_len or tk % part_len:
        raise ValueError("token counts must be multiples of part_len")
    blocks = list(blocks)
    arr = (_lib.Block * max(1, len(blocks)))()
    for i, b in enumerate(blocks):
        arr[i] = _lib.Block(*[int(x) for x in b])
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    desc = _lib.TileDesc(_dtype_code(q), part_len, tq // part_len, tk // part_len, hq, hkv, d,
                         scale, arr, len(blocks))
    desc._keep = arr  # the block array must outlive the call
    return desc


def tile_fwd(q, k, v, blocks, part_len, softmax_scale=None, out=None, lse=None, stream=None):
    """Forward of one tile.

    q: [n_q_slots*L, H_q, d], k/v: [n_kv_slots*L, H_kv, d] on the device
    (bf16 or f32, same dtype); blocks: iterable of (q_slot, kv_slot, q_part,
    kv_part, kind).  Returns (o [n_q_slots*L, H_q, d], lse [n_q_slots*L, H_q]
    float32), allocated with torch unless given.
    """
    import torch
    lib = _lib.load()
    desc = _tile_desc(q, k, v, blocks, part_len, softmax_scale)
    tq, hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    _require_device(q, k, v, out, lse)
    if out.shape != q.shape or out.dtype != q.dtype or lse.shape != (tq, hq) or \
            lse.dtype != torch.float32:
        raise ValueError("output buffers have the wrong shape or dtype")
    _no_overlap([out, lse], [q, k, v])
    _check(lib, lib.mesh_attn_tile_fwd(ctypes.byref(desc), q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                       _stream_handle(stream, q.device)))
    return out, lse


def lse_merge(o_parts, lse_parts, out=None, lse_out=None, want_lse=True, stream=None):
    """Merge n partial results: o_parts [n, rows, d] (bf16/f32), lse_parts
    [n, rows] float32 -> (o [rows, d], lse [rows] or None)."""
    import torch
    lib = _lib.load()
    _require_device(o_parts, lse_parts)
    if o_parts.dim() != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("expected o_parts [n, rows, d] and lse_parts [n, rows]")
    if lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be float32")
    n, rows, d = o_parts.shape
    if out is None:
        out = torch.empty((rows, d), dtype=o_parts.dtype, device=o_parts.device)
    if want_lse and lse_out is None:
        lse_out = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    outs = [out] + ([lse_out] if lse_out is not None else [])
    _require_device(o_parts, lse_parts, *outs)
    if out.shape != (rows, d) or out.dtype != o_parts.dtype:
        raise ValueError("output buffer has the wrong shape or dtype")
    if lse_out is not None and (lse_out.shape != (rows,) or lse_out.dtype != torch.float32):
        raise ValueError("lse_out must be float32 [rows]")
    _no_overlap(outs, [o_parts, lse_parts])
    _check(lib, lib.mesh_attn_lse_merge(n, rows, d, _dtype_code(o_parts), o_parts.data_ptr(),
                                        lse_parts.data_ptr(), out.data_ptr(),
                                        lse_out.data_ptr() if lse_out is not None else None,
                                        _stream_handle(stream, o_parts.device)))
    return out, lse_out


def bwd_delta(o, dout, out=None, stream=None):
    """D = sum over the last dimension of dout * o, float32: o, dout [..., d]
    (bf16 or f32, same shape) -> delta [...]."""
    import torch
    lib = _lib.load()
    _require_device(o, dout)
    if o.shape != dout.shape or o.dtype != dout.dtype:
        raise ValueError("o and dout must share shape and dtype")
    d = o.shape[-1]
    rows = o.numel() // d if d else 0
    if out is None:
        out = torch.empty(o.shape[:-1], dtype=torch.float32, device=o.device)
    _require_device(o, dout, out)
    if out.shape != o.shape[:-1] or out.dtype != torch.float32:
        raise ValueError("output buffer has the wrong shape or dtype")
    _no_overlap([out], [o, dout])
    _check(lib, lib.mesh_attn_bwd_delta(rows, d, _dtype_code(o), o.data_ptr(), dout.data_ptr(),
                                        out.data_ptr(), _stream_handle(stream, o.device)))
    return out


def tile_bwd(q, k, v, dout, lse, delta, blocks, part_len, softmax_scale=None, dq=None, dk=None,
             dv=None, stream=None):
    """One tile's share of the attention gradients.

    q, dout: [n_q_slots*L, H_q, d]; k, v: [n_kv_slots*L, H_kv, d] (bf16);
    lse, delta: [n_q_slots*L, H_q] float32 (the rows' final lse and
    rowsum(dout * o)).  Returns (dq, dk, dv) in float32, allocated with torch
    unless given.
    """
    import torch
    lib = _lib.load()
    desc = _tile_desc(q, k, v, blocks, part_len, softmax_scale)
    _require_device(dout, lse, delta)
    tq, hq = q.shape[0], q.shape[1]
    if dout.shape != q.shape or dout.dtype != q.dtype:
        raise ValueError("dout must match q")
    if lse.shape != (tq, hq) or delta.shape != (tq, hq) or lse.dtype != torch.float32 or \
            delta.dtype != torch.float32:
        raise ValueError("lse and delta must be float32 [Tq, Hq]")
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    _require_device(q, k, v, dout, lse, delta, dq, dk, dv)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape or \
            any(t.dtype != torch.float32 for t in (dq, dk, dv)):
        raise ValueError("gradient buffers have the wrong shape or dtype")
    _no_overlap([dq, dk, dv], [q, k, v, dout, lse, delta])
    _check(lib, lib.mesh_attn_tile_bwd(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       dout.data_ptr(), lse.data_ptr(), delta.data_ptr(),
                                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       _stream_handle(stream, q.device)))
    return dq, dk, dv


def plan(mesh_rows, mesh_cols, row, col, causal, kv_rotate, costs, delay=True):
    """Greedy communication/computation schedule of GPU (row, col).

    costs: mapping with recv_q_s, recv_kv_s, send_o_s, full_block_s and
    diag_block_s (seconds).  Returns a list of steps, each a dict: comm
    (COMM_NONE / COMM_RECV_Q / COMM_RECV_KV / COMM_SEND_O), slot (-1 for
    none), blocks (block tuples computed in the step, in order), comm_s,
    compute_s, start_s, end_s.  Host code; needs no GPU.
    """
    lib = _lib.load()
    c = _lib.PlanCosts(float(costs["recv_q_s"]), float(costs["recv_kv_s"]),
                       float(costs["send_o_s"]), float(costs["full_block_s"]),
                       float(costs["diag_block_s"]), int(bool(delay)))
    ns, no = ctypes.c_int32(0), ctypes.c_int32(0)
    args = (mesh_rows, mesh_cols, row, col, int(bool(causal)), int(bool(kv_rotate)), ctypes.byref(c))
    st = lib.mesh_attn_plan(*args, None, 0, ctypes.byref(ns), None, 0, ctypes.byref(no))
    if st != _lib.ERR_CAPACITY:
        _check(lib, st)
    steps = (_lib.PlanStep * max(1, ns.value))()
    order = (_lib.Block * max(1, no.value))()
    _check(lib, lib.mesh_attn_plan(*args, steps, ns.value, ctypes.byref(ns), order, no.value,
                                   ctypes.byref(no)))
    blocks = [(b.q_slot, b.kv_slot, b.q_part, b.kv_part, b.kind) for b in order[:no.value]]
    return [{"comm": s.comm, "slot": s.slot,
             "blocks": blocks[s.block_begin:s.block_begin + s.block_count],
             "comm_s": s.comm_s, "compute_s": s.compute_s, "start_s": s.start_s, "end_s": s.end_s}
            for s in steps[:ns.value]]
