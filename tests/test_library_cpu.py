"""The C-ABI library on the CPU: it loads, exports every declared symbol, its
block list equals the oracle's bit for bit, and every validation error path
returns its status before any HIP call.

No test here launches a kernel: every tile/merge call below is built to fail
validation (the fake device addresses are never dereferenced).
"""
import ctypes
import itertools
import os
import re

import pytest

import oracle
from long_context_distributed_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol(lib):
    with open(os.path.join(ROOT, "include", "mesh_attn.h")) as f:
        header = f.read()
    declared = set(re.findall(r"MESH_ATTN_API\s+[\w\s\*]+?\b(mesh_attn_\w+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.mesh_attn_version() == 100


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.mesh_attn_status_string(code)


def _lib_block_list(lib, R, C, r, c, causal, rot):
    n = ctypes.c_int32(0)
    st = lib.mesh_attn_block_list(R, C, r, c, causal, rot, None, 0, ctypes.byref(n))
    assert st == _lib.ERR_CAPACITY and n.value == R * C
    arr = (_lib.Block * n.value)()
    short = ctypes.c_int32(0)
    if n.value > 1:
        assert lib.mesh_attn_block_list(R, C, r, c, causal, rot, arr, n.value - 1,
                                        ctypes.byref(short)) == _lib.ERR_CAPACITY
        assert short.value == n.value
    assert lib.mesh_attn_block_list(R, C, r, c, causal, rot, arr, n.value, ctypes.byref(n)) == 0
    return [(b.q_slot, b.kv_slot, b.q_part, b.kv_part, b.kind) for b in arr]


def test_block_list_bit_exact_all_small_meshes(lib):
    for R, C in itertools.product(range(1, 9), repeat=2):
        for r, c in itertools.product(range(R), range(C)):
            for causal, rot in itertools.product((0, 1), repeat=2):
                assert _lib_block_list(lib, R, C, r, c, causal, rot) == \
                    oracle.block_list_ref(R, C, r, c, causal, rot), (R, C, r, c, causal, rot)


@pytest.mark.parametrize("R,C", [(16, 4), (4, 16), (16, 16), (13, 7)])
def test_block_list_bit_exact_larger_meshes(lib, R, C):
    for r, c in [(0, 0), (R // 2, C // 2), (R - 1, C - 1), (R - 1, 0), (1 % R, C - 1)]:
        for causal, rot in itertools.product((0, 1), repeat=2):
            assert _lib_block_list(lib, R, C, r, c, causal, rot) == \
                oracle.block_list_ref(R, C, r, c, causal, rot)


def test_block_list_pins_hold_for_the_library(lib):
    """The library's own lists satisfy the oracle's property pins directly
    (rotated geometry, causal counts, contiguous tiling, the fp32 workload's
    literal tile), not only equality with the oracle."""
    from tests import oracle_pins as pins

    def bl(R, C, r, c, causal, rot):
        return _lib_block_list(lib, R, C, r, c, int(causal), int(rot))
    for R, C in [(2, 2), (4, 4), (3, 5), (8, 8), (16, 4)]:
        pins.check_block_list_geometry(bl, R, C)
        pins.check_block_list_kinds(bl, R, C)
        pins.check_block_list_contiguous(bl, R, C)
    pins.check_block_list_fp32_workload_tile(bl)


def test_block_list_errors(lib):
    n = ctypes.c_int32(0)
    arr = (_lib.Block * 4)()
    assert lib.mesh_attn_block_list(0, 2, 0, 0, 1, 1, arr, 4, ctypes.byref(n)) == _lib.ERR_INVALID
    assert lib.mesh_attn_block_list(2, 2, 2, 0, 1, 1, arr, 4, ctypes.byref(n)) == _lib.ERR_INVALID
    assert lib.mesh_attn_block_list(2, 2, 0, -1, 1, 1, arr, 4, ctypes.byref(n)) == _lib.ERR_INVALID
    assert lib.mesh_attn_block_list(2, 2, 0, 0, 1, 1, arr, 4, None) == _lib.ERR_INVALID
    assert lib.mesh_attn_block_list(300, 300, 0, 0, 1, 1, arr, 4, ctypes.byref(n)) == \
        _lib.ERR_INVALID
    assert b"outside" in lib.mesh_attn_last_error() or lib.mesh_attn_last_error()


# ----------------------------------------------------------------------------- tile_fwd

FAKE = 0x100000  # 16-byte aligned fake address; never reaches a kernel


def _desc(blocks=None, **kw):
    base = dict(dtype=_lib.BF16, part_len=64, n_q_slots=2, n_kv_slots=2, heads_q=4, heads_kv=2,
                head_dim=128, softmax_scale=0.088)
    base.update(kw)
    if blocks is None:
        blocks = oracle.block_list_ref(2, 2, 0, 0, True, True)
    arr = (_lib.Block * max(1, len(blocks)))()
    for i, b in enumerate(blocks):
        arr[i] = _lib.Block(*b)
    d = _lib.TileDesc(base["dtype"], base["part_len"], base["n_q_slots"], base["n_kv_slots"],
                      base["heads_q"], base["heads_kv"], base["head_dim"], base["softmax_scale"],
                      arr, len(blocks))
    d._keep = arr
    return d


def _tile(lib, desc, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, by_ref=True):
    return lib.mesh_attn_tile_fwd(ctypes.byref(desc) if by_ref else None, q, k, v, o, lse, None)


INVALID_DESCS = {
    "dtype": dict(dtype=7),
    "part_len": dict(part_len=0),
    "n_q_slots": dict(n_q_slots=0),
    "n_q_slots too many": dict(n_q_slots=65),
    "n_kv_slots": dict(n_kv_slots=0),
    "heads_q not multiple": dict(heads_q=3, heads_kv=2),
    "heads_kv zero": dict(heads_kv=0),
    "scale zero": dict(softmax_scale=0.0),
    "scale negative": dict(softmax_scale=-1.0),
    "scale nan": dict(softmax_scale=float("nan")),
    "scale inf": dict(softmax_scale=float("inf")),
    "head_dim zero": dict(head_dim=0),
    "too many heads": dict(heads_q=4097 * 2, heads_kv=2),
    "tile too large": dict(part_len=1 << 30, n_q_slots=4),
}


@pytest.mark.parametrize("name", sorted(INVALID_DESCS))
def test_tile_invalid_desc(lib, name):
    assert _tile(lib, _desc(**INVALID_DESCS[name])) == _lib.ERR_INVALID
    assert lib.mesh_attn_last_error()


def test_tile_null_and_misaligned(lib):
    d = _desc()
    assert _tile(lib, d, by_ref=False) == _lib.ERR_INVALID
    for field in ("q", "k", "v", "o", "lse"):
        assert _tile(lib, d, **{field: None}) == _lib.ERR_INVALID
    for field in ("q", "k", "v", "o"):
        assert _tile(lib, d, **{field: FAKE + 4}) == _lib.ERR_INVALID
        assert b"16-byte" in lib.mesh_attn_last_error()
    assert _tile(lib, d, lse=FAKE + 2) == _lib.ERR_INVALID
    assert b"4-byte" in lib.mesh_attn_last_error()


def test_tile_lse_needs_only_four_byte_alignment(lib):
    """A tile's lse may start at any float of a merge's [n, rows] lse array.
    The block list here is invalid, so the call fails validation after the
    pointer checks and nothing is launched: the error is the block's, not
    the pointer's."""
    bad = [(0, 0, 0, 0, 0), (0, 0, 0, 0, 0)]  # duplicated block
    for off in (4, 8, 12):
        assert _tile(lib, _desc(blocks=bad), lse=FAKE + off) == _lib.ERR_INVALID
        assert b"duplicated" in lib.mesh_attn_last_error()
        assert _bwd(lib, _desc(blocks=bad), lse=FAKE + off, delta=FAKE + 16 + off) == \
            _lib.ERR_INVALID
        assert b"duplicated" in lib.mesh_attn_last_error()


def test_tile_unsupported(lib):
    assert _tile(lib, _desc(head_dim=64)) == _lib.ERR_UNSUPPORTED        # bf16 d=64
    assert _tile(lib, _desc(dtype=_lib.F32, head_dim=96)) == _lib.ERR_UNSUPPORTED


def _bad_blocks():
    good = oracle.block_list_ref(2, 2, 0, 0, True, True)  # q parts {0,1}, kv parts [0, 2]
    cases = {}
    b = list(good)
    b[0] = (2,) + b[0][1:]
    cases["q_slot out of range"] = b
    b = list(good)
    b[0] = (b[0][0], -1) + b[0][2:]
    cases["kv_slot negative"] = b
    b = list(good)
    b[1] = b[1][:4] + (3,)
    cases["kind out of range"] = b
    cases["duplicate block"] = good + [good[0]]
    b = list(good)
    b[2] = (b[2][0], b[2][1], 5, b[2][3], b[2][4])
    cases["q slot with two partitions"] = b
    b = list(good)
    b[1] = (b[1][0], b[1][1], b[1][2], 7, b[1][4])
    cases["kv slot with two partitions"] = b
    cases["diag on off-diagonal"] = [(0, 0, 0, 1, 1)]
    cases["two kv slots one partition"] = [(0, 0, 1, 0, 0), (0, 1, 1, 0, 0)]
    cases["two q slots one partition"] = [(0, 0, 1, 0, 0), (1, 0, 1, 0, 0)]
    cases["negative partition"] = [(0, 0, -1, 0, 0)]
    return cases


@pytest.mark.parametrize("name", sorted(_bad_blocks()))
def test_tile_invalid_blocks(lib, name):
    assert _tile(lib, _desc(blocks=_bad_blocks()[name])) == _lib.ERR_INVALID


def test_tile_too_many_blocks(lib):
    d = _desc()
    d.n_blocks = 1025
    assert _tile(lib, d) == _lib.ERR_INVALID
    d.n_blocks = 1
    d.blocks = None
    assert _tile(lib, d) == _lib.ERR_INVALID


# ----------------------------------------------------------------------------- lse_merge

def _merge(lib, n=4, rows=16, d=128, dtype=_lib.BF16, o=FAKE, l=FAKE, oo=FAKE, lo=FAKE):
    return lib.mesh_attn_lse_merge(n, rows, d, dtype, o, l, oo, lo, None)


@pytest.mark.parametrize("kw", [dict(n=0), dict(n=65), dict(rows=-1), dict(dtype=5), dict(d=0),
                                dict(d=12), dict(d=1024), dict(dtype=_lib.F32, d=6),
                                dict(o=None), dict(l=None), dict(oo=None), dict(o=FAKE + 8),
                                dict(oo=FAKE + 8), dict(l=FAKE + 2), dict(lo=FAKE + 1),
                                dict(rows=1 << 62)])
def test_merge_invalid(lib, kw):
    assert _merge(lib, **kw) == _lib.ERR_INVALID


def test_merge_zero_rows_is_a_noop(lib):
    assert _merge(lib, rows=0) == _lib.OK


# ----------------------------------------------------------------------------- backward

def _bwd(lib, desc, by_ref=True, **ptrs):
    names = ("q", "k", "v", "dout", "lse", "delta", "dq", "dk", "dv")
    args = [ptrs.get(n, FAKE) for n in names]
    return lib.mesh_attn_tile_bwd(ctypes.byref(desc) if by_ref else None, *args, None)


@pytest.mark.parametrize("name", sorted(INVALID_DESCS))
def test_tile_bwd_invalid_desc(lib, name):
    assert _bwd(lib, _desc(**INVALID_DESCS[name])) == _lib.ERR_INVALID
    assert lib.mesh_attn_last_error().startswith(b"tile_bwd")


@pytest.mark.parametrize("name", sorted(_bad_blocks()))
def test_tile_bwd_invalid_blocks(lib, name):
    assert _bwd(lib, _desc(blocks=_bad_blocks()[name])) == _lib.ERR_INVALID


def test_tile_bwd_null_misaligned_unsupported(lib):
    d = _desc()
    assert _bwd(lib, d, by_ref=False) == _lib.ERR_INVALID
    for field in ("q", "k", "v", "dout", "lse", "delta", "dq", "dk", "dv"):
        assert _bwd(lib, d, **{field: None}) == _lib.ERR_INVALID
    for field in ("q", "k", "v", "dout", "dq", "dk", "dv"):
        assert _bwd(lib, d, **{field: FAKE + 4}) == _lib.ERR_INVALID
    for field in ("lse", "delta"):
        assert _bwd(lib, d, **{field: FAKE + 2}) == _lib.ERR_INVALID
        assert b"4-byte" in lib.mesh_attn_last_error()
    assert _bwd(lib, _desc(head_dim=64)) == _lib.ERR_UNSUPPORTED
    assert _bwd(lib, _desc(dtype=_lib.F32)) == _lib.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(rows=-1), dict(dtype=5), dict(d=0), dict(d=12), dict(d=1024),
                                dict(dtype=_lib.F32, d=6), dict(o=None), dict(do=None),
                                dict(out=None), dict(o=FAKE + 8), dict(do=FAKE + 8),
                                dict(out=FAKE + 2), dict(rows=1 << 62)])
def test_bwd_delta_invalid(lib, kw):
    a = dict(rows=16, d=128, dtype=_lib.BF16, o=FAKE, do=FAKE, out=FAKE)
    a.update(kw)
    assert lib.mesh_attn_bwd_delta(a["rows"], a["d"], a["dtype"], a["o"], a["do"], a["out"],
                                   None) == _lib.ERR_INVALID


def test_bwd_delta_zero_rows_is_a_noop(lib):
    assert lib.mesh_attn_bwd_delta(0, 128, _lib.BF16, FAKE, FAKE, FAKE, None) == _lib.OK


# ----------------------------------------------------------------------------- threads

THREAD_CASES = [
    (dict(dtype=7), b"tile_fwd: unknown dtype"),
    (dict(part_len=0), b"tile_fwd: part_len must be >= 1"),
    (dict(heads_q=3, heads_kv=2), b"tile_fwd: heads_q must be a positive multiple of heads_kv"),
    (dict(softmax_scale=-1.0), b"tile_fwd: softmax_scale must be finite and > 0"),
]


def test_calls_are_thread_safe(lib):
    """Threads calling at once (ctypes drops the GIL around each call): every
    thread reads back its own last error, a successful block_list clears it,
    and the block lists computed concurrently equal the oracle's."""
    import threading
    meshes = [(4, 4, 2, 2), (8, 8, 4, 4), (16, 4, 8, 2), (3, 5, 1, 4)]
    want = {m: oracle.block_list_ref(*m, True, True) for m in meshes}
    failures = []
    start = threading.Barrier(8)

    def work(t):
        kw, msg = THREAD_CASES[t % len(THREAD_CASES)]
        m = meshes[t % len(meshes)]
        desc = _desc(**kw)
        start.wait()
        for it in range(300):
            if _tile(lib, desc) != _lib.ERR_INVALID:
                failures.append((t, it, "status"))
            err = lib.mesh_attn_last_error()
            if err != msg:
                failures.append((t, it, err))
            if _lib_block_list(lib, *m, 1, 1) != want[m]:
                failures.append((t, it, "block list"))
            if lib.mesh_attn_last_error() != b"":
                failures.append((t, it, "not cleared"))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not failures, failures[:5]


def test_binding_constants_match_the_header():
    """The limits the binding mirrors are the header's #defines."""
    text = open(os.path.join(ROOT, "include", "mesh_attn.h")).read()
    defines = dict(re.findall(r"#define MESH_ATTN_(MAX_\w+) (\d+)", text))
    assert set(defines) == {"MAX_Q_SLOTS", "MAX_KV_SLOTS", "MAX_BLOCKS", "MAX_HEADS"}
    for name, value in defines.items():
        assert getattr(_lib, name) == int(value), name
