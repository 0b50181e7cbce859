"""ctypes declarations of the C ABI in include/mesh_attn.h.

Loading the library needs only the HIP runtime shared library, not a GPU.
There is no fallback: if libmeshattn.so has not been built, loading fails
with an error that says how to build it.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmeshattn.so")

OK = 0
ERR_INVALID = -1
ERR_CAPACITY = -2
ERR_UNSUPPORTED = -3
ERR_HIP = -4

BF16 = 0
F32 = 1

FULL = 0
DIAG = 1
SKIP = 2

COMM_NONE = 0
COMM_RECV_Q = 1
COMM_RECV_KV = 2
COMM_SEND_O = 3

MAX_Q_SLOTS = 64
MAX_KV_SLOTS = 64
MAX_BLOCKS = 1024
MAX_HEADS = 4096

# Every symbol include/mesh_attn.h declares.
EXPORTS = ("mesh_attn_block_list", "mesh_attn_tile_fwd", "mesh_attn_lse_merge",
           "mesh_attn_bwd_delta", "mesh_attn_tile_bwd", "mesh_attn_plan",
           "mesh_attn_status_string", "mesh_attn_last_error", "mesh_attn_version")


class Block(ctypes.Structure):
    _fields_ = [("q_slot", ctypes.c_int32), ("kv_slot", ctypes.c_int32),
                ("q_part", ctypes.c_int32), ("kv_part", ctypes.c_int32),
                ("kind", ctypes.c_int32)]


class TileDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("part_len", ctypes.c_int32),
                ("n_q_slots", ctypes.c_int32), ("n_kv_slots", ctypes.c_int32),
                ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("blocks", ctypes.POINTER(Block)), ("n_blocks", ctypes.c_int32)]


class PlanCosts(ctypes.Structure):
    _fields_ = [("recv_q_s", ctypes.c_double), ("recv_kv_s", ctypes.c_double),
                ("send_o_s", ctypes.c_double), ("full_block_s", ctypes.c_double),
                ("diag_block_s", ctypes.c_double), ("delay", ctypes.c_int32)]


class PlanStep(ctypes.Structure):
    _fields_ = [("comm", ctypes.c_int32), ("slot", ctypes.c_int32),
                ("block_begin", ctypes.c_int32), ("block_count", ctypes.c_int32),
                ("comm_s", ctypes.c_double), ("compute_s", ctypes.c_double),
                ("start_s", ctypes.c_double), ("end_s", ctypes.c_double)]


_LIB = None


def load():
    """The loaded library (cached).  Raises RuntimeError if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m long_context_distributed_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.mesh_attn_block_list.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(Block), i32,
                                         ctypes.POINTER(i32)]
    lib.mesh_attn_block_list.restype = ctypes.c_int
    lib.mesh_attn_tile_fwd.argtypes = [ctypes.POINTER(TileDesc), vp, vp, vp, vp, vp, vp]
    lib.mesh_attn_tile_fwd.restype = ctypes.c_int
    lib.mesh_attn_lse_merge.argtypes = [i32, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.mesh_attn_lse_merge.restype = ctypes.c_int
    lib.mesh_attn_bwd_delta.argtypes = [i64, i32, i32, vp, vp, vp, vp]
    lib.mesh_attn_bwd_delta.restype = ctypes.c_int
    lib.mesh_attn_tile_bwd.argtypes = [ctypes.POINTER(TileDesc)] + [vp] * 10
    lib.mesh_attn_tile_bwd.restype = ctypes.c_int
    lib.mesh_attn_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(PlanCosts),
                                   ctypes.POINTER(PlanStep), i32, ctypes.POINTER(i32),
                                   ctypes.POINTER(Block), i32, ctypes.POINTER(i32)]
    lib.mesh_attn_plan.restype = ctypes.c_int
    lib.mesh_attn_status_string.argtypes = [ctypes.c_int]
    lib.mesh_attn_status_string.restype = ctypes.c_char_p
    lib.mesh_attn_last_error.argtypes = []
    lib.mesh_attn_last_error.restype = ctypes.c_char_p
    lib.mesh_attn_version.argtypes = []
    lib.mesh_attn_version.restype = i32
    _LIB = lib
    return lib
