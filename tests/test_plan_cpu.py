"""The library's greedy planner (mesh_attn_plan) on the CPU: bit-exact equal
to the oracle's plan (same transfers, same blocks in the same order, same
simulated times), the oracle's pins applied to it directly, its size query
and every validation error."""
import ctypes
import itertools
import math

import pytest

import long_context_distributed_amd as mat
import oracle
from long_context_distributed_amd import _lib
from tests import schedule_pins as pins


def lib_plan(R, C, r, c, causal, rot, costs, delay=True):
    return mat.plan(R, C, r, c, causal, rot, costs, delay)


def _same(a, b):
    assert len(a) == len(b), (len(a), len(b))
    for x, y in zip(a, b):
        assert (x["comm"], x["slot"]) == (y["comm"], y["slot"])
        assert [tuple(t) for t in x["blocks"]] == [tuple(t) for t in y["blocks"]]
        for key in ("comm_s", "compute_s", "start_s", "end_s"):
            assert x[key] == y[key], (key, x[key], y[key])


COSTS = list(pins.REGIMES.values()) + [
    dict(recv_q_s=0.0123, recv_kv_s=0.0061, send_o_s=0.0131, full_block_s=0.0037, diag_block_s=0.0019),
    dict(recv_q_s=0.0, recv_kv_s=0.0, send_o_s=0.0, full_block_s=1.0, diag_block_s=0.5),
]


def test_bit_exact_all_tiles_up_to_6x6():
    for R, C in itertools.product(range(1, 7), repeat=2):
        for r, c in itertools.product(range(R), range(C)):
            for causal, rot in itertools.product((False, True), repeat=2):
                for i, costs in enumerate(COSTS):
                    delay = i % 2 == 0
                    _same(lib_plan(R, C, r, c, causal, rot, costs, delay),
                          oracle.greedy_plan_ref(R, C, r, c, causal, rot, costs, delay))


@pytest.mark.parametrize("R,C", [(8, 8), (16, 4), (4, 16), (13, 7), (64, 1), (1, 64)])
def test_bit_exact_larger_meshes(R, C):
    for r, c in {(0, 0), (R // 2, C // 2), (R - 1, C - 1), (R - 1, 0), (1 % R, C - 1)}:
        for causal, rot in itertools.product((False, True), repeat=2):
            for costs in COSTS[:4]:
                for delay in (True, False):
                    _same(lib_plan(R, C, r, c, causal, rot, costs, delay),
                          oracle.greedy_plan_ref(R, C, r, c, causal, rot, costs, delay))


@pytest.mark.parametrize("R,C", [(2, 2), (3, 3), (4, 4), (8, 8), (16, 4)])
def test_pins_hold_for_the_library(R, C):
    for r, c in itertools.product(range(R), range(C)):
        for causal, rot in itertools.product((False, True), repeat=2):
            for costs in pins.REGIMES.values():
                pins.check_plan_valid(lib_plan, R, C, r, c, causal, rot, costs)
                pins.check_transfer_choice(lib_plan, R, C, r, c, causal, rot, costs)
                pins.check_delay_rule(lib_plan, R, C, r, c, causal, rot, costs)
    pins.check_ring_closed_form(lib_plan)


def test_library_against_exhaustive_optimum():
    mean, worst, _ = pins.check_against_optimum(lib_plan, oracle.optimal_makespan_ref)
    assert mean <= 1.02 and worst <= 1.2


def _raw(lib, R=2, C=2, r=0, c=0, causal=1, rot=1, costs=None, steps=None, scap=0, n_steps=True,
         order=None, ocap=0, n_order=True):
    ns, no = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = lib.mesh_attn_plan(R, C, r, c, causal, rot, ctypes.byref(costs) if costs is not None else None,
                            steps, scap, ctypes.byref(ns) if n_steps else None,
                            order, ocap, ctypes.byref(no) if n_order else None)
    return st, ns.value, no.value


def _costs(**kw):
    base = dict(recv_q_s=1.0, recv_kv_s=1.0, send_o_s=1.0, full_block_s=1.0, diag_block_s=0.5, delay=1)
    base.update(kw)
    return _lib.PlanCosts(base["recv_q_s"], base["recv_kv_s"], base["send_o_s"], base["full_block_s"],
                          base["diag_block_s"], base["delay"])


def test_size_query_and_capacity(lib):
    st, ns, no = _raw(lib, R=4, C=4, r=2, c=2, costs=_costs())
    assert st == _lib.ERR_CAPACITY and ns > 0 and no == 10  # 9 FULL + 1 DIAG blocks
    steps = (_lib.PlanStep * ns)()
    order = (_lib.Block * no)()
    st2, _, _ = _raw(lib, R=4, C=4, r=2, c=2, costs=_costs(), steps=steps, scap=ns - 1, order=order,
                     ocap=no)
    assert st2 == _lib.ERR_CAPACITY
    st3, ns3, no3 = _raw(lib, R=4, C=4, r=2, c=2, costs=_costs(), steps=steps, scap=ns, order=order,
                         ocap=no)
    assert st3 == _lib.OK and (ns3, no3) == (ns, no)
    assert lib.mesh_attn_last_error() == b""
    # a tile with no work and no transfer has an empty plan; NULL arrays still make a size query
    st4, ns4, no4 = _raw(lib, R=2, C=2, r=0, c=1, rot=0, costs=_costs())
    assert (ns4, no4) == (0, 0) and st4 == _lib.ERR_CAPACITY


@pytest.mark.parametrize("kw", [
    dict(costs=None), dict(n_steps=False), dict(n_order=False),
    dict(costs=_costs(recv_q_s=-1.0)), dict(costs=_costs(full_block_s=math.nan)),
    dict(costs=_costs(send_o_s=math.inf)), dict(costs=_costs(delay=2)),
    dict(R=65, C=1), dict(R=1, C=65), dict(R=0), dict(r=2), dict(c=-1),
])
def test_invalid_arguments(lib, kw):
    a = dict(costs=_costs())
    a.update(kw)
    st, _, _ = _raw(lib, **a)
    assert st == _lib.ERR_INVALID
    assert lib.mesh_attn_last_error()
