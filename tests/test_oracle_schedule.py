"""Pins of the schedule oracle (CPU only): validity of its plans, the two
greedy rules recounted from each plan, the ring's closed form, a hand-solved
optimum, the exhaustive optimum, and planted mistakes that the checks must
catch."""
import importlib.util
import itertools
import os
import sys

import pytest

import oracle
from tests import schedule_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def plan(R, C, r, c, causal, rot, costs, delay=True):
    return oracle.greedy_plan_ref(R, C, r, c, causal, rot, costs, delay)


MESHES = [(1, 1), (2, 2), (2, 3), (3, 2), (3, 3), (4, 4), (1, 5), (5, 1), (8, 8), (16, 4), (4, 16)]


@pytest.mark.parametrize("R,C", MESHES)
def test_plans_are_valid(R, C):
    tiles = list(itertools.product(range(R), range(C)))
    if len(tiles) > 12:
        tiles = tiles[::max(1, len(tiles) // 12)]
    for (r, c), causal, rot in itertools.product(tiles, (False, True), (False, True)):
        for costs in pins.REGIMES.values():
            for delay in (True, False):
                pins.check_plan_valid(plan, R, C, r, c, causal, rot, costs, delay)


@pytest.mark.parametrize("R,C", MESHES)
def test_greedy_rules_hold(R, C):
    tiles = list(itertools.product(range(R), range(C)))
    if len(tiles) > 12:
        tiles = tiles[::max(1, len(tiles) // 12)]
    for (r, c), causal, rot in itertools.product(tiles, (False, True), (False, True)):
        for costs in pins.REGIMES.values():
            pins.check_transfer_choice(plan, R, C, r, c, causal, rot, costs)
            pins.check_delay_rule(plan, R, C, r, c, causal, rot, costs)


def test_ring_closed_form():
    pins.check_ring_closed_form(plan)


def test_exhaustive_optimum_hand_solved_case():
    pins.check_one_by_two_optimum(oracle.optimal_makespan_ref)


def test_one_gpu_mesh():
    costs = pins.REGIMES["balanced"]
    assert oracle.optimal_makespan_ref(1, 1, 0, 0, True, True, costs) == costs["diag_block_s"]
    steps = plan(1, 1, 0, 0, True, True, costs)
    assert len(steps) == 1 and steps[0]["comm"] == pins.NONE
    assert steps[0]["end_s"] == costs["diag_block_s"]


def test_greedy_against_exhaustive_optimum():
    """Greedy within 1.2x of the optimum on every tile of meshes up to 3x3
    in five cost regimes, on average within 2%; holding compute back (rule
    2) never lengthens a plan and shortens many."""
    mean, worst, helped = pins.check_against_optimum(plan, oracle.optimal_makespan_ref)
    assert mean <= 1.02 and worst <= 1.2
    assert helped >= 100


# --------------------------------------------------------------------------- planted mistakes

def _mutant(replacements):
    """A copy of oracle/schedule.py with source replacements applied."""
    path = os.path.join(ROOT, "oracle", "schedule.py")
    src = open(path).read()
    for old, new in replacements:
        assert old in src, old
        src = src.replace(old, new)
    src = src.replace("from .block_list import", "from oracle.block_list import")
    spec = importlib.util.spec_from_loader("schedule_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, "schedule_mutant", "exec"), mod.__dict__)
    return mod


MUTANTS = {
    "transfer that unlocks the fewest blocks": [("key=lambda o: (-unlocks(o)", "key=lambda o: (unlocks(o)")],
    "every ready block at once": [("        if not delay:\n            chosen = ready",
                                   "        if True:\n            chosen = ready")],
    "send before the row is complete": [("ready_sends = [s for s in sends if row_left(s) == 0]",
                                         "ready_sends = list(sends)")],
    "data used in the step it arrives": [
        ("        ready = [b for b in need if (b[0], b[1]) not in done and q_present[b[0]] and kv_present[b[1]]]",
         "        if op[0] == RECV_KV:\n            kv_present[op[1]] = True\n"
         "        if op[0] == RECV_Q:\n            q_present[op[1]] = True\n"
         "        ready = [b for b in need if (b[0], b[1]) not in done and q_present[b[0]] and kv_present[b[1]]]")],
    "local partitions received again": [("if not kv_present[j]]", "]")],
    "more compute than the transfer needs": [("                if acc >= comm_s:\n                    break",
                                              "                if acc > 2 * comm_s:\n                    break")],
}

OPT_MUTANTS = {
    "optimum without sends": [("          [(SEND_O, s) for s in sorted({b[0] for b in need}) if q_part[s] != g]",
                               "          []")],
    "optimum with sends before rows complete": [("                if not all(comp >> k & 1 for k in row):",
                                                  "                if False:")],
}


def _caught_plan(mod):
    def p(R, C, r, c, causal, rot, costs, delay=True):
        return mod.greedy_plan_ref(R, C, r, c, causal, rot, costs, delay)
    checks = []
    for R, C in [(2, 2), (3, 3), (4, 4), (3, 2)]:
        for r, c in itertools.product(range(R), range(C)):
            for causal, rot in itertools.product((False, True), repeat=2):
                for costs in pins.REGIMES.values():
                    checks.append(lambda a=(R, C, r, c, causal, rot, costs): pins.check_plan_valid(p, *a))
                    checks.append(lambda a=(R, C, r, c, causal, rot, costs): pins.check_transfer_choice(p, *a))
                    checks.append(lambda a=(R, C, r, c, causal, rot, costs): pins.check_delay_rule(p, *a))
    checks.append(lambda: pins.check_ring_closed_form(p))
    failures = 0
    for chk in checks:
        try:
            chk()
        except (AssertionError, RuntimeError, ValueError, KeyError):
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_plan_mutant_is_caught(name):
    assert _caught_plan(_mutant(MUTANTS[name])) > 0, name


@pytest.mark.parametrize("name", sorted(OPT_MUTANTS))
def test_optimum_mutant_is_caught(name):
    mod = _mutant(OPT_MUTANTS[name])
    caught = 0
    for chk in (lambda: pins.check_one_by_two_optimum(mod.optimal_makespan_ref),
                lambda: pins.check_against_optimum(plan, mod.optimal_makespan_ref,
                                                   meshes=((2, 2), (1, 3)), bound=10.0)):
        try:
            chk()
        except AssertionError:
            caught += 1
    assert caught > 0, name


def test_real_oracle_passes_the_mutant_checks():
    assert _caught_plan(_mutant([])) == 0
