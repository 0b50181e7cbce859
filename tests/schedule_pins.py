"""Checks that pin a schedule planner (the oracle's or the library's) to the
rules it follows and to facts of the step model, independently of its own
code: validity of the plan, the greedy choice of each transfer recounted
from the plan's history, the compute-delay rule, the ring's closed form, and
the exhaustive optimum.

Each check takes ``plan(R, C, r, c, causal, rot, costs, delay=True)``
returning a list of step dicts (comm, slot, blocks, comm_s, compute_s,
start_s, end_s) and raises AssertionError on a violation.
"""
import itertools
import math

FULL, DIAG, SKIP = 0, 1, 2
NONE, RECV_Q, RECV_KV, SEND_O = 0, 1, 2, 3

REGIMES = {
    "comm-bound": dict(recv_q_s=4.0, recv_kv_s=4.0, send_o_s=4.0, full_block_s=1.0, diag_block_s=0.5),
    "balanced": dict(recv_q_s=1.0, recv_kv_s=1.0, send_o_s=1.0, full_block_s=1.0, diag_block_s=0.5),
    "compute-bound": dict(recv_q_s=0.25, recv_kv_s=0.5, send_o_s=0.25, full_block_s=1.0,
                          diag_block_s=0.5),
    "gqa": dict(recv_q_s=1.0, recv_kv_s=0.5, send_o_s=1.0, full_block_s=0.75, diag_block_s=0.375),
    "mixed": dict(recv_q_s=2.0, recv_kv_s=1.0, send_o_s=2.5, full_block_s=1.5, diag_block_s=0.75),
}


def _geometry(R, C, r, c, causal, rot):
    """Q and KV partitions of the tile and its non-SKIP blocks, straight from
    the definitions (mesh row for Q; the column, rotated or contiguous, for
    KV; the causal class from partition order)."""
    q_part = [r * C + t for t in range(C)]
    kv_part = [((r + k) % R) * C + c for k in range(R)] if rot else [c * R + k for k in range(R)]
    need = {}
    for j, kp in enumerate(kv_part):
        for s, qp in enumerate(q_part):
            kind = FULL if (not causal or kp < qp) else (DIAG if kp == qp else SKIP)
            if kind != SKIP:
                need[(s, j)] = kind
    return q_part, kv_part, need


def check_plan_valid(plan, R, C, r, c, causal, rot, costs, delay=True):
    """Every needed receive once and no other; every non-SKIP block once, and
    only once both its partitions are present (held from the start or
    received in an earlier step); each remote row's partial sent once, after
    its row is complete; step durations max(transfer, compute) and chained."""
    steps = plan(R, C, r, c, causal, rot, costs, delay)
    q_part, kv_part, need = _geometry(R, C, r, c, causal, rot)
    g = r * C + c
    q_have = [p == g for p in q_part]
    kv_have = [p == g for p in kv_part]
    rows = {s for s, _ in need}
    cols = {j for _, j in need}
    want_q = {s for s in rows if not q_have[s]}
    want_kv = {j for j in cols if not kv_have[j]}
    want_send = {s for s in rows if q_part[s] != g}
    got_q, got_kv, got_send, done = [], [], [], set()
    t = 0.0
    for st in steps:
        for b in st["blocks"]:
            s, j = b[0], b[1]
            assert (s, j) in need, f"block {b} is SKIP or outside the tile"
            assert b[2] == q_part[s] and b[3] == kv_part[j] and b[4] == need[(s, j)], b
            assert (s, j) not in done, f"block {b} computed twice"
            assert q_have[s] and kv_have[j], f"block {b} computed before its data arrived"
            done.add((s, j))
        comp = 0.0
        for b in st["blocks"]:
            comp += costs["full_block_s"] if b[4] == FULL else costs["diag_block_s"]
        assert math.isclose(st["compute_s"], comp, rel_tol=1e-12, abs_tol=1e-15)
        kind, slot = st["comm"], st["slot"]
        want_c = {NONE: 0.0, RECV_Q: costs["recv_q_s"], RECV_KV: costs["recv_kv_s"],
                  SEND_O: costs["send_o_s"]}[kind]
        assert st["comm_s"] == want_c
        if kind == NONE:
            assert slot == -1 and st["blocks"], "empty step"
        elif kind == RECV_Q:
            got_q.append(slot)
        elif kind == RECV_KV:
            got_kv.append(slot)
        else:
            row = {k for k in need if k[0] == slot}
            assert row <= done - {(b[0], b[1]) for b in st["blocks"]}, \
                f"partial of Q slot {slot} sent before its row was complete"
            got_send.append(slot)
        assert math.isclose(st["start_s"], t, rel_tol=1e-12, abs_tol=1e-12)
        t = t + max(st["comm_s"], st["compute_s"])
        assert math.isclose(st["end_s"], t, rel_tol=1e-12, abs_tol=1e-12)
        # data of this step's receive is usable from the next step on
        if kind == RECV_Q:
            q_have[slot] = True
        elif kind == RECV_KV:
            kv_have[slot] = True
    assert sorted(got_q) == sorted(want_q) and len(got_q) == len(set(got_q)), "Q receives"
    assert sorted(got_kv) == sorted(want_kv) and len(got_kv) == len(set(got_kv)), "KV receives"
    assert sorted(got_send) == sorted(want_send) and len(got_send) == len(set(got_send)), "sends"
    assert done == set(need), "not every non-SKIP block computed"
    return steps


def check_transfer_choice(plan, R, C, r, c, causal, rot, costs):
    """Rule 1 recounted from the plan's own history: each receive made
    computable at least as many blocks as any other pending receive would
    have, and sends come only when no pending receive would unlock a block."""
    steps = plan(R, C, r, c, causal, rot, costs, True)
    q_part, kv_part, need = _geometry(R, C, r, c, causal, rot)
    g = r * C + c
    q_have = [p == g for p in q_part]
    kv_have = [p == g for p in kv_part]
    pending = {(RECV_Q, s) for s, _ in need if not q_have[s]} | \
              {(RECV_KV, j) for _, j in need if not kv_have[j]}

    def unlocks(op):
        kind, slot = op
        if kind == RECV_KV:
            return sum(1 for (s, j) in need if j == slot and q_have[s])
        return sum(1 for (s, j) in need if s == slot and kv_have[j])

    for st in steps:
        op = (st["comm"], st["slot"])
        if op[0] in (RECV_Q, RECV_KV):
            assert op in pending
            best = max(unlocks(o) for o in pending)
            assert unlocks(op) == best, f"receive {op} unlocks {unlocks(op)} < {best}"
            pending.discard(op)
            if op[0] == RECV_Q:
                q_have[op[1]] = True
            else:
                kv_have[op[1]] = True
        elif op[0] == SEND_O and pending:
            assert max(unlocks(o) for o in pending) == 0, "send taken while a receive unlocks work"
        elif op[0] == NONE:
            assert not pending, "a step without a transfer while receives are pending"


def check_delay_rule(plan, R, C, r, c, causal, rot, costs):
    """Rule 2: a step with a transfer computes just enough ready blocks to
    cover it: its compute covers the transfer unless it took every ready
    block, and without its last block it would not cover it."""
    steps = plan(R, C, r, c, causal, rot, costs, True)
    q_part, kv_part, need = _geometry(R, C, r, c, causal, rot)
    g = r * C + c
    q_have = [p == g for p in q_part]
    kv_have = [p == g for p in kv_part]
    done = set()
    for st in steps:
        ready = {k for k in need if k not in done and q_have[k[0]] and kv_have[k[1]]}
        blocks = [(b[0], b[1]) for b in st["blocks"]]
        if st["comm"] != NONE:
            if st["compute_s"] < st["comm_s"]:
                assert set(blocks) == ready, "transfer left uncovered while ready blocks wait"
            if blocks:
                last = st["blocks"][-1]
                t_last = costs["full_block_s"] if last[4] == FULL else costs["diag_block_s"]
                assert st["compute_s"] - t_last < st["comm_s"], "more compute than the transfer needs"
        done.update(blocks)
        if st["comm"] == RECV_Q:
            q_have[st["slot"]] = True
        elif st["comm"] == RECV_KV:
            kv_have[st["slot"]] = True


def check_ring_closed_form(plan):
    """A C = 1 mesh is Ring-Attention: one Q partition, all KV partitions in
    rotation.  Non-causal, the plan is the ring's 'compute one step,
    transfer one step' and its makespan is (R-1) max(t_kv, t_block) +
    t_block, which is also the least any schedule can take (R-1 receives
    in sequence, each block after its data, the last one after all)."""
    for R in (2, 3, 5, 8):
        for tkv, tb in [(1.0, 1.0), (3.0, 1.0), (0.5, 2.0)]:
            costs = dict(recv_q_s=9.0, recv_kv_s=tkv, send_o_s=9.0, full_block_s=tb, diag_block_s=tb / 2)
            steps = plan(R, 1, 0, 0, False, True, costs, True)
            assert [(s["comm"], s["slot"]) for s in steps] == \
                [(RECV_KV, j) for j in range(1, R)] + [(NONE, -1)]
            assert [[(b[0], b[1]) for b in s["blocks"]] for s in steps] == [[(0, j)] for j in range(R)]
            assert math.isclose(steps[-1]["end_s"], (R - 1) * max(tkv, tb) + tb, rel_tol=1e-12)


def check_one_by_two_optimum(optimal):
    """Pin of the exhaustive search by a case solved by hand: a 1 x 2 mesh,
    tile (0,0), non-causal.  The GPU holds Q0 and KV0; it must receive Q1,
    compute (1,0) after that, and then send row 1's partial; block (0,0)
    can go beside the receive or beside the send.  Optimum:
    min(max(tq, tb) + tb + to, tq + tb + max(to, tb))."""
    for tq, to, tb in [(1.0, 1.0, 1.0), (2.0, 1.0, 1.0), (1.0, 3.0, 2.0), (0.5, 0.5, 2.0),
                       (3.0, 0.25, 1.0)]:
        costs = dict(recv_q_s=tq, recv_kv_s=7.0, send_o_s=to, full_block_s=tb, diag_block_s=tb)
        want = min(max(tq, tb) + tb + to, tq + tb + max(to, tb))
        assert math.isclose(optimal(1, 2, 0, 0, False, True, costs), want, rel_tol=1e-12), (tq, to, tb)


def check_against_optimum(plan, optimal, meshes=((2, 2), (2, 3), (3, 2), (3, 3), (1, 3), (3, 1)),
                          bound=1.2):
    """On every tile of tiny meshes: the exhaustive optimum is at most the
    greedy plan's makespan, which is at most the eager variant's and within
    `bound` of the optimum; the optimum is at least the busier resource's
    total.  Returns (mean ratio, worst ratio, cases where delay helps)."""
    ratios, helped = [], 0
    for R, C in meshes:
        for r, c in itertools.product(range(R), range(C)):
            for causal, rot in itertools.product((False, True), repeat=2):
                for costs in REGIMES.values():
                    steps = plan(R, C, r, c, causal, rot, costs, True)
                    eager = plan(R, C, r, c, causal, rot, costs, False)
                    gm = steps[-1]["end_s"] if steps else 0.0
                    em = eager[-1]["end_s"] if eager else 0.0
                    opt = optimal(R, C, r, c, causal, rot, costs)
                    comm = sum(s["comm_s"] for s in steps)
                    comp = sum(s["compute_s"] for s in steps)
                    assert opt >= max(comm, comp) - 1e-12, "optimum below the busier resource's total"
                    assert opt <= gm + 1e-12, "greedy plan beats the exhaustive optimum"
                    assert gm <= em + 1e-12, "delaying compute made the plan longer"
                    helped += gm < em - 1e-12
                    if opt == 0:
                        assert gm == 0
                        continue
                    ratios.append(gm / opt)
                    assert gm <= bound * opt + 1e-12, (R, C, r, c, causal, rot, costs, gm, opt)
    return sum(ratios) / len(ratios), max(ratios), helped
