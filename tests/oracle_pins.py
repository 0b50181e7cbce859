"""Checks that pin the oracle to facts other than itself.

Each ``check_*`` takes the oracle functions it exercises as arguments, so the
same checks run against the real oracle (``test_oracle_*.py``) and against
planted mistakes (``test_oracle_mutations.py``), which must each fail at least
one check.  Every check raises AssertionError on failure.

Sources of truth used here, none of which is the oracle's own formula:

* torch's scaled_dot_product_attention (CPU, float64) and scipy's logsumexp
  / numpy's logaddexp - library routines for the whole-matrix special case;
* closed forms: Q = 0 gives the mean of the visible values and lse = ln(count);
  one visible key gives O = v and lse = its score; equal lse merges are means;
* invariants: affine equivariance in V, permutation of keys, head grouping,
  split-then-merge equals the unsplit result;
* brute force in pure Python (math.exp / math.fsum, no max shift) on tiny
  inputs;
* mesh facts: tiles partition the matrix, row/column-only peers, a GPU's own
  block is in its tile, rotation steps are permutations, block counts in
  closed form.
"""

import itertools
import math

import numpy as np

FULL, DIAG, SKIP = 0, 1, 2


def _rng(seed):
    return np.random.default_rng(seed)


def _positions(parts, L):
    return np.concatenate([np.arange(p * L, (p + 1) * L) for p in parts]) if len(parts) else \
        np.zeros((0,), dtype=np.int64)


# --------------------------------------------------------------------------- attention

def check_sdpa(attention, causal, hq=4, hkv=2, nq=9, nk=9, d=16, seed=0):
    """Whole contiguous matrix: equals torch SDPA (float64, CPU math path)."""
    import torch
    import torch.nn.functional as F
    r = _rng(seed)
    q = r.standard_normal((nq, hq, d))
    k = r.standard_normal((nk, hkv, d))
    v = r.standard_normal((nk, hkv, d))
    scale = 1.0 / math.sqrt(d)
    pos = np.arange(nq)
    o, lse = attention(q, k, v, pos, np.arange(nk), causal, scale)
    g = hq // hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)[None].contiguous()
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)[None].contiguous()
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12), "output differs from torch SDPA"
    # lse against scipy's logsumexp of the masked scaled scores
    from scipy.special import logsumexp
    for i in range(nq):
        for h in range(hq):
            s = scale * (k[:, h // g, :] @ q[i, h, :])
            if causal:
                s = s[:i + 1]
            assert abs(lse[i, h] - logsumexp(s)) < 1e-12, "lse differs from scipy logsumexp"


def check_zero_query(attention, L=5, q_parts=(1, 2), kv_parts=(2, 0, 3, 1), hq=2, hkv=1, d=8,
                     seed=1):
    """Q = 0: every visible score is 0, so O = mean of the visible values and
    lse = ln(count); the count is n_before*L + (u+1 when the own partition is
    in the KV set), which pins the causal rule exactly."""
    r = _rng(seed)
    nq, nk = len(q_parts) * L, len(kv_parts) * L
    q = np.zeros((nq, hq, d))
    k = r.standard_normal((nk, hkv, d))
    v = r.standard_normal((nk, hkv, d))
    qp, kp = _positions(q_parts, L), _positions(kv_parts, L)
    o, lse = attention(q, k, v, qp, kp, True, 0.125)
    g = hq // hkv
    for s, part in enumerate(q_parts):
        n_before = sum(1 for x in kv_parts if x < part)
        own = part in kv_parts
        for u in range(L):
            count = n_before * L + (u + 1 if own else 0)
            i = s * L + u
            for h in range(hq):
                if count == 0:
                    assert lse[i, h] == -np.inf and np.all(o[i, h] == 0), "empty row not (0, -inf)"
                    continue
                assert abs(lse[i, h] - math.log(count)) < 1e-12, "lse != ln(visible count)"
                vis = kp <= qp[i]
                mean = v[vis, h // g, :].mean(axis=0)
                assert np.allclose(o[i, h], mean, atol=1e-12), "Q=0 output != mean of visible V"


def check_single_key(attention, d=8, seed=2):
    """A query that sees exactly one key gets that key's value and score."""
    r = _rng(seed)
    q = r.standard_normal((1, 1, d))
    k = r.standard_normal((4, 1, d))
    v = r.standard_normal((4, 1, d))
    scale = 0.3
    o, lse = attention(q, k, v, np.array([10]), np.array([10, 11, 12, 13]), True, scale)
    assert np.allclose(o[0, 0], v[0, 0], atol=1e-14), "single visible key: O != v"
    assert abs(lse[0, 0] - scale * float(q[0, 0] @ k[0, 0])) < 1e-13, "single key: lse != score"


def check_affine_values(attention, causal, seed=3):
    """O is affine-equivariant in V (rows of the softmax sum to one)."""
    r = _rng(seed)
    q = r.standard_normal((6, 2, 8))
    k = r.standard_normal((7, 2, 8))
    v = r.standard_normal((7, 2, 8))
    qp, kp = np.arange(3, 9), np.arange(0, 7)
    o1, l1 = attention(q, k, v, qp, kp, causal, 0.4)
    o2, l2 = attention(q, k, 2.5 * v - 0.75, qp, kp, causal, 0.4)
    assert np.allclose(o2, 2.5 * o1 - 0.75, atol=1e-12), "O not affine in V"
    assert np.array_equal(l1, l2), "lse depends on V"
    o3, _ = attention(q, k, np.ones_like(v), qp, kp, causal, 0.4)
    assert np.allclose(o3, 1.0, atol=1e-13), "softmax rows do not sum to one"


def check_gqa_mapping(attention, hq=8, hkv=2, seed=4):
    """Query head h reads KV head h // (hq/hkv): with V constant per KV head,
    O equals that constant."""
    r = _rng(seed)
    q = r.standard_normal((3, hq, 4))
    k = r.standard_normal((5, hkv, 4))
    v = np.broadcast_to(np.arange(hkv, dtype=np.float64)[None, :, None], (5, hkv, 4)).copy()
    o, _ = attention(q, k, v, np.arange(3), np.arange(5), False, 0.5)
    g = hq // hkv
    for h in range(hq):
        assert np.allclose(o[:, h, :], h // g, atol=1e-13), "wrong KV head for query head"


def check_brute_force(attention, causal, seed=5):
    """Pure-Python evaluation of the definition, without max subtraction."""
    r = _rng(seed)
    nq, nk, hq, hkv, d = 3, 4, 2, 1, 3
    q = r.standard_normal((nq, hq, d))
    k = r.standard_normal((nk, hkv, d))
    v = r.standard_normal((nk, hkv, d))
    qp, kp = np.array([2, 4, 5]), np.array([1, 2, 4, 6])
    scale = 0.7
    o, lse = attention(q, k, v, qp, kp, causal, scale)
    for i in range(nq):
        for h in range(hq):
            ws, idx = [], []
            for j in range(nk):
                if causal and kp[j] > qp[i]:
                    continue
                s = scale * math.fsum(float(q[i, h, t]) * float(k[j, 0, t]) for t in range(d))
                ws.append(math.exp(s))
                idx.append(j)
            tot = math.fsum(ws)
            assert abs(lse[i, h] - math.log(tot)) < 1e-12, "lse != brute force"
            for t in range(d):
                ref = math.fsum(w * float(v[j, 0, t]) for w, j in zip(ws, idx)) / tot
                assert abs(o[i, h, t] - ref) < 1e-12, "O != brute force"


def check_large_scores(attention, seed=6):
    """Scores near +-1e3 neither overflow nor lose the dominant key."""
    r = _rng(seed)
    d = 4
    k = 0.1 * r.standard_normal((6, 1, d))
    k[:, 0, 0] = [0.2, -0.5, 0.8, 1.0, 0.1, 0.95]
    v = r.standard_normal((6, 1, d))
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 400.0
    scale = 2.5  # scores 1000 * k[:, 0, 0]: 1000 for key 3, 950 next
    pos = np.zeros(6, dtype=np.int64)
    o, lse = attention(q, k, v, np.array([0]), pos, False, scale)
    s = scale * (k[:, 0, :] @ q[0, 0, :])
    assert np.all(np.isfinite(o)) and np.isfinite(lse[0, 0]), "overflow on large scores"
    m = s.max()
    ref_lse = m + math.log(math.fsum(math.exp(x - m) for x in s))
    assert abs(lse[0, 0] - ref_lse) < 1e-12 * abs(ref_lse), "large-score lse wrong"
    assert np.allclose(o[0, 0], v[3, 0], atol=1e-12), "dominant key lost"
    o2, lse2 = attention(-q, k, v, np.array([0]), pos, False, scale)
    assert np.all(np.isfinite(o2)) and np.isfinite(lse2[0, 0]), "underflow on negative scores"
    assert np.allclose(o2[0, 0], v[1, 0], atol=1e-12), "dominant key lost (negative q)"


def check_key_permutation(attention, seed=7):
    """Non-causal attention does not depend on key order."""
    r = _rng(seed)
    q = r.standard_normal((4, 2, 8))
    k = r.standard_normal((9, 2, 8))
    v = r.standard_normal((9, 2, 8))
    perm = r.permutation(9)
    o1, l1 = attention(q, k, v, np.arange(4), np.arange(9), False, 0.3)
    o2, l2 = attention(q, k[perm], v[perm], np.arange(4), np.arange(9)[perm], False, 0.3)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13), "order dependence"


def check_scale_on_scores(attention, seed=8):
    """The scale multiplies the scores: scale s on q equals scale 1 on s*q."""
    r = _rng(seed)
    q = r.standard_normal((4, 1, 8))
    k = r.standard_normal((6, 1, 8))
    v = r.standard_normal((6, 1, 8))
    o1, l1 = attention(q, k, v, np.arange(4), np.arange(6), True, 0.37)
    o2, l2 = attention(0.37 * q, k, v, np.arange(4), np.arange(6), True, 1.0)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13), "scale misplaced"


# --------------------------------------------------------------------------- merge

def check_merge_closed_forms(merge, seed=9):
    r = _rng(seed)
    o = r.standard_normal((3, 5, 4))
    lse = np.full((3, 5), 1.7)
    mo, ml = merge(o, lse)
    assert np.allclose(mo, o.mean(axis=0), atol=1e-14), "equal lse: merge != mean"
    assert np.allclose(ml, 1.7 + math.log(3), atol=1e-14), "equal lse: lse != lse+ln n"
    l1 = lse[:1] + r.standard_normal(5)
    mo, ml = merge(o[:1], l1)
    assert np.allclose(mo, o[0], atol=1e-15) and np.allclose(ml, l1[0], atol=1e-15), \
        "n=1 merge is not the identity"
    l2 = r.standard_normal((3, 5))
    l2[1, :] = -np.inf
    o_bad = o.copy()
    o_bad[1] = np.nan
    mo, ml = merge(o_bad, l2)
    ro, rl = merge(o[[0, 2]], l2[[0, 2]])
    assert np.allclose(mo, ro, atol=1e-14) and np.allclose(ml, rl, atol=1e-14), "-inf partial used"
    mo, ml = merge(np.ones((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(mo == 0) and np.all(ml == -np.inf), "all -inf must give (0, -inf)"
    big = np.full((3, 5), 1000.0)
    mo, ml = merge(o, big)
    assert np.allclose(mo, o.mean(axis=0), atol=1e-14), "large equal lse: merge != mean"
    assert np.allclose(ml, 1000.0 + math.log(3), atol=1e-12), "large equal lse overflows"


def check_merge_logaddexp(merge, seed=10):
    r = _rng(seed)
    lse = 50.0 * r.standard_normal((6, 7))
    _, ml = merge(r.standard_normal((6, 7, 3)), lse)
    assert np.allclose(ml, np.logaddexp.reduce(lse, axis=0), rtol=1e-13), "lse != logaddexp"


def check_merge_associative(merge, seed=11):
    r = _rng(seed)
    o = r.standard_normal((4, 6, 5))
    lse = 3.0 * r.standard_normal((4, 6))
    mo, ml = merge(o, lse)
    ao, al = merge(o[:2], lse[:2])
    bo, bl = merge(o[2:], lse[2:])
    co, cl = merge(np.stack([ao, bo]), np.stack([al, bl]))
    assert np.allclose(mo, co, atol=1e-13) and np.allclose(ml, cl, atol=1e-13), "not associative"


def check_split_merge(attention, merge, causal, seed=12):
    """Splitting the keys anywhere (empty and one-key pieces included) and
    merging the partial results reproduces attention over all keys."""
    r = _rng(seed)
    nq, nk, hq, hkv, d = 7, 13, 4, 2, 6
    q = r.standard_normal((nq, hq, d))
    k = r.standard_normal((nk, hkv, d))
    v = r.standard_normal((nk, hkv, d))
    qp = np.sort(r.integers(0, 20, nq))
    kp = r.permutation(20)[:nk]
    full_o, full_l = attention(q, k, v, qp, kp, causal, 0.45)
    for cuts in ([0, 0, 1, 13], [0, 5, 6, 6, 13], [0, 13], [0, 2, 4, 8, 12, 13]):
        os, ls = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o_i, l_i = attention(q, k[a:b], v[a:b], qp, kp[a:b], causal, 0.45)
            os.append(o_i.reshape(nq * hq, d))
            ls.append(l_i.reshape(nq * hq))
        mo, ml = merge(np.stack(os), np.stack(ls))
        assert np.allclose(mo, full_o.reshape(-1, d), atol=1e-12), "split+merge O != full"
        fl = full_l.reshape(-1)
        fin = np.isfinite(fl)
        assert np.array_equal(np.isfinite(ml), fin), "split+merge -inf pattern != full"
        assert np.allclose(ml[fin], fl[fin], atol=1e-12), "split+merge lse != full"


# --------------------------------------------------------------------------- block list

def _tile_sets(block_list, R, C, r, c, causal, rot):
    bl = block_list(R, C, r, c, causal, rot)
    qs = {}
    ks = {}
    for q_slot, kv_slot, qp, kp, kind in bl:
        assert qs.setdefault(q_slot, qp) == qp, "q slot maps to two partitions"
        assert ks.setdefault(kv_slot, kp) == kp, "kv slot maps to two partitions"
    return bl, [qs[i] for i in range(len(qs))], [ks[i] for i in range(len(ks))]


def check_block_list_geometry(block_list, R, C):
    """Tiles partition the matrix; rotated tiles hold their own block, read Q
    only from their mesh row and KV only from their mesh column; every
    rotation step is a permutation of senders."""
    P = R * C
    seen = {}
    for r, c in itertools.product(range(R), range(C)):
        bl, qset, kvset = _tile_sets(block_list, R, C, r, c, False, True)
        assert len(bl) == R * C, "tile must hold C*R blocks"
        g = r * C + c
        assert g in qset and g in kvset, "own block (g,g) missing from rotated tile"
        assert all(p // C == r for p in qset), "Q from outside the mesh row"
        assert all(p % C == c for p in kvset), "KV from outside the mesh column"
        assert kvset[0] == g, "rotation does not start at the local partition"
        for _, _, qp, kp, _ in bl:
            seen[(qp, kp)] = seen.get((qp, kp), 0) + 1
    assert len(seen) == P * P and set(seen.values()) == {1}, "tiles do not partition the matrix"
    for step in range(R):
        senders = []
        for r, c in itertools.product(range(R), range(C)):
            _, _, kvset = _tile_sets(block_list, R, C, r, c, False, True)
            senders.append(kvset[step])  # partition p lives on GPU p
        assert sorted(senders) == list(range(P)), "rotation step is not a permutation"
    # Communication: C-1 remote Q plus R-1 remote KV partitions, against P-1 for a ring.
    _, qset, kvset = _tile_sets(block_list, R, C, 0, 0, False, True)
    assert len(set(qset) - {0}) + len(set(kvset) - {0}) == (C - 1) + (R - 1)


def check_block_list_kinds(block_list, R, C):
    """Causal classes: closed-form counts for rotated tiles and the
    partition-order rule; non-causal tiles are all FULL; slot order is
    KV-slot major."""
    for r, c in itertools.product(range(R), range(C)):
        bl, qset, kvset = _tile_sets(block_list, R, C, r, c, True, True)
        kinds = [b[4] for b in bl]
        assert kinds.count(FULL) == r * C + (C - 1 - c), "FULL count"
        assert kinds.count(DIAG) == 1, "DIAG count"
        assert kinds.count(SKIP) == c + (R - 1 - r) * C, "SKIP count"
        for q_slot, kv_slot, qp, kp, kind in bl:
            want = FULL if kp < qp else (DIAG if kp == qp else SKIP)
            assert kind == want, "kind disagrees with partition order"
        order = [(b[1], b[0]) for b in bl]
        assert order == sorted(order) and len(order) == len(set(order)), "not kv-slot major"
        nc = block_list(R, C, r, c, False, True)
        assert all(b[4] == FULL for b in nc), "non-causal tile must be all FULL"


def check_block_list_contiguous(block_list, R, C):
    """Contiguous (un-rotated) tiles: plain 2-D block tiling of the Q-KV
    matrix, checked by properties rather than by the index formula.

    * Every tile's Q set is the C partitions of its own mesh row, in order
      (a GPU receives Q only from its mesh-row peers; tutorial page, "From
      1-D ring to 2-D mesh", panel (b)).
    * Every tile's KV set is a run of R consecutive partitions in increasing
      order ("contiguous" taken literally: no stride, no rotation).
    * The tiles of the mesh cover each (Q partition, KV partition) block of
      the P x P matrix exactly once.
    * Tiles of one mesh row take their runs left to right: column c's run
      lies before column c+1's.
    * Causal classes follow the partition order, and a contiguous tile may
      hold more than one diagonal block (e.g. 2x2 tile (0,0)).
    """
    P = R * C
    seen = {}
    for r, c in itertools.product(range(R), range(C)):
        bl, qset, kvset = _tile_sets(block_list, R, C, r, c, False, False)
        assert len(bl) == R * C, "tile must hold C*R blocks"
        assert sorted(qset) == qset and all(p // C == r for p in qset) and len(set(qset)) == C, \
            "contiguous Q set is not the mesh row"
        assert len(kvset) == R and all(b - a == 1 for a, b in zip(kvset, kvset[1:])), \
            "contiguous KV set is not a run of consecutive partitions"
        assert 0 <= kvset[0] and kvset[-1] < P, "KV partition outside the sequence"
        for _, _, qp, kp, _ in bl:
            seen[(qp, kp)] = seen.get((qp, kp), 0) + 1
        if c + 1 < C:
            _, _, right = _tile_sets(block_list, R, C, r, c + 1, False, False)
            assert kvset[-1] < right[0], "column runs not ordered left to right"
        cbl = block_list(R, C, r, c, True, False)
        for q_slot, kv_slot, qp, kp, kind in cbl:
            want = FULL if kp < qp else (DIAG if kp == qp else SKIP)
            assert kind == want, "contiguous causal kind disagrees with partition order"
    assert len(seen) == P * P and set(seen.values()) == {1}, \
        "contiguous tiles do not partition the matrix"


def check_block_list_fp32_workload_tile(block_list):
    """The literal geometry the fp32 workload statement gives: a 2x2 mesh
    with contiguous KV partitions, whose tile (0,0) holds Q partitions {0,1}
    against KV partitions {0,1}, merged with the partial of the tile that
    holds KV partitions {2,3} (its mesh-row sibling (0,1))."""
    bl, qset, kvset = _tile_sets(block_list, 2, 2, 0, 0, False, False)
    assert qset == [0, 1] and kvset == [0, 1], "fp32 workload tile (0,0)"
    assert sorted((b[2], b[3]) for b in bl) == [(0, 0), (0, 1), (1, 0), (1, 1)]
    assert all(b[4] == FULL for b in bl), "non-causal tile must be all FULL"
    _, qset1, kvset1 = _tile_sets(block_list, 2, 2, 0, 1, False, False)
    assert qset1 == [0, 1] and kvset1 == [2, 3], "fp32 workload sibling tile (0,1)"
    # Causal 2x2 tile (0,0) holds both diagonal blocks of its Q partitions.
    kinds = {(b[2], b[3]): b[4] for b in block_list(2, 2, 0, 0, True, False)}
    assert kinds == {(0, 0): DIAG, (0, 1): SKIP, (1, 0): FULL, (1, 1): DIAG}


# --------------------------------------------------------------------------- backward

def _torch_full_grads(q, k, v, do, q_pos, k_pos, causal, scale):
    """Gradients of sum(O * dO) by torch autograd (float64, CPU), with lse
    from torch.logsumexp and D from the autograd forward's output."""
    import torch
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    g = q.shape[1] // k.shape[1]
    kk = tk.repeat_interleave(g, dim=1)              # [Nk, Hq, d]
    vv = tv.repeat_interleave(g, dim=1)
    s = scale * torch.einsum("ihd,jhd->hij", tq, kk)
    if causal:
        mask = torch.tensor(k_pos[None, :] <= q_pos[:, None])
        s = s.masked_fill(~mask[None], float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("hij,jhd->ihd", p, vv)
    (o * torch.tensor(do)).sum().backward()
    lse = torch.logsumexp(s, dim=-1).T.detach().numpy()
    delta = (o.detach() * torch.tensor(do)).sum(-1).numpy()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), lse, delta


def check_bwd_autograd(bwd, causal, hq=4, hkv=2, nq=11, nk=11, d=16, seed=20):
    """Whole contiguous matrix: the oracle's gradients equal torch autograd's."""
    r = _rng(seed)
    q, k, v = (r.standard_normal(s) for s in ((nq, hq, d), (nk, hkv, d), (nk, hkv, d)))
    do = r.standard_normal((nq, hq, d))
    qp, kp = np.arange(nq), np.arange(nk)
    scale = 1.0 / math.sqrt(d)
    rdq, rdk, rdv, lse, delta = _torch_full_grads(q, k, v, do, qp, kp, causal, scale)
    dq, dk, dv = bwd(q, k, v, do, lse, delta, qp, kp, causal, scale)
    for name, a, b in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-11), f"{name} differs from torch autograd"


def check_bwd_finite_differences(bwd, seed=21):
    """Tiny case, positions not contiguous, causal: central differences of the
    loss sum(O * dO), with O computed by brute force in pure Python (math.exp,
    no max shift), match the oracle's gradients."""
    r = _rng(seed)
    nq, nk, hq, hkv, d = 3, 5, 2, 1, 3
    q, k, v = (r.standard_normal(s) for s in ((nq, hq, d), (nk, hkv, d), (nk, hkv, d)))
    do = r.standard_normal((nq, hq, d))
    qp, kp = np.array([4, 7, 9]), np.array([0, 5, 6, 7, 9])
    scale = 0.7

    def forward(q_, k_, v_):
        o = np.zeros((nq, hq, d))
        lse = np.zeros((nq, hq))
        for i in range(nq):
            for h in range(hq):
                js = [j for j in range(nk) if kp[j] <= qp[i]]
                e = [math.exp(scale * sum(q_[i, h, t] * k_[j, 0, t] for t in range(d))) for j in js]
                z = math.fsum(e)
                lse[i, h] = math.log(z)
                for t in range(d):
                    o[i, h, t] = math.fsum(ej * v_[j, 0, t] for ej, j in zip(e, js)) / z
        return o, lse

    def loss(q_, k_, v_):
        return math.fsum((forward(q_, k_, v_)[0] * do).ravel())

    o, lse = forward(q, k, v)
    delta = (o * do).sum(-1)
    grads = bwd(q, k, v, do, lse, delta, qp, kp, True, scale)
    eps = 1e-6
    for x, g in zip((q, k, v), grads):
        for idx in itertools.product(*(range(n) for n in x.shape)):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = loss(q, k, v)
            x[idx] = x0 - eps
            lm = loss(q, k, v)
            x[idx] = x0
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(fd)), f"finite difference mismatch at {idx}"


def check_bwd_zero_query(bwd, n=7, d=5, seed=22):
    """Q = 0, no mask: P = 1/n everywhere, so dV_j = mean_i dO_i, dK = 0 and
    dQ_i = (scale / n) sum_j <dO_i, v_j - mean v> k_j (closed forms)."""
    r = _rng(seed)
    q = np.zeros((n, 1, d))
    k, v, do = (r.standard_normal((n, 1, d)) for _ in range(3))
    scale = 0.9
    lse = np.full((n, 1), math.log(n))
    vbar = v[:, 0].mean(axis=0)
    delta = (do[:, 0] @ vbar)[:, None]
    dq, dk, dv = bwd(q, k, v, do, lse, delta, np.arange(n), np.arange(n), False, scale)
    assert np.allclose(dv[:, 0], np.broadcast_to(do[:, 0].mean(axis=0), (n, d)), atol=1e-13), \
        "Q=0: dV != mean of dO"
    assert np.allclose(dk, 0.0, atol=1e-14), "Q=0: dK != 0"
    want = (scale / n) * ((do[:, 0] @ (v[:, 0] - vbar).T) @ k[:, 0])
    assert np.allclose(dq[:, 0], want, atol=1e-13), "Q=0: dQ closed form"


def check_bwd_tile_sum(tile_bwd, tile_sets, R, C, causal=True, rot=True, L=3, hq=2, hkv=1, d=4,
                       seed=23):
    """The gradient shares of all tiles of an R x C mesh add up to the
    gradient of full attention (torch autograd); each tile is given the
    rows' full lse and D."""
    r = _rng(seed)
    P = R * C
    N = P * L
    q, do = (r.standard_normal((N, hq, d)) for _ in range(2))
    k, v = (r.standard_normal((N, hkv, d)) for _ in range(2))
    scale = 0.5
    pos = np.arange(N)
    rdq, rdk, rdv, lse, delta = _torch_full_grads(q, k, v, do, pos, pos, causal, scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for rr in range(R):
        for cc in range(C):
            q_parts, kv_parts = tile_sets(R, C, rr, cc, rot)
            qi = _positions(q_parts, L)
            ki = _positions(kv_parts, L)
            a, b, c = tile_bwd(q[qi], k[ki], v[ki], do[qi], lse[qi], delta[qi], q_parts, kv_parts,
                               L, causal, scale)
            np.add.at(dq, qi, a)
            np.add.at(dk, ki, b)
            np.add.at(dv, ki, c)
    for name, a, b in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-11), f"tile shares of {name} do not sum to the gradient"


def check_bwd_empty_rows(bwd, seed=24):
    """Rows with lse = -inf (no visible key anywhere) contribute nothing."""
    r = _rng(seed)
    q, do = (r.standard_normal((4, 1, 3)) for _ in range(2))
    k, v = (r.standard_normal((4, 1, 3)) for _ in range(2))
    lse = np.full((4, 1), -np.inf)
    dq, dk, dv = bwd(q, k, v, do, lse, np.zeros((4, 1)), np.arange(4), np.arange(4), False, 0.5)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0), "empty rows contributed"
