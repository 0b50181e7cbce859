"""Planted mistakes in the oracle must each be caught by at least one pin.

The mutants wrap or re-implement oracle functions on the CPU with one
plausible error each (a dropped term, a wrong sign or index, a swapped
operand); every one must make some check in ``oracle_pins`` fail.
"""
import math

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

A = oracle.attention_ref


def _per_head_mod(q, k, v, qp, kp, causal, scale):
    hq, hkv = q.shape[1], k.shape[1]
    outs = [A(q[:, h:h + 1], k[:, h % hkv:h % hkv + 1], v[:, h % hkv:h % hkv + 1], qp, kp, causal,
              scale) for h in range(hq)]
    return np.concatenate([o for o, _ in outs], axis=1), np.concatenate([l for _, l in outs], axis=1)


ATTENTION_MUTANTS = {
    "scale dropped": lambda q, k, v, qp, kp, c, s: A(q, k, v, qp, kp, c, 1.0),
    "scale squared": lambda q, k, v, qp, kp, c, s: A(q, k, v, qp, kp, c, s * s),
    "causal excludes self": lambda q, k, v, qp, kp, c, s: A(q, k, v, qp, np.asarray(kp) + 1, c, s),
    "causal off by one the other way": lambda q, k, v, qp, kp, c, s:
        A(q, k, v, qp, np.asarray(kp) - 1, c, s),
    "head h % Hkv": _per_head_mod,
    "lse in log2": lambda q, k, v, qp, kp, c, s:
        (lambda r: (r[0], r[1] / math.log(2)))(A(q, k, v, qp, kp, c, s)),
    "k and v swapped": lambda q, k, v, qp, kp, c, s: A(q, v, k, qp, kp, c, s),
    "key positions reversed": lambda q, k, v, qp, kp, c, s: A(q, k, v, qp, np.asarray(kp)[::-1], c, s),
    "uniform weights": lambda q, k, v, qp, kp, c, s: A(np.zeros_like(q), k, v, qp, kp, c, s),
    "lse shifted": lambda q, k, v, qp, kp, c, s:
        (lambda r: (r[0], r[1] + 1e-6))(A(q, k, v, qp, kp, c, s)),
}


def _merge_unweighted(o, l):
    _, ml = oracle.lse_merge_ref(o, l)
    return np.asarray(o).mean(axis=0), ml


def _merge_unnormalised(o, l):
    l = np.asarray(l)
    m = l.max(axis=0)
    w = np.exp(l - m)
    return np.einsum("nr,nrd->rd", w, np.asarray(o)), m + np.log(w.sum(axis=0))


def _merge_no_shift(o, l):
    w = np.exp(np.asarray(l))
    return np.einsum("nr,nrd->rd", w / w.sum(axis=0), np.asarray(o)), np.log(w.sum(axis=0))


MERGE_MUTANTS = {
    "unweighted mean": _merge_unweighted,
    "weights not normalised": _merge_unnormalised,
    "lse forgets the sum": lambda o, l: (oracle.lse_merge_ref(o, l)[0], np.asarray(l).max(axis=0)),
    "no max shift": _merge_no_shift,
}


def _bl_rot_row_major(R, C, r, c, causal, rot):
    """Rotation that steps through the row-major GPU index instead of the column."""
    out = []
    for (qs, ks, qp, kp, kind) in oracle.block_list_ref(R, C, r, c, causal, rot):
        if rot:
            kp = (r * C + c + ks) % (R * C)
            kind = oracle.FULL if not causal else (0 if kp < qp else (1 if kp == qp else 2))
        out.append((qs, ks, qp, kp, kind))
    return out


def _bl_kind_flipped(R, C, r, c, causal, rot):
    return [(a, b, qp, kp, (oracle.SKIP if k == oracle.FULL and causal else
                            oracle.FULL if k == oracle.SKIP else k))
            for (a, b, qp, kp, k) in oracle.block_list_ref(R, C, r, c, causal, rot)]


def _bl_q_major(R, C, r, c, causal, rot):
    return sorted(oracle.block_list_ref(R, C, r, c, causal, rot), key=lambda b: (b[0], b[1]))


def _bl_modes_swapped(R, C, r, c, causal, rot):
    return oracle.block_list_ref(R, C, r, c, causal, not rot)


def _bl_q_from_column(R, C, r, c, causal, rot):
    out = []
    for (qs, ks, qp, kp, kind) in oracle.block_list_ref(R, C, r, c, causal, rot):
        qp = (qs % R) * C + c
        kind = oracle.FULL if not causal else (0 if kp < qp else (1 if kp == qp else 2))
        out.append((qs, ks, qp, kp, kind))
    return out


def _bl_contiguous_strided(R, C, r, c, causal, rot):
    """Contiguous mode read as a column stride: KV partitions c + k*C."""
    if rot:
        return oracle.block_list_ref(R, C, r, c, causal, rot)
    out = []
    for (qs, ks, qp, kp, kind) in oracle.block_list_ref(R, C, r, c, causal, rot):
        kp = c + ks * C
        kind = oracle.FULL if not causal else (0 if kp < qp else (1 if kp == qp else 2))
        out.append((qs, ks, qp, kp, kind))
    return out


def _bl_contiguous_columns_reversed(R, C, r, c, causal, rot):
    """Contiguous runs handed to the mesh columns right to left."""
    if rot:
        return oracle.block_list_ref(R, C, r, c, causal, rot)
    out = []
    for (qs, ks, qp, kp, kind) in oracle.block_list_ref(R, C, r, c, causal, rot):
        kp = (C - 1 - c) * R + ks
        kind = oracle.FULL if not causal else (0 if kp < qp else (1 if kp == qp else 2))
        out.append((qs, ks, qp, kp, kind))
    return out


BLOCK_MUTANTS = {
    "rotation along the row-major index": _bl_rot_row_major,
    "kinds flipped": _bl_kind_flipped,
    "q-slot major order": _bl_q_major,
    "rotated and contiguous swapped": _bl_modes_swapped,
    "Q set taken from the column": _bl_q_from_column,
    "contiguous KV strided by the column count": _bl_contiguous_strided,
    "contiguous KV runs in reversed column order": _bl_contiguous_columns_reversed,
}


BW = oracle.attention_bwd_ref


def _bwd_per_head_mod(q, k, v, do, lse, delta, qp, kp, c, s):
    hq, hkv = q.shape[1], k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(hq):
        hk = h % hkv
        a, b, cc = BW(q[:, h:h + 1], k[:, hk:hk + 1], v[:, hk:hk + 1], do[:, h:h + 1], lse[:, h:h + 1],
                      delta[:, h:h + 1], qp, kp, c, s)
        dq[:, h:h + 1] += a
        dk[:, hk:hk + 1] += b
        dv[:, hk:hk + 1] += cc
    return dq, dk, dv


def _bwd_dk_unscaled(*a):
    dq, dk, dv = BW(*a)
    return dq, dk / a[-1], dv


BWD_MUTANTS = {
    "delta dropped": lambda q, k, v, do, l, dl, qp, kp, c, s: BW(q, k, v, do, l, 0 * dl, qp, kp, c, s),
    "lse shifted": lambda q, k, v, do, l, dl, qp, kp, c, s: BW(q, k, v, do, l + 1e-6, dl, qp, kp, c, s),
    "causal excludes self": lambda q, k, v, do, l, dl, qp, kp, c, s:
        BW(q, k, v, do, l, dl, qp, np.asarray(kp) + 1, c, s),
    "k and v swapped": lambda q, k, v, do, l, dl, qp, kp, c, s: BW(q, v, k, do, l, dl, qp, kp, c, s),
    "dS sign flipped": lambda *a: (lambda r: (-r[0], -r[1], r[2]))(BW(*a)),
    "dK without the scale": _bwd_dk_unscaled,
    "head h % Hkv": _bwd_per_head_mod,
    "dO taken as O's gradient twice": lambda q, k, v, do, l, dl, qp, kp, c, s:
        BW(q, k, v, 2 * do, l, dl, qp, kp, c, s),
}


def _attention_checks(att):
    yield lambda: pins.check_sdpa(att, False)
    yield lambda: pins.check_sdpa(att, True)
    yield lambda: pins.check_zero_query(att)
    yield lambda: pins.check_single_key(att)
    yield lambda: pins.check_affine_values(att, True)
    yield lambda: pins.check_gqa_mapping(att)
    yield lambda: pins.check_brute_force(att, True)
    yield lambda: pins.check_large_scores(att)
    yield lambda: pins.check_scale_on_scores(att)


def _merge_checks(mg):
    yield lambda: pins.check_merge_closed_forms(mg)
    yield lambda: pins.check_merge_logaddexp(mg)
    yield lambda: pins.check_merge_associative(mg)
    yield lambda: pins.check_split_merge(A, mg, True)


def _block_checks(bl):
    for R, C in [(4, 4), (3, 5), (2, 3)]:
        yield lambda R=R, C=C: pins.check_block_list_geometry(bl, R, C)
        yield lambda R=R, C=C: pins.check_block_list_kinds(bl, R, C)
        yield lambda R=R, C=C: pins.check_block_list_contiguous(bl, R, C)
    yield lambda: pins.check_block_list_fp32_workload_tile(bl)


def _bwd_checks(bw):
    yield lambda: pins.check_bwd_autograd(bw, False)
    yield lambda: pins.check_bwd_autograd(bw, True)
    yield lambda: pins.check_bwd_finite_differences(bw)
    yield lambda: pins.check_bwd_zero_query(bw)
    yield lambda: pins.check_bwd_empty_rows(bw)


def _caught(checks):
    failures = 0
    for chk in checks:
        try:
            with np.errstate(all="ignore"):
                chk()
        except (AssertionError, ValueError, FloatingPointError):
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(ATTENTION_MUTANTS))
def test_attention_mutant_is_caught(name):
    assert _caught(_attention_checks(ATTENTION_MUTANTS[name])) > 0, name


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_mutant_is_caught(name):
    assert _caught(_merge_checks(MERGE_MUTANTS[name])) > 0, name


@pytest.mark.parametrize("name", sorted(BLOCK_MUTANTS))
def test_block_list_mutant_is_caught(name):
    assert _caught(_block_checks(BLOCK_MUTANTS[name])) > 0, name


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name):
    assert _caught(_bwd_checks(BWD_MUTANTS[name])) > 0, name


def test_real_oracle_passes_every_check():
    assert _caught(_attention_checks(A)) == 0
    assert _caught(_merge_checks(oracle.lse_merge_ref)) == 0
    assert _caught(_block_checks(oracle.block_list_ref)) == 0
    assert _caught(_bwd_checks(BW)) == 0
