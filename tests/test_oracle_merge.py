"""Pins of the merge oracle, alone and against attention (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def attention(q, k, v, qp, kp, causal, scale):
    return oracle.attention_ref(q, k, v, qp, kp, causal, scale)


def test_closed_forms():
    pins.check_merge_closed_forms(oracle.lse_merge_ref)


def test_lse_is_logaddexp():
    pins.check_merge_logaddexp(oracle.lse_merge_ref)


def test_associative():
    pins.check_merge_associative(oracle.lse_merge_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_split_then_merge_is_full_attention(causal):
    pins.check_split_merge(attention, oracle.lse_merge_ref, causal)


@pytest.mark.parametrize("R,C,row", [(2, 2, 0), (4, 4, 2), (3, 2, 1)])
def test_mesh_row_siblings_merge_to_full_causal_attention(R, C, row):
    """The C tiles of one mesh row, merged, give causal attention of the row's
    Q partitions over the whole sequence."""
    L, hq, hkv, d = 3, 2, 1, 4
    r = np.random.default_rng(R * 10 + C)
    P = R * C
    Q = r.standard_normal((P * L, hq, d))
    K = r.standard_normal((P * L, hkv, d))
    V = r.standard_normal((P * L, hkv, d))
    def parts(x, ps):
        return np.concatenate([x[p * L:(p + 1) * L] for p in ps])
    os, ls = [], []
    for col in range(C):
        qset, kvset = oracle.mesh_tile_sets_ref(R, C, row, col, True)
        o, l = oracle.tile_rows_ref(parts(Q, qset), parts(K, kvset), parts(V, kvset), qset, kvset,
                                    L, True, 0.5)
        os.append(o.reshape(-1, d))
        ls.append(l.reshape(-1))
    mo, ml = oracle.lse_merge_ref(np.stack(os), np.stack(ls))
    qset, _ = oracle.mesh_tile_sets_ref(R, C, row, 0, True)
    fo, fl = oracle.tile_rows_ref(parts(Q, qset), K, V, qset, list(range(P)), L, True, 0.5)
    assert np.allclose(mo, fo.reshape(-1, d), atol=1e-12)
    assert np.allclose(ml, fl.reshape(-1), atol=1e-12)
