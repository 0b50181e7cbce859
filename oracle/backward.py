"""Oracle: gradients of softmax attention, split into one tile's share (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages aim Mesh-Attention at long-context training (tutorial page, the
closing section "总结", and the greedy-scheduling section, which speaks of
distributed training), so a GPU's tile has a backward pass as well as a
forward one.  The pages print no formula for it; the oracle takes the plain
definition.  With O = softmax(scale Q K^T + causal mask) V (the decomposition
on the Ring-Attention page, section "理论奠基：注意力分解的数学突破") and a loss
whose gradient with respect to O is dO, differentiating gives, per query row i
(token, head) and key j, with s_ij = scale <q_i, k_j>:

    P_ij  = exp(s_ij - lse_i)            lse_i: the row's log-sum-exp over ALL
                                         its visible keys (the final one)
    D_i   = <dO_i, O_i>                  O_i: the row's final output
    dV_j += P_ij dO_i
    dS_ij = P_ij (<dO_i, v_j> - D_i)
    dQ_i += scale dS_ij k_j
    dK_j += scale dS_ij q_i

Each term belongs to one visible (query, key) pair, and every pair belongs to
exactly one tile of the mesh, so a tile's share is the sum over its own
visible pairs and the shares of all tiles add up to the full gradient.  A row
with lse = -inf has no visible key anywhere and contributes nothing.  With GQA
the key and value gradients of a KV head collect the terms of all query heads
that share it (query head h uses KV head h // G).

Functions:

* ``bwd_delta_ref(o, do)``  - D per row;
* ``attention_bwd_ref(...)`` - the share of the pairs between the given query
  rows and keys (positions decide causality), given lse and D;
* ``tile_bwd_ref(...)`` - the same for a tile's Q and KV partition sets;
* ``full_grads_ref(...)`` - forward (exact lse and O) plus backward over all
  keys: the gradient of full attention.
"""

import numpy as np

from .attention import _as_f64, attention_ref, tile_positions_ref

_CHUNK_ELEMS = 1 << 24


def bwd_delta_ref(o, do):
    """D = sum over the head dimension of dO * O, per (token, head) row."""
    o = _as_f64(o)
    do = _as_f64(do)
    if o.shape != do.shape:
        raise ValueError("O and dO shapes differ")
    return (o * do).sum(axis=-1)


def attention_bwd_ref(q, k, v, do, lse, delta, q_pos, k_pos, causal, scale):
    """Gradient share of the visible pairs between rows of q and keys k.

    q, do: [Nq, Hq, d]; k, v: [Nk, Hkv, d]; lse, delta: [Nq, Hq];
    q_pos: [Nq], k_pos: [Nk].  Returns (dq [Nq, Hq, d], dk [Nk, Hkv, d],
    dv [Nk, Hkv, d]) in float64.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    lse, delta = _as_f64(lse), _as_f64(delta)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    n_q, h_q, d = q.shape
    n_k, h_kv, _ = k.shape
    if do.shape != q.shape or v.shape != k.shape or k.shape[2] != d:
        raise ValueError("shapes disagree")
    if lse.shape != (n_q, h_q) or delta.shape != (n_q, h_q):
        raise ValueError("lse / delta shapes disagree")
    if h_q % h_kv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = h_q // h_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    chunk = max(1, _CHUNK_ELEMS // max(1, n_k))
    for h in range(h_q):
        hk = h // group
        k_h, v_h = k[:, hk, :], v[:, hk, :]
        for r0 in range(0, n_q, chunk):
            r1 = min(n_q, r0 + chunk)
            q_r, do_r = q[r0:r1, h, :], do[r0:r1, h, :]
            lse_r, d_r = lse[r0:r1, h], delta[r0:r1, h]
            if causal:
                allowed = k_pos[None, :] <= q_pos[r0:r1][:, None]
            else:
                allowed = np.ones((r1 - r0, n_k), dtype=bool)
            allowed &= np.isfinite(lse_r)[:, None]
            s = scale * (q_r @ k_h.T)
            p = np.where(allowed, np.exp(np.where(allowed, s - lse_r[:, None], 0.0)), 0.0)
            dv[:, hk, :] += p.T @ do_r
            ds = p * (do_r @ v_h.T - d_r[:, None])
            dq[r0:r1, h, :] += scale * (ds @ k_h)
            dk[:, hk, :] += scale * (ds.T @ q_r)
    return dq, dk, dv


def tile_bwd_ref(q, k, v, do, lse, delta, q_parts, kv_parts, part_len, causal, scale):
    """A tile's gradient share: Q slots hold ``q_parts``, KV slots ``kv_parts``."""
    q_pos = tile_positions_ref(q_parts, part_len)
    k_pos = tile_positions_ref(kv_parts, part_len)
    return attention_bwd_ref(q, k, v, do, lse, delta, q_pos, k_pos, causal, scale)


def full_grads_ref(q, k, v, do, q_pos, k_pos, causal, scale):
    """Exact forward over all keys, then the backward of full attention.

    Returns (dq, dk, dv, o, lse, delta)."""
    o, lse = attention_ref(q, k, v, q_pos, k_pos, causal, scale)
    delta = bwd_delta_ref(o, do)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, lse, delta, q_pos, k_pos, causal, scale)
    return dq, dk, dv, o, lse, delta
