"""Oracle: exact softmax attention of query rows over a set of keys (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed is the left-hand side of the attention decomposition printed
on the Ring-Attention page ("环形注意力", section "理论奠基：注意力分解的数学突破"):
softmax(Q K^T / sqrt(d_k)) V, row by row.  The max-subtracted form with a
running maximum m and exponent sum l is the one that page describes for
FlashAttention in section "数值稳定性：Log-Sum-Exp技术的分布式应用"; here it is
evaluated in two plain passes (maximum first, then exponentials), never
online.

For each query row (token i at global position p_i, query head h):

* kv head  = h // G with G = H_q / H_kv (consecutive query heads share a KV
  head; GQA is only cited by title on the mlsanity page, "Builds on");
* allowed  = { key j : not causal or pos_j <= p_i };
* s_j      = scale * sum_d q[i,h,d] * k[j,h_kv,d]   (float64);
* if allowed is empty: O = 0, lse = -inf;
* else m = max s_j, e_j = exp(s_j - m), l = sum e_j,
  O = sum e_j v_j / l, lse = m + ln(l)  (natural log of the scaled scores).
"""

import numpy as np

# Rows are processed in chunks so that one chunk's score matrix stays below
# this many float64 elements (256 MiB).
_CHUNK_ELEMS = 1 << 25


def tile_positions_ref(parts, part_len):
    """Global token positions of the concatenated partitions ``parts``."""
    parts = np.asarray(parts, dtype=np.int64).reshape(-1)
    offs = np.arange(part_len, dtype=np.int64)
    return (parts[:, None] * part_len + offs[None, :]).reshape(-1)


def _as_f64(x):
    if hasattr(x, "detach"):  # torch tensor: bf16/fp32 -> fp64 is exact
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def attention_ref(q, k, v, q_pos, k_pos, causal, scale, rows=None):
    """Exact attention rows.

    q: [Nq, Hq, d]; k, v: [Nk, Hkv, d]; q_pos: [Nq]; k_pos: [Nk] (integers).
    rows: None for every (token, head) row, else an int array [n, 2] of
    (token, head) pairs.  Returns (O, lse): [Nq, Hq, d] and [Nq, Hq] when
    rows is None, else [n, d] and [n].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    n_q, h_q, d = q.shape
    n_k, h_kv, d_k = k.shape
    if d_k != d or v.shape != k.shape:
        raise ValueError("q, k, v head dimensions disagree")
    if h_q % h_kv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if q_pos.shape != (n_q,) or k_pos.shape != (n_k,):
        raise ValueError("position arrays do not match token counts")
    group = h_q // h_kv

    full = rows is None
    if full:
        tok = np.repeat(np.arange(n_q), h_q)
        head = np.tile(np.arange(h_q), n_q)
    else:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        tok, head = rows[:, 0], rows[:, 1]
    n_rows = tok.shape[0]
    out = np.zeros((n_rows, d), dtype=np.float64)
    lse = np.full((n_rows,), -np.inf, dtype=np.float64)

    kv_head = head // group
    chunk = max(1, _CHUNK_ELEMS // max(1, n_k))
    for hk in range(h_kv):
        sel = np.nonzero(kv_head == hk)[0]
        k_h = k[:, hk, :]
        v_h = v[:, hk, :]
        for c0 in range(0, sel.shape[0], chunk):
            idx = sel[c0:c0 + chunk]
            qr = q[tok[idx], head[idx], :]                  # [n, d]
            s = scale * (qr @ k_h.T)                         # [n, Nk]
            if causal:
                allowed = k_pos[None, :] <= q_pos[tok[idx]][:, None]
            else:
                allowed = np.ones(s.shape, dtype=bool)
            s = np.where(allowed, s, -np.inf)
            any_allowed = allowed.any(axis=1)
            m = np.where(any_allowed, s.max(axis=1, initial=-np.inf), 0.0)  # pass 1: maximum
            e = np.where(allowed, np.exp(s - m[:, None]), 0.0)  # pass 2
            l = e.sum(axis=1)
            o = e @ v_h
            safe_l = np.where(any_allowed, l, 1.0)
            out[idx] = np.where(any_allowed[:, None], o / safe_l[:, None], 0.0)
            lse[idx] = np.where(any_allowed, m + np.log(safe_l), -np.inf)

    if full:
        return out.reshape(n_q, h_q, d), lse.reshape(n_q, h_q)
    return out, lse


def tile_rows_ref(q, k, v, q_parts, kv_parts, part_len, causal, scale, rows=None):
    """Attention of a tile: Q slots hold partitions ``q_parts`` and KV slots
    hold ``kv_parts``, each ``part_len`` tokens, concatenated in slot order.

    The causal rule uses global positions part*part_len + offset, so the
    result does not depend on any block classification.
    """
    q_pos = tile_positions_ref(q_parts, part_len)
    k_pos = tile_positions_ref(kv_parts, part_len)
    return attention_ref(q, k, v, q_pos, k_pos, causal, scale, rows=rows)
