"""Oracle: log-sum-exp merge of partial attention results (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Mesh-Attention returns partial outputs along a mesh row to the owner of the
Q partition (Mesh-Attention tutorial page, section on the greedy algorithm:
a GPU receives Q, KV and partial output results).  The Ring-Attention page
says partial states are combined with log-sum-exp bookkeeping (section
"数值稳定性：Log-Sum-Exp技术的分布式应用") and prints a decomposition of
attention over KV blocks (section "理论奠基：注意力分解的数学突破") that is
wrong as printed: a plain sum of separately normalised softmaxes is not
attention.  The correct combination weights each partial by its share of the
total exponent mass:

  M   = max_i lse_i
  if M = -inf:  O = 0, lse = -inf          (no partial saw any key)
  w_i = exp(lse_i - M)
  O   = sum_i (w_i / sum_j w_j) O_i
  lse = M + ln(sum_i w_i)
"""

import numpy as np


def lse_merge_ref(o_parts, lse_parts):
    """o_parts: [n, rows, d]; lse_parts: [n, rows] -> (O [rows, d], lse [rows])."""
    if hasattr(o_parts, "detach"):
        o_parts = o_parts.detach().to("cpu").double().numpy()
    if hasattr(lse_parts, "detach"):
        lse_parts = lse_parts.detach().to("cpu").double().numpy()
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.ndim != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("expected o_parts [n, rows, d] and lse_parts [n, rows]")
    if o_parts.shape[0] < 1:
        raise ValueError("need at least one partial")
    m = lse_parts.max(axis=0)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[None, :]), 0.0)
    total = w.sum(axis=0)
    total_safe = np.where(live, total, 1.0)
    # A partial whose lse is -inf saw no key; it carries no weight, whatever
    # its output rows hold.
    o_live = np.where((w > 0)[:, :, None], o_parts, 0.0)
    out = np.einsum("nr,nrd->rd", w / total_safe[None, :], o_live)
    out = np.where(live[:, None], out, 0.0)
    lse = np.where(live, m_safe + np.log(total_safe), -np.inf)
    return out, lse
