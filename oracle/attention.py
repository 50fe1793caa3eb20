"""Packed draft attention (oracle side).

One drafter attention layer of the packed async forward ([D3D, 核心方法] and
[D3D, 方法步骤详情 step 4]): every packed query attends, with scaled-dot-product softmax
attention, to the keys its visibility row allows (see ``packing.visible_mask``). Query heads are
grouped over key/value heads in consecutive groups of H_q / H_kv (grouped-query attention, the
drafter being initialised from a grouped-query target-family model).

o[t, h] = softmax_j( scale * q[t, h] . k[j, g(h)] over visible j ) @ v[:, g(h)],  g(h) = h // (H_q/H_kv)

computed in float64 on the exact input values. Rotary embedding and any q/k normalisation happen
upstream of this layer (the inputs are already rotated).

TEST INFRASTRUCTURE: see the package docstring.
"""

import numpy as np


def packed_attention(q, k_prefix, v_prefix, k_new, v_new, mask, scale, rows=None):
    """Attention of one request's packed queries.

    q: [n_q, H_q, d]; k_prefix, v_prefix: [L, H_kv, d]; k_new, v_new: [n_q, H_kv, d] (the packed
    rows' own keys/values); mask: bool [n_q, L + n_q] from ``packing.visible_mask``.
    rows: optional iterable of packed-row indices to evaluate (all rows when None).
    Returns float64 [len(rows), H_q, d].
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.concatenate([np.asarray(k_prefix, np.float64), np.asarray(k_new, np.float64)], axis=0)
    vals = np.concatenate([np.asarray(v_prefix, np.float64), np.asarray(v_new, np.float64)], axis=0)
    n_q, h_q, d = q.shape
    h_kv = keys.shape[1]
    if h_q % h_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    if mask.shape != (n_q, keys.shape[0]):
        raise ValueError("mask shape does not match the packed queries and keys")
    group = h_q // h_kv
    sel = np.arange(n_q) if rows is None else np.asarray(list(rows), dtype=np.int64)
    out = np.empty((sel.size, h_q, d), dtype=np.float64)
    m = mask[sel]
    for h in range(h_q):
        g = h // group
        s = (q[sel, h, :] @ keys[:, g, :].T) * float(scale)
        s = np.where(m, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vals[:, g, :]
    return out
