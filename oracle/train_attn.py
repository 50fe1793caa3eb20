"""Training-time packed attention, forward and backward (oracle side).

[D3D, 方法步骤详情 step 2] and [D3D, 核心方法]: anchors are drawn in each training response; every
anchor starts a diffusion block of B tokens (the anchor itself visible, the B-1 positions after it
masked); all blocks are packed into one sequence after the response; the response is encoded
causally once and shared as the prefix of every block, and attention inside a block is
bidirectional. The clean response rows are computed too (they carry the autoregressive loss).
[DScout, 方法步骤详情 step 2]: the horizon B is drawn per update from {8, 16, 24, 32}.

Reading (the pages leave the layout open): packed rows 0..L-1 are the response; block i occupies rows
L + i*B .. L + i*B + B - 1 and its anchor sits at response position a_i. A response row p sees the
response keys j <= p. A row of block i sees the response keys j < a_i (the tokens before its anchor)
and every row of block i. No row sees another block.

Forward, per query head h with key/value head g(h) = h // (H_q / H_kv):
    s = scale * q k^T (masked to -inf),  lse = log sum_j exp(s),  o = exp(s - lse) v.
Backward of a scalar loss with upstream gradient do: with P = exp(s - lse) and D_r = sum_d do_r o_r,
    dS = P * (do v^T - D),  dq = scale dS k,  dk = scale dS^T q,  dv = P^T do,
dk and dv summed over the query heads of a group. Everything in float64 on the exact input values.

TEST INFRASTRUCTURE: see the package docstring.
"""

import numpy as np


def n_rows(L, n_blocks, B):
    return L + n_blocks * B


def visible_mask(L, anchors, B):
    """bool [N, N]: mask[r, j] is True when packed row r sees packed key j (the reading above)."""
    anchors = [int(a) for a in anchors]
    n = n_rows(L, len(anchors), B)
    mask = np.zeros((n, n), dtype=bool)
    for p in range(L):
        mask[p, :p + 1] = True
    for i, a in enumerate(anchors):
        r0 = L + i * B
        mask[r0:r0 + B, :a] = True
        mask[r0:r0 + B, r0:r0 + B] = True
    return mask


def _group(hq, hkv):
    if hq % hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return hq // hkv


def forward(q, k, v, L, anchors, B, scale):
    """q [N, H_q, d], k, v [N, H_kv, d] -> (o float64 [N, H_q, d], lse float64 [N, H_q])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, hq, d = q.shape
    grp = _group(hq, k.shape[1])
    mask = visible_mask(L, anchors, B)
    if mask.shape[0] != n:
        raise ValueError("row count does not match L + n_blocks * B")
    o = np.empty_like(q)
    lse = np.empty((n, hq))
    for h in range(hq):
        g = h // grp
        s = np.where(mask, (q[:, h] @ k[:, g].T) * float(scale), -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        tot = e.sum(axis=1, keepdims=True)
        lse[:, h] = (m + np.log(tot))[:, 0]
        o[:, h] = (e / tot) @ v[:, g]
    return o, lse


def backward(q, k, v, do, L, anchors, B, scale):
    """Gradients (dq [N, H_q, d], dk, dv [N, H_kv, d]) of sum(o * do), float64."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n, hq, d = q.shape
    hkv = k.shape[1]
    grp = _group(hq, hkv)
    mask = visible_mask(L, anchors, B)
    o, lse = forward(q, k, v, L, anchors, B, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        g = h // grp
        s = np.where(mask, (q[:, h] @ k[:, g].T) * float(scale), -np.inf)
        p = np.exp(s - lse[:, h:h + 1])
        dp = do[:, h] @ v[:, g].T
        dd = np.sum(do[:, h] * o[:, h], axis=1, keepdims=True)
        ds = p * (dp - dd)
        dq[:, h] = float(scale) * (ds @ k[:, g])
        dk[:, g] += float(scale) * (ds.T @ q[:, h])
        dv[:, g] += p.T @ do[:, h]
    return dq, dk, dv


def _rows_forward(q, k, v, vis, scale, rows):
    """o, lse of the query rows `rows` whose visibility rows are `vis` (float64 inputs)."""
    hq = q.shape[1]
    grp = _group(hq, k.shape[1])
    o = np.empty((len(rows), hq, q.shape[2]))
    lse = np.empty((len(rows), hq))
    for h in range(hq):
        g = h // grp
        s = np.where(vis, (q[rows, h] @ k[:, g].T) * float(scale), -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        tot = e.sum(axis=1, keepdims=True)
        lse[:, h] = (m + np.log(tot))[:, 0]
        o[:, h] = (e / tot) @ v[:, g]
    return o, lse


def forward_rows(q, k, v, L, anchors, B, scale, rows):
    """forward() restricted to the packed query rows `rows`: (o [R, H_q, d], lse [R, H_q]). A row's
    softmax involves only its own scores, so this is the same definition on fewer rows (for shapes
    where every row would be too much work)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    rows = np.asarray(rows, dtype=np.int64)
    return _rows_forward(q, k, v, visible_mask(L, anchors, B)[rows], scale, rows)


def backward_rows(q, k, v, do, L, anchors, B, scale, rows):
    """dq of the packed query rows `rows` only, [R, H_q, d]: a row's dq involves only its own scores,
    probabilities and D_r = sum_d do_r o_r."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    rows = np.asarray(rows, dtype=np.int64)
    hq = q.shape[1]
    grp = _group(hq, k.shape[1])
    vis = visible_mask(L, anchors, B)[rows]
    o, lse = _rows_forward(q, k, v, vis, scale, rows)
    dq = np.empty((len(rows), hq, q.shape[2]))
    for h in range(hq):
        g = h // grp
        s = np.where(vis, (q[rows, h] @ k[:, g].T) * float(scale), -np.inf)
        p = np.exp(s - lse[:, h:h + 1])
        dp = do[rows, h] @ v[:, g].T
        dd = np.sum(do[rows, h] * o[:, h], axis=1, keepdims=True)
        dq[:, h] = float(scale) * ((p * (dp - dd)) @ k[:, g])
    return dq


def backward_keys(q, k, v, do, L, anchors, B, scale, keys):
    """(dk, dv) of the packed keys `keys` only, [K, H_kv, d]: each is a sum over the rows that see the
    key (and the query heads of its group), with every viewer's own lse and o."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    keys = np.asarray(keys, dtype=np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    grp = _group(hq, hkv)
    mask = visible_mask(L, anchors, B)
    dk = np.zeros((len(keys), hkv, k.shape[2]))
    dv = np.zeros((len(keys), hkv, v.shape[2]))
    # every viewer's o and lse once (the keys share most of their viewers)
    seen = np.nonzero(mask[:, keys].any(axis=1))[0]
    if len(seen) == 0:
        return dk, dv
    o_all, lse_all = _rows_forward(q, k, v, mask[seen], scale, seen)
    for i, kj in enumerate(keys):
        sel = np.nonzero(mask[seen, kj])[0]
        viewers, o, lse = seen[sel], o_all[sel], lse_all[sel]
        for h in range(hq):
            g = h // grp
            p = np.exp((q[viewers, h] @ k[kj, g]) * float(scale) - lse[:, h])
            dp = do[viewers, h] @ v[kj, g]
            dd = np.sum(do[viewers, h] * o[:, h], axis=1)
            dv[i, g] += p @ do[viewers, h]
            dk[i, g] += float(scale) * ((p * (dp - dd)) @ q[viewers, h])
    return dk, dv
