"""Pins of the training-time packed attention oracle (oracle/train_attn.py): a hand-written
visibility table, torch's scaled-dot-product attention and its autograd gradients (float64, CPU),
central finite differences, and the independence properties the packing implies."""

import numpy as np
import pytest
import torch

from oracle import train_attn as ta


def _inputs(rng, n, hq, hkv, d):
    return (rng.normal(size=(n, hq, d)), rng.normal(size=(n, hkv, d)), rng.normal(size=(n, hkv, d)))


def test_visibility_table_by_hand():
    # response of 6 tokens, anchors at positions 2 and 4, blocks of 2 -> rows 6, 7 (anchor 2) and 8, 9
    want = [
        "1000000000",
        "1100000000",
        "1110000000",
        "1111000000",
        "1111100000",
        "1111110000",
        "1100001100",  # block 0 sees response keys 0, 1 (before its anchor) and its own rows 6, 7
        "1100001100",
        "1111000011",  # block 1 sees response keys 0..3 and its own rows 8, 9
        "1111000011",
    ]
    got = ta.visible_mask(6, [2, 4], 2)
    assert ["".join("1" if x else "0" for x in row) for row in got] == want


def test_anchor_zero_sees_only_its_block():
    m = ta.visible_mask(4, [0], 3)
    assert not m[4:, :4].any() and m[4:, 4:].all()


def _torch_sdpa(q, k, v, mask, scale, grad_out=None):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    grp = q.shape[1] // k.shape[1]
    kk = kt.repeat_interleave(grp, dim=1)
    vv = vt.repeat_interleave(grp, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.transpose(0, 1), kk.transpose(0, 1), vv.transpose(0, 1),
        attn_mask=torch.tensor(mask)[None], scale=scale).transpose(0, 1)
    if grad_out is None:
        return o.detach().numpy()
    o.backward(torch.tensor(grad_out, dtype=torch.float64))
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("L,anchors,B,hq,hkv,d", [
    (40, [3, 17, 17, 30, 39], 8, 4, 2, 16),
    (64, [0, 5, 60], 16, 8, 2, 32),
    (24, [10, 2, 23], 24, 2, 1, 8),   # unsorted anchors, B = 24
])
def test_forward_and_gradients_match_torch(L, anchors, B, hq, hkv, d):
    rng = np.random.default_rng(L + B)
    n = ta.n_rows(L, len(anchors), B)
    q, k, v = _inputs(rng, n, hq, hkv, d)
    do = rng.normal(size=(n, hq, d))
    scale = d ** -0.5
    o, lse = ta.forward(q, k, v, L, anchors, B, scale)
    mask = ta.visible_mask(L, anchors, B)
    t_o, t_dq, t_dk, t_dv = _torch_sdpa(q, k, v, mask, scale, grad_out=do)
    assert np.allclose(o, t_o, rtol=1e-12, atol=1e-12)
    dq, dk, dv = ta.backward(q, k, v, do, L, anchors, B, scale)
    assert np.allclose(dq, t_dq, rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, t_dk, rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, t_dv, rtol=1e-10, atol=1e-12)
    # lse: the row's log-partition, checked against its definition on one row per head
    s = (q[n - 1, 0] @ k[:, 0].T) * scale
    assert np.isclose(lse[n - 1, 0], np.log(np.exp(s[mask[n - 1]]).sum()), rtol=1e-13)


def test_gradients_match_finite_differences():
    rng = np.random.default_rng(7)
    L, anchors, B, hq, hkv, d = 5, [1, 3], 2, 2, 1, 3
    n = ta.n_rows(L, len(anchors), B)
    q, k, v = _inputs(rng, n, hq, hkv, d)
    do = rng.normal(size=(n, hq, d))
    scale = 0.7
    dq, dk, dv = ta.backward(q, k, v, do, L, anchors, B, scale)
    f = lambda q_, k_, v_: float(np.sum(ta.forward(q_, k_, v_, L, anchors, B, scale)[0] * do))
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0), (n - 1, hq - 1 if name == "q" else 0, d - 1), (L + 1, 0, 1), (2, 0, 2)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(num - g[idx]) < 1e-6, (name, idx, num, g[idx])


def test_what_a_row_may_depend_on():
    """Response rows ignore every block; a block ignores the response from its anchor on and every
    other block (perturbing those keys / values changes nothing)."""
    rng = np.random.default_rng(3)
    L, anchors, B, hq, hkv, d = 20, [4, 12, 15], 4, 2, 1, 8
    n = ta.n_rows(L, len(anchors), B)
    q, k, v = _inputs(rng, n, hq, hkv, d)
    o, _ = ta.forward(q, k, v, L, anchors, B, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[L:] += 5.0
    v2[L:] -= 3.0
    o2, _ = ta.forward(q, k2, v2, L, anchors, B, 0.5)
    assert np.array_equal(o[:L], o2[:L])
    i = 1
    r0 = L + i * B
    k3, v3 = k.copy(), v.copy()
    keep = np.zeros(n, bool)
    keep[:anchors[i]] = True
    keep[r0:r0 + B] = True
    k3[~keep] = rng.normal(size=k3[~keep].shape)
    v3[~keep] = rng.normal(size=v3[~keep].shape)
    o3, _ = ta.forward(q, k3, v3, L, anchors, B, 0.5)
    assert np.allclose(o3[r0:r0 + B], o[r0:r0 + B], rtol=0, atol=1e-14)


def test_row_and_key_restrictions_match_torch():
    """forward_rows / backward_rows / backward_keys (the oracle evaluated on some rows or keys only, for
    shapes where every row would be too much work) against torch's autograd on the whole problem."""
    rng = np.random.default_rng(21)
    L, anchors, B, hq, hkv, d = 48, [5, 20, 20, 47], 8, 4, 2, 16
    n = ta.n_rows(L, len(anchors), B)
    q, k, v = _inputs(rng, n, hq, hkv, d)
    do = rng.normal(size=(n, hq, d))
    scale = d ** -0.5
    mask = ta.visible_mask(L, anchors, B)
    t_o, t_dq, t_dk, t_dv = _torch_sdpa(q, k, v, mask, scale, grad_out=do)
    rows = [0, 1, 19, L - 1, L, L + 9, n - 1]
    o, lse = ta.forward_rows(q, k, v, L, anchors, B, scale, rows)
    assert np.allclose(o, t_o[rows], rtol=1e-12, atol=1e-12)
    s = (q[rows[3], 1] @ k[:, 0].T) * scale
    assert np.isclose(lse[3, 1], np.log(np.exp(s[mask[rows[3]]]).sum()), rtol=1e-13)
    assert np.allclose(ta.backward_rows(q, k, v, do, L, anchors, B, scale, rows), t_dq[rows], rtol=1e-10, atol=1e-12)
    keys = [0, 4, 5, 30, L - 1, L, L + 17, n - 1]
    dk, dv = ta.backward_keys(q, k, v, do, L, anchors, B, scale, keys)
    assert np.allclose(dk, t_dk[keys], rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, t_dv[keys], rtol=1e-10, atol=1e-12)
