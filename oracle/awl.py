"""Acceptance-weighted loss (AWL) of block-diffusion drafter training (oracle side).

[DScout, 前置知识: 接受加权损失 AWL 与推测采样接受规则]: the acceptance score of draft token y_j is
alpha_j = min(1, P_j(y_j) / Q_j(y_j)) (P the target, Q the draft distribution); AWL weights the loss of
block position k by the cumulative product of the earlier positions' scores, with a stop-gradient:
w_k = sg[prod_{j<k} alpha_j]. [DScout, 方法步骤详情, step 4]: the training objective is
L = sum_{r,k} I_{r,k} w_{r,k} CE(Q_{r,k}, y*_{r,k}) / (sum_{r,k} I_{r,k} w_{r,k} + eps), eps = 1e-6, over
blocks r and positions k, with I the inclusion indicator (revealed positions are context only and not
in the loss).

Readings where the pages leave a step open:

* Positions k = 0..n_pos-1 are a block's future tokens (block position k+1; position 0 of the block
  is the anchor, never predicted). w_0 = 1 (empty product), w_k = prod_{j<k} alpha_j -- the verify
  step's S(k) for k >= 1 (S(0) = 1).
* P and Q are softmaxes of the target and draft logits at temperature 1; alpha_j = 1 when
  Q_j(y_j) = 0 (as in verify); CE(Q, y*) = -log Q(y*).
* The gradient flows into the draft logits only (w is a stop-gradient; P is the frozen target):
  dL/dz^Q_{r,k,v} = I_{r,k} w_{r,k} / (sum I w + eps) * (Q_{r,k}(v) - [v = y*_{r,k}]).

TEST INFRASTRUCTURE: see the package docstring.
"""

import numpy as np

from . import verify


def _softmax(z):
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def awl_weights(alpha):
    """w_k = prod_{j<k} alpha_j for k = 0..n-1 (w_0 = 1)."""
    alpha = np.asarray(alpha, dtype=np.float64)
    return np.concatenate([[1.0], np.cumprod(alpha)[:-1]]) if alpha.size else alpha


def awl_loss(z_target, z_draft, draft_tokens, labels, include=None, eps=1e-6):
    """z_target, z_draft: [n_blocks, n_pos, V]; draft_tokens, labels: [n_blocks, n_pos] ints;
    include: [n_blocks, n_pos] bools (all when None). Returns dict(loss, weights, ce, grad)."""
    zt = np.asarray(z_target, dtype=np.float64)
    zd = np.asarray(z_draft, dtype=np.float64)
    n_blocks, n_pos, V = zd.shape
    inc = np.ones((n_blocks, n_pos), bool) if include is None else np.asarray(include, bool)
    weights = np.zeros((n_blocks, n_pos))
    ce = np.zeros((n_blocks, n_pos))
    q = _softmax(zd)
    for r in range(n_blocks):
        alpha = verify.acceptance_ratios(zt[r], zd[r], draft_tokens[r], 1.0)
        weights[r] = awl_weights(alpha)
        ce[r] = -np.log(q[r, np.arange(n_pos), labels[r]])
    num = float(np.sum(inc * weights * ce))
    den = float(np.sum(inc * weights))
    loss = num / (den + eps)
    onehot = np.zeros_like(q)
    for r in range(n_blocks):
        onehot[r, np.arange(n_pos), labels[r]] = 1.0
    grad = (inc * weights)[..., None] / (den + eps) * (q - onehot)
    return dict(loss=loss, weights=weights, ce=ce, grad=grad, num=num, den=den)
