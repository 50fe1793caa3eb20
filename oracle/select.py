"""Drafter token selection (oracle side).

[D3D, 方法步骤详情 step 4]: while the target verifies the current block, one packed drafter forward
drafts continuation blocks for each of the first C-1 rejection positions with F alternative
anchors each, plus a full-accept block. [D3D, 前置知识: 异步起草与缓存命中]: a branch is reused
when the verified prefix starts like it. The pages do not say how the anchors or the drafted tokens
are chosen; the readings taken here:

* The drafted token of a masked position is the most likely token of its logits (greedy drafting,
  the pages' own evaluation setting).
* The F anchors of rejection position k (1-based; rejecting draft d_k) are the F most likely tokens
  of the draft distribution Q_{k-1} (0-based row k-1, the row that judges d_k) other than d_k: a
  rejection replaces d_k by a draw from max(0, P - Q), which is zero at d_k, so d_k can never be the
  replacement. The full-accept anchor is the most likely token of the position after the block.
* Order: larger logit first, ties to the lower token id (softmax at any temperature is monotone in
  the logit, so this is the order of the probabilities). NaN logits count as -inf.
* Sampled drafting at temperature T > 0 (R21; [DScout] 实验结果 reports temperature-1 decoding):
  the token of a row is a draw from softmax(z / T), taken by the Gumbel-max rule: the token with the
  largest z_v / T + G_v, G_v = -ln(-ln u_v), ties to the lower id. The uniforms are counter-based so
  that both sides draw the same ones: u_v = ((w >> 8) + 1/2) / 2^24 with w word (v mod 4) of
  Philox4x32-10 at counter (v div 4, row index, round, 2) under the 64-bit seed.

TEST INFRASTRUCTURE: see the package docstring.
"""

import numpy as np

from . import philox


def topk(row, k, exclude=-1):
    """The k best tokens of one logit row other than `exclude`, larger logit first, ties to the lower
    id; -1 pads the result when the row has fewer than k candidates."""
    z = np.asarray(row, dtype=np.float64)
    z = np.where(np.isnan(z), -np.inf, z)
    order = np.lexsort((np.arange(z.size), -z))  # primary key -z (descending logit), then the id
    order = order[order != exclude][:k]
    out = np.full(k, -1, dtype=np.int64)
    out[:order.size] = order
    return out


def alt_anchors(z_draft, tokens, z_next, coverage, fanout):
    """Anchors of one request's branches in pack order: F per rejection position k = 1..C-1 (from
    draft row k-1, excluding d_k = tokens[k-1]), then the full-accept anchor (from z_next)."""
    out = []
    for k in range(1, coverage):
        out.extend(int(t) for t in topk(z_draft[k - 1], fanout, exclude=int(tokens[k - 1])))
    out.append(int(topk(z_next, 1)[0]))
    return np.array(out, dtype=np.int64)


def gumbel_scores(row, temperature, seed, round_, row_index):
    """z_v / T + G_v for every token of one row (float64; NaN logits count as -inf)."""
    z = np.asarray(row, dtype=np.float64)
    z = np.where(np.isnan(z), -np.inf, z)
    v = np.arange(z.size, dtype=np.uint64)
    seed = int(seed)
    words = philox.philox4x32_10(v >> np.uint64(2), int(row_index), int(round_), philox.PURPOSE_DRAFT,
                                 seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.choose((v & np.uint64(3)).astype(np.int64), words)
    u = philox.uniform24(w)
    return z / float(temperature) - np.log(-np.log(u))


def sample_token(row, temperature, seed, round_, row_index):
    """The sampled token of one row at temperature T > 0 (Gumbel-max; ties to the lower id), or -1
    when every logit is -inf."""
    s = gumbel_scores(row, temperature, seed, round_, row_index)
    if not np.isfinite(s).any() and not (s == np.inf).any():
        return -1
    return int(np.argmax(s))
