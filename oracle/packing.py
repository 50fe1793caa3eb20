"""Packing of one asynchronous draft forward (oracle side).

[D3D, 方法步骤详情 step 4] and [D3D, 技术新颖性]: while the target verifies the current B-token
block, one packed drafter forward pre-drafts a successor block for each of the first C-1
rejection positions, with F alternative anchors each, plus one block for the full-accept case;
the budget is N_async = B[(C-1)F + 2] tokens (384 at B=16, C=12, F=2).
[D3D, 核心方法]: the prefix is shared and causally encoded; attention inside a block is
bidirectional. [D3D, 前置知识: 异步起草与缓存命中]: a branch is reused when the verified prefix
equals the start of that branch.

Readings where the pages leave a step open:

* The "+2" is the full-accept block plus the current block itself (block 0): the branches need
  the current block's own key/value rows for the accepted slice, so they are produced in this pass.
* Block 0 is causal inside itself (its rows are the causal context the branches read); branch and
  full-accept blocks are bidirectional.
* Position 0 of a block is its anchor and positions 1..B-1 its drafts. The branch for rejection
  position k (draft k rejected, k = 1..C-1) keeps the accepted slice a0, d_1..d_{k-1}, i.e. the
  first r = k rows of block 0; the full-accept branch has r = B.
* Blocks are ordered: block 0, then (k, f) for k = 1..C-1 and f = 1..F with k major, then the
  full-accept block.

TEST INFRASTRUCTURE: see the package docstring.
"""

import numpy as np


def n_async(B, C, F):
    """Token budget of one packed async draft forward: B[(C-1)F + 2]."""
    return B * ((C - 1) * F + 2)


def pack_blocks(B, C, F, cur_anchor, alt_anchors):
    """Blocks of one packed forward in pack order, as (r, anchor, causal) triples.

    alt_anchors holds (C-1)*F branch anchors, k-major, followed by the full-accept anchor.
    """
    if not (2 <= C <= B and F >= 1):
        raise ValueError("need 2 <= C <= B and F >= 1")
    alt_anchors = list(alt_anchors)
    if len(alt_anchors) != (C - 1) * F + 1:
        raise ValueError("need (C-1)*F + 1 anchors")
    blocks = [(0, int(cur_anchor), True)]
    for k in range(1, C):
        for f in range(F):
            blocks.append((k, int(alt_anchors[(k - 1) * F + f]), False))
    blocks.append((B, int(alt_anchors[(C - 1) * F]), False))
    return blocks


def visible_mask(B, blocks, prefix_len):
    """Dense visibility of one request's packed forward: bool [n_q, prefix_len + n_q].

    Key index j < prefix_len is prefix token j; key index prefix_len + t is packed row t.
    Row t = b*B + i (block b, position i) sees: every prefix token; when b >= 1, rows [0, r_b)
    of block 0 (the accepted slice its branch assumes); and the rows of its own block -- all of
    them if the block is bidirectional, rows 0..i if it is causal.
    """
    n_q = len(blocks) * B
    L = int(prefix_len)
    mask = np.zeros((n_q, L + n_q), dtype=bool)
    mask[:, :L] = True
    for b, (r, _anchor, causal) in enumerate(blocks):
        own = L + b * B
        for i in range(B):
            t = b * B + i
            if b >= 1 and r > 0:
                mask[t, L:L + r] = True
            if causal:
                mask[t, own:own + i + 1] = True
            else:
                mask[t, own:own + B] = True
    return mask
