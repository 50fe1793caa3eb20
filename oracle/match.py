"""Branch-cache hit test (oracle side).

[D3D, 前置知识: 异步起草与缓存命中]: after verification, if the verified prefix equals the
start of one of the pre-drafted branches, the branch is a cache hit and its remaining draft tokens
are reused; otherwise ([D3D, 核心方法]) a synchronous draft round is run.

Reading (the pages leave this open): the verified prefix is the accepted slice a0, y_1..y_n (n =
n_accepted) followed by the resampled or bonus token t. The branch with rejection position r and
anchor a assumes the slice is the first r rows of block 0 and that its anchor comes next, so it is
a hit exactly when r = n_accepted + 1 and a = t. The first such block in pack order wins; block 0
(the current block) is never a branch.

TEST INFRASTRUCTURE: see the package docstring.
"""


def match_request(blocks, n_accepted, next_token):
    """Index (within the request's pack) of the first hit branch, or -1 on a miss.

    blocks: the request's blocks as (r, anchor, causal) triples in pack order.
    """
    for b in range(1, len(blocks)):
        r, anchor, _causal = blocks[b]
        if r == n_accepted + 1 and anchor == next_token:
            return b
    return -1
