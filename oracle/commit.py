"""KV commit of the accepted slice and promotion of the hit branch (oracle side).

[D3D, 前置知识: 异步起草与缓存命中]: after verification the verified prefix grows, and when it
starts like a pre-drafted branch that branch's remaining draft is reused (a cache hit); otherwise a
synchronous draft round runs. [D3D, 方法步骤详情 step 4]: the packed forward that drafted the
branches also ran the current block under prefix-shared causal encoding. Readings where the
pages leave a step open:

* The verified prefix grows by the anchor and the accepted drafts (a0, d_1 .. d_{n_acc}); the
  resampled or bonus token is the next block's anchor, whose keys / values the next forward computes.
* Their drafter keys / values are rows 0 .. n_acc of the request's block 0 in the packed rows: block 0
  is causal (R2), so row j saw exactly the prefix and rows 0 .. j, as a prefix token does.
* They are written to the paged cache at token positions prefix_len .. prefix_len + n_acc (token t
  lives in page page_table[t // page_size], slot t % page_size). A row without a slot (page index past
  the table, or page id outside the cache) is skipped; the prefix grows by the rows before the first
  such row and the request is flagged.
* Promotion: on a hit the next round's current block is the hit branch's B packed tokens (its anchor
  and its remaining draft); on a miss there is none (-1).

TEST INFRASTRUCTURE: see the package docstring.
"""

import numpy as np


def kv_commit(k_new, v_new, k_cache, v_cache, page_table, req_block_off, prefix_len, n_accepted, B):
    """Returns (k_cache, v_cache, prefix_len, status) after the commit; the inputs are not modified.
    k_new / v_new [N_q, H_kv, d]; caches [pages, page_size, H_kv, d]; page_table [n_req, max_pages]."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    num_pages, page_size = kc.shape[0], kc.shape[1]
    n_req, max_pages = len(n_accepted), page_table.shape[1]
    new_len = np.array(prefix_len, dtype=np.int64, copy=True)
    status = np.zeros(n_req, dtype=np.int64)
    for i in range(n_req):
        n = min(max(int(n_accepted[i]), 0), B - 1) + 1
        first = n
        for j in range(n):
            t = int(prefix_len[i]) + j
            page = int(page_table[i, t // page_size]) if 0 <= t and t // page_size < max_pages else -1
            if not 0 <= page < num_pages:
                first = min(first, j)
                continue
            src = int(req_block_off[i]) * B + j
            kc[page, t % page_size] = k_new[src]
            vc[page, t % page_size] = v_new[src]
        new_len[i] = int(prefix_len[i]) + first
        status[i] = 1 if first < n else 0
    return kc, vc, new_len, status


def promote(packed_tokens, req_block_off, hit, B):
    """The next round's current block per request: the hit branch's B packed tokens, or -1s."""
    n_req = len(hit)
    out = np.full((n_req, B), -1, dtype=np.int64)
    for i in range(n_req):
        h, blocks = int(hit[i]), int(req_block_off[i + 1]) - int(req_block_off[i])
        if 1 <= h < blocks:
            b = int(req_block_off[i]) + h
            out[i] = packed_tokens[b * B:(b + 1) * B]
    return out
