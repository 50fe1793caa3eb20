"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no step of the method itself: it only draws logits, activations, draft tokens,
anchors and page layouts of the shapes and distributions of the workloads below, and converts
float32 to bfloat16 bit patterns. Both the HIP path and the CPU oracle consume what it returns.

The workloads stand in for the pages' benchmarks (GSM8K ... MT-Bench), which are not used: only
their shapes are taken, with a Qwen3-8B-shaped drafter attention layer (32 query heads, 8 key/value
heads, head dim 128) and a 151936-token vocabulary.

Distributions:
* attention activations: q, k, v ~ N(0, 1) (standard deviation 1), rounded to bfloat16 by
  round-to-nearest-even (float32 for the tiny workload);
* vocabulary logits: either i.i.d. N(0, sigma) for target and draft rows, or target rows
  N(0, 2) - 1.1 * ln(rank) with rank a seeded random permutation of 1..V per row (a Zipf(1.1)
  rank bias) and draft rows = target rows + N(0, sigma_noise);
* draft tokens are sampled from softmax(z_draft / T) by the Gumbel-max construction (argmax for
  T = 0), from NumPy's generator (not from the generator the verify step uses);
* anchors for rejection position k: the F highest draft logits of row k-1 other than the draft token
  there (ties to the lower id); the full-accept anchor is the argmax of one extra draft row;
* prefix lengths of the serving batch are uniform on [1024, 16384]; paged key/value caches use
  16-token pages whose physical order is a seeded random permutation; a last page may be partial.
"""

from dataclasses import dataclass, field

import numpy as np


# --------------------------------------------------------------------------------------------
# bfloat16 bit patterns (NumPy has no bfloat16 dtype)
# --------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x):
    """float32 values rounded to the nearest bfloat16 value."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# --------------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "bf16" or "f32": activations and logits
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    block_size: int            # B
    coverage: int              # C (rejection positions 1..C-1 get branches); 0 = one sync block
    fanout: int                # F
    prefix: tuple              # prefix length per request (resolved), or () for serving draws
    n_req: int
    paged: bool
    vocab: int
    logits: str                # "iid" or "zipf"
    logit_sigma: float         # iid sigma, or the draft-noise sigma for "zipf"
    temperature: float
    seed: int                  # NumPy seed of every draw
    philox_seed: int           # key of the verify step's uniforms
    page_size: int = 16
    extra: dict = field(default_factory=dict, compare=False, hash=False)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-fp32-h1-d64-L128-V1024", "f32", 1, 1, 64, 16, 0, 0, (128,), 1, False,
                 1024, "iid", 1.5, 1.0, 1, 0xD3D0),
        Workload("sync-bf16-L2048-V151936", "bf16", 32, 8, 128, 16, 0, 0, (2048,), 1, False,
                 151936, "zipf", 0.5, 1.0, 2, 0xD3D1),
        Workload("async-B16C12F2-L4096-V151936", "bf16", 32, 8, 128, 16, 12, 2, (4096,), 1, False,
                 151936, "zipf", 0.5, 1.0, 3, 0xD3D2),
        Workload("long-B32C16F5-L8192-V151936", "bf16", 32, 8, 128, 32, 16, 5, (8192,), 1, False,
                 151936, "zipf", 1.0, 1.0, 4, 0xD3D3),
        Workload("serve-16req-B16C12F2-paged16-V151936", "bf16", 32, 8, 128, 16, 12, 2, (), 16, True,
                 151936, "zipf", 0.5, 1.0, 5, 0xD3D4),
    ]
}

ASYNC = "async-B16C12F2-L4096-V151936"


def n_blocks(w):
    """Blocks per request: one synchronous block, or the async pack's (C-1)F + 2."""
    return 1 if w.coverage == 0 else (w.coverage - 1) * w.fanout + 2


def prefix_lengths(w):
    """Prefix length of every request (serving draws are seeded and inclusive on [1024, 16384])."""
    if w.prefix:
        return list(w.prefix)
    rng = np.random.default_rng([w.seed, 17])
    return [int(x) for x in rng.integers(1024, 16384, size=w.n_req, endpoint=True)]


def _cast(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def device_bits(x, dtype):
    """Host buffer the library reads: bfloat16 bit patterns (uint16) or float32."""
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


# --------------------------------------------------------------------------------------------
# Verify inputs
# --------------------------------------------------------------------------------------------

def _gumbel_argmax(rng, z, temperature):
    if temperature == 0.0:
        return np.argmax(z, axis=-1)
    g = -np.log(-np.log(rng.random(z.shape)))
    return np.argmax(z.astype(np.float64) / temperature + g, axis=-1)


def _top_excluding(row, exclude, k):
    order = np.lexsort((np.arange(row.size), -row.astype(np.float64)))  # descending, ties to low id
    order = order[order != exclude]
    return [int(v) for v in order[:k]]


def verify_inputs(w, n_req=None, vocab=None, block_size=None, seed=None, temperature=None):
    """Logits, draft tokens and anchors for one verification round.

    Returns a dict with float32 (bf16-exact for bf16 workloads) arrays:
      z_target [n_req, B, V], z_draft [n_req, B-1, V], tokens int32 [n_req, B-1],
      cur_anchor int32 [n_req], alt_anchors int32 [n_req, (C-1)F+1] (async workloads),
      temperature, philox_seed.
    """
    n_req = w.n_req if n_req is None else n_req
    V = w.vocab if vocab is None else vocab
    B = w.block_size if block_size is None else block_size
    T = w.temperature if temperature is None else temperature
    rng = np.random.default_rng([w.seed if seed is None else seed, 1])
    if w.logits == "iid":
        zt = rng.normal(0.0, w.logit_sigma, size=(n_req, B, V))
        zd = rng.normal(0.0, w.logit_sigma, size=(n_req, B - 1, V))
        zx = rng.normal(0.0, w.logit_sigma, size=(n_req, V))
    else:
        zt = rng.normal(0.0, 2.0, size=(n_req, B, V)).astype(np.float32)
        ranks = np.empty((n_req, B, V), dtype=np.float32)
        base = np.arange(1, V + 1, dtype=np.float32)
        for i in range(n_req):
            for j in range(B):
                ranks[i, j] = rng.permutation(base)
        zt -= np.float32(1.1) * np.log(ranks)
        zd = zt[:, :B - 1] + rng.normal(0.0, w.logit_sigma, size=(n_req, B - 1, V)).astype(np.float32)
        zx = zt[:, B - 1] + rng.normal(0.0, w.logit_sigma, size=(n_req, V)).astype(np.float32)
    zt = _cast(zt, w.dtype)
    zd = _cast(zd, w.dtype)
    zx = _cast(zx, w.dtype)
    tokens = _gumbel_argmax(rng, zd, T).astype(np.int32)
    out = dict(z_target=zt, z_draft=zd, tokens=tokens, temperature=float(T),
               philox_seed=w.philox_seed, vocab=V, block_size=B)
    out["cur_anchor"] = rng.integers(0, V, size=n_req).astype(np.int32)
    if w.coverage:
        C, F = w.coverage, w.fanout
        alt = np.empty((n_req, (C - 1) * F + 1), dtype=np.int32)
        for i in range(n_req):
            for k in range(1, C):
                alt[i, (k - 1) * F:k * F] = _top_excluding(zd[i, k - 1], tokens[i, k - 1], F)
            alt[i, (C - 1) * F] = int(np.argmax(zx[i]))
        out["alt_anchors"] = alt
        out["z_next"] = zx  # the draft row of the position after the block (full-accept anchor)
    return out


# --------------------------------------------------------------------------------------------
# Drafter-training loss inputs
# --------------------------------------------------------------------------------------------

def awl_inputs(n_blocks, n_pos, vocab, dtype="bf16", seed=0, sigma=2.0, noise=1.0, greedy=0.7, include=0.85):
    """Logits and labels of one training step's diffusion blocks (n_pos future positions each).

    Target logits are iid N(0, sigma); the draft's are the target's plus N(0, noise), so the two
    distributions agree only roughly. Draft tokens are the draft's most likely token with probability
    `greedy`, else uniform; labels are the target's most likely token with probability `greedy`, else
    uniform; each position is in the loss with probability `include`. Rows are drawn in slices so
    that no float64 copy of the whole batch is made. Returns float32 (bf16-exact for bf16) arrays
    z_target, z_draft [n_blocks, n_pos, V] and int32 tokens, labels, include [n_blocks, n_pos]."""
    rng = np.random.default_rng([seed, 23])
    rows = n_blocks * n_pos
    zt = np.empty((rows, vocab), dtype=np.float32)
    zd = np.empty((rows, vocab), dtype=np.float32)
    step = max(1, (1 << 24) // max(vocab, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        t = rng.standard_normal((r1 - r0, vocab), dtype=np.float32) * np.float32(sigma)
        d = t + rng.standard_normal((r1 - r0, vocab), dtype=np.float32) * np.float32(noise)
        zt[r0:r1] = _cast(t, dtype)
        zd[r0:r1] = _cast(d, dtype)
    pick = lambda z: np.where(rng.random(rows) < greedy, np.argmax(z, axis=1), rng.integers(0, vocab, size=rows))
    tokens = pick(zd).astype(np.int32).reshape(n_blocks, n_pos)
    labels = pick(zt).astype(np.int32).reshape(n_blocks, n_pos)
    inc = (rng.random(rows) < include).astype(np.int32).reshape(n_blocks, n_pos)
    return dict(z_target=zt.reshape(n_blocks, n_pos, vocab), z_draft=zd.reshape(n_blocks, n_pos, vocab),
                tokens=tokens, labels=labels, include=inc)


# --------------------------------------------------------------------------------------------
# Attention inputs
# --------------------------------------------------------------------------------------------

def attention_inputs(w, prefix=None, n_q=None, n_heads_q=None, n_heads_kv=None, head_dim=None,
                     seed=None, needles=0):
    """Activations of one drafter attention layer for every request of the workload.

    Returns a dict: q [N_q_total, H_q, d], k_new / v_new [N_q_total, H_kv, d] (requests packed one
    after another), k_prefix / v_prefix (list per request of [L_i, H_kv, d]), prefix (list of L_i),
    q_per_req (list). With needles > 0, that many queries per request get a planted prefix key
    aligned with them (peaky softmax, outputs of order one).
    """
    Hq = w.n_heads_q if n_heads_q is None else n_heads_q
    Hkv = w.n_heads_kv if n_heads_kv is None else n_heads_kv
    d = w.head_dim if head_dim is None else head_dim
    lens = prefix_lengths(w) if prefix is None else list(prefix)
    nq = w.block_size * n_blocks(w) if n_q is None else n_q
    rng = np.random.default_rng([w.seed if seed is None else seed, 2])
    tot = nq * len(lens)
    q = _cast(rng.standard_normal((tot, Hq, d), dtype=np.float32), w.dtype)
    k_new = _cast(rng.standard_normal((tot, Hkv, d), dtype=np.float32), w.dtype)
    v_new = _cast(rng.standard_normal((tot, Hkv, d), dtype=np.float32), w.dtype)
    kp, vp = [], []
    for i, L in enumerate(lens):
        k = rng.standard_normal((L, Hkv, d), dtype=np.float32)
        v = rng.standard_normal((L, Hkv, d), dtype=np.float32)
        if needles and L > 0:
            group = Hq // Hkv
            rows = rng.choice(nq, size=min(needles, nq), replace=False)
            for t in rows:
                h = int(rng.integers(0, Hq))
                pos = int(rng.integers(0, L))
                k[pos, h // group] = 3.0 * q[i * nq + t, h]
        kp.append(_cast(k, w.dtype))
        vp.append(_cast(v, w.dtype))
    return dict(q=q, k_new=k_new, v_new=v_new, k_prefix=kp, v_prefix=vp, prefix=lens,
                q_per_req=[nq] * len(lens), n_heads_q=Hq, n_heads_kv=Hkv, head_dim=d)


def paginate(prefixes, page_size, seed):
    """Scatter per-request prefixes [L_i, H, d] into a shared page pool in a random physical order.

    Returns (pages [n_pages, page_size, H, d], page_table int32 [n_req, max_pages]); unused table
    entries are -1 and the unused tail of a partial last page is zero.
    """
    counts = [-(-p.shape[0] // page_size) for p in prefixes]
    total = sum(counts)
    max_pages = max(max(counts), 1)
    rng = np.random.default_rng([seed, 3])
    phys = rng.permutation(total)
    h, d = prefixes[0].shape[1:]
    pages = np.zeros((total, page_size, h, d), dtype=prefixes[0].dtype)
    table = np.full((len(prefixes), max_pages), -1, dtype=np.int32)
    nxt = 0
    for i, p in enumerate(prefixes):
        for j in range(counts[i]):
            page = phys[nxt]
            nxt += 1
            chunk = p[j * page_size:(j + 1) * page_size]
            pages[page, :chunk.shape[0]] = chunk
            table[i, j] = page
    return pages, table
