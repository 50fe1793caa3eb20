"""GPU parity of draft_attn_packed against the oracle (through the C ABI).

Bar: bf16 inputs (fp32 accumulation) within 2e-2 absolute and 1e-2 relative Frobenius of the
float64 oracle; fp32 within 1e-4 absolute. Full-size workloads compare sampled rows (always including
the first and last row of every block kind)."""

import sys

import numpy as np
import pytest

from block_diffusion_drafting_draft_amd import synth
from gpu_util import AttnProblem, attn_close, host, require_gpu

pytestmark = pytest.mark.gpu

BF16_ATOL, BF16_FRO = 2e-2, 1e-2
F32_ATOL, F32_FRO = 1e-4, 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tol(dtype):
    return (BF16_ATOL, BF16_FRO) if dtype == "bf16" else (F32_ATOL, F32_FRO)


def _sample_rows(n_q, B, k, rng):
    edges = {0, B - 1, B, 2 * B - 1, n_q - B, n_q - 1}
    extra = rng.choice(n_q, size=min(k, n_q), replace=False)
    return np.array(sorted({r for r in edges if 0 <= r < n_q} | set(int(x) for x in extra)))


def _check(prob, rows_per_req=None, name=""):
    got = prob.run()
    import torch
    torch.cuda.synchronize()
    want, rows = prob.oracle(rows_per_req)
    g = host(got)[rows]
    ok, emax, fro = attn_close(g, want, *_tol(prob.dtype))
    _say(f"  {name}: max|err|={emax:.3g} rel_fro={fro:.3g} |want|max={np.abs(want).max():.3g}")
    assert ok, (name, emax, fro)
    # non-vacuity: an all-zero output must fail the same bar
    assert not attn_close(np.zeros_like(want), want, *_tol(prob.dtype))[0]
    return emax, fro


def _workload_problem(name, sample=None, needles=0):
    w = synth.WORKLOADS[name]
    inp = synth.attention_inputs(w, needles=needles)
    lens = inp["prefix"]
    if w.coverage:
        reqs = [dict(L=L, kind="async", C=w.coverage, F=w.fanout) for L in lens]
    else:
        reqs = [dict(L=L, kind="sync") for L in lens]
    prob = AttnProblem(w.dtype, w.block_size, reqs, inp, paged=w.paged, page_size=w.page_size, seed=w.seed)
    rows = None
    if sample:
        rng = np.random.default_rng(w.seed)
        rows = [_sample_rows(inp["q_per_req"][i], w.block_size, sample, rng) for i in range(len(lens))]
    return prob, rows


@pytest.mark.parametrize("name,sample", [
    ("tiny-fp32-h1-d64-L128-V1024", None),
    ("sync-bf16-L2048-V151936", None),
    ("async-B16C12F2-L4096-V151936", None),
    ("long-B32C16F5-L8192-V151936", 192),
    ("serve-16req-B16C12F2-paged16-V151936", 24),
])
def test_workload_parity(name, sample):
    require_gpu()
    _say(f"attention parity: {name}")
    prob, rows = _workload_problem(name, sample)
    _check(prob, rows, name)


def test_async_needles_peaky_softmax():
    """Planted keys aligned with queries give peaky attention and outputs of order one."""
    require_gpu()
    _say("attention parity: async with needles")
    prob, _ = _workload_problem("async-B16C12F2-L4096-V151936", needles=96)
    got = host(prob.run())
    want, rows = prob.oracle()
    assert np.abs(want).max() > 0.5
    ok, emax, fro = attn_close(got[rows], want, BF16_ATOL, BF16_FRO)
    _say(f"  needles: max|err|={emax:.3g} rel_fro={fro:.3g}")
    assert ok


FUZZ = [
    # dtype, B, C, F, L, Hq, Hkv, d
    ("bf16", 16, 12, 2, 0, 32, 8, 128),
    ("bf16", 16, 12, 2, 1, 32, 8, 128),
    ("bf16", 16, 12, 2, 63, 32, 8, 128),
    ("bf16", 16, 12, 2, 65, 32, 8, 128),
    ("bf16", 8, 3, 1, 200, 8, 1, 64),
    ("bf16", 24, 5, 3, 130, 4, 1, 128),
    ("bf16", 32, 16, 5, 77, 32, 8, 128),
    ("bf16", 8, 8, 5, 1000, 8, 8, 64),
    ("bf16", 16, 2, 1, 513, 16, 1, 128),
    ("bf16", 24, 24, 1, 64, 2, 1, 64),
    # plans with 3-8 key splits (split 0 also walks the in-pack tail), ragged and whole prefixes
    ("bf16", 16, 12, 2, 1024, 32, 8, 128),
    ("bf16", 16, 12, 2, 2500, 32, 8, 128),
    ("bf16", 16, 4, 2, 700, 8, 2, 128),
    ("bf16", 8, 3, 1, 1900, 8, 1, 128),
    ("bf16", 24, 5, 3, 1300, 16, 4, 128),
    ("f32", 16, 4, 2, 100, 8, 2, 64),
    ("f32", 8, 3, 2, 0, 4, 4, 128),
]


@pytest.mark.parametrize("case", FUZZ, ids=lambda c: "-".join(map(str, c)))
def test_fuzz_shapes(case):
    require_gpu()
    dtype, B, C, F, L, hq, hkv, d = case
    _say(f"attention fuzz: {case}")
    w = synth.WORKLOADS["async-B16C12F2-L4096-V151936"]
    nq = B * ((C - 1) * F + 2)
    inp = synth.attention_inputs(w, prefix=[L], n_q=nq, n_heads_q=hq, n_heads_kv=hkv, head_dim=d,
                                 seed=B * 100000 + C * 1000 + F * 100 + L + d)
    if dtype == "f32":
        for k in ("q", "k_new", "v_new"):
            inp[k] = np.random.default_rng(7).standard_normal(inp[k].shape).astype(np.float32)
        inp["k_prefix"] = [np.random.default_rng(8).standard_normal(x.shape).astype(np.float32) for x in inp["k_prefix"]]
        inp["v_prefix"] = [np.random.default_rng(9).standard_normal(x.shape).astype(np.float32) for x in inp["v_prefix"]]
    prob = AttnProblem(dtype, B, [dict(L=L, kind="async", C=C, F=F)], inp)
    _check(prob, None, str(case))


def test_multi_request_contiguous_mixed_blocks():
    """Three requests with different prefixes and block counts in one call (kv_stride > every L),
    including a synchronous single-block request and generic descriptors."""
    require_gpu()
    _say("attention: mixed multi-request contiguous")
    w = synth.WORKLOADS["async-B16C12F2-L4096-V151936"]
    B = 16
    reqs = [dict(L=300, kind="async", C=4, F=2), dict(L=0, kind="sync"),
            dict(L=129, blocks=[(0, 5, True), (3, 6, False), (16, 7, True), (0, 8, False), (9, 9, True)])]
    nblk = [8, 1, 5]
    rng = np.random.default_rng(11)
    tot = sum(nblk) * B
    inp = dict(q=synth.round_bf16(rng.standard_normal((tot, 32, 128)).astype(np.float32)),
               k_new=synth.round_bf16(rng.standard_normal((tot, 8, 128)).astype(np.float32)),
               v_new=synth.round_bf16(rng.standard_normal((tot, 8, 128)).astype(np.float32)),
               k_prefix=[synth.round_bf16(rng.standard_normal((r["L"], 8, 128)).astype(np.float32)) for r in reqs],
               v_prefix=[synth.round_bf16(rng.standard_normal((r["L"], 8, 128)).astype(np.float32)) for r in reqs])
    prob = AttnProblem("bf16", B, reqs, inp, kv_stride=512)
    _check(prob, None, "mixed")
    del w


def test_paged_small_ragged_pages():
    require_gpu()
    _say("attention: small paged batch with ragged pages")
    rng = np.random.default_rng(12)
    B, lens = 16, [1, 17, 250, 33]
    reqs = [dict(L=L, kind="async", C=3, F=2) for L in lens]
    tot = len(lens) * 6 * B
    mk = lambda *s: synth.round_bf16(rng.standard_normal(s).astype(np.float32))
    inp = dict(q=mk(tot, 8, 64), k_new=mk(tot, 2, 64), v_new=mk(tot, 2, 64),
               k_prefix=[mk(L, 2, 64) for L in lens], v_prefix=[mk(L, 2, 64) for L in lens])
    prob = AttnProblem("bf16", B, reqs, inp, paged=True, page_size=16, seed=3)
    _check(prob, None, "paged-small")


@pytest.mark.parametrize("page_size,d", [(8, 64), (4, 128), (32, 128), (5, 128), (3, 64), (1, 128)])
def test_paged_page_sizes(page_size, d):
    """Page sizes that are multiples of the rows one 16-byte-per-lane copy instruction covers
    (4 at d = 128, 8 at d = 64) take the wave-uniform page path; the others (5, 3, 1) the per-lane
    path. Prefix lengths straddle page and tile boundaries."""
    require_gpu()
    _say(f"attention: paged, page_size {page_size}, d {d}")
    rng = np.random.default_rng(100 + page_size + d)
    B, lens = 16, [70, 129, 3, 300]
    reqs = [dict(L=L, kind="async", C=3, F=2) for L in lens]
    tot = len(lens) * 6 * B
    mk = lambda *s: synth.round_bf16(rng.standard_normal(s).astype(np.float32))
    inp = dict(q=mk(tot, 8, d), k_new=mk(tot, 2, d), v_new=mk(tot, 2, d),
               k_prefix=[mk(L, 2, d) for L in lens], v_prefix=[mk(L, 2, d) for L in lens])
    prob = AttnProblem("bf16", B, reqs, inp, paged=True, page_size=page_size, seed=page_size)
    _check(prob, None, f"paged-ps{page_size}-d{d}")
