"""GPU parity of draft_topk (drafter token selection) against the oracle, through the C ABI.

Bar: bit-exact token ids (integer work; the order is a strict total order on (logit, id))."""

import sys

import numpy as np
import pytest
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from gpu_util import dev, require_gpu
from oracle import select as o_sel

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rows(rng, n, V, kind, dtype):
    if kind == "ties":  # few distinct values: ties everywhere
        z = rng.integers(-4, 5, size=(n, V)).astype(np.float32)
    elif kind == "masked":  # -inf tail and a planted NaN
        z = rng.normal(0, 2, size=(n, V)).astype(np.float32)
        z[:, V // 2:] = -np.inf
        z[0, 0] = np.nan
    else:
        z = rng.normal(0, 2, size=(n, V)).astype(np.float32)
    return synth.round_bf16(z) if dtype == "bf16" else z


CASES = [
    # dtype, n_rows, V, k, exclude, kind
    ("bf16", 5, 1000, 1, False, "normal"),
    ("bf16", 5, 1000, 2, True, "ties"),
    ("bf16", 3, 1003, 5, True, "ties"),      # V not a multiple of 8: scalar path
    ("bf16", 4, 64, 8, True, "normal"),
    ("bf16", 2, 7, 8, True, "normal"),        # fewer candidates than k: -1 padding
    ("bf16", 1, 1, 1, False, "normal"),
    ("f32", 6, 4096, 3, True, "ties"),
    ("f32", 3, 50, 8, False, "masked"),
    ("bf16", 4, 151936, 2, True, "ties"),
    ("bf16", 3, 151936, 8, True, "masked"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_topk_parity(case):
    require_gpu()
    dtype, n, V, k, use_ex, kind = case
    _say(f"draft_topk: {case}")
    rng = np.random.default_rng(V * 10 + k)
    z = _rows(rng, n, V, kind, dtype)
    ex = rng.integers(-1, V, size=n).astype(np.int32) if use_ex else None
    if use_ex and kind == "ties":
        ex[0] = int(o_sel.topk(z[0], 1)[0])  # exclude a row's own best token
    got = _binding.draft_topk(dev(z, dtype), k, exclude=None if ex is None else torch.from_numpy(ex).cuda())
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for r in range(n):
        want = o_sel.topk(z[r], k, exclude=-1 if ex is None else int(ex[r]))
        assert got[r].tolist() == want.tolist(), (r, got[r], want)


@pytest.mark.parametrize("name", ["async-B16C12F2-L4096-V151936", "long-B32C16F5-L8192-V151936",
                                  "serve-16req-B16C12F2-paged16-V151936"])
def test_branch_anchors_in_builder_layout(name):
    """The anchors of every request's branches, written by two calls straight into the
    [n_req, (C-1)F + 1] layout the descriptor builder takes: F from draft row k-1 excluding d_k for
    k = 1..C-1 (row gather + output offsets), then the full-accept anchor from the next row."""
    require_gpu()
    w = synth.WORKLOADS[name]
    _say(f"draft_topk: branch anchors of {name}")
    vin = synth.verify_inputs(w)
    n_req, nd = vin["tokens"].shape
    C, F = w.coverage, w.fanout
    per = (C - 1) * F + 1
    rows = np.array([i * nd + (k - 1) for i in range(n_req) for k in range(1, C)], dtype=np.int32)
    excl = np.array([vin["tokens"][i, k - 1] for i in range(n_req) for k in range(1, C)], dtype=np.int32)
    offs = np.array([i * per + (k - 1) * F for i in range(n_req) for k in range(1, C)], dtype=np.int32)
    alt = torch.full((n_req, per), -7, dtype=torch.int32, device="cuda")
    zd = dev(vin["z_draft"].reshape(n_req * nd, -1), w.dtype)
    _binding.draft_topk(zd, F, rows=torch.from_numpy(rows).cuda(), exclude=torch.from_numpy(excl).cuda(), out=alt,
                        out_off=torch.from_numpy(offs).cuda())
    _binding.draft_topk(dev(vin["z_next"], w.dtype), 1, out=alt,
                        out_off=torch.from_numpy(np.arange(n_req, dtype=np.int32) * per + (C - 1) * F).cuda())
    torch.cuda.synchronize()
    got = alt.cpu().numpy()
    for i in range(n_req):
        want = o_sel.alt_anchors(vin["z_draft"][i], vin["tokens"][i], vin["z_next"][i], C, F)
        assert got[i].tolist() == want.tolist(), i


def test_drafted_tokens_of_a_packed_forward():
    """Greedy drafted tokens of all 384 packed positions over a 151936-token vocabulary (k = 1)."""
    require_gpu()
    _say("draft_topk: 384 x 151936 argmax")
    rng = np.random.default_rng(11)
    z = synth.round_bf16(rng.normal(0, 3, size=(384, 151936)).astype(np.float32))
    got = _binding.draft_topk(dev(z, "bf16"), 1)
    torch.cuda.synchronize()
    want = np.argmax(z, axis=1)
    assert np.array_equal(got.cpu().numpy()[:, 0], want)


def test_bad_arguments_raise():
    require_gpu()
    z = torch.zeros((2, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        _binding.draft_topk(z, 9)
    with pytest.raises(ValueError):
        _binding.draft_topk(z, 0)
