"""GPU parity of kv_commit (the accepted slice appended to the paged cache, the hit branch promoted)
against the oracle, through the C ABI. Bar: bit-exact (copies and integers)."""

import sys

import numpy as np
import pytest
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from gpu_util import dev, require_gpu
from oracle import commit as o_commit

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _host(t, dtype):
    return t.float().cpu().numpy() if dtype == "bf16" else t.cpu().numpy()


@pytest.mark.parametrize("dtype,n_req,B,ps,hkv,d,max_pages", [
    ("bf16", 4, 16, 16, 8, 128, 6),
    ("bf16", 3, 8, 5, 2, 64, 9),
    ("f32", 2, 4, 3, 1, 4, 5),
    ("bf16", 16, 16, 16, 8, 128, 40),
])
def test_commit_parity(dtype, n_req, B, ps, hkv, d, max_pages):
    require_gpu()
    _say(f"kv_commit: {dtype} n_req {n_req} B {B} page {ps} H_kv {hkv} d {d}")
    rng = np.random.default_rng(n_req * 100 + B + ps)
    blocks = rng.integers(1, 6, size=n_req)
    off = np.concatenate([[0], np.cumsum(blocks)]).astype(np.int32)
    nq = int(off[-1]) * B
    cast = synth.round_bf16 if dtype == "bf16" else (lambda x: x.astype(np.float32))
    k_new = cast(rng.normal(size=(nq, hkv, d)).astype(np.float32))
    v_new = cast(rng.normal(size=(nq, hkv, d)).astype(np.float32))
    n_pages = n_req * max_pages
    kc = cast(rng.normal(size=(n_pages, ps, hkv, d)).astype(np.float32))
    vc = cast(rng.normal(size=(n_pages, ps, hkv, d)).astype(np.float32))
    table = rng.permutation(n_pages).reshape(n_req, max_pages).astype(np.int32)
    cap = max_pages * ps
    lens = rng.integers(0, cap - B + 1, size=n_req).astype(np.int32)
    lens[0] = cap - 2  # runs out of slots: only the leading rows are committed
    n_acc = rng.integers(-1, B + 1, size=n_req).astype(np.int32)  # clamped to [0, B-1]
    hit = np.array([int(rng.integers(-1, blocks[i])) for i in range(n_req)], dtype=np.int32)
    tokens = rng.integers(0, 151936, size=nq).astype(np.int32)

    kc_d, vc_d = dev(kc, dtype), dev(vc, dtype)
    lens_d = torch.from_numpy(lens.copy()).cuda()
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    nxt, status = _binding.kv_commit(dev(k_new, dtype), dev(v_new, dtype), kc_d, vc_d, i32(table), i32(off), lens_d,
                                     i32(n_acc), B, hit=i32(hit), packed_tokens=i32(tokens))
    torch.cuda.synchronize()
    want_k, want_v, want_len, want_status = o_commit.kv_commit(k_new, v_new, kc, vc, table, off, lens, n_acc, B)
    assert np.array_equal(_host(kc_d, dtype), want_k)
    assert np.array_equal(_host(vc_d, dtype), want_v)
    assert lens_d.cpu().numpy().tolist() == want_len.tolist()
    assert status.cpu().numpy().tolist() == want_status.tolist()
    assert want_status[0] == 1 or n_acc[0] <= 1  # two slots left for request 0
    assert np.array_equal(nxt.cpu().numpy(), o_commit.promote(tokens, off, hit, B))


def test_commit_without_promotion_and_bad_arguments():
    require_gpu()
    _say("kv_commit: no promotion, argument checks")
    B, hkv, d = 4, 2, 8
    k_new = torch.randn((2 * B, hkv, d), device="cuda").to(torch.bfloat16)
    kc = torch.zeros((4, 4, hkv, d), device="cuda", dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    table = torch.tensor([[1, 3], [0, 2]], dtype=torch.int32, device="cuda")
    off = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    lens = torch.tensor([0, 2], dtype=torch.int32, device="cuda")
    n_acc = torch.tensor([3, 0], dtype=torch.int32, device="cuda")
    nxt, status = _binding.kv_commit(k_new, k_new, kc, vc, table, off, lens, n_acc, B)
    torch.cuda.synchronize()
    assert nxt is None and status.cpu().tolist() == [0, 0] and lens.cpu().tolist() == [4, 3]
    assert torch.equal(kc[1], k_new[0:4]) and torch.equal(kc[0, 2], k_new[4])
    with pytest.raises(ValueError):
        _binding.kv_commit(k_new, k_new, kc, vc, table, off, lens, n_acc, B, hit=n_acc)
    with pytest.raises(TypeError):
        _binding.kv_commit(k_new, k_new, kc.float(), vc, table, off, lens, n_acc, B)
