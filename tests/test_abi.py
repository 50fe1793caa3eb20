"""The C-ABI library loads and exports every symbol include/d3d.h declares; host-side logic
(descriptor builder, argument validation, workspace sizing) checked without a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

from block_diffusion_drafting_draft_amd import _binding
from oracle import packing

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "d3d.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"sizeof"})


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ("d3d_build_branch_descs", "d3d_build_branch_descs_batch", "d3d_build_branch_descs_device",
                 "draft_attn_packed", "draft_attn_packed_workspace",
                 "spec_verify", "spec_verify_workspace", "branch_cache_match", "draft_topk", "draft_topk_workspace",
                 "draft_sample", "draft_sample_workspace",
                 "kv_commit", "awl_loss", "awl_loss_workspace", "train_attn_workspace", "train_attn_fwd",
                 "train_attn_bwd", "spec_verify_match", "draft_attn_packed_join", "d3d_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_binding.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_binding.EXPORTS) == set(_declared_functions())


def test_binding_has_every_entry_point_by_name():
    """The Python binding carries a function of the same name for every declared entry point, and the
    package re-exports each of them."""
    import block_diffusion_drafting_draft_amd as pkg
    for name in _declared_functions():
        if name == "d3d_status_string":
            continue
        assert callable(getattr(_binding, name, None)), name
        assert name in pkg.__all__, name
        assert getattr(pkg, name) is getattr(_binding, name)


@pytest.mark.parametrize("B,C,F,L", [(16, 12, 2, 4096), (32, 16, 5, 8192), (4, 3, 1, 0), (8, 8, 3, 7)])
def test_descriptor_builder_matches_oracle_packing(B, C, F, L):
    rng = np.random.default_rng(B * 100 + C)
    anchors = rng.integers(0, 151936, size=(C - 1) * F + 1)
    a0 = int(rng.integers(0, 151936))
    d = _binding.d3d_build_branch_descs(B, C, F, L, a0, anchors)
    blocks = packing.pack_blocks(B, C, F, a0, anchors)
    assert d.shape == (len(blocks), 4)
    assert len(blocks) * B == packing.n_async(B, C, F)
    for row, (r, anchor, causal) in zip(d, blocks):
        assert tuple(int(x) for x in row) == (L, r, anchor, 1 if causal else 0)


@pytest.mark.parametrize("B,C,F", [(16, 12, 2), (32, 16, 5), (4, 3, 1)])
def test_batched_descriptor_builder_matches_per_request(B, C, F):
    rng = np.random.default_rng(7 * B + C)
    n_req = 5
    lens = rng.integers(0, 9000, size=n_req)
    cur = rng.integers(0, 151936, size=n_req)
    alt = rng.integers(0, 151936, size=(n_req, (C - 1) * F + 1))
    out = np.full((n_req * ((C - 1) * F + 2) + 3, 4), -7, dtype=np.int32)
    d, off = _binding.d3d_build_branch_descs_batch(B, C, F, lens, cur, alt, out=out)
    want = [_binding.d3d_build_branch_descs(B, C, F, int(lens[i]), int(cur[i]), alt[i]) for i in range(n_req)]
    assert np.array_equal(d, np.concatenate(want))
    assert off.tolist() == np.concatenate([[0], np.cumsum([len(w) for w in want])]).tolist()
    assert (out[len(d):] == -7).all()  # nothing written past the batch
    with pytest.raises(RuntimeError, match="status -1"):
        _binding.d3d_build_branch_descs_batch(B, C, F, lens, cur, alt, out=out[:len(d) - 1])
    with pytest.raises(RuntimeError, match="status -1"):
        _binding.d3d_build_branch_descs_batch(B, C, F, np.r_[lens[:-1], -1], cur, alt)


def test_descriptor_builder_rejects_bad_arguments():
    with pytest.raises(RuntimeError, match="status -1"):
        _binding.d3d_build_branch_descs(16, 17, 2, 0, 0, np.zeros(40))
    with pytest.raises(RuntimeError, match="status -1"):
        _binding.d3d_build_branch_descs(16, 1, 2, 0, 0, np.zeros(40))
    with pytest.raises(RuntimeError, match="status -1"):
        _binding.d3d_build_branch_descs(16, 12, 0, 0, 0, np.zeros(40))


def test_status_strings():
    lib = _binding.load()
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.d3d_status_string(code)


def test_host_validation_returns_before_launch():
    """Bad shapes are rejected on the host (no device pointer is touched)."""
    lib = _binding.load()
    off = (ctypes.c_int32 * 2)(0, 24)
    pre = (ctypes.c_int32 * 1)(4096)
    fake = ctypes.c_void_p(256)
    args = dict(page_table=None, page_size=16, max_pages=0, num_pages=0, kv_stride=4096)

    def attn(hq=32, hkv=8, d=128, B=16, n_req=1, scale=0.088):
        return lib.draft_attn_packed(0, fake, fake, fake, fake, fake, None, 16, 0, 0, 4096, fake, off, pre,
                                     n_req, B, hq, hkv, d, scale, fake, None, 0, None)

    assert attn(d=96) == -2           # head_dim not in {64, 128}
    assert attn(hq=24, hkv=8) == -2   # group size 3
    assert attn(hq=30, hkv=8) == -1   # not a multiple
    assert attn(B=65) == -1
    assert attn(n_req=0) == -1
    assert attn(scale=0.0) == -1
    assert attn() == -4               # the 8-way split needs a workspace
    assert lib.spec_verify(0, fake, fake, fake, 1, 64, 100, 1.0, 0, 0, fake, fake, None, None, None, None,
                           fake, 1 << 20, None) == -1
    assert lib.spec_verify(0, fake, fake, fake, 1, 15, 100, -1.0, 0, 0, fake, fake, None, None, None, None,
                           fake, 1 << 20, None) == -1
    assert lib.spec_verify(0, fake, fake, fake, 1, 15, 100, 1.0, 0, 0, fake, fake, None, None, None, None,
                           fake, 16, None) == -4
    assert lib.branch_cache_match(fake, 0, fake, 1, fake, fake, fake, None) == -1


def test_workspace_sizes():
    # async pack, 384 queries, 4096-token prefix: too few (row tile, head) items for the device, so the
    # prefix is cut into s key splits; the workspace holds s fp32 partial rows (d values + max + sum)
    # per query-head row
    per_split = 384 * 32 * 130 * 4
    for dt in ("bf16", "f32"):
        ws = _binding.draft_attn_packed_workspace(dt, [0, 24], [4096], 16, 32, 8, 128)
        assert ws % per_split == 0 and 2 <= ws // per_split <= 16, (dt, ws)
    # a serving batch of 16 requests has enough items that no request is split
    assert _binding.draft_attn_packed_workspace("bf16", list(range(0, 17 * 24, 24)), [4096] * 16, 16, 32, 8, 128) == 0
    # no prefix: nothing to split
    assert _binding.draft_attn_packed_workspace("bf16", [0, 24], [0], 16, 32, 8, 128) == 0
    # invalid head shape
    assert _binding.draft_attn_packed_workspace("bf16", [0, 24], [4096], 16, 32, 8, 96) == 0
    assert _binding.spec_verify_workspace(16, 15, 151936) > 0
    assert _binding.spec_verify_workspace(1, 64, 10) == 0
    # statistics partials (16 B per row and chunk), sample records (40 B per request and 2048-token
    # chunk), per-request counters (256 B apart), each region 256-aligned. The statistics grid stays
    # within 1024 workgroups: 2 chunks per row for the serving batch's 496 rows, the cap of 8 for one
    # request's 31 rows.
    align = lambda x: (x + 255) // 256 * 256
    assert _binding.spec_verify_workspace(16, 15, 151936) == align(16 * 496 * 2) + align(40 * 16 * 75) + 16 * 256
    assert _binding.spec_verify_workspace(1, 15, 151936) == align(16 * 31 * 8) + align(40 * 75) + 256


def test_topk_workspace():
    # rows x chunks x k candidates of 8 bytes, 256-byte aligned; chunks fill 4096 workgroups (two
    # rounds of 8 per CU; at most 32 per row, at least 1024 tokens each): 4096 // 384 = 10 per row
    assert _binding.draft_topk_workspace(384, 151936, 1) == 384 * 10 * 8
    assert _binding.draft_topk_workspace(11, 151936, 2) % 256 == 0
    assert _binding.draft_topk_workspace(11, 151936, 2) >= 11 * 32 * 2 * 8
    assert _binding.draft_topk_workspace(1, 7, 8) == 256
    for bad in ((0, 10, 1), (1, 0, 1), (1, 10, 0), (1, 10, 9)):
        assert _binding.draft_topk_workspace(*bad) == 0


def test_noalloc_verify_rejects_calls_beyond_its_scratch():
    """spec_verify_noalloc checks the call's workspace against its static scratch on the host and
    returns D3D_ESCRATCH before anything runs (the pointers below are never dereferenced)."""
    lib = _binding.load()
    n_req, nd, V = 4096, 15, 151936
    need = lib.spec_verify_workspace(n_req, nd, V)
    assert need > (6 << 20)
    fake = ctypes.c_void_p(1 << 40)
    st = lib.spec_verify_noalloc(_binding.D3D_BF16, fake, fake, fake, n_req, nd, V, 1.0, 1, 0, fake, fake, None,
                                 None, None, None, None)
    assert st == -5
    assert b"scratch" in lib.d3d_status_string(st)


def test_device_descriptor_builder_rejects_bad_arguments_before_launching():
    """d3d_build_branch_descs_device validates on the host (the fake pointers are never used)."""
    lib = _binding.load()
    fake = ctypes.c_void_p(1 << 40)
    for n_req, B, C, F in ((0, 16, 12, 2), (1, 65, 12, 2), (1, 16, 17, 2), (1, 16, 1, 2), (1, 16, 12, 0),
                           (1 << 26, 64, 64, 1000)):
        st = lib.d3d_build_branch_descs_device(n_req, B, C, F, fake, fake, fake, fake, None, None)
        assert st == -1, (n_req, B, C, F, st)
    assert lib.d3d_build_branch_descs_device(4, 16, 12, 2, None, fake, fake, fake, None, None) == -1
    assert lib.d3d_build_branch_descs_device(4, 16, 12, 2, fake, fake, fake, None, None, None) == -1
