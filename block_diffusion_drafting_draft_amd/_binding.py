"""ctypes binding of libd3d.so: argument marshalling only.

Every function here has the name of the C entry point it wraps and does nothing but check the
tensors it is handed, allocate outputs with torch (device memory is plumbing), pass raw pointers and
torch's current HIP stream, and raise on a negative status. All arithmetic happens in the HIP
kernels. There is no fallback: without the built library every call raises.
"""

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libd3d.so")

D3D_BF16, D3D_F32 = 0, 1
BLOCK_CAUSAL = 1
MAX_REQ = 64

_c = ctypes
_i32p = _c.c_void_p  # host int32 array, passed as its address

_SIGNATURES = {
    "d3d_build_branch_descs": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int32, _i32p,
                                           _c.c_void_p, _c.c_int, _c.POINTER(_c.c_int)]),
    "d3d_build_branch_descs_batch": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _i32p, _i32p, _i32p,
                                                 _c.c_void_p, _c.c_int, _i32p]),
    "d3d_build_branch_descs_device": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p,
                                                  _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "draft_attn_packed_workspace": (_c.c_size_t, [_c.c_int, _i32p, _i32p, _c.c_int, _c.c_int, _c.c_int,
                                                  _c.c_int, _c.c_int]),
    "draft_attn_packed": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                     _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                     _c.c_void_p, _i32p, _i32p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                     _c.c_int, _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                     _c.c_void_p]),
    "draft_attn_packed_join": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                          _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                          _c.c_void_p, _i32p, _i32p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                          _c.c_int, _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                          _c.c_void_p, _c.c_void_p]),
    "spec_verify_workspace": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int]),
    "spec_verify": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                               _c.c_int, _c.c_float, _c.c_uint64, _c.c_uint32, _c.c_void_p, _c.c_void_p,
                               _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                               _c.c_size_t, _c.c_void_p]),
    "spec_verify_match": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                                     _c.c_int, _c.c_float, _c.c_uint64, _c.c_uint32, _c.c_void_p, _c.c_void_p,
                                     _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                     _c.c_size_t, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "spec_verify_noalloc": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                                       _c.c_int, _c.c_float, _c.c_uint64, _c.c_uint32, _c.c_void_p, _c.c_void_p,
                                       _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "branch_cache_match": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p,
                                      _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "draft_topk_workspace": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int]),
    "draft_topk": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int,
                              _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "draft_sample_workspace": (_c.c_size_t, [_c.c_int, _c.c_int]),
    "draft_sample": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p, _c.c_float, _c.c_uint64,
                                _c.c_uint32, _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "kv_commit": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int,
                             _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int,
                             _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "awl_loss_workspace": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int]),
    "awl_loss": (_c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int,
                            _c.c_int, _c.c_int, _c.c_double, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                            _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "train_attn_workspace": (_c.c_size_t, [_c.c_int] * 5),
    "train_attn_fwd": (_c.c_int, [_c.c_int] + [_c.c_void_p] * 4 + [_c.c_int] * 6 + [_c.c_float] + [_c.c_void_p] * 3),
    "train_attn_bwd": (_c.c_int, [_c.c_int] + [_c.c_void_p] * 7 + [_c.c_int] * 6 + [_c.c_float] + [_c.c_void_p] * 4
                       + [_c.c_size_t, _c.c_void_p]),
    "d3d_status_string": (_c.c_char_p, [_c.c_int]),
}
EXPORTS = tuple(_SIGNATURES)

_lib = None


def load():
    """Load libd3d.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_diffusion_drafting_draft_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status, what):
    if status != 0:
        msg = load().d3d_status_string(status).decode()
        raise RuntimeError(f"{what} failed: status {status} ({msg})")


def _host_i32(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    """d3d_dtype of a tensor, a torch dtype, "bf16" / "f32", or an existing code."""
    if isinstance(t, int):
        if t in (D3D_BF16, D3D_F32):
            return t
        raise TypeError(f"unsupported dtype code {t}")
    dt = t.dtype if hasattr(t, "dtype") else t
    if dt in (torch.bfloat16, "bf16"):
        return D3D_BF16
    if dt in (torch.float32, "f32"):
        return D3D_F32
    raise TypeError(f"unsupported dtype {dt}")


def _dev(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t


# ------------------------------------------------------------------------------------------------
def d3d_build_branch_descs(block_size, coverage, fanout, prefix_len, cur_anchor, alt_anchors):
    """Host descriptor builder -> int32 array [(C-1)F + 2, 4] of (prefix_len, rej_pos, anchor, flags)."""
    alt, alt_p = _host_i32(alt_anchors)
    cap = max(0, (coverage - 1) * fanout + 2)
    out = np.zeros((max(cap, 1), 4), dtype=np.int32)
    n = ctypes.c_int(0)
    _check(load().d3d_build_branch_descs(block_size, coverage, fanout, prefix_len, int(cur_anchor), alt_p,
                                         out.ctypes.data, cap, ctypes.byref(n)),
           "d3d_build_branch_descs")
    return out[:n.value]


def d3d_build_branch_descs_batch(block_size, coverage, fanout, prefix_len, cur_anchor, alt_anchors, out=None,
                                 req_block_off=None):
    """Batched host descriptor builder. prefix_len / cur_anchor: [n_req]; alt_anchors: [n_req, (C-1)F + 1].
    out: optional int32 array [>= n_req ((C-1)F + 2), 4] (a numpy view of pinned memory works);
    req_block_off: optional int32 array [n_req + 1]. Returns (descs, req_block_off) as numpy arrays."""
    pre, pre_p = _host_i32(prefix_len)
    cur, cur_p = _host_i32(cur_anchor)
    alt, alt_p = _host_i32(alt_anchors)
    n_req = pre.size
    per = (coverage - 1) * fanout + 2
    if cur.size != n_req or alt.size != n_req * (per - 1):
        raise ValueError("cur_anchor / alt_anchors do not match prefix_len")
    if out is None:
        out = np.zeros((max(n_req * per, 1), 4), dtype=np.int32)
    if out.dtype != np.int32 or not out.flags.c_contiguous or out.ndim != 2 or out.shape[1] != 4:
        raise ValueError("out must be a C-contiguous int32 array [cap, 4]")
    if req_block_off is None:
        req_block_off = np.zeros(n_req + 1, dtype=np.int32)
    if req_block_off.dtype != np.int32 or not req_block_off.flags.c_contiguous or req_block_off.size < n_req + 1:
        raise ValueError("req_block_off must be a C-contiguous int32 array of n_req + 1 entries")
    _check(load().d3d_build_branch_descs_batch(n_req, block_size, coverage, fanout, pre_p, cur_p, alt_p,
                                               out.ctypes.data, out.shape[0],
                                               req_block_off.ctypes.data),
           "d3d_build_branch_descs_batch")
    return out[:n_req * per], req_block_off[:n_req + 1]


def draft_attn_packed_workspace(dtype, req_block_off, req_prefix_len, block_size, n_heads_q, n_heads_kv,
                                head_dim):
    """Workspace bytes for draft_attn_packed on the current device; dtype is torch.bfloat16 /
    torch.float32 or "bf16" / "f32"."""
    off, off_p = _host_i32(req_block_off)
    pre, pre_p = _host_i32(req_prefix_len)
    return int(load().draft_attn_packed_workspace(_dtype_code(dtype), off_p, pre_p, len(pre), block_size, n_heads_q,
                                                  n_heads_kv, head_dim))


def draft_attn_packed(q, k_new, v_new, k_cache, v_cache, descs, req_block_off, req_prefix_len, block_size,
                      scale=None, page_table=None, page_size=16, kv_stride=None, out=None, ws=None,
                      stream=None, join=None):
    """Packed draft attention. q [N_q, H_q, d]; k_new/v_new [N_q, H_kv, d]; k_cache/v_cache either
    [n_req, kv_stride, H_kv, d] (page_table None) or [n_pages, page_size, H_kv, d]; descs: device int32
    [n_blocks, 4]; req_block_off / req_prefix_len: host ints. Returns out [N_q, H_q, d]. join: a
    recorded torch.cuda.Event the stream waits for before the call's last launch
    (draft_attn_packed_join)."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (descs, "descs")):
        _dev(t, n)
    dt = _dtype_code(q)
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise TypeError("q, k_new, v_new must share a dtype")
    n_q, hq, d = q.shape
    hkv = k_new.shape[1]
    off, off_p = _host_i32(req_block_off)
    pre, pre_p = _host_i32(req_prefix_len)
    n_req = len(pre)
    if off.size != n_req + 1 or int(off[-1]) * block_size != n_q:
        raise ValueError("req_block_off does not match the packed query count")
    if descs.dtype != torch.int32 or descs.shape != (int(off[-1]), 4):
        raise ValueError("descs must be int32 [n_blocks, 4]")
    if k_new.shape != (n_q, hkv, d) or v_new.shape != (n_q, hkv, d):
        raise ValueError("k_new / v_new shape mismatch")
    has_prefix = bool(pre.max(initial=0) > 0)
    if has_prefix:
        _dev(k_cache, "k_cache")
        _dev(v_cache, "v_cache")
        if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or k_cache.shape != v_cache.shape:
            raise TypeError("k_cache / v_cache must match q's dtype and each other")
        if k_cache.shape[-2:] != (hkv, d):
            raise ValueError("k_cache / v_cache trailing dims must be [H_kv, d]")
    if page_table is not None:
        _dev(page_table, "page_table")
        if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != n_req:
            raise ValueError("page_table must be int32 [n_req, max_pages]")
        max_pages, num_pages = page_table.shape[1], (k_cache.shape[0] if has_prefix else 1)
        if has_prefix and k_cache.shape[1] != page_size:
            raise ValueError("k_cache page dimension does not match page_size")
        stride = 0
    else:
        max_pages, num_pages = 0, 0
        stride = (k_cache.shape[1] if has_prefix else 0) if kv_stride is None else kv_stride
        if has_prefix and k_cache.shape[0] != n_req:
            raise ValueError("contiguous caches must be [n_req, kv_stride, H_kv, d]")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out")
    need = draft_attn_packed_workspace(dt, off, pre, block_size, hq, hkv, d)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = d ** -0.5 if scale is None else scale
    args = (dt, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache) if has_prefix else None,
            _ptr(v_cache) if has_prefix else None, _ptr(page_table), page_size, max_pages, num_pages, stride,
            _ptr(descs), off_p, pre_p, n_req, block_size, hq, hkv, d, float(scale), _ptr(out),
            _ptr(ws) if need else None, need)
    if join is None:
        st = load().draft_attn_packed(*args, _stream(stream))
    else:
        st = load().draft_attn_packed_join(*args, join.cuda_event, _stream(stream))
    _check(st, "draft_attn_packed")
    return out


def draft_attn_packed_join(q, k_new, v_new, k_cache, v_cache, descs, req_block_off, req_prefix_len, block_size,
                           join, **kw):
    """draft_attn_packed whose stream waits for the recorded torch.cuda.Event `join` before the call's
    last launch (the C entry point of the same name)."""
    if join is None:
        raise ValueError("draft_attn_packed_join needs a recorded event")
    return draft_attn_packed(q, k_new, v_new, k_cache, v_cache, descs, req_block_off, req_prefix_len, block_size,
                             join=join, **kw)


def spec_verify_workspace(n_req, n_draft, vocab):
    return int(load().spec_verify_workspace(n_req, n_draft, vocab))


def spec_verify(target_logits, draft_logits, draft_tokens, temperature, seed, round_, ws=None, out=None,
                stream=None, match=None):
    """Speculative-sampling verify. target_logits [n_req, B, V], draft_logits [n_req, B-1, V],
    draft_tokens int32 [n_req, B-1]. Returns a dict of device tensors: n_accepted, next_token, alpha,
    survival, tau, flags. With match=(descs, req_block_off) (int32 GPU tensors as for
    branch_cache_match) the cache match runs inside the verify launches (spec_verify_match) and the
    dict also holds hit_branch."""
    _dev(target_logits, "target_logits")
    _dev(draft_tokens, "draft_tokens")
    dt = _dtype_code(target_logits)
    n_req, b, vocab = target_logits.shape
    nd = b - 1
    if draft_tokens.dtype != torch.int32 or draft_tokens.shape != (n_req, nd):
        raise ValueError("draft_tokens must be int32 [n_req, B-1]")
    if float(temperature) != 0.0 or draft_logits is not None:
        _dev(draft_logits, "draft_logits")
        if draft_logits.dtype != target_logits.dtype or draft_logits.shape != (n_req, nd, vocab):
            raise ValueError("draft_logits must match target_logits' dtype and be [n_req, B-1, V]")
    dev = target_logits.device
    if out is None:
        out = dict(n_accepted=torch.empty(n_req, dtype=torch.int32, device=dev),
                   next_token=torch.empty(n_req, dtype=torch.int32, device=dev),
                   alpha=torch.empty(n_req, nd, dtype=torch.float32, device=dev),
                   survival=torch.empty(n_req, nd, dtype=torch.float32, device=dev),
                   tau=torch.empty(n_req, dtype=torch.float32, device=dev),
                   flags=torch.empty(n_req, dtype=torch.int32, device=dev))
    need = spec_verify_workspace(n_req, nd, vocab)
    if need == 0:
        raise ValueError("unsupported verify shape")
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    args = (dt, _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), n_req, nd, vocab, float(temperature),
            int(seed) & (2**64 - 1), int(round_) & 0xFFFFFFFF, _ptr(out["n_accepted"]), _ptr(out["next_token"]),
            _ptr(out["alpha"]), _ptr(out["survival"]), _ptr(out["tau"]), _ptr(out["flags"]), _ptr(ws), need)
    if match is None:
        st = load().spec_verify(*args, _stream(stream))
        _check(st, "spec_verify")
        return out
    descs, req_block_off = match
    for t, n in ((descs, "descs"), (req_block_off, "req_block_off")):
        _dev(t, n)
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
    if req_block_off.numel() != n_req + 1:
        raise ValueError("req_block_off must have n_req + 1 entries")
    if out.get("hit_branch") is None:
        out["hit_branch"] = torch.empty(n_req, dtype=torch.int32, device=dev)
    st = load().spec_verify_match(*args, _ptr(descs), descs.shape[0], _ptr(req_block_off), _ptr(out["hit_branch"]),
                                  _stream(stream))
    _check(st, "spec_verify_match")
    return out


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, temperature, seed, round_, out=None,
                        stream=None):
    """spec_verify whose workspace is the library's static per-GPU scratch (the C entry point of the
    same name allocates nothing; calls that overlap on one GPU race). Arguments and the returned
    dict as spec_verify; `out` may hold preallocated output tensors."""
    _dev(target_logits, "target_logits")
    _dev(draft_tokens, "draft_tokens")
    dt = _dtype_code(target_logits)
    n_req, b, vocab = target_logits.shape
    nd = b - 1
    if draft_tokens.dtype != torch.int32 or draft_tokens.shape != (n_req, nd):
        raise ValueError("draft_tokens must be int32 [n_req, B-1]")
    if float(temperature) != 0.0 or draft_logits is not None:
        _dev(draft_logits, "draft_logits")
        if draft_logits.dtype != target_logits.dtype or draft_logits.shape != (n_req, nd, vocab):
            raise ValueError("draft_logits must match target_logits' dtype and be [n_req, B-1, V]")
    dev = target_logits.device
    if out is None:
        out = dict(n_accepted=torch.empty(n_req, dtype=torch.int32, device=dev),
                   next_token=torch.empty(n_req, dtype=torch.int32, device=dev),
                   alpha=torch.empty(n_req, nd, dtype=torch.float32, device=dev),
                   survival=torch.empty(n_req, nd, dtype=torch.float32, device=dev),
                   tau=torch.empty(n_req, dtype=torch.float32, device=dev),
                   flags=torch.empty(n_req, dtype=torch.int32, device=dev))
    st = load().spec_verify_noalloc(dt, _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), n_req, nd,
                                    vocab, float(temperature), int(seed) & (2**64 - 1), int(round_) & 0xFFFFFFFF,
                                    _ptr(out["n_accepted"]), _ptr(out["next_token"]), _ptr(out["alpha"]),
                                    _ptr(out["survival"]), _ptr(out["tau"]), _ptr(out["flags"]), _stream(stream))
    _check(st, "spec_verify_noalloc")
    return out


def spec_verify_match(target_logits, draft_logits, draft_tokens, temperature, seed, round_, descs, req_block_off,
                      **kw):
    """spec_verify with the cache match inside its launches (the C entry point of the same name):
    the returned dict also holds hit_branch."""
    return spec_verify(target_logits, draft_logits, draft_tokens, temperature, seed, round_,
                       match=(descs, req_block_off), **kw)


def d3d_build_branch_descs_device(block_size, coverage, fanout, prefix_len, cur_anchor, alt_anchors, out=None,
                                  req_block_off=None, stream=None):
    """Batched descriptor builder on the GPU. prefix_len / cur_anchor: int32 [n_req]; alt_anchors: int32
    [n_req, (C-1)F + 1]; all GPU tensors. out: optional int32 [>= n_req ((C-1)F + 2), 4]; req_block_off:
    optional int32 [n_req + 1]. Returns (descs, req_block_off) as GPU tensors."""
    for t, n in ((prefix_len, "prefix_len"), (cur_anchor, "cur_anchor"), (alt_anchors, "alt_anchors")):
        _dev(t, n)
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 tensor")
    n_req = prefix_len.numel()
    per = (coverage - 1) * fanout + 2
    if cur_anchor.numel() != n_req or alt_anchors.numel() != n_req * (per - 1):
        raise ValueError("cur_anchor / alt_anchors do not match prefix_len")
    if out is None:
        out = torch.empty((n_req * per, 4), dtype=torch.int32, device=prefix_len.device)
    if req_block_off is None:
        req_block_off = torch.empty(n_req + 1, dtype=torch.int32, device=prefix_len.device)
    for t, n, size in ((out, "out", 4 * n_req * per), (req_block_off, "req_block_off", n_req + 1)):
        _dev(t, n)
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < size:
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor of at least {size} entries")
    _check(load().d3d_build_branch_descs_device(n_req, block_size, coverage, fanout, _ptr(prefix_len),
                                                _ptr(cur_anchor), _ptr(alt_anchors), _ptr(out),
                                                _ptr(req_block_off), _stream(stream)),
           "d3d_build_branch_descs_device")
    return out, req_block_off


def branch_cache_match(descs, req_block_off, n_accepted, next_token, hit=None, stream=None):
    """descs int32 [n_blocks, 4], req_block_off int32 [n_req+1], n_accepted / next_token int32 [n_req],
    all on the GPU. Returns hit_branch int32 [n_req] (-1 = miss)."""
    for t, n in ((descs, "descs"), (req_block_off, "req_block_off"), (n_accepted, "n_accepted"),
                 (next_token, "next_token")):
        _dev(t, n)
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
    n_req = n_accepted.numel()
    if hit is None:
        hit = torch.empty(n_req, dtype=torch.int32, device=n_accepted.device)
    st = load().branch_cache_match(_ptr(descs), descs.shape[0], _ptr(req_block_off), n_req, _ptr(n_accepted),
                                   _ptr(next_token), _ptr(hit), _stream(stream))
    _check(st, "branch_cache_match")
    return hit


def draft_topk_workspace(n_rows, vocab, k):
    return int(load().draft_topk_workspace(n_rows, vocab, k))


def draft_topk(logits, k, rows=None, exclude=None, out=None, out_off=None, n_rows=None, ws=None, stream=None):
    """The k best tokens of logit rows (larger logit first, ties to the lower id), skipping exclude[r].
    logits [rows_in, V] on the GPU; rows / exclude / out_off: int32 GPU tensors or None. Returns out
    (int32 [n_rows, k] when allocated here)."""
    _dev(logits, "logits")
    dt = _dtype_code(logits)
    vocab = logits.shape[-1]
    for t, n in ((rows, "rows"), (exclude, "exclude"), (out_off, "out_off")):
        if t is not None:
            _dev(t, n)
            if t.dtype != torch.int32:
                raise TypeError(f"{n} must be int32")
    if n_rows is None:
        n_rows = rows.numel() if rows is not None else logits.numel() // vocab
    if out is None:
        if out_off is not None:
            raise ValueError("pass out together with out_off")
        out = torch.empty((n_rows, k), dtype=torch.int32, device=logits.device)
    _dev(out, "out")
    need = draft_topk_workspace(n_rows, vocab, k)
    if need == 0:
        raise ValueError("unsupported draft_topk shape")
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
    st = load().draft_topk(dt, _ptr(logits), vocab, n_rows, _ptr(rows), _ptr(exclude), k, _ptr(out), _ptr(out_off),
                           _ptr(ws), need, _stream(stream))
    _check(st, "draft_topk")
    return out


def draft_sample_workspace(n_rows, vocab):
    return int(load().draft_sample_workspace(n_rows, vocab))


def draft_sample(logits, temperature, seed, round_, rows=None, out=None, n_rows=None, ws=None, stream=None):
    """One token per logit row drawn from softmax(z / T) (Gumbel-max over Philox uniforms, decided in
    fp64). logits [rows_in, V] on the GPU; rows: int32 GPU tensor or None. Returns out (int32 [n_rows])."""
    _dev(logits, "logits")
    dt = _dtype_code(logits)
    vocab = logits.shape[-1]
    if rows is not None:
        _dev(rows, "rows")
        if rows.dtype != torch.int32:
            raise TypeError("rows must be int32")
    if n_rows is None:
        n_rows = rows.numel() if rows is not None else logits.numel() // vocab
    if out is None:
        out = torch.empty(n_rows, dtype=torch.int32, device=logits.device)
    _dev(out, "out")
    need = draft_sample_workspace(n_rows, vocab)
    if need == 0:
        raise ValueError("unsupported draft_sample shape")
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
    st = load().draft_sample(dt, _ptr(logits), vocab, n_rows, _ptr(rows), float(temperature), int(seed),
                             int(round_) & 0xFFFFFFFF, _ptr(out), _ptr(ws), need, _stream(stream))
    _check(st, "draft_sample")
    return out


def kv_commit(k_new, v_new, k_cache, v_cache, page_table, req_block_off, prefix_len, n_accepted, block_size,
              hit=None, packed_tokens=None, next_block=None, status=None, stream=None):
    """Append each request's accepted slice to the paged cache (prefix_len updated in place) and, with
    hit / packed_tokens, promote the hit branch. k_new / v_new [N_q, H_kv, d]; caches [pages, page, H_kv,
    d]; page_table [n_req, max_pages]; req_block_off [n_req + 1]; prefix_len, n_accepted, hit [n_req];
    packed_tokens [N_q]; all int32 / GPU. Returns (next_block or None, status)."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (page_table, "page_table"), (req_block_off, "req_block_off"), (prefix_len, "prefix_len"),
                 (n_accepted, "n_accepted")):
        _dev(t, n)
    dt = _dtype_code(k_new)
    if not (k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("k_new, v_new and the caches must share a dtype")
    hkv, d = k_new.shape[1], k_new.shape[2]
    if k_cache.shape != v_cache.shape or k_cache.shape[2:] != (hkv, d):
        raise ValueError("caches must be [pages, page_size, H_kv, d] like k_new's rows")
    n_req = n_accepted.numel()
    for t, n in ((page_table, "page_table"), (req_block_off, "req_block_off"), (prefix_len, "prefix_len"),
                 (n_accepted, "n_accepted")):
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
    if page_table.dim() != 2 or page_table.shape[0] != n_req or req_block_off.numel() != n_req + 1 \
            or prefix_len.numel() != n_req:
        raise ValueError("page_table / req_block_off / prefix_len do not match n_accepted")
    if (hit is None) != (packed_tokens is None):
        raise ValueError("pass hit and packed_tokens together")
    if hit is not None:
        _dev(hit, "hit")
        _dev(packed_tokens, "packed_tokens")
        if next_block is None:
            next_block = torch.empty((n_req, block_size), dtype=torch.int32, device=k_new.device)
    if status is None:
        status = torch.empty(n_req, dtype=torch.int32, device=k_new.device)
    st = load().kv_commit(dt, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                          k_cache.shape[1], page_table.shape[1], k_cache.shape[0], _ptr(req_block_off),
                          _ptr(prefix_len), _ptr(n_accepted), n_req, block_size, hkv, d, _ptr(hit),
                          _ptr(packed_tokens), _ptr(next_block), _ptr(status), _stream(stream))
    _check(st, "kv_commit")
    return next_block, status


def awl_loss_workspace(n_blocks, n_pos, vocab):
    return int(load().awl_loss_workspace(n_blocks, n_pos, vocab))


def awl_loss(target_logits, draft_logits, draft_tokens, labels, include=None, eps=1e-6, grad=False, out=None,
             ws=None, stream=None):
    """Acceptance-weighted loss. target / draft logits [n_blocks, n_pos, V]; draft_tokens, labels,
    include int32 [n_blocks, n_pos] (include None: all), all on the GPU. Returns a dict of device
    tensors: loss (float64 [1]), weights, ce (float32 [n_blocks, n_pos]) and grad (like draft_logits)
    when grad=True."""
    for t, n in ((target_logits, "target_logits"), (draft_logits, "draft_logits"), (draft_tokens, "draft_tokens"),
                 (labels, "labels")):
        _dev(t, n)
    dt = _dtype_code(draft_logits)
    if target_logits.dtype != draft_logits.dtype or target_logits.shape != draft_logits.shape:
        raise ValueError("target and draft logits must share dtype and shape")
    n_blocks, n_pos, vocab = draft_logits.shape
    for t, n in ((draft_tokens, "draft_tokens"), (labels, "labels"), (include, "include")):
        if t is not None:
            _dev(t, n)
            if t.dtype != torch.int32 or t.shape != (n_blocks, n_pos):
                raise ValueError(f"{n} must be int32 [n_blocks, n_pos]")
    dev = draft_logits.device
    if out is None:
        out = dict(loss=torch.empty(1, dtype=torch.float64, device=dev),
                   weights=torch.empty((n_blocks, n_pos), dtype=torch.float32, device=dev),
                   ce=torch.empty((n_blocks, n_pos), dtype=torch.float32, device=dev))
        if grad:
            out["grad"] = torch.empty_like(draft_logits)
    else:
        _like(out["loss"], (1,), torch.float64, "loss")
        _like(out["weights"], (n_blocks, n_pos), torch.float32, "weights")
        if out.get("ce") is not None:
            _like(out["ce"], (n_blocks, n_pos), torch.float32, "ce")
        if out.get("grad") is not None:
            _like(out["grad"], draft_logits.shape, draft_logits.dtype, "grad")
    need = awl_loss_workspace(n_blocks, n_pos, vocab)
    if need == 0:
        raise ValueError("unsupported awl_loss shape")
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().awl_loss(dt, _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(labels), _ptr(include),
                         n_blocks, n_pos, vocab, float(eps), _ptr(out["weights"]), _ptr(out.get("ce")),
                         _ptr(out["loss"]), _ptr(out.get("grad")), _ptr(ws), need, _stream(stream))
    _check(st, "awl_loss")
    return out


def _like(t, shape, dtype, name):
    """Check a caller-supplied tensor: contiguous, on the GPU, of this shape and dtype."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}")
    return t


def _train_shape(q, k, anchors, L, block_size):
    for t, n in ((q, "q"), (k, "k"), (anchors, "anchors")):
        _dev(t, n)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise TypeError("training attention takes bf16 tensors")
    if anchors.dtype != torch.int32 or anchors.dim() != 1:
        raise ValueError("anchors must be int32 [n_blocks]")
    n_blocks = anchors.numel()
    N, hq, d = q.shape
    if N != L + n_blocks * block_size or k.shape[0] != N or k.shape[2] != d:
        raise ValueError("q / k rows must be L + n_blocks * block_size")
    return n_blocks, N, hq, k.shape[1], d


def train_attn_workspace(L, n_blocks, block_size, n_heads_q, n_heads_kv):
    return int(load().train_attn_workspace(L, n_blocks, block_size, n_heads_q, n_heads_kv))


def train_attn_fwd(q, k, v, anchors, L, block_size, scale=None, out=None, lse=None, stream=None):
    """Training-time packed attention forward. q [N, H_q, d], k, v [N, H_kv, d] bf16, anchors int32
    [n_blocks] (all on the GPU). Returns (out [N, H_q, d] bf16, lse [N, H_q] f32)."""
    n_blocks, N, hq, hkv, d = _train_shape(q, k, anchors, L, block_size)
    _like(v, k.shape, torch.bfloat16, "v")
    scale = d ** -0.5 if scale is None else scale
    out = torch.empty_like(q) if out is None else _like(out, q.shape, torch.bfloat16, "out")
    lse = (torch.empty((N, hq), dtype=torch.float32, device=q.device) if lse is None
           else _like(lse, (N, hq), torch.float32, "lse"))
    st = load().train_attn_fwd(D3D_BF16, _ptr(q), _ptr(k), _ptr(v), _ptr(anchors), L, n_blocks, block_size, hq, hkv, d,
                               float(scale), _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "train_attn_fwd")
    return out, lse


def train_attn_bwd(q, k, v, out, dout, lse, anchors, L, block_size, scale=None, dq=None, dk=None, dv=None, ws=None,
                   stream=None):
    """Training-time packed attention backward: (dq, dk, dv) from the forward's out, lse and the
    upstream gradient dout (bf16 tensors on the GPU)."""
    n_blocks, N, hq, hkv, d = _train_shape(q, k, anchors, L, block_size)
    _like(v, k.shape, torch.bfloat16, "v")
    for t, n in ((out, "out"), (dout, "dout")):
        _like(t, q.shape, torch.bfloat16, n)
    _like(lse, (N, hq), torch.float32, "lse")
    scale = d ** -0.5 if scale is None else scale
    dq = torch.empty_like(q) if dq is None else _like(dq, q.shape, torch.bfloat16, "dq")
    dk = torch.empty_like(k) if dk is None else _like(dk, k.shape, torch.bfloat16, "dk")
    dv = torch.empty_like(v) if dv is None else _like(dv, k.shape, torch.bfloat16, "dv")
    need = train_attn_workspace(L, n_blocks, block_size, hq, hkv)
    if need == 0:
        raise RuntimeError("train_attn_bwd: unsupported shape")
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = load().train_attn_bwd(D3D_BF16, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(anchors), L,
                               n_blocks, block_size, hq, hkv, d, float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                               need, _stream(stream))
    _check(st, "train_attn_bwd")
    return dq, dk, dv
