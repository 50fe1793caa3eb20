"""MI355X-native hot path of asynchronous block-diffusion speculative decoding.

The entry points live in the HIP library ``libd3d.so`` (C ABI in ``include/d3d.h``); the functions
exported here are its thin Python binding with the same names. Build the library with
``python -m block_diffusion_drafting_draft_amd.build``.
"""

_BOUND = ("d3d_build_branch_descs", "d3d_build_branch_descs_batch", "d3d_build_branch_descs_device", "draft_attn_packed_workspace", "draft_attn_packed", "draft_attn_packed_join",
          "spec_verify_workspace", "spec_verify", "spec_verify_match", "spec_verify_noalloc", "branch_cache_match", "draft_topk_workspace", "draft_topk",
          "draft_sample_workspace", "draft_sample", "kv_commit", "awl_loss_workspace", "awl_loss",
          "train_attn_workspace", "train_attn_fwd", "train_attn_bwd")

__all__ = list(_BOUND)


def __getattr__(name):
    if name in _BOUND:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
