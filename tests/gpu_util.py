"""Helpers for the GPU parity tests: moving seeded inputs to the device, building the device-side
problem through the library's own descriptor builder, and the oracle side of the same problem."""

import numpy as np
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from oracle import attention as o_attn
from oracle import packing as o_pack


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    _binding.load()  # fail loudly when the HIP library is missing


def dev(x, dtype):
    """float32 host array (bf16-exact for bf16) -> contiguous device tensor of that dtype."""
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32).copy()).cuda()


def host(t):
    return t.detach().float().cpu().numpy()


class AttnProblem:
    """One packed attention call: per-request block lists (oracle side) and device tensors built with
    the library's descriptor builder (GPU side)."""

    def __init__(self, dtype, B, reqs, inputs, paged=False, page_size=16, seed=0, kv_stride=None):
        # reqs: list of dicts {L, kind: "sync"|"async", C, F, a0, anchors} or {"blocks": [...]}
        self.dtype, self.B = dtype, B
        self.inputs = inputs
        self.reqs = reqs
        descs, off, pre, self.blocks = [], [0], [], []
        for r in reqs:
            if "blocks" in r:  # explicit descriptors (r, anchor, causal)
                blocks = list(r["blocks"])
                d = np.array([[r["L"], rr, a, 1 if c else 0] for rr, a, c in blocks], dtype=np.int32)
            elif r["kind"] == "sync":
                blocks = [(0, r.get("a0", 0), False)]
                d = np.array([[r["L"], 0, r.get("a0", 0), 0]], dtype=np.int32)
            else:
                C, F = r["C"], r["F"]
                anchors = r.get("anchors", list(range((C - 1) * F + 1)))
                d = _binding.d3d_build_branch_descs(B, C, F, r["L"], r.get("a0", 0), anchors)
                blocks = o_pack.pack_blocks(B, C, F, r.get("a0", 0), anchors)
            descs.append(d)
            self.blocks.append(blocks)
            off.append(off[-1] + len(blocks))
            pre.append(r["L"])
        self.off, self.pre = off, pre
        self.descs = torch.from_numpy(np.concatenate(descs)).cuda()
        self.q = dev(inputs["q"], dtype)
        self.k_new = dev(inputs["k_new"], dtype)
        self.v_new = dev(inputs["v_new"], dtype)
        hkv, d = inputs["k_new"].shape[1:]
        self.page_table = None
        self.page_size = page_size
        if paged:
            kp, table = synth.paginate(inputs["k_prefix"], page_size, seed)
            vp, _ = synth.paginate(inputs["v_prefix"], page_size, seed)
            self.k_cache, self.v_cache = dev(kp, dtype), dev(vp, dtype)
            self.page_table = torch.from_numpy(table).cuda()
        else:
            stride = max(max(pre), 1) if kv_stride is None else kv_stride
            kc = np.zeros((len(pre), stride, hkv, d), dtype=np.float32)
            vc = np.zeros_like(kc)
            for i, (k, v) in enumerate(zip(inputs["k_prefix"], inputs["v_prefix"])):
                kc[i, :k.shape[0]] = k
                vc[i, :v.shape[0]] = v
            self.k_cache, self.v_cache = dev(kc, dtype), dev(vc, dtype)

    def run(self, scale=None):
        return _binding.draft_attn_packed(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache, self.descs,
                                          self.off, self.pre, self.B, scale=scale, page_table=self.page_table,
                                          page_size=self.page_size)

    def oracle(self, rows_per_req=None, scale=None):
        """Oracle outputs for every request (all rows, or the given local row lists)."""
        d = self.inputs["q"].shape[2]
        scale = d ** -0.5 if scale is None else scale
        outs, rows_all = [], []
        for i, blocks in enumerate(self.blocks):
            q0, q1 = self.off[i] * self.B, self.off[i + 1] * self.B
            mask = o_pack.visible_mask(self.B, blocks, self.pre[i])
            rows = None if rows_per_req is None else rows_per_req[i]
            outs.append(o_attn.packed_attention(
                self.inputs["q"][q0:q1], self.inputs["k_prefix"][i], self.inputs["v_prefix"][i],
                self.inputs["k_new"][q0:q1], self.inputs["v_new"][q0:q1], mask, scale, rows=rows))
            rows_all.append(np.arange(q0, q1) if rows is None else q0 + np.asarray(rows))
        return np.concatenate(outs), np.concatenate(rows_all)


def attn_close(got, want, atol, rel_fro):
    """Element-wise |got - want| <= atol and ||got - want||_F <= rel_fro ||want||_F."""
    err = np.abs(got - want)
    fro = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    return bool(err.max() <= atol and fro <= rel_fro), float(err.max()), float(fro)
