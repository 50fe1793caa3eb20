"""GPU parity of the training-time packed attention (train_attn_fwd / train_attn_bwd) against the
oracle, through the C ABI.

Inputs are bf16-exact N(0, 1) values; the kernels multiply bf16 operands with fp32 accumulation and
round the probabilities (and dS) to bf16 before the second product. Bar, per tensor: the
element-wise error within 2e-2 of the tensor's largest magnitude and the Frobenius error within
1.5e-2 of its norm (o, lse within 2e-2 / 1e-2 absolute as for the draft attention)."""

import sys

import numpy as np
import pytest
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from gpu_util import dev, host, require_gpu
from oracle import train_attn as ta

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _close(got, want, rel_max=2e-2, rel_fro=1.5e-2):
    scale = max(float(np.abs(want).max()), 1e-30)
    err = np.abs(got - want)
    fro = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    return bool(err.max() <= rel_max * scale and fro <= rel_fro), float(err.max() / scale), float(fro)


def _anchors(rng, L, n, B, kind):
    if kind == "sorted":
        return np.sort(rng.integers(0, L + 1, size=n)).astype(np.int32)
    a = rng.integers(0, L + 1, size=n).astype(np.int32)
    a[0], a[-1] = 0, L  # an empty prefix and the whole response
    return a


def _problem(L, n_blocks, B, hq, hkv, kind, seed):
    rng = np.random.default_rng(seed)
    N = L + n_blocks * B
    q, k, v, do = (synth.round_bf16(rng.standard_normal((N, h, 128), dtype=np.float32)) for h in (hq, hkv, hkv, hq))
    return q, k, v, do, _anchors(rng, L, n_blocks, B, kind)


CASES = [
    # L, n_blocks, B, H_q, H_kv, anchors
    (256, 16, 16, 8, 2, "sorted"),
    (256, 24, 8, 8, 2, "sorted"),
    (200, 7, 24, 8, 2, "mixed"),    # ragged response, unsorted anchors with 0 and L
    (320, 6, 32, 8, 2, "sorted"),
    (128, 9, 16, 2, 2, "mixed"),    # one head per group
    (192, 5, 16, 16, 2, "sorted"),  # eight heads per group
    (0, 4, 16, 8, 2, "sorted"),     # no response: blocks only
    (100, 0, 16, 8, 2, "sorted"),   # response only (the autoregressive rows)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_train_attention_parity(case):
    require_gpu()
    L, nb, B, hq, hkv, kind = case
    _say(f"train_attn: {case}")
    q, k, v, do, anchors = _problem(L, nb, B, hq, hkv, kind, seed=L + 7 * nb + B)
    scale = 128 ** -0.5
    qd, kd, vd, dod = (dev(x, "bf16") for x in (q, k, v, do))
    an = torch.from_numpy(anchors).cuda() if nb else torch.zeros(0, dtype=torch.int32, device="cuda")
    out, lse = _binding.train_attn_fwd(qd, kd, vd, an, L, B, scale=scale)
    dq, dk, dv = _binding.train_attn_bwd(qd, kd, vd, out, dod, lse, an, L, B, scale=scale)
    torch.cuda.synchronize()
    want_o, want_lse = ta.forward(q, k, v, L, anchors, B, scale)
    ok, e, f = _close(host(out), want_o, 2e-2, 1e-2)
    assert ok, ("o", e, f)
    assert np.abs(lse.cpu().numpy() - want_lse).max() < 2e-2
    # the backward from the kernel's own (bf16) forward output, as training runs it; the oracle's
    # gradient takes its exact forward
    wdq, wdk, wdv = ta.backward(q, k, v, do, L, anchors, B, scale)
    for name, got, want in (("dq", dq, wdq), ("dk", dk, wdk), ("dv", dv, wdv)):
        ok, e, f = _close(host(got), want)
        assert ok, (name, e, f)


def test_train_attention_clamps_anchors():
    """Anchors outside [0, L] are clamped (an empty prefix, the whole response): the result equals
    the oracle's on the clamped anchors."""
    require_gpu()
    L, nb, B, hq, hkv = 96, 4, 16, 8, 2
    _say("train_attn: anchors outside [0, L]")
    q, k, v, do, _ = _problem(L, nb, B, hq, hkv, "sorted", seed=17)
    raw = np.array([-5, 40, L + 30, 10**6], dtype=np.int32)
    clamped = np.clip(raw, 0, L)
    scale = 128 ** -0.5
    qd, kd, vd, dod = (dev(x, "bf16") for x in (q, k, v, do))
    an = torch.from_numpy(raw).cuda()
    out, lse = _binding.train_attn_fwd(qd, kd, vd, an, L, B, scale=scale)
    dq, dk, dv = _binding.train_attn_bwd(qd, kd, vd, out, dod, lse, an, L, B, scale=scale)
    torch.cuda.synchronize()
    want_o, _ = ta.forward(q, k, v, L, clamped, B, scale)
    assert _close(host(out), want_o, 2e-2, 1e-2)[0]
    for got, want in zip((dq, dk, dv), ta.backward(q, k, v, do, L, clamped, B, scale)):
        assert _close(host(got), want)[0]


def test_train_attention_training_step_shape_sampled():
    """One training sample at B = 16: a 4096-token response with 128 anchors, 32 query / 8 key-value
    heads. Sampled rows of o, lse and dq against the oracle row by row; dk and dv on keys whose
    viewers are few (the last 64 response keys and the keys of four blocks), every viewer's
    partition computed exactly."""
    require_gpu()
    L, nb, B, hq, hkv = 4096, 128, 16, 32, 8
    _say(f"train_attn: {L} + {nb} x {B}, {hq}/{hkv} heads")
    q, k, v, do, anchors = _problem(L, nb, B, hq, hkv, "sorted", seed=11)
    scale = 128 ** -0.5
    qd, kd, vd, dod = (dev(x, "bf16") for x in (q, k, v, do))
    an = torch.from_numpy(anchors).cuda()
    out, lse = _binding.train_attn_fwd(qd, kd, vd, an, L, B, scale=scale)
    dq, dk, dv = _binding.train_attn_bwd(qd, kd, vd, out, dod, lse, an, L, B, scale=scale)
    torch.cuda.synchronize()
    N = ta.n_rows(L, nb, B)
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, L - 1, L, L + B - 1, N - 1]) | set(int(x) for x in rng.choice(N, 40, replace=False)))
    heads = sorted(set([0, hq - 1]) | set(int(x) for x in rng.choice(hq, 2, replace=False)))
    want_o, want_lse = ta.forward_rows(q, k, v, L, anchors, B, scale, rows)
    want_dq = ta.backward_rows(q, k, v, do, L, anchors, B, scale, rows)
    o_h, lse_h, dq_h = host(out)[rows], lse.cpu().numpy()[rows], host(dq)[rows]
    for h in heads:
        assert np.abs(lse_h[:, h] - want_lse[:, h]).max() < 2e-2, h
        assert np.abs(o_h[:, h] - want_o[:, h]).max() < 2e-2, h
        for i, r in enumerate(rows):
            w = want_dq[i, h]
            assert np.abs(dq_h[i, h] - w).max() <= 2e-2 * max(np.abs(w).max(), 1e-3), (r, h)
    keys = list(range(L - 64, L)) + [L + b * B + j for b in (0, 5, 77, nb - 1) for j in range(B)]
    want_dk, want_dv = ta.backward_keys(q, k, v, do, L, anchors, B, scale, keys)
    dk_h, dv_h = host(dk)[keys], host(dv)[keys]
    for i, kj in enumerate(keys):
        for g in (0, hkv - 1):
            for got, want in ((dk_h[i, g], want_dk[i, g]), (dv_h[i, g], want_dv[i, g])):
                assert np.abs(got - want).max() <= 2e-2 * max(np.abs(want).max(), 1e-3), (kj, g)


def test_train_attention_bad_arguments():
    require_gpu()
    q = torch.zeros((48, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((48, 2, 128), dtype=torch.bfloat16, device="cuda")
    an = torch.tensor([3, 9], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):  # 16 + 2 x 16 = 48 rows, not 16 + 2 x 8
        _binding.train_attn_fwd(q, k, k, an, 16, 8)
    q3 = torch.zeros((48, 6, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):  # 3 heads per group does not divide 32
        _binding.train_attn_fwd(q3, k, k, an, 16, 16)
    with pytest.raises(ValueError):  # an output of the wrong shape is refused before any launch
        _binding.train_attn_fwd(q, k, k, an, 16, 16, out=torch.zeros((40, 8, 128), dtype=torch.bfloat16, device="cuda"))
