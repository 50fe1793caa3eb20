"""GPU parity of awl_loss (acceptance-weighted drafter-training loss and its gradient) against the
oracle, through the C ABI.

Bar: weights (products of up to 63 acceptance scores, fp32 exp with fp64 accumulation on the GPU)
relative 1e-6 per factor; CE and the loss 1e-5; the gradient within one rounding of its stored type
(2^-8 relative for bf16, 1e-5 for fp32) plus 1e-5 of the row's coefficient I w / (sum I w + eps)."""

import sys

import numpy as np
import pytest
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from gpu_util import dev, host, require_gpu
from oracle import awl as o_awl

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(x, dtype, include=True, grad=True, eps=1e-6):
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    out = _binding.awl_loss(dev(x["z_target"], dtype), dev(x["z_draft"], dtype), i32(x["tokens"]), i32(x["labels"]),
                            include=i32(x["include"]) if include else None, eps=eps, grad=grad)
    torch.cuda.synchronize()
    return out


def _check(out, want, dtype, n_pos, inc_mask=None):
    w_got = out["weights"].cpu().numpy().astype(np.float64)
    tol_w = 1e-6 * (np.arange(n_pos) + 2) * want["weights"] + 1e-9
    assert np.all(np.abs(w_got - want["weights"]) <= tol_w), np.max(np.abs(w_got - want["weights"]))
    ce_got = out["ce"].cpu().numpy().astype(np.float64)
    assert np.allclose(ce_got, want["ce"], rtol=1e-6, atol=1e-5)
    loss = float(out["loss"].cpu().numpy()[0])
    assert abs(loss - want["loss"]) <= 1e-5 * max(1.0, abs(want["loss"])), (loss, want["loss"])
    if "grad" in out:
        g = host(out["grad"]).astype(np.float64)
        coef = (want["weights"] * (1.0 if inc_mask is None else inc_mask)) / (want["den"] + 1e-6)
        rt = 2.0 ** -8 if dtype == "bf16" else 1e-5
        tol = rt * np.abs(want["grad"]) + 1e-5 * coef[..., None] + 1e-30
        err = np.abs(g - want["grad"])
        assert np.all(err <= tol), float(np.max(err / tol))


CASES = [
    # dtype, n_blocks, n_pos, V
    ("bf16", 3, 15, 1000),
    ("bf16", 4, 7, 1003),      # V * 2 bytes not a multiple of 16: scalar path
    ("f32", 2, 63, 4096),      # longest block
    ("f32", 5, 1, 333),        # one position: every weight is 1
    ("bf16", 8, 15, 151936),   # Qwen3 vocabulary
    ("bf16", 2, 31, 151936),   # B = 32 horizon
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_awl_parity(case):
    require_gpu()
    dtype, nb, npos, V = case
    _say(f"awl_loss: {case}")
    x = synth.awl_inputs(nb, npos, V, dtype=dtype, seed=nb * 100 + npos)
    out = _run(x, dtype)
    want = o_awl.awl_loss(x["z_target"], x["z_draft"], x["tokens"], x["labels"], x["include"])
    _check(out, want, dtype, npos, inc_mask=x["include"])
    # the weights span (0, 1]: early rejections and long accepted prefixes both occur
    if npos > 1:
        assert want["weights"].min() < 0.5


def test_awl_without_mask_and_without_gradient():
    require_gpu()
    _say("awl_loss: include NULL, no gradient")
    x = synth.awl_inputs(3, 15, 2048, dtype="bf16", seed=5)
    out = _run(x, "bf16", include=False, grad=False)
    assert "grad" not in out
    want = o_awl.awl_loss(x["z_target"], x["z_draft"], x["tokens"], x["labels"], None)
    _check(out, want, "bf16", 15)


def test_awl_nothing_included_and_identical_models():
    """No position in the loss: L = 0 / eps = 0 and a zero gradient. P = Q: every alpha is 1, so every
    weight is 1 and L is the plain mean CE over the included positions."""
    require_gpu()
    _say("awl_loss: empty inclusion, P = Q")
    x = synth.awl_inputs(2, 15, 1000, dtype="f32", seed=9)
    x["include"][:] = 0
    out = _run(x, "f32")
    assert float(out["loss"].cpu()[0]) == 0.0 and not torch.any(out["grad"] != 0)
    x = synth.awl_inputs(2, 15, 1000, dtype="f32", seed=10)
    x["z_target"] = x["z_draft"].copy()
    out = _run(x, "f32")
    assert np.allclose(out["weights"].cpu().numpy(), 1.0, rtol=0, atol=1e-6)
    want = o_awl.awl_loss(x["z_target"], x["z_draft"], x["tokens"], x["labels"], x["include"])
    _check(out, want, "f32", 15, inc_mask=x["include"])


def test_awl_masked_vocabulary():
    """Logits at -inf (a masked vocabulary tail) take no probability: they add nothing to either
    softmax and get a zero gradient."""
    require_gpu()
    _say("awl_loss: masked vocabulary")
    x = synth.awl_inputs(3, 15, 1024, dtype="f32", seed=12)
    x["z_target"][..., 700:] = -np.inf
    x["z_draft"][..., 700:] = -np.inf
    x["tokens"] %= 700
    x["labels"] %= 700
    out = _run(x, "f32")
    want = o_awl.awl_loss(x["z_target"], x["z_draft"], x["tokens"], x["labels"], x["include"])
    _check(out, want, "f32", 15, inc_mask=x["include"])
    assert not torch.any(out["grad"][..., 700:] != 0)


def test_awl_training_step_shape_sampled():
    """128 anchor blocks x 15 future positions x 151936 (one training sample at B = 16): every weight,
    CE and the loss against the oracle block by block, the gradient on sampled rows."""
    require_gpu()
    nb, npos, V = 128, 15, 151936
    _say(f"awl_loss: {nb} x {npos} x {V}")
    x = synth.awl_inputs(nb, npos, V, dtype="bf16", seed=1)
    out = _run(x, "bf16")
    w_got = out["weights"].cpu().numpy().astype(np.float64)
    ce_got = out["ce"].cpu().numpy().astype(np.float64)
    num = den = 0.0
    wants = {}
    for b in range(nb):
        wb = o_awl.awl_loss(x["z_target"][b:b + 1], x["z_draft"][b:b + 1], x["tokens"][b:b + 1],
                            x["labels"][b:b + 1], x["include"][b:b + 1])
        tol_w = 1e-6 * (np.arange(npos) + 2) * wb["weights"][0] + 1e-9
        assert np.all(np.abs(w_got[b] - wb["weights"][0]) <= tol_w), b
        assert np.allclose(ce_got[b], wb["ce"][0], rtol=1e-6, atol=1e-5), b
        num += wb["num"]
        den += wb["den"]
        if b in (0, 77, nb - 1):
            wants[b] = wb
    loss = float(out["loss"].cpu()[0])
    want_loss = num / (den + 1e-6)
    assert abs(loss - want_loss) <= 1e-5 * max(1.0, want_loss)
    for b, wb in wants.items():
        g = host(out["grad"][b]).astype(np.float64)
        coef = x["include"][b] * wb["weights"][0] / (den + 1e-6)
        want_g = wb["grad"][0] * (wb["den"] + 1e-6) / (den + 1e-6)  # the block alone normalised by its own sum
        tol = 2.0 ** -8 * np.abs(want_g) + 1e-5 * coef[:, None] + 1e-30
        assert np.all(np.abs(g - want_g) <= tol), b


def test_awl_bad_arguments():
    require_gpu()
    z = torch.zeros((2, 64, 16), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((2, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):  # more than 63 positions
        _binding.awl_loss(z, z, t, t)
    z = torch.zeros((2, 4, 16), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        _binding.awl_loss(z, z.float(), t, t)
    with pytest.raises(ValueError):
        _binding.awl_loss(z, z, t.long(), t)
