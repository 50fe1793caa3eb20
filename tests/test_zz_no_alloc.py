"""The allocation-free verify entry point (spec_verify_noalloc, static per-GPU scratch) against
spec_verify with its own workspace, through the C ABI: every output identical, on two calls in a row
(the second with a smaller input, so stale scratch contents of the first call are present), sampled
and greedy."""

import sys

import numpy as np
import pytest
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from gpu_util import dev, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(name, n_req, vocab, T):
    w = synth.WORKLOADS[name]
    inp = synth.verify_inputs(w, n_req=n_req, vocab=vocab, temperature=T)
    return (dev(inp["z_target"], w.dtype), dev(inp["z_draft"], w.dtype),
            torch.from_numpy(inp["tokens"]).cuda(), T, inp["philox_seed"])


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_noalloc_equals_spec_verify_on_two_calls(T):
    require_gpu()
    cases = [("serve-16req-B16C12F2-paged16-V151936", 16, 151936),  # the serving batch's verify
             ("long-B32C16F5-L8192-V151936", 3, 40000)]            # then a smaller one
    for k, (name, n_req, vocab) in enumerate(cases):
        print(f"noalloc call {k}: {name} n_req={n_req} V={vocab} T={T}", flush=True)
        sys.stdout.flush()
        zt, zd, tok, temp, seed = _inputs(name, n_req, vocab, T)
        want = _binding.spec_verify(zt, zd, tok, temp, seed, 7)
        got = _binding.spec_verify_noalloc(zt, zd, tok, temp, seed, 7)
        torch.cuda.synchronize()
        for key in ("n_accepted", "next_token", "alpha", "survival", "tau", "flags"):
            a, b = got[key].cpu().numpy(), want[key].cpu().numpy()
            assert np.array_equal(a, b), (name, key, a, b)
