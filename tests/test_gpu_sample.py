"""GPU parity of draft_sample (sampled drafting at temperature T) against the oracle, through the C ABI.

Bar: bit-exact token ids. Both sides decide the Gumbel-max winner in fp64 on the same Philox uniforms;
their fp64 logarithms may differ in the last bit, so a row whose two best oracle scores lie within
1e-9 (relative) of each other is reported and not compared (none is expected at these sizes)."""

import sys

import numpy as np
import pytest
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from gpu_util import dev, require_gpu
from oracle import select as o_sel

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-9


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _compare(z, T, seed, round_, got, row_index=None):
    """Compare got[r] with the oracle's draw for each row r of z (float32 host rows); returns the
    number of rows skipped as near ties."""
    skipped = 0
    for r in range(z.shape[0]):
        ri = r if row_index is None else int(row_index[r])
        s = o_sel.gumbel_scores(z[r], np.float32(T), seed, round_, ri)
        want = o_sel.sample_token(z[r], np.float32(T), seed, round_, ri)
        if want >= 0:
            fin = np.sort(s[np.isfinite(s)])
            if fin.size >= 2 and np.isfinite(s[want]) and fin[-1] - fin[-2] < NEAR_TIE * max(1.0, abs(fin[-1])):
                skipped += 1
                continue
        assert int(got[r]) == want, (r, int(got[r]), want)
    # near ties are rare (the two best of many continuous scores); a comparison that skipped most
    # rows would prove nothing
    assert skipped <= max(1, z.shape[0] // 10), skipped
    return skipped


def _zipf_rows(rng, n, V):
    """Drafter-like logit rows: N(0, 2) plus a -1.1 ln(rank) bias over a random permutation."""
    z = rng.normal(0, 2, size=(n, V)).astype(np.float32)
    for r in range(n):
        z[r] -= 1.1 * np.log(rng.permutation(V) + 1.0).astype(np.float32)
    return z


CASES = [
    # dtype, n_rows, V, T, kind
    ("bf16", 6, 151936, 1.0, "zipf"),
    ("bf16", 5, 1003, 0.7, "normal"),      # V not a multiple of 8: scalar path
    ("bf16", 4, 64, 2.0, "normal"),
    ("bf16", 3, 1, 1.0, "normal"),         # one token
    ("f32", 6, 4096, 1.0, "normal"),
    ("f32", 4, 5000, 1.0, "masked"),       # -inf tail, a NaN, one row all -inf
    ("f32", 4, 4096, 1e-3, "normal"),      # near-greedy: scores of order 1e3
    ("f32", 4, 4096, 50.0, "normal"),      # flat: the noise decides
    ("f32", 3, 4096, 1.0, "wide"),         # logits of order 1e4: the margin's relative part
    ("bf16", 4, 2048, 1.0, "ties"),        # few distinct logits
    ("f32", 3, 777, 1.0, "posinf"),        # +inf logits: the first one wins
]


def _make(rng, n, V, kind, dtype):
    if kind == "zipf":
        z = _zipf_rows(rng, n, V)
    elif kind == "ties":
        z = rng.integers(-3, 4, size=(n, V)).astype(np.float32)
    elif kind == "wide":
        z = rng.normal(0, 1e4, size=(n, V)).astype(np.float32)
    else:
        z = rng.normal(0, 2, size=(n, V)).astype(np.float32)
    if kind == "masked":
        z[:, V // 3:] = -np.inf
        z[0, 5] = np.nan
        z[-1, :] = -np.inf
    if kind == "posinf":
        z[0, [17, 400]] = np.inf
        z[1, V - 1] = np.inf
    return synth.round_bf16(z) if dtype == "bf16" else z


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_sample_parity(case):
    require_gpu()
    dtype, n, V, T, kind = case
    _say(f"draft_sample: {case}")
    rng = np.random.default_rng(V + n)
    z = _make(rng, n, V, kind, dtype)
    seed, round_ = 0xD3D5 + n, 3
    got = _binding.draft_sample(dev(z, dtype), T, seed, round_)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    skipped = _compare(z, T, seed, round_, got)
    _say(f"  near ties skipped: {skipped}")
    if kind == "masked":
        assert got[-1] == -1
    if kind == "posinf":
        assert got[0] == 17 and got[1] == V - 1


def test_row_gather_uses_the_row_index_as_counter():
    """rows[] picks logit rows; the counter word is the logits row index, so a row gathered twice draws
    the same token and the result does not depend on the gather order."""
    require_gpu()
    _say("draft_sample: row gather")
    rng = np.random.default_rng(5)
    z = synth.round_bf16(rng.normal(0, 2, size=(10, 8192)).astype(np.float32))
    rows = np.array([7, 2, 2, 9, 0], dtype=np.int32)
    got = _binding.draft_sample(dev(z, "bf16"), 1.0, 99, 1, rows=torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert got[1] == got[2]
    _compare(z[rows], 1.0, 99, 1, got, row_index=rows)


def test_drafted_tokens_of_a_packed_forward_sampled():
    """Sampled drafted tokens of the 384 packed positions over a 151936-token vocabulary at T = 1 (the
    launch the bench times), compared on 24 sampled rows, plus the remaining rows' validity."""
    require_gpu()
    _say("draft_sample: 384 x 151936 at T = 1")
    rng = np.random.default_rng(12)
    z = synth.round_bf16(_zipf_rows(rng, 384, 151936))
    got = _binding.draft_sample(dev(z, "bf16"), 1.0, 0xD3D2, 0)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert ((got >= 0) & (got < 151936)).all()
    pick = np.sort(rng.choice(384, size=24, replace=False))
    skipped = _compare(z[pick], 1.0, 0xD3D2, 0, got[pick], row_index=pick)
    _say(f"  near ties skipped: {skipped}")


def test_draws_follow_the_softmax():
    """40000 identical rows of a 5-token vocabulary: the draw frequencies match softmax(z / T) (chi-square
    at 4 degrees of freedom, fixed seed)."""
    require_gpu()
    _say("draft_sample: frequencies")
    z0 = np.array([0.3, -1.0, 1.2, 0.0, -0.4], dtype=np.float32)
    T, n = 0.8, 40000
    z = np.tile(z0, (n, 1))
    got = _binding.draft_sample(dev(z, "f32"), T, 2024, 0)
    torch.cuda.synchronize()
    counts = np.bincount(got.cpu().numpy(), minlength=5)
    p = np.exp(z0 / T - np.max(z0 / T))
    p /= p.sum()
    chi2 = float((((counts - n * p) ** 2) / (n * p)).sum())
    assert chi2 < 18.47, (counts, n * p, chi2)  # p = 0.001 at 4 degrees of freedom


def test_bad_arguments_raise():
    require_gpu()
    z = torch.zeros((2, 16), dtype=torch.bfloat16, device="cuda")
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(RuntimeError):
            _binding.draft_sample(z, T, 1, 0)
