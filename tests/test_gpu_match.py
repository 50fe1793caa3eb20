"""GPU parity of branch_cache_match and of one whole device round against the oracle."""

import sys

import numpy as np
import pytest
import torch

from block_diffusion_drafting_draft_amd import _binding, synth
from gpu_util import AttnProblem, attn_close, dev, host, require_gpu
from oracle import match as o_match
from oracle import packing as o_pack
from oracle import verify as o_ver

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _match(descs, off, n_acc, tok):
    return _binding.branch_cache_match(
        torch.from_numpy(np.ascontiguousarray(descs, np.int32)).cuda(),
        torch.from_numpy(np.asarray(off, np.int32)).cuda(),
        torch.from_numpy(np.asarray(n_acc, np.int32)).cuda(),
        torch.from_numpy(np.asarray(tok, np.int32)).cuda()).cpu().numpy()


def test_random_outcomes_match_oracle():
    require_gpu()
    _say("match: random outcomes, forced hits and misses")
    rng = np.random.default_rng(1)
    B, C, F = 16, 12, 2
    descs, blocks, off = [], [], [0]
    n_req = 200
    for i in range(n_req):
        anchors = rng.integers(0, 50, size=(C - 1) * F + 1)  # small id range: duplicates happen
        descs.append(_binding.d3d_build_branch_descs(B, C, F, 100 + i, int(rng.integers(0, 50)), anchors))
        blocks.append(o_pack.pack_blocks(B, C, F, 0, anchors))
        off.append(off[-1] + len(blocks[-1]))
    n_acc = rng.integers(0, B, size=n_req)
    tok = rng.integers(0, 50, size=n_req)
    # force hits on every 3rd request, misses (uncovered position) on every 7th
    for i in range(0, n_req, 3):
        b = int(rng.integers(1, len(blocks[i])))
        n_acc[i], tok[i] = blocks[i][b][0] - 1, blocks[i][b][1]
    for i in range(0, n_req, 7):
        n_acc[i] = C  # rejection position C + 1 is not covered
    got = _match(np.concatenate(descs), off, n_acc, tok)
    want = np.array([o_match.match_request(blocks[i], int(n_acc[i]), int(tok[i])) for i in range(n_req)])
    np.testing.assert_array_equal(got, want)
    forced_hit = [i for i in range(0, n_req, 3) if i % 7]
    assert (want[forced_hit] >= 0).all() and (want[::7] == -1).all()


@pytest.mark.parametrize("n_req,B,C,F", [(1, 2, 2, 1), (16, 16, 12, 2), (3, 64, 64, 3), (1000, 16, 4, 5),
                                          (7, 8, 8, 1)])
def test_device_descriptor_builder_matches_oracle(n_req, B, C, F):
    """d3d_build_branch_descs_device against the oracle's pack order, field by field, plus the block
    offsets; a second call into a larger, pre-filled buffer writes exactly its own entries."""
    require_gpu()
    _say(f"device descriptor build: n_req {n_req}, B {B}, C {C}, F {F}")
    rng = np.random.default_rng(n_req * 131 + B)
    per = (C - 1) * F + 2
    lens = rng.integers(0, 1 << 20, size=n_req).astype(np.int32)
    cur = rng.integers(-5, 151936, size=n_req).astype(np.int32)
    alt = rng.integers(-5, 151936, size=(n_req, per - 1)).astype(np.int32)
    want = np.zeros((n_req * per, 4), np.int32)
    for i in range(n_req):
        for b, (r, anchor, causal) in enumerate(o_pack.pack_blocks(B, C, F, int(cur[i]), alt[i])):
            want[i * per + b] = (lens[i], r, anchor, 1 if causal else 0)
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    descs, off = _binding.d3d_build_branch_descs_device(B, C, F, to(lens), to(cur), to(alt))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(descs.cpu().numpy(), want)
    np.testing.assert_array_equal(off.cpu().numpy(), np.arange(n_req + 1, dtype=np.int32) * per)
    big = torch.full((n_req * per + 5, 4), -7, dtype=torch.int32, device="cuda")
    _binding.d3d_build_branch_descs_device(B, C, F, to(lens), to(cur), to(alt), out=big)
    torch.cuda.synchronize()
    got = big.cpu().numpy()
    np.testing.assert_array_equal(got[:n_req * per], want)
    assert (got[n_req * per:] == -7).all()


def test_one_device_round_async():
    """Descriptor build -> packed attention -> verify -> match for the async workload, each against
    the oracle; the match is fed the GPU verify outcome and compared with the oracle match of the
    oracle outcome."""
    require_gpu()
    name = "async-B16C12F2-L4096-V151936"
    _say(f"device round: {name}")
    w = synth.WORKLOADS[name]
    vin = synth.verify_inputs(w)
    ain = synth.attention_inputs(w)
    a0 = int(vin["cur_anchor"][0])
    anchors = vin["alt_anchors"][0]
    prob = AttnProblem("bf16", w.block_size,
                       [dict(L=w.prefix[0], kind="async", C=w.coverage, F=w.fanout, a0=a0, anchors=anchors)], ain)
    out = host(prob.run())
    want, rows = prob.oracle()
    ok, emax, fro = attn_close(out[rows], want, 2e-2, 1e-2)
    _say(f"  attention max|err|={emax:.3g} rel_fro={fro:.3g}")
    assert ok
    res = _binding.spec_verify(dev(vin["z_target"], "bf16"), dev(vin["z_draft"], "bf16"),
                               torch.from_numpy(vin["tokens"]).cuda(), 1.0, vin["philox_seed"], 0)
    hit = _binding.branch_cache_match(prob.descs, torch.tensor(prob.off, dtype=torch.int32).cuda(),
                                      res["n_accepted"], res["next_token"]).cpu().numpy()
    o = o_ver.verify_request(vin["z_target"][0], vin["z_draft"][0], vin["tokens"][0], 1.0, vin["philox_seed"], 0, 0)
    blocks = o_pack.pack_blocks(w.block_size, w.coverage, w.fanout, a0, anchors)
    if not o.flags & 3:
        assert int(res["n_accepted"][0]) == o.n_accepted and int(res["next_token"][0]) == o.next_token
        assert int(hit[0]) == o_match.match_request(blocks, o.n_accepted, o.next_token)
    _say(f"  n_acc={o.n_accepted} token={o.next_token} hit={int(hit[0])}")


def test_graph_replays_match_eager():
    """The device round captured in a HIP graph gives, on every replay, exactly the eager results
    (the kernels are deterministic); eager work and synchronisations run between the replays."""
    require_gpu()
    _say("graph capture: replays vs eager")
    B, C, F, L = 16, 4, 2, 300
    w = synth.Workload("graph", "bf16", 32, 8, 128, B, C, F, (L,), 1, False, 4096, "zipf", 0.8, 1.0, 21, 0x77)
    ain, vin = synth.attention_inputs(w), synth.verify_inputs(w)
    prob = AttnProblem("bf16", B, [dict(L=L, kind="async", C=C, F=F, a0=int(vin["cur_anchor"][0]),
                                        anchors=vin["alt_anchors"][0])], ain)
    zt, zd = dev(vin["z_target"], "bf16"), dev(vin["z_draft"], "bf16")
    tok = torch.from_numpy(vin["tokens"]).cuda()
    off_dev = torch.tensor(prob.off, dtype=torch.int32).cuda()
    out = torch.empty_like(prob.q)
    need = _binding.draft_attn_packed_workspace("bf16", prob.off, prob.pre, B, 32, 8, 128)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    vws = torch.empty(_binding.spec_verify_workspace(1, B - 1, 4096), dtype=torch.uint8, device="cuda")
    res = dict(n_accepted=torch.empty(1, dtype=torch.int32, device="cuda"),
               next_token=torch.empty(1, dtype=torch.int32, device="cuda"),
               alpha=torch.empty(1, B - 1, device="cuda"), survival=torch.empty(1, B - 1, device="cuda"),
               tau=torch.empty(1, device="cuda"), flags=torch.empty(1, dtype=torch.int32, device="cuda"))
    hit = torch.empty(1, dtype=torch.int32, device="cuda")

    def device_round():
        _binding.draft_attn_packed(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.descs,
                                   prob.off, prob.pre, B, out=out, ws=ws)
        _binding.spec_verify(zt, zd, tok, 1.0, 0x77, 3, ws=vws, out=res)
        _binding.branch_cache_match(prob.descs, off_dev, res["n_accepted"], res["next_token"], hit=hit)

    def snapshot():
        torch.cuda.synchronize()
        return [out.clone(), hit.clone()] + [v.clone() for v in res.values()]

    device_round()
    eager = snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device_round()
    for rep in range(3):
        out.zero_()
        hit.fill_(-7)
        for v in res.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a, b in zip(eager, got):
            assert torch.equal(a, b), rep
        device_round()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("temperature", [1.0, 0.0])
def test_fused_verify_match_equals_the_two_calls(temperature):
    """spec_verify_match gives exactly spec_verify followed by branch_cache_match: 16 requests whose
    branch lists are built (from a first verify of the same inputs) so that some hold the verified
    outcome at various positions and the others miss."""
    require_gpu()
    _say(f"fused verify + match, T = {temperature}")
    w = synth.WORKLOADS["serve-16req-B16C12F2-paged16-V151936"]
    vin = synth.verify_inputs(w, vocab=8192, temperature=temperature)
    zt, zd = dev(vin["z_target"], "bf16"), dev(vin["z_draft"], "bf16")
    tok = torch.from_numpy(vin["tokens"]).cuda()
    first = _binding.spec_verify(zt, zd, tok, temperature, vin["philox_seed"], 5)
    n_acc = first["n_accepted"].cpu().numpy()
    nxt = first["next_token"].cpu().numpy()
    B, C, F = w.block_size, w.coverage, w.fanout
    rng = np.random.default_rng(3)
    descs, off = [], [0]
    for i in range(w.n_req):
        anchors = rng.integers(0, 8192, size=(C - 1) * F + 1).astype(np.int32)
        k = int(n_acc[i]) + 1
        if i % 3 != 2 and k <= C - 1:  # plant the outcome at rejection position k (fan-out slot i % F)
            anchors[(k - 1) * F + i % F] = nxt[i]
        elif i % 3 != 2 and k == B:  # full accept: the full-accept branch's anchor
            anchors[(C - 1) * F] = nxt[i]
        d = _binding.d3d_build_branch_descs(B, C, F, 1000 + i, int(rng.integers(0, 8192)), anchors)
        descs.append(d)
        off.append(off[-1] + len(d))
    descs_d = torch.from_numpy(np.ascontiguousarray(np.concatenate(descs), np.int32)).cuda()
    off_d = torch.tensor(off, dtype=torch.int32, device="cuda")
    sep = _binding.spec_verify(zt, zd, tok, temperature, vin["philox_seed"], 5)
    hit_sep = _binding.branch_cache_match(descs_d, off_d, sep["n_accepted"], sep["next_token"])
    fused = _binding.spec_verify(zt, zd, tok, temperature, vin["philox_seed"], 5, match=(descs_d, off_d))
    torch.cuda.synchronize()
    for key in ("n_accepted", "next_token", "alpha", "survival", "tau", "flags"):
        assert torch.equal(fused[key], sep[key]), key
    assert torch.equal(fused["hit_branch"], hit_sep)
    h = hit_sep.cpu().numpy()
    assert (h >= 0).sum() >= 4 and (h == -1).sum() >= 2, h


def test_round_with_join_equals_sequential_calls():
    """The round as the bench runs it when the attention merges splits: verify + match on a second
    stream, the attention stream joining it before its merge launch (draft_attn_packed_join). Outputs
    equal the plain calls in sequence, eagerly and on graph replays."""
    require_gpu()
    _say("two-stream round with the join before the merge")
    B, C, F, L = 16, 4, 2, 3000
    w = synth.Workload("join", "bf16", 32, 8, 128, B, C, F, (L,), 1, False, 4096, "zipf", 0.8, 1.0, 23, 0x79)
    ain, vin = synth.attention_inputs(w), synth.verify_inputs(w)
    prob = AttnProblem("bf16", B, [dict(L=L, kind="async", C=C, F=F, a0=int(vin["cur_anchor"][0]),
                                        anchors=vin["alt_anchors"][0])], ain)
    need = _binding.draft_attn_packed_workspace("bf16", prob.off, prob.pre, B, 32, 8, 128)
    assert need > 0  # the call merges splits
    zt, zd = dev(vin["z_target"], "bf16"), dev(vin["z_draft"], "bf16")
    tok = torch.from_numpy(vin["tokens"]).cuda()
    off_dev = torch.tensor(prob.off, dtype=torch.int32).cuda()
    ref_out = _binding.draft_attn_packed(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.descs,
                                         prob.off, prob.pre, B)
    ref = _binding.spec_verify(zt, zd, tok, 1.0, 0x79, 2)
    ref_hit = _binding.branch_cache_match(prob.descs, off_dev, ref["n_accepted"], ref["next_token"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    out = torch.empty_like(prob.q)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    res = {}

    def round_():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            res.update(_binding.spec_verify(zt, zd, tok, 1.0, 0x79, 2, out=res or None,
                                            match=(prob.descs, off_dev)))
            ev.record(side)
        _binding.draft_attn_packed(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.descs,
                                   prob.off, prob.pre, B, out=out, ws=ws, join=ev)
        cur.wait_stream(side)

    def check():
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        assert torch.equal(res["hit_branch"], ref_hit)
        for k in ("n_accepted", "next_token", "alpha", "survival", "tau", "flags"):
            assert torch.equal(res[k], ref[k]), k

    round_()
    check()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        round_()
    for _ in range(3):
        out.zero_()
        res["hit_branch"].fill_(-7)
        g.replay()
        check()
