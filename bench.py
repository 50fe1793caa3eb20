#!/usr/bin/env python3
"""Benchmark of one packed async draft round on one MI355X.

A step is one pass of the whole hot path over one synthetic round of the async workload
(B = 16, C = 12, F = 2: 24 blocks, 384 packed queries; 32 query / 8 key-value heads, head dim 128,
4096-token prefix; verify of 16 target + 15 draft rows over a 151936-token vocabulary):
  1. branch descriptors of every request built on the GPU (d3d_build_branch_descs_device) from the
     device-resident prefix lengths and anchors (in a serving loop the anchors come from draft_topk
     on the GPU and the prefix lengths from kv_commit),
  2. draft_attn_packed (one drafter attention layer, all heads),
  3. spec_verify (stats; decide, split residual sums and the draw in one launch),
  4. branch_cache_match.
Inputs are resident in HBM before the timed region. A step (1-4) is captured once in a HIP graph,
with 2 and 3 on two streams (they are independent within a round: drafting the next block's branches
overlaps verifying the current block) joined before 4; each step replays the graph. The host
builder's CPU time and the copy a host-built batch would need are reported beside it
(calls_us.descriptor_build_host, descriptor_copy).
W untimed warm-up steps, then K timed steps between device synchronisations. Per-call durations
come from HIP events recorded on the launch stream around K replays of a graph holding only that
call. Prints one JSON line. `--call NAME` replays only that call's graph (the command to profile one
call's kernels alone).

`python bench.py --gpus N --steps K --warmup W [--workload NAME] [--no-cpu-baseline] [--call NAME]`
"""

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (2.5 PFLOP/s)
MFMA_F32_PEAK_TFLOPS = 157.3
METRIC = "µs per packed draft round (384 q) + attn TFLOP/s % MFMA peak; verify GB/s % HBM"


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="async-B16C12F2-L4096-V151936")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on the oracle's timed CPU work")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB three times (the reference "
                        "dispatch that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--no-serve-verify", action="store_true",
                   help="skip the serving batch's verify measurement (warm and cold) and the synchronous "
                        "draft's attention call")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip the next-row measurements (token selection, KV commit, AWL, training attention)")
    p.add_argument("--call", choices=("round", "descriptor_build_device", "draft_attn_packed", "spec_verify",
                                     "branch_cache_match", "awl_loss",
                                     "train_attn_fwd", "train_attn_bwd", "draft_topk_tokens", "draft_topk_anchors",
                                     "draft_sample_tokens",
                                     "kv_commit"),
                   default=None,
                   help="only replay this call's graph (warmup + steps times, nothing else on the GPU) and print "
                        "its event-timed duration: the command to profile one call's kernels alone")
    p.add_argument("--calls-per-graph", type=int, default=1,
                   help="with --call: capture this many back-to-back copies of the call in its graph and "
                        "report the time per copy (a small call's own graph replay is bounded below by the "
                        "graph launch, ~10-15 us on this system)")
    return p.parse_args()


def visible_pairs(B, blocks, L):
    """(query, key) pairs one request's packed attention actually scores (the algorithmic work)."""
    n = 0
    for b, (r, causal) in enumerate(blocks):
        for i in range(B):
            n += L + (r if b > 0 else 0) + (i + 1 if causal else B)
    return n


class Round:
    """Device-resident inputs of one round plus the calls of one step."""

    def __init__(self, w):
        import torch
        from block_diffusion_drafting_draft_amd import _binding, synth
        self.torch, self.lib, self.w = torch, _binding, w
        _binding.load()
        self.ain = synth.attention_inputs(w)
        self.vin = synth.verify_inputs(w)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        bits = (lambda x: torch.from_numpy(synth.f32_to_bf16_bits(x).view(np.int16).copy()).view(torch.bfloat16)) \
            if w.dtype == "bf16" else (lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)))
        cu = lambda x: bits(x).cuda()
        self.B = w.block_size
        self.lens = self.ain["prefix"]
        self.lens_i32 = np.asarray(self.lens, dtype=np.int32)
        self.n_req = len(self.lens)
        self.q, self.k_new, self.v_new = cu(self.ain["q"]), cu(self.ain["k_new"]), cu(self.ain["v_new"])
        if w.paged:
            kp, table = synth.paginate(self.ain["k_prefix"], w.page_size, w.seed)
            vp, _ = synth.paginate(self.ain["v_prefix"], w.page_size, w.seed)
            self.k_cache, self.v_cache = cu(kp), cu(vp)
            self.page_table = torch.from_numpy(table).cuda()
        else:
            stride = max(self.lens)
            kc = np.zeros((self.n_req, stride) + self.ain["k_prefix"][0].shape[1:], np.float32)
            vc = np.zeros_like(kc)
            for i in range(self.n_req):
                kc[i, :self.lens[i]] = self.ain["k_prefix"][i]
                vc[i, :self.lens[i]] = self.ain["v_prefix"][i]
            self.k_cache, self.v_cache = cu(kc), cu(vc)
            self.page_table = None
        self.z_t, self.z_d = cu(self.vin["z_target"]), cu(self.vin["z_draft"])
        self.tokens = torch.from_numpy(self.vin["tokens"]).cuda()
        # descriptors: host build each step into pinned memory, async copy to the device
        self.blocks_per_req = [(w.coverage - 1) * w.fanout + 2 if w.coverage else 1] * self.n_req
        self.off = np.concatenate([[0], np.cumsum(self.blocks_per_req)]).astype(np.int32)
        n_blk = int(self.off[-1])
        self.desc_host = torch.empty((n_blk, 4), dtype=torch.int32, pin_memory=True)
        self.descs = torch.empty((n_blk, 4), dtype=torch.int32, device="cuda")
        self.off_dev = torch.from_numpy(self.off).cuda()
        self.off_scratch = np.zeros(self.n_req + 1, dtype=np.int32)
        self.cur_anchor = np.ascontiguousarray(self.vin["cur_anchor"], dtype=np.int32)
        self.alt_anchors = np.ascontiguousarray(self.vin["alt_anchors"], dtype=np.int32) if w.coverage else None
        # the device builder's inputs, resident like the round's other inputs
        self.lens_dev = torch.from_numpy(self.lens_i32.copy()).cuda()
        self.cur_dev = torch.from_numpy(self.cur_anchor.copy()).cuda()
        self.alt_dev = torch.from_numpy(self.alt_anchors.copy()).cuda() if w.coverage else None
        self.out = torch.empty_like(self.q)
        need = _binding.draft_attn_packed_workspace(self.q.dtype, self.off, self.lens, self.B, self.q.shape[1],
                                                    self.k_new.shape[1], self.q.shape[2])
        self.attn_ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.attn_merges = need > 0  # split partials: the call ends with its merge launch
        nd = self.B - 1
        self.ver_ws = torch.empty(_binding.spec_verify_workspace(self.n_req, nd, w.vocab), dtype=torch.uint8,
                                  device="cuda")
        self.ver_out = dict(n_accepted=torch.empty(self.n_req, dtype=torch.int32, device="cuda"),
                            next_token=torch.empty(self.n_req, dtype=torch.int32, device="cuda"),
                            alpha=torch.empty(self.n_req, nd, dtype=torch.float32, device="cuda"),
                            survival=torch.empty(self.n_req, nd, dtype=torch.float32, device="cuda"),
                            tau=torch.empty(self.n_req, dtype=torch.float32, device="cuda"),
                            flags=torch.empty(self.n_req, dtype=torch.int32, device="cuda"))
        self.hit = torch.empty(self.n_req, dtype=torch.int32, device="cuda")
        self.ver_out["hit_branch"] = self.hit  # the fused verify + match writes the same hit tensor
        self.round = 0

    def build_descs_device(self):
        """The round's descriptors built on the GPU from the device-resident prefix lengths and anchors.
        A workload without branches has one descriptor per request, {prefix_len, 0, anchor, 0}: its
        two varying fields are copied in (rej_pos and flags stay 0)."""
        if self.w.coverage:
            self.lib.d3d_build_branch_descs_device(self.B, self.w.coverage, self.w.fanout, self.lens_dev,
                                                   self.cur_dev, self.alt_dev, out=self.descs,
                                                   req_block_off=self.off_dev)
        else:
            self.descs[:, 0].copy_(self.lens_dev)
            self.descs[:, 2].copy_(self.cur_dev)

    def build_descs(self, pinned=None):
        w = self.w
        host = (self.desc_host if pinned is None else pinned).numpy()
        if w.coverage:
            self.lib.d3d_build_branch_descs_batch(self.B, w.coverage, w.fanout, self.lens_i32, self.cur_anchor,
                                                  self.alt_anchors, out=host, req_block_off=self.off_scratch)
        else:
            host[:, 0], host[:, 1], host[:, 2], host[:, 3] = self.lens, 0, self.cur_anchor, 0
        if pinned is None:
            self.descs.copy_(self.desc_host, non_blocking=True)

    def attention(self, join=None):
        self.lib.draft_attn_packed(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache, self.descs,
                                   self.off, self.lens_i32, self.B, page_table=self.page_table,
                                   page_size=self.w.page_size, out=self.out, ws=self.attn_ws, join=join)

    def verify(self, match=False):
        """spec_verify; with match=True the cache match runs inside it (spec_verify_match)."""
        self.lib.spec_verify(self.z_t, self.z_d, self.tokens, self.vin["temperature"], self.vin["philox_seed"],
                             self.round, ws=self.ver_ws, out=self.ver_out,
                             match=(self.descs, self.off_dev) if match else None)
        self.round += 1

    def match(self):
        self.lib.branch_cache_match(self.descs, self.off_dev, self.ver_out["n_accepted"],
                                    self.ver_out["next_token"], hit=self.hit)

    def work(self):
        """Algorithmic FLOPs / bytes per call, counted from the pages' definitions."""
        w = self.w
        d, hq, hkv = self.q.shape[2], self.q.shape[1], self.k_new.shape[1]
        es = 2 if w.dtype == "bf16" else 4
        if w.coverage:
            blocks = [(0, True)] + [(k, False) for k in range(1, w.coverage) for _ in range(w.fanout)] + \
                     [(self.B, False)]
        else:
            blocks = [(0, False)]
        pairs = sum(visible_pairs(self.B, blocks, L) for L in self.lens)
        nq = self.q.shape[0]
        attn_flops = 4 * d * hq * pairs
        attn_bytes = es * (2 * nq * hq * d + 2 * nq * hkv * d + 2 * sum(self.lens) * hkv * d)
        nd = self.B - 1
        ver_bytes = es * self.n_req * (2 * nd + 1) * w.vocab + 4 * self.n_req * nd + \
            self.n_req * (4 + 4 + 4 * nd + 4 * nd + 4 + 4)
        return attn_flops, attn_bytes, ver_bytes


def cpu_baseline(w, budget_s):
    """The oracle as it stands, on the same round: packing + attention + verify + match, repeated
    until `budget_s` seconds of CPU work; reports the median per round."""
    from threadpoolctl import threadpool_info
    from block_diffusion_drafting_draft_amd import synth
    from oracle import attention, match, packing, verify
    ain, vin = synth.attention_inputs(w), synth.verify_inputs(w)
    B, d = w.block_size, ain["q"].shape[2]
    nq = ain["q_per_req"][0]
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        for i, L in enumerate(ain["prefix"]):
            if w.coverage:
                blocks = packing.pack_blocks(B, w.coverage, w.fanout, int(vin["cur_anchor"][i]), vin["alt_anchors"][i])
            else:
                blocks = [(0, int(vin["cur_anchor"][i]), False)]
            mask = packing.visible_mask(B, blocks, L)
            sl = slice(i * nq, (i + 1) * nq)
            attention.packed_attention(ain["q"][sl], ain["k_prefix"][i], ain["v_prefix"][i], ain["k_new"][sl],
                                       ain["v_new"][sl], mask, d ** -0.5)
            o = verify.verify_request(vin["z_target"][i], vin["z_draft"][i], vin["tokens"][i], vin["temperature"],
                                      vin["philox_seed"], 0, i)
            match.match_request(blocks, o.n_accepted, o.next_token)
        times.append(time.perf_counter() - t0)
    info = threadpool_info()
    threads = max([p["num_threads"] for p in info] or [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=statistics.median(times) * 1e6, unit="µs per packed draft round", cores=threads,
                kind="oracle", cpu_model=model, cpu_count=os.cpu_count(),
                affinity=len(os.sched_getaffinity(0)),
                blas=sorted({f"{p.get('internal_api')} {p.get('version')}" for p in info if p.get("user_api") == "blas"}),
                sample=f"{len(times)} full rounds of the same workload (all queries and heads, verify of every row, "
                       f"match), float64 NumPy, median; not a tuned CPU implementation")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the path is built and measured on a single GPU, so --gpus {args.gpus} "
              f"is not run (it would shard by request or key/value head).", file=sys.stderr)
        return 2
    import torch
    from block_diffusion_drafting_draft_amd import synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "dispatches": 3}), flush=True)
        return 0
    w = synth.WORKLOADS[args.workload]
    r = Round(w)
    ring = [torch.empty_like(r.desc_host).pin_memory() for _ in range(3)]  # host-path copy timing only

    side = torch.cuda.Stream()  # default priority
    verified = torch.cuda.Event()

    def device_round():
        # The drafter's packed attention (branches for the next block) and the target's verify of the
        # current block are independent within a round: they run on two streams. The cache match needs
        # the verify outcome and the branch descriptors (built before the round), not the drafted
        # branches. When the attention ends with its split merge, the match runs inside the verify
        # launches (spec_verify_match) and the attention stream joins the verify stream just before
        # the merge launch (draft_attn_packed_join): the round ends with that kernel. Without a merge,
        # the match kernel follows the join (a graph that ends on a bare join measured slower).
        # The descriptors are built first, on the GPU; both streams wait for them.
        cur = torch.cuda.current_stream()
        r.build_descs_device()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            r.verify(match=r.attn_merges)
            verified.record(side)
        if r.attn_merges:
            r.attention(join=verified)
            cur.wait_stream(side)
        else:
            r.attention()
            cur.wait_stream(side)
            r.match()

    r.build_descs()  # host build + copy: the fixed descriptors of a workload without branches
    torch.cuda.synchronize()
    for _ in range(3):  # eager warm-up (first launches, code-object loads)
        device_round()
    torch.cuda.synchronize()
    graphs = {}
    calls = [("round", device_round), ("draft_attn_packed", r.attention), ("spec_verify", r.verify),
             ("branch_cache_match", r.match)]
    calls.append(("descriptor_build_device", r.build_descs_device))
    for name, fn in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    if args.call:
        if args.call == "awl_loss":
            g = awl_graph(r, torch)[0]
        elif args.call in ("draft_topk_tokens", "draft_topk_anchors", "draft_sample_tokens"):
            tg = topk_graphs(r, torch)
            if tg is None:
                print("this workload drafts no branches", file=sys.stderr)
                return 2
            g = tg[{"draft_topk_tokens": "tokens", "draft_topk_anchors": "anchors",
                    "draft_sample_tokens": "sampled"}[args.call]][0]
        elif args.call == "kv_commit":
            g = next_row_commit(r, torch, None, graph_only=True)
        elif args.call in ("train_attn_fwd", "train_attn_bwd"):
            g = train_attn_graphs(r, torch)[0 if args.call == "train_attn_fwd" else 1]
        else:
            g = graphs[args.call]
        n_copies = max(1, args.calls_per_graph)
        if n_copies > 1:
            fn = dict(calls)[args.call] if args.call in dict(calls) else None
            if fn is None:
                print("--calls-per-graph applies to round, descriptor_build_device, draft_attn_packed, spec_verify "
                      "and branch_cache_match", file=sys.stderr)
                return 2
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(n_copies):
                    fn()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(cur)
        for _ in range(args.steps):
            g.replay()
        e1.record(cur)
        e1.synchronize()
        print(json.dumps({"workload": w.name, "call": args.call, "replays": args.steps, "calls_per_graph": n_copies,
                          "us_per_call": round(e0.elapsed_time(e1) * 1e3 / max(args.steps * n_copies, 1), 3)}),
              flush=True)
        return 0

    def step(k):
        graphs["round"].replay()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    def per_replay_us(g, reps, warmup=10, before=None):
        """HIP-event duration (µs) of each of `reps` replays of graph g on the launch stream, after
        `warmup` untimed replays; `before(k)`, if given, is enqueued (untimed) ahead of replay k."""
        for _ in range(warmup):
            g.replay()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for k, (e0, e1) in enumerate(evs):
            if before is not None:
                before(k)
            e0.record(cur)
            g.replay()
            e1.record(cur)
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])

    def summary(x):
        return float(np.median(x)), float(np.percentile(x, 10)), float(np.percentile(x, 90))

    def mean_us(g, reps, warmup=10):
        """Average duration (µs) of `reps` back-to-back replays of graph g between two HIP events on
        the launch stream: the per-launch time a kernel profiler reports, launch latency amortised."""
        for _ in range(warmup):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(cur)
        for _ in range(reps):
            g.replay()
        e1.record(cur)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    reps = 100
    names = ("draft_attn_packed", "spec_verify", "branch_cache_match", "round")
    t_attn, t_ver, t_match, t_round = (mean_us(graphs[n], reps) for n in names)
    # Device time of one call without a graph replay's launch latency: graphs of n_copy back-to-back
    # copies of the call, per copy. A small call's own replay is bounded below by the graph launch.
    n_copy = 10
    in_graph = {}
    for name, fn in (("descriptor_build_device", r.build_descs_device), ("draft_attn_packed", r.attention),
                     ("spec_verify", r.verify), ("branch_cache_match", r.match)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_copy):
                fn()
        torch.cuda.synchronize()
        in_graph[name] = mean_us(g, 30) / n_copy
        del g
    stats = {n: summary(per_replay_us(graphs[n], reps)) for n in names}
    t_ver_cold = summary(verify_cold_us(r.lib, r.z_t, r.z_d, r.tokens, r.vin["temperature"], r.vin["philox_seed"],
                                        r.round, r.ver_ws, r.ver_out, per_replay_us, reps))
    serve = None if args.no_serve_verify else verify_serve(torch, mean_us, per_replay_us, summary, reps)
    sync = sync_attention(torch, mean_us, reps) if w.coverage and not args.no_serve_verify else None
    # the host path for comparison: CPU time of the batched host builder, and the copy of its batch
    scratch = torch.empty_like(r.desc_host)
    n_host = 2000
    t_h = time.perf_counter()
    for _ in range(n_host):
        r.build_descs(scratch)
    t_desc_host = (time.perf_counter() - t_h) * 1e6 / n_host
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(cur)
    for k in range(reps):
        r.descs.copy_(ring[k % len(ring)], non_blocking=True)
    e1.record(cur)
    e1.synchronize()
    t_desc = e0.elapsed_time(e1) * 1e3 / reps
    r.build_descs()  # the copies above overwrote the device descriptors with a host batch
    torch.cuda.synchronize()
    t_desc_dev = mean_us(graphs["descriptor_build_device"], reps)
    attn_flops, attn_bytes, ver_bytes = r.work()
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    attn_tflops = attn_flops / (in_graph["draft_attn_packed"] * 1e-6) / 1e12
    ver_gbs = ver_bytes / (in_graph["spec_verify"] * 1e-6) / 1e9
    traffic = None
    tf = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "attn_traffic.json")
    if os.path.exists(tf):
        with open(tf) as fh:
            rec = json.load(fh)
        if rec.get("workload") == w.name and rec.get("source_digest") == _kernel_digest():
            traffic = rec.get("bytes_per_launch")
    out = {
        "metric": METRIC,
        "value": round(ms_step * 1e3, 3),
        "unit": "µs",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_req": r.n_req, "block_size": w.block_size, "coverage": w.coverage,
                   "fanout": w.fanout, "prefix": r.lens if r.n_req > 1 else r.lens[0],
                   "packed_queries": int(r.q.shape[0]), "heads_q": int(r.q.shape[1]),
                   "heads_kv": int(r.k_new.shape[1]), "head_dim": int(r.q.shape[2]), "vocab": w.vocab,
                   "paged": w.paged},
        "calls_us": {"descriptor_build_device": round(t_desc_dev, 3),
                     "descriptor_build_host": round(t_desc_host, 3),
                     "descriptor_copy": round(t_desc, 3), "draft_attn_packed": round(t_attn, 3),
                     "spec_verify": round(t_ver, 3), "branch_cache_match": round(t_match, 3),
                     "device_round": round(t_round, 3)},
        "calls_us_median_p10_p90": {("device_round" if n == "round" else n): [round(v[0], 3), round(v[1], 3),
                                                                              round(v[2], 3)]
                                    for n, v in stats.items()},
        "timing": "value: wall time per step over K back-to-back steps, each one replay of the round graph "
                  "(descriptors built on the GPU inside it); "
                  "calls_us: mean of 100 back-to-back graph replays between two HIP events on the launch "
                  "stream after 10 warm-up replays (each replay's launch latency included); "
                  "calls_us_in_graph: the same over 30 replays of a graph holding 10 back-to-back copies of "
                  "the call, per copy (the call's device time; used for the percentages and the roofline); "
                  "descriptor_build_host: CPU time of the batched host builder per call; "
                  "calls_us_median_p10_p90: HIP events around each of 100 replays (includes each launch's "
                  "latency)",
        "attn": {"tflops": round(attn_tflops, 2), "pct_mfma_peak": round(100 * attn_tflops / peak, 2),
                 "flops": attn_flops, "bytes": attn_bytes},
        "verify": {"gbs": round(ver_gbs, 1), "pct_hbm_peak": round(100 * ver_gbs / HBM_PEAK_GBS, 2),
                   "bytes": ver_bytes},
        "verify_cold": {"us": round(t_ver_cold[0], 3), "p10_p90": [round(t_ver_cold[1], 3), round(t_ver_cold[2], 3)],
                        "gbs": round(ver_bytes / (t_ver_cold[0] * 1e-6) / 1e9, 1),
                        "pct_hbm_peak": round(100 * ver_bytes / (t_ver_cold[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                        "protocol": "512 MiB read before each call (untimed) to flush the MALL; logits rotate "
                                    "over 3 copies; HIP events around each call; median of 100"},
        "calls_us_in_graph": {n: round(v, 3) for n, v in in_graph.items()},
        "roofline": {"bound": "mfma", "kernel": "draft_attn_packed (attn_kernel + combine_kernel)",
                     "achieved": round(attn_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4), "traffic": traffic},
    }
    if serve is not None:
        out["verify_serve"] = serve
    if sync is not None:
        out["sync_attention"] = sync
    if not args.no_next_rows:
        out["next_rows"] = {"draft_topk": next_row_topk(r, torch, cur, mean_us),
                            "kv_commit": next_row_commit(r, torch, mean_us),
                            "awl_loss": next_row_awl(r, torch, mean_us),
                            "train_attn": next_row_train_attn(r, torch, mean_us)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def verify_cold_us(lib, zt, zd, tokens, temperature, seed, round_, ws, out, per_replay_us, reps):
    """HIP-event duration (µs) of `reps` spec_verify calls, each after the MALL has been flushed by
    reading 512 MiB (untimed; a read leaves no dirty lines whose write-back would compete with the
    timed reads), the logits rotating over three copies."""
    import torch
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    copies = [(zt.clone(), zd.clone(), tokens.clone()) for _ in range(3)]
    graphs = []
    for a, b, c in copies:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lib.spec_verify(a, b, c, temperature, seed, round_, ws=ws, out=out)
        graphs.append(g)
    torch.cuda.synchronize()
    cold = []
    for k in range(reps):
        torch.sum(flush, dim=0, out=sink)
        cold.append(per_replay_us(graphs[k % 3], 1, warmup=0)[0])
    del flush, sink, copies, graphs
    return np.array(cold)


def sync_attention(torch, mean_us, reps):
    """draft_attn_packed of the synchronous draft a cache miss falls back to (one request, one
    16-query block, 32/8 heads, d = 128, 2048-token prefix): device time per call in a graph of 10
    back-to-back copies, and per replay of a one-call graph."""
    from block_diffusion_drafting_draft_amd import synth
    w = synth.WORKLOADS["sync-bf16-L2048-V151936"]
    r = Round(w)
    r.build_descs()
    for _ in range(3):
        r.attention()
    torch.cuda.synchronize()
    g1, g10 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        r.attention()
    with torch.cuda.graph(g10):
        for _ in range(10):
            r.attention()
    torch.cuda.synchronize()
    t1 = mean_us(g1, reps)
    t10 = mean_us(g10, 30) / 10
    flops = r.work()[0]
    del g1, g10, r
    return {"workload": w.name, "us_in_graph": round(t10, 3), "us_single_replay": round(t1, 3),
            "tflops_in_graph": round(flops / (t10 * 1e-6) / 1e12, 2),
            "pct_mfma_peak_in_graph": round(100 * flops / (t10 * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2)}


def verify_serve(torch, mean_us, per_replay_us, summary, reps):
    """spec_verify on the serving batch's verify (16 requests x (16 target + 15 draft rows) over
    V = 151936, bf16: 150,720,512 bytes), the largest verify here, against the HBM peak: warm (mean of
    back-to-back replays) and cold (MALL flushed before each call, median)."""
    from block_diffusion_drafting_draft_amd import _binding, synth
    w = synth.WORKLOADS["serve-16req-B16C12F2-paged16-V151936"]
    vin = synth.verify_inputs(w)
    cu = lambda x: torch.from_numpy(synth.f32_to_bf16_bits(x).view(np.int16).copy()).view(torch.bfloat16).cuda()
    zt, zd = cu(vin["z_target"]), cu(vin["z_draft"])
    tok = torch.from_numpy(vin["tokens"]).cuda()
    n_req, nd = tok.shape
    ws = torch.empty(_binding.spec_verify_workspace(n_req, nd, w.vocab), dtype=torch.uint8, device="cuda")
    out = _binding.spec_verify(zt, zd, tok, vin["temperature"], vin["philox_seed"], 0, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _binding.spec_verify(zt, zd, tok, vin["temperature"], vin["philox_seed"], 0, ws=ws, out=out)
    warm = mean_us(g, reps)
    cold = summary(verify_cold_us(_binding, zt, zd, tok, vin["temperature"], vin["philox_seed"], 0, ws, out,
                                  per_replay_us, reps))
    nbytes = 2 * n_req * (2 * nd + 1) * w.vocab + 4 * n_req * nd + n_req * (4 + 4 + 4 * nd + 4 * nd + 4 + 4)
    del g, zt, zd, tok, ws, out
    gbs = lambda t: nbytes / (t * 1e-6) / 1e9
    return {"workload": w.name, "bytes": nbytes,
            "warm_us": round(warm, 3), "warm_gbs": round(gbs(warm), 1),
            "warm_pct_hbm_peak": round(100 * gbs(warm) / HBM_PEAK_GBS, 2),
            "cold_us": round(cold[0], 3), "cold_p10_p90": [round(cold[1], 3), round(cold[2], 3)],
            "cold_gbs": round(gbs(cold[0]), 1), "cold_pct_hbm_peak": round(100 * gbs(cold[0]) / HBM_PEAK_GBS, 2),
            "protocol": "warm: mean of 100 back-to-back graph replays; cold: 512 MiB read before each call "
                        "(untimed), logits rotating over 3 copies, HIP events around each call, median of 100"}


def awl_graph(r, torch, n_blocks=128, n_pos=15):
    """Graph of one awl_loss call with its gradient at one training sample's shape: 128 anchor blocks
    x 15 future positions (B = 16) over the workload's vocabulary. Logits, tokens, labels and the
    inclusion mask are drawn on the device (timing only; the tests check this shape against the
    oracle). HBM bytes = rows x V x 2 B x 4: target and draft logits read for the statistics, the
    draft logits read again and the gradient written. Returns (graph, bytes, shape), or None when the
    workload's logits are not bf16."""
    w, lib = r.w, r.lib
    if w.dtype != "bf16":
        return None
    V = w.vocab
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 4)
    zt = (torch.randn((n_blocks, n_pos, V), generator=gen, device="cuda") * 2.0).to(torch.bfloat16)
    zd = (zt.float() + torch.randn((n_blocks, n_pos, V), generator=gen, device="cuda")).to(torch.bfloat16)
    tok = zd.argmax(dim=-1).to(torch.int32)
    lab = zt.argmax(dim=-1).to(torch.int32)
    inc = (torch.rand((n_blocks, n_pos), generator=gen, device="cuda") < 0.85).to(torch.int32)
    out = lib.awl_loss(zt, zd, tok, lab, include=inc, grad=True)
    ws = torch.empty(lib.awl_loss_workspace(n_blocks, n_pos, V), dtype=torch.uint8, device="cuda")

    def fn():
        lib.awl_loss(zt, zd, tok, lab, include=inc, grad=True, out=out, ws=ws)

    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.keep = (zt, zd, tok, lab, inc, out, ws)
    return g, n_blocks * n_pos * V * 2 * 4, [n_blocks, n_pos, V]


def train_attn_graphs(r, torch, L=4096, n_blocks=128, B=16):
    """Graphs of the training-time packed attention forward and backward at one training sample's
    shape: a 4096-token response with 128 anchors (sorted, drawn uniformly), B = 16, the drafter's
    32 query / 8 key-value heads of dimension 128. q, k, v, dout are N(0, 1) bf16 drawn on the device
    (timing only; the tests check this shape against the oracle). Returns (fwd graph, bwd graph,
    visible (row, key) pairs per query head)."""
    gen = torch.Generator(device="cuda").manual_seed(r.w.seed + 5)
    hq, hkv, d = 32, 8, 128
    N = L + n_blocks * B
    q = torch.randn((N, hq, d), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((N, hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((N, hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
    dout = torch.randn((N, hq, d), generator=gen, device="cuda").to(torch.bfloat16)
    anchors = torch.sort(torch.randint(0, L + 1, (n_blocks,), generator=gen, device="cuda"))[0].to(torch.int32)
    lib = r.lib
    out, lse = lib.train_attn_fwd(q, k, v, anchors, L, B)
    dq, dk, dv = lib.train_attn_bwd(q, k, v, out, dout, lse, anchors, L, B)
    ws = torch.empty(lib.train_attn_workspace(L, n_blocks, B, hq, hkv), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    gf, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf):
        lib.train_attn_fwd(q, k, v, anchors, L, B, out=out, lse=lse)
    with torch.cuda.graph(gb):
        lib.train_attn_bwd(q, k, v, out, dout, lse, anchors, L, B, dq=dq, dk=dk, dv=dv, ws=ws)
    keep = (q, k, v, dout, anchors, out, lse, dq, dk, dv, ws)
    gf.keep = gb.keep = keep
    a = anchors.cpu().numpy().astype(np.int64)
    pairs = L * (L + 1) // 2 + int(np.sum(B * (a + B)))
    return gf, gb, pairs * hq


def next_row_train_attn(r, torch, mean_us):
    """Training-time packed attention (the third next row): forward and backward, each the mean of
    back-to-back graph replays. Algorithmic FLOPs per visible (row, key) pair and query head: 4 d
    forward (q.k and p.v), 10 d backward (s recomputed, dP, dV, dK, dQ)."""
    gf, gb, pairs = train_attn_graphs(r, torch)
    d = 128
    tf, tb = mean_us(gf, 20), mean_us(gb, 20)
    ff, fb = 4 * d * pairs, 10 * d * pairs
    peak = MFMA_BF16_PEAK_TFLOPS
    return {"shape": "L 4096 + 128 x 16, 32/8 heads, d 128", "visible_pairs_per_head": pairs // 32,
            "fwd_us": round(tf, 2), "bwd_us": round(tb, 2),
            "fwd_tflops": round(ff / tf / 1e6, 1), "bwd_tflops": round(fb / tb / 1e6, 1),
            "fwd_pct_mfma_peak": round(100 * ff / tf / 1e6 / peak, 2),
            "bwd_pct_mfma_peak": round(100 * fb / tb / 1e6 / peak, 2)}


def next_row_awl(r, torch, mean_us):
    """Acceptance-weighted drafter-training loss with its gradient (the fourth next row, not part of
    the step), timed as the mean of back-to-back graph replays."""
    made = awl_graph(r, torch)
    if made is None:
        return None
    g, nbytes, shape = made
    t = mean_us(g, 50)
    gbs = nbytes / (t * 1e-6) / 1e9
    return {"shape": shape, "us": round(t, 3), "bytes": nbytes, "gbs": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}


def next_row_commit(r, torch, mean_us, graph_only=False):
    """KV commit (the second next row, not part of the step): each request's accepted slice (n_acc + 1
    rows of block 0, n_acc from this round's verify outputs) appended to a paged cache at the end of
    its prefix, plus promotion of the hit branch. The page table maps the pages around each prefix
    end to a small pool (timing only); the prefix lengths are restored inside the graph before
    each commit. Bytes = sum (n_acc + 1) x H_kv x d x 2 B x 2 (keys, values) x 2 (read, write)."""
    B, n_req = r.B, r.n_req
    hkv, d = int(r.k_new.shape[1]), int(r.k_new.shape[2])
    ps = 16
    lens0 = torch.tensor(r.lens_i32, dtype=torch.int32, device="cuda")
    span = (B + ps - 1) // ps + 1  # pages a slice of at most B tokens can touch
    max_pages = max(r.lens) // ps + span
    table = torch.full((n_req, max_pages), -1, dtype=torch.int32)
    for i, L in enumerate(r.lens):
        for p in range(span):
            table[i, L // ps + p] = span * i + p
    table = table.cuda()
    kc = torch.zeros((span * n_req, ps, hkv, d), dtype=r.k_new.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    lens = lens0.clone()
    tokens = torch.zeros(int(r.q.shape[0]), dtype=torch.int32, device="cuda")
    nxt = torch.empty((n_req, B), dtype=torch.int32, device="cuda")
    status = torch.empty(n_req, dtype=torch.int32, device="cuda")
    n_acc = r.ver_out["n_accepted"]

    def fn():
        lens.copy_(lens0)
        r.lib.kv_commit(r.k_new, r.v_new, kc, vc, table, r.off_dev, lens, n_acc, B, hit=r.hit, packed_tokens=tokens,
                        next_block=nxt, status=status)

    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.keep = (lens0, table, kc, vc, lens, tokens, nxt, status)
    if graph_only:
        return g
    t = mean_us(g, 100)
    g10 = torch.cuda.CUDAGraph()  # 10 back-to-back copies: the call's device time
    with torch.cuda.graph(g10):
        for _ in range(10):
            fn()
    t10 = mean_us(g10, 30) / 10
    rows = int((n_acc.clamp(0, B - 1) + 1).sum().item())
    nbytes = rows * hkv * d * r.k_new.element_size() * 2 * 2
    return {"rows": rows, "us": round(t, 3), "gbs": round(nbytes / (t * 1e-6) / 1e9, 2),
            "us_in_graph": round(t10, 3),
            "note": "graph also restores the prefix lengths (one small device copy)"}


def topk_graphs(r, torch):
    """Graphs of drafter token selection: greedy tokens of every masked position of the packed blocks
    (k = 1 over rows of drafter logits; synthetic N(0, 3) bf16 logits drawn on the device: timing
    only) and the branch anchors in the builder's layout (top-F of draft rows 1..C-1 excluding the
    drafts, then the full-accept anchor), and the sampled tokens of the same masked positions at
    temperature 1 (draft_sample). Returns {"tokens" | "anchors" | "sampled": (graph, rows read)}, or
    None for workloads without branches."""
    w, lib = r.w, r.lib
    if not w.coverage or w.dtype != "bf16":
        return None
    B, C, F, V = r.B, w.coverage, w.fanout, w.vocab
    n_pos = int(r.q.shape[0])
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    logits = (torch.randn((n_pos, V), generator=gen, device="cuda") * 3.0).to(torch.bfloat16)
    masked = torch.tensor([p for p in range(n_pos) if p % B != 0], dtype=torch.int32, device="cuda")
    toks = torch.empty((masked.numel(), 1), dtype=torch.int32, device="cuda")
    n_req, nd = r.tokens.shape
    per = (C - 1) * F + 1
    rows = torch.tensor([i * nd + k - 1 for i in range(n_req) for k in range(1, C)], dtype=torch.int32, device="cuda")
    excl = r.tokens[:, :C - 1].reshape(-1).contiguous()
    offs = torch.tensor([i * per + (k - 1) * F for i in range(n_req) for k in range(1, C)], dtype=torch.int32,
                        device="cuda")
    offs_full = torch.arange(n_req, dtype=torch.int32, device="cuda") * per + (C - 1) * F
    z_next = r.z_d[:, nd - 1].contiguous()  # stands in for the row after the block
    alt = torch.empty((n_req, per), dtype=torch.int32, device="cuda")
    zd_rows = r.z_d.reshape(n_req * nd, V)
    ws_t = torch.empty(lib.draft_topk_workspace(masked.numel(), V, 1), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(lib.draft_topk_workspace(rows.numel(), V, F), lib.draft_topk_workspace(n_req, V, 1)),
                       dtype=torch.uint8, device="cuda")

    toks_s = torch.empty(masked.numel(), dtype=torch.int32, device="cuda")
    ws_s = torch.empty(lib.draft_sample_workspace(masked.numel(), V), dtype=torch.uint8, device="cuda")

    def tokens():
        lib.draft_topk(logits, 1, rows=masked, out=toks, ws=ws_t)

    def sampled():
        lib.draft_sample(logits, 1.0, 0xD3D0 + w.seed, 0, rows=masked, out=toks_s, ws=ws_s)

    def anchors():
        lib.draft_topk(zd_rows, F, rows=rows, exclude=excl, out=alt, out_off=offs, ws=ws_a)
        lib.draft_topk(z_next, 1, out=alt, out_off=offs_full, ws=ws_a)

    out = {}
    keep = (logits, masked, toks, rows, excl, offs, offs_full, z_next, alt, ws_t, ws_a, toks_s, ws_s)
    for name, fn, n_rows in (("tokens", tokens, masked.numel()), ("anchors", anchors, rows.numel() + n_req),
                             ("sampled", sampled, masked.numel())):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.keep = keep
        g10 = torch.cuda.CUDAGraph()  # 10 back-to-back copies: the call's device time
        with torch.cuda.graph(g10):
            for _ in range(10):
                fn()
        g10.keep = keep
        out[name] = (g, g10, int(n_rows))
    return out


def next_row_topk(r, torch, cur, mean_us):
    """Drafter token selection (the first next row, not part of the step), timed as the mean of
    back-to-back graph replays. HBM bytes = rows x V x 2. The sampled tokens are ALU-bound (a Philox
    block per 4 tokens and two logarithms per token): also reported in tokens scored per second."""
    graphs = topk_graphs(r, torch)
    if graphs is None:
        return None
    V = r.w.vocab
    res = {}
    for name, (g, g10, n_rows) in graphs.items():
        t = mean_us(g, 100)
        t10 = mean_us(g10, 30) / 10
        nbytes = n_rows * V * 2
        res[name] = {"rows": int(n_rows), "us": round(t, 3), "gbs": round(nbytes / (t * 1e-6) / 1e9, 1),
                     "pct_hbm_peak": round(100 * nbytes / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                     "us_in_graph": round(t10, 3),
                     "pct_hbm_peak_in_graph": round(100 * nbytes / (t10 * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        if name == "sampled":
            res[name]["gtokens_per_s"] = round(n_rows * V / (t * 1e-6) / 1e9, 1)
            res[name]["gtokens_per_s_in_graph"] = round(n_rows * V / (t10 * 1e-6) / 1e9, 1)
    return res


def _kernel_digest():
    from block_diffusion_drafting_draft_amd import traffic
    return traffic.source_digest()


if __name__ == "__main__":
    sys.exit(main())
