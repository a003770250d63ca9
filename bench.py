"""Benchmark of the DFlash2 draft-block hot path on one MI355X.

A step is one dfs_draft_block call: grouped causal conv, vocabulary head,
log-softmax, per-slot top-K, transition scores and the Viterbi walk, over one
batch of synthetic inputs already resident in HBM.  The default workload is
the page drafter shape at batch 1 (hidden 5120, vocab 248 320, block 8, K 16,
rank 256).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "draft blocks/sec & µs/block (conv+head+top-K+select), % HBM/MFMA roofline"

WORKLOAD_NAMES = {
    0: "tiny oracle check (batch 1, B 4, D 64, V 1000, K 4, r 16, fp32)",
    1: "small drafter shape (batch 1, B 8, D 2560, V 151936, K 16, r 256, bf16)",
    2: "page drafter shape, batch 1 (B 8, D 5120, V 248320, K 16, r 256, bf16)",
    3: "page drafter shape, batch 32 (B 8, D 5120, V 248320, K 16, r 256, bf16)",
    4: "long block, batch 8 (B 16, D 5120, V 248320, K 16, r 256, bf16)",
    5: "selector only, conv off: page drafter shape, batch 1 (B 8, D 5120, V 248320, K 16, r 256, bf16, 1 tap)",
}


def head_stage_bytes(s) -> int:
    """Algorithmic bytes of the lm_head + top-K stage: the weight once, the
    conv output once, the candidates and lse out."""
    esz = 2 if s.dtype == "bf16" else 4
    return s.vocab * s.hidden * esz + s.rows * s.hidden * esz + s.rows * s.top_k * 8 + s.rows * 4


def block_bytes(s) -> int:
    """Algorithmic bytes of a whole draft block: conv (h in, generator, y
    out), the head stage, and the gathered selector rows."""
    esz = 2 if s.dtype == "bf16" else 4
    conv = s.rows * s.hidden * esz * 2 + s.groups * s.ksize * s.hidden * esz
    sel = s.batch * ((1 + s.top_k * (s.block - 2)) + s.top_k * (s.block - 1)) * s.rank * esz
    return conv + head_stage_bytes(s) + sel


def head_flops(s) -> int:
    return 2 * s.rows * s.hidden * s.vocab


def recorded_traffic(workload: int):
    """HBM bytes per launch of the head + top-K stage from the committed
    rocprofv3 counter records, or None if there is no record for this
    workload or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "head_traffic.json")
    if not os.path.exists(path):
        return None
    for rec in json.load(open(path))["records"]:
        if rec["workload"] != workload:
            continue
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None
    return None


def uses_gemm_head(s) -> bool:
    """More than 8 rows in bf16: the library's GEMM head writes the logits
    and the slice top-K ranks them."""
    return s.dtype == "bf16" and s.rows > 8


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(s, inp, budget_s: float) -> dict:
    """The oracle, as it is, on the host cores: whole draft blocks of the
    same workload until about budget_s seconds have passed (at least one)."""
    import oracle
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], inp["Q"])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    blocks = n * s.batch
    return {"value": blocks / el, "unit": "blocks/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{n} full call(s) of the same workload ({blocks} blocks) in {el:.1f} s; CPU: {cpu_model()}"}


def graph_steps(step, stream, steps: int, per_graph: int = 20):
    """Times exactly ``steps`` steps replayed from captured HIP graphs: one
    graph of ``per_graph`` steps back to back replayed steps // per_graph
    times, and one graph of the remaining steps.  Each graph is replayed
    twice untimed first.  Several steps per replay spread the host's cost of
    issuing a replay, so for shapes whose GPU work is shorter than a host call
    this measures the GPU.  Returns (ms per step, wall seconds of the timed
    region)."""
    import torch

    full, rem = divmod(steps, per_graph)
    gstream = torch.cuda.Stream()
    gstream.wait_stream(stream)
    with torch.cuda.stream(gstream):
        step(gstream)  # once eagerly on the capture stream
    stream.wait_stream(gstream)
    torch.cuda.synchronize()
    graphs = []
    for n in ([per_graph] if full else []) + ([rem] if rem else []):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            for _ in range(n):
                step(gstream)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
        g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(full):
        graphs[0].replay()
    if rem:
        graphs[-1].replay()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = g0.elapsed_time(g1) / steps
    del graphs
    return ms, wall


def dev_tensor(a):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def head_roofline(s, us_head: float) -> dict:
    """The lm_head + top-K stage against both roofs: algorithmic bytes (the
    weight once, y in, candidates and lse out) over 8 TB/s, and the GEMM's
    flops over the bf16 MFMA peak."""
    hb, fl = head_stage_bytes(s), head_flops(s)
    gbs = hb / (us_head * 1e-6) / 1e9
    tfl = fl / (us_head * 1e-6) / 1e12
    return {"head_topk_us": round(us_head, 2), "head_GBps": round(gbs, 1), "head_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "head_tflops": round(tfl, 1), "head_mfma_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
            "bound": "latency" if s.dtype != "bf16" else ("mfma" if uses_gemm_head(s) and s.rows >= 256 else "hbm")}


def cpu_sample(s, inp, calls: int, blocks=None) -> dict:
    """The oracle as it is on a bounded sample of a workload: the median of
    ``calls`` whole calls on ``blocks`` of its blocks (default: all)."""
    import oracle
    if blocks is not None:
        rows = np.concatenate([np.arange(b * s.block, (b + 1) * s.block) for b in blocks])
        s2 = s.with_(batch=len(blocks))
        h, anchor = np.ascontiguousarray(inp["h"][rows]), inp["anchor"][blocks]
    else:
        s2, h, anchor = s, inp["h"], inp["anchor"]
    times = []
    for _ in range(calls):
        t0 = time.perf_counter()
        oracle.draft_block(s2, h, anchor, inp["wg"], inp["W"], inp["P"], inp["Q"])
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {"value": round(s2.batch / med, 3), "unit": "blocks/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"median of {calls} call(s) on {s2.batch} of the {s.batch} block(s) ({med * 1e3:.1f} ms each)"}


def workload_line(wid: int, inp: dict, steps: int, cpu_calls: int, cpu_blocks=None, graph: bool = False) -> dict:
    """One workload timed on its own inputs (the h, anchors and weights in
    ``inp``): µs per block and blocks/s of whole dfs_draft_block steps, the
    head stage against its roofs, optionally the step replayed from a HIP
    graph, and a short oracle sample."""
    import torch

    import block_drafter_grouped_amd as dfs

    s = wl.shape_of(wid)
    d = {k: dev_tensor(inp[k]) for k in ("h", "W", "P", "Q", "anchor")}
    wg_cm = dev_tensor(np.ascontiguousarray(inp["wg"].T))
    cfg = dfs.Config.of(s)
    ws = torch.empty(dfs.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    tdt = torch.int16 if s.dtype == "bf16" else torch.float32
    path = torch.empty((s.batch, s.block), dtype=torch.int32, device="cuda")
    score = torch.empty((s.batch,), dtype=torch.float32, device="cuda")
    ids = torch.empty((s.rows, s.top_k), dtype=torch.int32, device="cuda")
    lp = torch.empty((s.rows, s.top_k), dtype=torch.float32, device="cuda")
    lse = torch.empty((s.rows,), dtype=torch.float32, device="cuda")
    y = torch.empty((s.rows, s.hidden), dtype=tdt, device="cuda")
    stream = torch.cuda.current_stream()

    def step(st=stream):
        dfs.draft_block(cfg, d["h"], d["anchor"], wg_cm, d["W"], d["P"], d["Q"], path, score, ws, stream=st)

    def timed(fn, n) -> float:
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3  # us

    us_eager = timed(step, steps)
    us_step = graph_steps(step, stream, steps)[0] * 1e3 if graph else us_eager
    dfs.conv(cfg, d["h"], wg_cm, y, ws)
    us_head = timed(lambda: dfs.head_topk(cfg, y, d["W"], ids, lp, lse, ws), steps)
    gate = (0.5 + torch.rand((s.rows, s.rank), generator=torch.Generator().manual_seed(7))).cuda()
    us_sel = timed(lambda: dfs.select(cfg, d["anchor"], ids, lp, d["P"], d["Q"], path, score, ws), steps)
    us_sel_g = timed(lambda: dfs.select(cfg, d["anchor"], ids, lp, d["P"], d["Q"], path, score, ws, gate=gate), steps)
    out = {"workload": WORKLOAD_NAMES[wid], "steps": steps,
           "timing": "graph replay (20 steps per captured HIP graph)" if graph else "eager launches",
           "us_per_block": round(us_step / s.batch, 3),
           "us_per_step": round(us_step, 2), "blocks_per_s": round(s.batch / (us_step * 1e-6), 1),
           **head_roofline(s, us_head), "outside_head_us": round(us_step - us_head, 2),
           "select_us": round(us_sel, 2), "select_gated_us": round(us_sel_g, 2),
           "eager": {"us_per_step": round(us_eager, 2), "blocks_per_s": round(s.batch / (us_eager * 1e-6), 1)}}
    if cpu_calls > 0:
        out["cpu_baseline"] = cpu_sample(s, inp, cpu_calls, cpu_blocks)
    del d, wg_cm, ws
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(wl.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline (0: skip)")
    ap.add_argument("--stage-steps", type=int, default=None, help="calls per stage timing loop")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run 4 plain 1 GiB device copies (counter calibration for profiles)")
    ap.add_argument("--timing", choices=("graph", "eager"), default="graph",
                    help="time the K steps replayed from captured HIP graphs (default) or as eager launches")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-layer conv, vocabulary-shard and other-workload timings (for profiler runs: "
                         "their launches of the same kernels at other sizes would mix into per-kernel means)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the draft-block path runs on one GPU; a run across several GPUs is not "
              "implemented. Use --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import block_drafter_grouped_amd as dfs

    s = wl.shape_of(args.workload)
    inp = wl.make_inputs(args.workload)

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

    h, W, P, Q, anchor = (dev(inp[k]) for k in ("h", "W", "P", "Q", "anchor"))
    wg_cm = dev(np.ascontiguousarray(inp["wg"].T))
    cfg = dfs.Config.of(s)
    ws = torch.empty(dfs.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    tdt = torch.int16 if s.dtype == "bf16" else torch.float32
    path = torch.empty((s.batch, s.block), dtype=torch.int32, device="cuda")
    score = torch.empty((s.batch,), dtype=torch.float32, device="cuda")
    ids = torch.empty((s.rows, s.top_k), dtype=torch.int32, device="cuda")
    lp = torch.empty((s.rows, s.top_k), dtype=torch.float32, device="cuda")
    lse = torch.empty((s.rows,), dtype=torch.float32, device="cuda")
    y = torch.empty((s.rows, s.hidden), dtype=tdt, device="cuda")
    stream = torch.cuda.current_stream()

    def step(st=stream):
        dfs.draft_block(cfg, h, anchor, wg_cm, W, P, Q, path, score, ws, cand_ids=ids, cand_logp=lp,
                        stream=st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    ms_eager = e0.elapsed_time(e1) / args.steps
    # The headline: the same K steps replayed from captured HIP graphs (the
    # library takes the caller's stream and never allocates or synchronises,
    # so a serving loop can capture its draft step; the release-note article's
    # cost section times the conv the same way).  --timing eager keeps eager
    # launches (profiler runs).
    if args.timing == "graph":
        ms_step, wall = graph_steps(step, stream, args.steps)
    else:
        ms_step, wall = ms_eager, wall_eager

    # Per-stage split, each stage timed alone with HIP events on the same stream.
    n_stage = args.stage_steps or args.steps

    def timed(fn) -> float:
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_stage):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n_stage * 1e3  # us

    us_conv = timed(lambda: dfs.conv(cfg, h, wg_cm, y, ws, stream=stream))
    NL = 5
    us_layers = us_separate = us_shard = None
    if not args.no_extras:
        # One conv per drafter layer: five layers in one dfs_conv_layers call
        # against five dfs_conv calls (inputs: the workload's tensors repeated).
        hL, wgL = h.repeat(NL, 1, 1).contiguous(), wg_cm.repeat(NL, 1, 1).contiguous()
        yL = torch.empty((NL, s.rows, s.hidden), dtype=tdt, device="cuda")
        wsL = torch.empty(dfs.conv_layers_workspace_size(cfg, NL), dtype=torch.uint8, device="cuda")
        us_layers = timed(lambda: dfs.conv_layers(cfg, NL, hL, wgL, yL, wsL, stream=stream))

        def separate():
            for layer in range(NL):
                dfs.conv(cfg, hL[layer], wgL[layer], yL[layer], ws, stream=stream)

        us_separate = timed(separate)
        del hL, wgL, yL, wsL
    us_head = timed(lambda: dfs.head_topk(cfg, y, W, ids, lp, lse, ws, stream=stream))
    us_sel = timed(lambda: dfs.select(cfg, anchor, ids, lp, P, Q, path, score, ws, stream=stream))
    # The selector with a context gate (the Inco AI post's H(h_t); random
    # fp32 rows in [0.5, 1.5), since the pages give no form for it).
    gate = (0.5 + torch.rand((s.rows, s.rank), generator=torch.Generator().manual_seed(7))).cuda()
    us_sel_gated = timed(lambda: dfs.select(cfg, anchor, ids, lp, P, Q, path, score, ws, stream=stream, gate=gate))
    vs = s.vocab // 8
    if not args.no_extras:
        # One GPU's share under vocabulary sharding over 8 GPUs: the head +
        # top-K stage on an eighth of the weight (the merge of the shards'
        # partials is a few KB per row, left out).
        cfg8 = dfs.Config.of(s.with_(vocab=vs))
        ws8 = torch.empty(dfs.workspace_size(cfg8), dtype=torch.uint8, device="cuda")
        us_shard = timed(lambda: dfs.head_topk(cfg8, y, W[:vs], ids, lp, lse, ws8, stream=stream))
        del ws8

    # The other workloads, each on its own seeded inputs: µs per block (timed
    # as the headline is), the head stage against both roofs, and a short
    # oracle sample.
    others = None
    if not args.no_extras:
        others = {}
        plan = {0: (500, 5, None), 1: (200, 5, None), 3: (40, 1, [0, 1]), 4: (40, 1, [0])}
        for wid, (n, calls, blocks) in plan.items():
            if wid == args.workload:
                continue
            winp = wl.make_inputs(wid)
            others[str(wid)] = workload_line(wid, winp, n, calls if args.cpu_seconds > 0 else 0, blocks,
                                             graph=args.timing == "graph")
            del winp

    hb = head_stage_bytes(s)
    traffic = recorded_traffic(args.workload)
    traffic_gbs = round(traffic / (us_head * 1e-6) / 1e9, 1) if traffic else None
    if uses_gemm_head(s):
        # The contraction is large enough to be bound by the matrix cores.
        fl = head_flops(s)
        achieved = fl / (us_head * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic_gbs,
                "traffic_unit": "GB/s", "traffic_bytes_per_launch": traffic,
                "kernel": "lm_head + top-K stage (head_gemm_kernel with segment partials + merge_seg_kernel, "
                          "one dfs_head_topk call)" if s.top_k <= 16 else
                          "lm_head + top-K stage (head_gemm_kernel + slice_topk_kernel + merge64_kernel, "
                          "one dfs_head_topk call)",
                "flops_per_launch": fl, "bytes_per_launch": hb, "us_per_launch": round(us_head, 2)}
    else:
        achieved = hb / (us_head * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_gbs,
                "traffic_bytes_per_launch": traffic,
                "kernel": "lm_head + top-K stage (head_pair_kernel + merge16_kernel, one dfs_head_topk call)",
                "bytes_per_launch": hb, "us_per_launch": round(us_head, 2)}
    if s.dtype != "bf16":
        roof["bound"] = "latency"

    out = {
        "metric": METRIC,
        "value": round(s.batch / (ms_step * 1e-3), 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Philox normals: h~N(0,1), Wg~N(0,1/D), W~N(0,9/D), P,Q~N(0,1/r))",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "batch": s.batch, "block": s.block,
                   "hidden": s.hidden, "vocab": s.vocab, "top_k": s.top_k, "rank": s.rank,
                   "conv_group_size": s.group, "conv_kernel_size": s.ksize, "parallelism": "none (1 GPU)"},
        "us_per_block": round(ms_step * 1e3 / s.batch, 3),
        "stage_us": {"conv": round(us_conv, 2), "head_topk": round(us_head, 2), "select": round(us_sel, 2),
                     "select_gated": round(us_sel_gated, 2)},
        "conv_layers_us": None if us_layers is None else
        {"layers": NL, "one_call": round(us_layers, 2), "separate_calls": round(us_separate, 2)},
        "vocab_shard_of_8": None if us_shard is None else
        {"vocab": vs, "head_topk_us": round(us_shard, 2),
         "GBps": round((vs * s.hidden + s.rows * s.hidden) * (2 if s.dtype == "bf16" else 4)
                       / (us_shard * 1e-6) / 1e9, 1)},
        "block_hbm_frac": round(block_bytes(s) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "head_mfma_frac": round(head_flops(s) / (us_head * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "timing": "graph replay: the K steps captured 20 to a HIP graph, replayed; eager launches below"
        if args.timing == "graph" else "eager launches",
        "eager": {"ms_per_step": round(ms_eager, 5), "value": round(s.batch / (ms_eager * 1e-3), 2),
                  "wall_s_timed": round(wall_eager, 3)},
        "workloads": others,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.copy_probe:
        # A plain copy of known size: HBM counters of a profiled run divided
        # by 1 GiB read + 1 GiB written give the counters' scale.
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(s, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
