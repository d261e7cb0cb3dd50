"""Benchmark of the routed-expert path of one MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--skew S]

One step = route -> permute -> plan -> expert FFN (FC1, FC2) -> combine over one batch of
seeded synthetic input already resident in HBM, timed as eager calls on one stream (--graph:
as HIP-graph replays of the whole path; the eager figure is then reported beside it).  The
default layer is the largest one that fits one GPU: one GPU's 32-expert share of a
DeepSeek-V3-sized layer (T=32768, H=7168, I=2048, top-8 of 256) at Zipf skew 1.0.
Protocol: a settle phase of whole steps (--settle-s seconds), W warm-up steps, then exactly
K timed steps, each bracketed by HIP events; ms_per_step is the median step.
Prints ONE JSON line: whole-path tokens/s, the grouped GEMM's TFLOP/s, the dominant kernel
(FC1, the gate/up GEMM with fused SwiGLU) against the bf16 MFMA peak, per-call times, and the
CPU oracle timed on a bounded sample of the same workload on the host cores (all threads,
and one thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-expert layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak) vs skew"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (the MX path's FP4 x FP8 products)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a few hundred warm-up steps: the GPU's clocks take on the order of 100 ms to settle
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="deepseek_v3_share",
                    help="layer shape (default: the largest one-GPU layer, one GPU's 32-expert share "
                         "of a DeepSeek-V3-sized layer, T=32768, H=7168, I=2048)")
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of whole steps run before the warm-up steps, outside the timed "
                         "region, so that the GPU clock has settled under this load")
    ap.add_argument("--skew", default=None, help="Zipf exponent or 'hot4' (default: middle skew)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--planner", choices=("moonep", "megaflux"), default="moonep",
                    help="moe_plan (exact per-rank entry capacity, the default) or moe_plan_blocks "
                         "(block-granular replicas, budget E_loc / (4P))")
    ap.add_argument("--materialize", action="store_true",
                    help="write the permuted copy xp of x (moe_permute with xp, moe_expert_ffn) "
                         "instead of gathering x rows inside the gate/up GEMM")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the whole path instead of eager calls")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the oracle's sizing pass (the measured sample is scaled to "
                         "about 12 s of CPU work)")
    ap.add_argument("--no-all-skews", action="store_true",
                    help="skip timing every skew of the workload (the by_skew field)")
    ap.add_argument("--precision", choices=("bf16", "mx"), default="bf16",
                    help="bf16 expert GEMMs (the default) or the MX path: MXFP4 weights, MXFP8 "
                         "activations (x quantized inside the step)")
    ap.add_argument("--no-router", action="store_true",
                    help="skip timing moe_router_topk (router scores + top-k) beside the step")
    ap.add_argument("--no-mx-summary", action="store_true",
                    help="skip the MX path's summary (mx_path) in a bf16 run")
    ap.add_argument("--direct", choices=("auto", "on", "off"), default="auto",
                    help="on: the rows of one-entry tokens go to out from the down GEMM's epilogue "
                         "(moe_expert_ffn_fc2_direct + moe_combine_multi); off: the down GEMM stores "
                         "every row to yp and the combine sums every token; auto (default): on where "
                         "a token can have exactly one local entry (a share of the experts, or top-1)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a reference for "
                         "hardware byte counters)")
    return ap.parse_args()


def pick_skew(w, s):
    if s is None:
        return w.skews[len(w.skews) // 2]
    if s == "hot4":
        return s
    for cand in w.skews:
        if not isinstance(cand, str) and abs(cand - float(s)) < 1e-9:
            return cand
    raise SystemExit(f"skew {s} is not one of {w.skews} for {w.name}")


class Step:
    """The path's calls on one stream, with optional HIP events between them."""

    CALLS = ("route", "permute", "plan", "fc1", "fc2", "combine")
    CALLS_MX = ("route", "permute", "quantize_x", "plan", "fc1", "fc2", "combine")

    def __init__(self, layer, logits, x, W1, W2):
        self.layer, self.logits, self.x, self.W1, self.W2 = layer, logits, x, W1, W2
        self.calls = self.CALLS_MX if layer.precision == "mx" else self.CALLS

    def run(self, events=None):
        L = self.layer
        fns = {"route": lambda: L.route(self.logits), "permute": lambda: L.permute(self.x),
               "quantize_x": lambda: L.quantize_x(self.x), "plan": L.plan,
               "fc1": lambda: L.expert_ffn_fc1(self.W1), "fc2": lambda: L.expert_ffn_fc2(self.W2),
               "combine": L.combine}
        if events is not None:
            events[0].record()
        for i, c in enumerate(self.calls):
            fns[c]()
            if events is not None:
                events[i + 1].record()


def settle(run, seconds, torch):
    """Whole steps for about `seconds` of wall time (outside the timed region): the GPU's
    clock takes on the order of a second to settle under a sustained load.  Returns (steps,
    seconds)."""
    if seconds <= 0:
        return 0, 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(4):
            run()
        n += 4
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def time_steps(step, steps, warmup, torch, graph=None, settle_s=0.0):
    """Times exactly `steps` steps (HIP-graph replays of the whole path if `graph`, else eager
    calls) after a settle phase and `warmup` untimed steps.  Every timed step is bracketed by
    HIP events on the stream the kernels run on (eager steps: also between its calls), so the
    per-step and per-call figures are medians over the timed steps themselves; the wall clock
    around the timed region (synchronised on both sides) is reported beside them."""
    run = graph.replay if graph is not None else step.run
    n_settle, t_settle = settle(run, settle_s, torch)
    for _ in range(warmup):
        run()
    ncall = len(step.calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ncall + 1 if graph is None else 2)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if graph is None:
            step.run(ev[i])
        else:
            ev[i][0].record()
            graph.replay()
            ev[i][1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    step_ms = [e[0].elapsed_time(e[-1]) for e in ev]
    if graph is not None:
        # per-call durations from event-bracketed eager steps after the timed region
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ncall + 1)] for _ in range(steps)]
        for i in range(steps):
            step.run(ev[i])
        torch.cuda.synchronize()
    per = {c: float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)])) * 1e3
           for j, c in enumerate(step.calls)}
    # the FC1 call starts with the tile-schedule kernel: time it alone on the same table, so
    # that the FC1 GEMM kernel's own duration is fc1 - schedule
    if step.layer.dtype == torch.bfloat16:
        per["fc1_schedule"] = schedule_us(step.layer, torch)
    return {"median_s": float(np.median(step_ms)) * 1e-3, "mean_s": float(np.mean(step_ms)) * 1e-3,
            "wall_s": wall, "per": per, "settle_steps": n_settle, "settle_s": t_settle}


def schedule_us(layer, torch, n=50, reps=8):
    """GPU time of one tile-schedule launch: a HIP graph of n back-to-back launches, replayed
    reps times between two events, so that the host's per-call overhead (longer than this
    small kernel) is not counted as the kernel's time."""
    layer.tile_schedule()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            layer.tile_schedule()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / (n * reps) * 1e3


def ffn_roofline(w, n_loc, eb, peak=PEAK_BF16_TFLOPS):
    """Per-expert roofline of the two expert GEMMs: each touched expert costs the larger of
    its valid-row flops at the MFMA peak and one read of its weights (3 H I values) at the
    HBM peak.  Returns (t_roof seconds, touched experts, weight bytes of touched experts,
    bound of the sum: 'mfma' or 'hbm')."""
    per_flop = 6.0 * w.H * w.I / (peak * 1e12)
    wbytes = 3.0 * w.H * w.I * eb
    per_byte = wbytes / (PEAK_HBM_GBS * 1e9)
    touched = [int(n) for n in n_loc if n > 0]
    t_mfma = sum(n * per_flop for n in touched)
    t_roof = sum(max(n * per_flop, per_byte) for n in touched)
    bound = "hbm" if len(touched) * per_byte > t_mfma else "mfma"
    return t_roof, len(touched), len(touched) * wbytes, bound


def ffn_traffic(workload: str, precision: str = "bf16"):
    """HBM bytes per FC1 launch from committed rocprofv3 counter runs, if they were taken on
    the current FC1 kernel source; else None."""
    tag = "fc1_mx" if precision == "mx" else "fc1"
    path = os.path.join(ROOT, "profiles", f"{tag}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("ffn_source_sha256") != ffn_source_sha256(precision):
        return None
    return rec.get("bytes_per_launch")


def ffn_source_sha256(precision: str = "bf16") -> str:
    """SHA-256 over the FC1 kernel's sources (the kernel file, then the headers it includes)."""
    files = (("ffn_mx.hip", "moe_lds.h", "moe_ffn_ws.h", "moe_mx.h") if precision == "mx" else
             ("ffn.hip", "moe_lds.h", "moe_ffn_ws.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "mixture_experts_routed_router_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def hbm_reference(torch, dev, mib=1024, reps=20):
    """The box's practical HBM rates, measured live: a device-to-device copy of `mib` MiB
    (bytes read + written per second) and a read-only pass over the same buffer (an int64
    sum), each the median of `reps` event-timed launches."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    out = {}
    for name, fn, bytes_ in (("copy", lambda: b.copy_(a), 2 * n),
                             ("read", lambda: a.view(torch.int64).sum(), n)):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        t = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3
        out[name + "_gbs"] = round(bytes_ / t / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def gemm_reference(torch, dev, w, n_loc, reps=20):
    """The vendor library's rate (torch.bmm, hipBLASLt) on a batched GEMM of the same
    per-expert shape as the two expert GEMMs: one batch entry per touched expert with the
    mean of their rows (FC1: [m, H] x [H, 2I]; FC2: [m, I] x [I, H]), bf16, operands
    contiguous; median of `reps` event-timed launches after 3 warm-ups.  Neither fuses the
    gather or the SwiGLU.  Returns TFLOP/s per GEMM."""
    touched = [int(n) for n in n_loc if n > 0]
    if not touched:
        return {}
    b, m = len(touched), max(1, round(sum(touched) / len(touched)))
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for name, k, n in (("fc1", w.H, 2 * w.I), ("fc2", w.I, w.H)):
        a = torch.randn(b, m, k, device=dev, dtype=torch.bfloat16, generator=g)
        bm = torch.randn(b, k, n, device=dev, dtype=torch.bfloat16, generator=g)
        for _ in range(3):
            torch.bmm(a, bm)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            torch.bmm(a, bm)
            e1.record()
        torch.cuda.synchronize()
        t = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3
        out[name + "_tflops"] = round(2.0 * b * m * k * n / t / 1e12, 1)
        del a, bm
    out["shape"] = f"{b} x [{m} x K] x [K x N] (experts x mean rows)"
    torch.cuda.empty_cache()
    return out


def read_rate_at(torch, dev, nbytes, reps=20):
    """The box's read rate for a working set of `nbytes` read again pass after pass, as the
    weight-bound FFN re-reads its touched experts' weights every step: a read-only int64 sum over
    a buffer of that size, median of `reps` event-timed launches after 3 warm-ups (GB/s).  The
    rate depends on the size: sets that fit the last-level cache read faster than 8 TB/s allows
    for HBM alone, sets of a few times its size slower than very large ones."""
    n = max(1, int(nbytes) // 8)
    a = torch.ones(n, dtype=torch.int64, device=dev)
    for _ in range(3):
        a.sum()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        a.sum()
        e1.record()
    torch.cuda.synchronize()
    t = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3
    del a
    torch.cuda.empty_cache()
    return n * 8 / t / 1e9


def router_measured(torch, dev, w, x, binding, inputs, reps=200):
    """moe_router_topk (router scores x . W_r^T with the top-k fused) on the batch's x and a
    seeded router matrix, apart from the measured step (which starts from given logits): the
    mean of `reps` back-to-back calls between two events, after as many warm-ups (a pair of
    events around each call would add the launch gap to calls of a few microseconds).  Bytes: x
    and W_r read once, the ids and weights written (T H b + E H b + 8 T K)."""
    wr = inputs.make_router_weights(w).to(dev)
    ids = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    tw = torch.empty((w.T, w.K), dtype=torch.float32, device=dev)
    cnt = torch.empty((w.E,), dtype=torch.int32, device=dev)
    for _ in range(reps):
        binding.moe_router_topk(x, wr, w.K, w.K, ids, tw, cnt)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        binding.moe_router_topk(x, wr, w.K, w.K, ids, tw, cnt)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    b = x.element_size()
    nbytes = w.T * w.H * b + w.E * w.H * b + 8 * w.T * w.K
    return {"us": round(t * 1e6, 2), "bytes": nbytes, "gbs": round(nbytes / t / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
            "calls": reps}


def plan_comparison(layer, w, steps, torch):
    """Both planners on the layer's current expert counts: plan kernel time (HIP events over
    back-to-back calls), blocks in the table, the busiest rank's blocks and rows, partial
    blocks, and weight copies (moe_plan: expert slices moved; moe_plan_blocks: replicas)."""
    res = {}
    saved = layer.planner
    for name in ("moonep", "megaflux"):
        layer.planner = name
        layer.plan()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            layer.plan()
        e1.record()
        torch.cuda.synchronize()
        nb = int(layer.n_blocks.item())
        bl = layer.blocks[:nb].cpu().long()
        per_blocks = torch.bincount(bl[:, 0], minlength=w.P)
        per_rows = torch.zeros(w.P, dtype=torch.long).index_add_(0, bl[:, 0], bl[:, 3])
        res[name] = {"plan_us": round(e0.elapsed_time(e1) / steps * 1e3, 2), "blocks": nb,
                     "max_rank_blocks": int(per_blocks.max()),
                     "max_rank_rows": int(per_rows.max()),
                     "partial_blocks": int((bl[:, 3] < w.beta).sum()),
                     "weight_copies": int(layer.n_moves.item())}
    res["megaflux"]["replica_budget"] = layer.replica_budget
    layer.planner = saved
    layer.plan()
    torch.cuda.synchronize()
    return res


def cpu_baseline(w, skew, T_s, target_s=12.0, precision="bf16"):
    """The CPU oracle, as it stands, over the first tokens of the same batch (whole path).
    A first pass over T_s tokens sizes the measured sample to about target_s seconds of CPU
    work (at most the whole batch, a multiple of P tokens).  precision "mx": the oracle's MX
    path (x quantized to MXFP8 inside the timed pass; the weights' MXFP4 codes prepared once,
    outside it, as the GPU path's are)."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle
    from mixture_experts_routed_router_amd import inputs

    logits_all = inputs.make_logits(w, skew)
    x_all = inputs.as_oracle_array(inputs.make_x(w))
    W1, W2 = (inputs.as_oracle_array(t) for t in inputs.make_weights(w, threads=16))
    oracle.build()
    if precision == "mx":
        w1q, w1s = oracle.mx_quantize(W1.reshape(-1, w.H), oracle.MX_FP4)
        w2q, w2s = oracle.mx_quantize(W2.reshape(-1, w.I), oracle.MX_FP4)
        del W1, W2

    def ffn_mx(xp, blocks):
        rows = np.concatenate([np.arange(b0, b0 + m) for _, _, b0, m in blocks.tolist()]
                              + [np.zeros(0, np.int64)]).astype(np.int32)
        ex = np.concatenate([np.full(m, l) for _, l, _, m in blocks.tolist()]
                            + [np.zeros(0, np.int64)]).astype(np.int32)
        xq, xs = oracle.mx_quantize(xp, oracle.MX_FP8)
        _, _, y = oracle.ffn_mx_rows(xq, xs, w1q, w1s, w2q, w2s, w.H, w.I, rows, ex)
        yp = np.zeros((xp.shape[0], w.H), np.uint16)
        yp[rows] = y
        return yp

    steps_s = {"route": 0.0, "permute": 0.0, "plan": 0.0, "ffn": 0.0, "combine": 0.0}

    def run(n):
        logits = np.ascontiguousarray(logits_all[:n])
        x = np.ascontiguousarray(x_all[:n])
        t = [time.perf_counter()]
        ids, wt, counts = oracle.route(logits, w.K)
        t.append(time.perf_counter())
        _, ep, _, xp = oracle.permute(ids, counts, w.E, w.expert_begin, w.expert_stride,
                                      w.n_local, w.beta, x)
        t.append(time.perf_counter())
        _, _, blocks = oracle.plan(counts, w.E, w.expert_begin, w.expert_stride, w.n_local, w.P,
                                   w.beta)
        t.append(time.perf_counter())
        if precision == "mx":
            yp = ffn_mx(xp, blocks)
        else:
            _, yp = oracle.ffn_blocks(xp, W1, W2, blocks)
        t.append(time.perf_counter())
        oracle.combine(yp, wt, ep, n, w.K)
        t.append(time.perf_counter())
        for k, name in enumerate(steps_s):
            steps_s[name] += t[k + 1] - t[k]
        return t[-1] - t[0]

    def sized(t_probe_tokens, target):
        """Sizes a sample from a probe run to about `target` seconds and runs it; returns
        (tokens, repetitions, seconds, description, per-step seconds)."""
        t_probe = run(t_probe_tokens)
        for name in steps_s:
            steps_s[name] = 0.0
        want = int(t_probe_tokens * target / max(t_probe, 1e-6))
        n = max(w.P, min(w.T, want) // w.P * w.P)
        # a whole batch that takes less than the target is run again until the target is reached
        reps, dt = 0, 0.0
        while reps == 0 or (n == w.T and dt < target):
            dt += run(n)
            reps += 1
        what = (f"first {n} of {w.T} tokens of the same batch" if reps == 1 else
                f"the whole batch of {w.T} tokens, {reps} times")
        per_step = {k: round(v, 3) for k, v in steps_s.items()}
        return n, reps, dt, what, per_step

    cores = oracle.num_threads()
    n, reps, dt, what, per_step = sized(T_s, target_s)
    # the same oracle on one thread, over a shorter sample
    oracle.set_num_threads(1)
    try:
        n1, reps1, dt1, what1, per_step1 = sized(w.P, target_s / 2)
    finally:
        oracle.set_num_threads(cores)
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    kind = f"{'MX ' if precision == 'mx' else ''}FFN"
    return {"value": round(n * reps / dt, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model, "per_step_s": per_step,
            "sample": f"{what}, whole path (route, permute, plan, {kind}, combine), float64 plain C "
                      f"with OpenMP on {cores} threads, {dt:.1f} s",
            "one_thread": {"value": round(n1 * reps1 / dt1, 3), "unit": "tokens/s", "cores": 1,
                           "per_step_s": per_step1,
                           "sample": f"{what1}, the same path on one thread, {dt1:.1f} s"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_routed_router_amd import binding, inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = inputs.WORKLOADS[args.workload]
    skew = pick_skew(w, args.skew)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    mx = args.precision == "mx"
    if mx and (dt != torch.bfloat16 or args.materialize):
        raise SystemExit("--precision mx takes a bf16 workload and gathers its input rows")
    W1, W2 = inputs.make_weights(w, threads=16)
    W1, W2 = W1.to(dev), W2.to(dev)
    x = inputs.make_x(w).to(dev)
    wmx = None
    if mx or (dt == torch.bfloat16 and not args.no_mx_summary):
        wmx = binding.mx_quantize_weights(W1, W2)  # MXFP4 weights, prepared once
    if mx:
        W1, W2 = wmx
    direct = args.direct == "on" or (args.direct == "auto" and (w.n_local < w.E or w.K == 1))
    layer = binding.RoutedExperts(w.T, w.H, w.E, w.K, w.I, w.P, dtype=dt, E_loc=w.n_local,
                                  expert_begin=w.expert_begin, expert_stride=w.expert_stride,
                                  block_m=w.beta, gather=not args.materialize,
                                  planner=args.planner, precision=args.precision, direct=direct)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def measure(sk, steps, warmup, lay=None, w1=None, w2=None, settle_s=0.0):
        lay = lay or layer
        w1, w2 = (w1, w2) if w1 is not None else (W1, W2)
        logits = torch.from_numpy(inputs.make_logits(w, sk)).to(dev)
        step = Step(lay, logits, x, w1, w2)
        graph = lay.capture(logits, x, w1, w2) if args.graph else None
        tm = time_steps(step, steps, warmup, torch, graph, settle_s)
        tm["eager_median_s"] = (time_steps(step, steps, 1, torch)["median_s"] if graph is not None
                                else tm["median_s"])
        counts = lay.counts.cpu()
        N = int(counts[w.expert_begin::w.expert_stride][: w.n_local].sum())
        nb = int(lay.n_blocks.item())
        del graph
        return tm, N, nb, counts

    tm, N, nb, counts = measure(skew, args.steps, args.warmup, settle_s=args.settle_s)
    wall, per = tm["median_s"], tm["per"]
    flops_fc1 = 4.0 * w.H * w.I * N
    flops_ffn = 6.0 * w.H * w.I * N
    fc1_s = (per["fc1"] - per.get("fc1_schedule", 0.0)) * 1e-6  # the FC1 GEMM kernel alone
    ffn_s = (per["fc1"] + per["fc2"]) * 1e-6
    achieved = flops_fc1 / fc1_s / 1e12
    loc = counts[w.expert_begin::w.expert_stride][: w.n_local].double()
    maxvio = float(loc.max() / loc.mean() - 1.0)
    rows_pad = int(layer.offsets[-1].item())
    eb = 2 if dt == torch.bfloat16 else 4
    permute_bytes = (w.T + N) * w.H * eb + 4 * (w.T * w.K + rows_pad)
    # tokens with exactly one local entry: with direct rows the down GEMM stores their out rows
    # and the combine neither reads their expert row nor writes their out row
    n_one = int(((layer.entry_pos.view(w.T, w.K) >= 0).sum(dim=1) == 1).sum().item())
    combine_bytes = (N + w.T) * w.H * eb + 8 * w.T * w.K
    if direct:
        combine_bytes -= 2 * n_one * w.H * eb
    traffic = ffn_traffic(w.name, args.precision)
    t_roof, touched, wbytes, bound = ffn_roofline(w, loc.tolist(), eb)
    fc1_kernel = ("ffn_bf16_kernel<true, false>, the FC1 GEMM of moe_expert_ffn_fc1 (gate/up + SwiGLU)"
                  if args.materialize else
                  "ffn_bf16_kernel<true, true>, the FC1 GEMM of moe_expert_ffn_fc1_gather (gate/up + SwiGLU, "
                  "rows gathered from x)")
    if dt == torch.float32:
        fc1_kernel = ("ffn_f32_kernel<true>, the FC1 of moe_expert_ffn_fc1_gather on the float32 layer "
                      "(gate/up + SwiGLU, fp32 FMAs, rows gathered from x)")
    peak_mfma = PEAK_BF16_TFLOPS
    if mx:
        fc1_kernel = ("ffn_mx_kernel<true>, the FC1 GEMM of moe_expert_ffn_mx_fc1 (MXFP4 gate/up "
                      "weights x MXFP8 rows gathered from x, SwiGLU, MXFP8 activation out)")
        peak_mfma = PEAK_FP8_TFLOPS
        # weights are 4.25 bits per value (codes + one E8M0 scale per 32): 17/32 byte
        eb = 17.0 / 32.0
        t_roof, touched, wbytes, bound = ffn_roofline(w, loc.tolist(), eb, PEAK_FP8_TFLOPS)
    if bound == "hbm":
        # weight-read bound (decode): FC1 streams the gate/up weights of every touched expert
        fc1_bytes = wbytes * 2.0 / 3.0
        roofline = {"kernel": fc1_kernel,
                    "bound": "hbm", "achieved": round(fc1_bytes / fc1_s / 1e9, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(fc1_bytes / fc1_s / 1e9 / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roofline = {"kernel": fc1_kernel,
                    "bound": "mfma", "achieved": round(achieved, 1),
                    "peak": peak_mfma, "unit": "TFLOP/s",
                    "frac": round(achieved / peak_mfma, 4), "traffic": traffic}

    line = {
        "metric": METRIC,
        "value": round(w.T / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "timing": {"ms_per_step": "median of the timed steps' HIP-event durations",
                   "mean_ms_per_step": round(tm["mean_s"] * 1e3, 4),
                   "wall_ms_per_step": round(tm["wall_s"] * 1e3, 4),
                   "eager_median_ms_per_step": round(tm["eager_median_s"] * 1e3, 4),
                   "per_call_us": "medians over the timed steps",
                   "settle_s": round(tm["settle_s"], 3), "settle_steps": tm["settle_steps"]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4 weights x mxfp8 activations (f32 accumulation), bf16 in/out" if mx else
                  "bf16" if dt == torch.bfloat16 else "f32"),
        "data": "synthetic (seeded Zipf-skewed router logits, N(0,1) activations, "
                "N(0,0.02^2) expert weights)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "E_loc": w.n_local,
                   "K": w.K, "I": w.I, "P": w.P, "block_m": w.beta,
                   "skew": w.skew_label(skew), "local_entries": N, "blocks": nb,
                   "maxvio": round(maxvio, 3), "planner": args.planner,
                   "precision": "f32" if dt == torch.float32 else args.precision,
                   "parallelism": "single GPU",
                   "launch": "hip graph replay" if args.graph else "eager",
                   "dispatch": "materialised xp" if args.materialize else
                               "gather-on-load (FC1 reads x rows through row_token)",
                   "combine": ("direct rows: the down GEMM stores the weighted out rows of the "
                               f"{n_one} one-entry tokens, the combine sums the other "
                               f"{w.T - n_one}" if direct else
                               "every token summed by the combine")},
        "gemm_tflops": round(flops_ffn / ffn_s / 1e12, 1),
        "gemm_frac_of_peak": round(flops_ffn / ffn_s / 1e12 / peak_mfma, 4),
        "per_call_us": {k: round(v, 2) for k, v in per.items()},
        "permute_gbs": (round(permute_bytes / (per["permute"] * 1e-6) / 1e9, 1)
                        if args.materialize else None),
        # gather-on-load: the permute is index work only (topk_ids read, entry_pos and row_token
        # written); a few MB over three small kernels, so its rate is launch- and latency-bound
        "permute_index_bytes": 4 * (2 * w.T * w.K + rows_pad),
        "permute_index_gbs": round(4 * (2 * w.T * w.K + rows_pad) / (per["permute"] * 1e-6) / 1e9, 1),
        "combine_gbs": round(combine_bytes / (per["combine"] * 1e-6) / 1e9, 1),
        "combine_bytes": combine_bytes,
        "ffn_t_roof_us": round(t_roof * 1e6, 2),
        "ffn_frac_of_t_roof": round(t_roof / ffn_s, 4),
        "touched_experts": touched,
        "ffn_weight_gbs": round(wbytes / ffn_s / 1e9, 1),
        "ffn_weight_frac_of_hbm": round(wbytes / ffn_s / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": roofline,
        "roofline_kernel_us": round(fc1_s * 1e6, 2),
    }
    if wmx is not None and not mx:
        # the same step on the MX path (MXFP4 weights, MXFP8 activations), same batch
        lay_mx = binding.RoutedExperts(w.T, w.H, w.E, w.K, w.I, w.P, dtype=dt, E_loc=w.n_local,
                                       expert_begin=w.expert_begin,
                                       expert_stride=w.expert_stride, block_m=w.beta,
                                       planner=args.planner, precision="mx", direct=direct)
        st = max(20, min(args.steps, 100))
        tm_mx, n_mx, _, _ = measure(skew, st, st, lay_mx, wmx[0], wmx[1], settle_s=0.5)
        wl_mx, pr_mx = tm_mx["median_s"], tm_mx["per"]
        f1 = (pr_mx["fc1"] - pr_mx.get("fc1_schedule", 0.0)) * 1e-6
        line["mx_path"] = {
            "tokens_per_s": round(w.T / wl_mx, 1), "ms_per_step": round(wl_mx * 1e3, 4),
            "fc1_kernel": "ffn_mx_kernel<true>",
            "combine": "direct rows (one-entry tokens stored by the MX down GEMM)" if direct else
                       "every token summed by the combine",
            "fc1_tflops": round(4.0 * w.H * w.I * n_mx / f1 / 1e12, 1),
            "fc1_frac_of_fp8_peak": round(4.0 * w.H * w.I * n_mx / f1 / 1e12 / PEAK_FP8_TFLOPS, 4),
            "gemm_tflops": round(6.0 * w.H * w.I * n_mx / ((pr_mx["fc1"] + pr_mx["fc2"]) * 1e-6) / 1e12, 1),
            "per_call_us": {k: round(v, 2) for k, v in pr_mx.items()},
            "steps": st}
        del lay_mx
        torch.cuda.empty_cache()
    if w.n_local // w.P <= 64 and w.n_local * w.P <= 4096:
        line["plan_comparison"] = plan_comparison(layer, w, max(20, args.steps // 4), torch)
    if not args.no_router:
        line["router_topk"] = {**router_measured(torch, dev, w, x, binding, inputs),
                               "what": "moe_router_topk (scores and top-k in one kernel) on the batch's x and "
                                       "a seeded W_r, outside the measured step; mean of back-to-back calls"}
    # the practical HBM rates of this machine (after the timed steps), beside the 8 TB/s spec
    ref = hbm_reference(torch, dev)
    line["hbm_measured"] = {**ref, "what": "1 GiB device copy (read + written bytes) and a 1 GiB "
                                           "read-only sum, median of 20 event-timed launches"}
    line["combine_frac_of_measured_copy"] = round(combine_bytes / (per["combine"] * 1e-6) / 1e9
                                                  / ref["copy_gbs"], 4)
    if bound == "mfma" and dt == torch.bfloat16 and not mx:
        # the vendor library on the same per-expert shapes, beside the 2.5 PFLOP/s peak
        gref = gemm_reference(torch, dev, w, loc.tolist())
        fc2_s = per["fc2"] * 1e-6
        gref["fc1_frac"] = round(achieved / gref["fc1_tflops"], 4)
        gref["fc2_frac"] = round(2.0 * w.H * w.I * N / fc2_s / 1e12 / gref["fc2_tflops"], 4)
        line["gemm_measured"] = {**gref, "what": "torch.bmm (hipBLASLt) bf16 on the same per-expert "
                                                 "shapes; *_frac = this path's GEMM kernel rate over it"}
    if not args.no_all_skews:
        by = []
        for sk in w.skews:
            tm_, n_, nb_, cnt_ = measure(sk, max(10, args.steps // 4), max(10, args.warmup // 4),
                                         settle_s=0.5)
            wl, pr = tm_["median_s"], tm_["per"]
            f = 6.0 * w.H * w.I * n_
            ffn_t = (pr["fc1"] + pr["fc2"]) * 1e-6
            loc_ = cnt_[w.expert_begin::w.expert_stride][: w.n_local].tolist()
            tr, tch, wb, bound_ = ffn_roofline(w, loc_, eb, peak_mfma)
            entry = {"skew": w.skew_label(sk), "tokens_per_s": round(w.T / wl, 1),
                     "ms_per_step": round(wl * 1e3, 4),
                     "gemm_tflops": round(f / ffn_t / 1e12, 1),
                     "ffn_frac_of_t_roof": round(tr / ffn_t, 4),
                     "touched_experts": tch,
                     "ffn_weight_gbs": round(wb / ffn_t / 1e9, 1)}
            if bound_ == "hbm":
                # the same weight stream against what this machine reads for a working set of
                # that size (re-read pass after pass), beside the 8 TB/s of t_roof
                rr = read_rate_at(torch, dev, wb)
                entry["read_ref_gbs"] = round(rr, 1)
                entry["ffn_frac_of_read_ref"] = round(wb / ffn_t / 1e9 / rr, 4)
            by.append(entry)
        line["by_skew"] = by
    if not args.no_cpu_baseline:
        T_s = args.cpu_tokens or {"tiny_f32": 64, "olmoe_shaped": 256,
                                  "qwen3_30b_a3b_shaped": 256, "gpt_oss_120b_shaped": 64,
                                  "gpt_oss_120b_decode": 64, "deepseek_v3_share": 256}[w.name]
        T_s = max(w.P, T_s // w.P * w.P)
        del layer
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline(w, skew, T_s, precision=args.precision)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
