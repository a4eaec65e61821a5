#!/usr/bin/env python3
"""Benchmark of the W4AFP8 fused-MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one fused-MoE call (align -> quant -> gate_up + SwiGLU + requant ->
down -> combine; w4a8_fused_moe_prepacked on weights re-laid out once before
timing, or w4a8_fused_moe with --layout canonical) on the decode workload: T=64 tokens, H=7168,
I=2048, top-8 of 256 experts, this GPU's share = experts 0..31.  Inputs are
seeded synthetic data already resident in HBM; successive steps rotate over
distinct weight sets (>= 1 GB in total, so the weights stream from HBM rather
than from the 256 MB last-level cache).  The same calls replayed from HIP
graphs (one captured call per weight set, as a serving decode loop may run
them) are reported too.

Printed: one JSON line with the headline (decode µs per call), the roofline
of the dominant kernel (timed live with HIP events on the library's stream),
the prefill workloads (T=4096 and the EP8 rank share T=32768) and the CPU
oracle baseline.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA (published, no sparsity)
F16_PEAK_TFLOPS = 2500.0       # dense fp16 MFMA
METRIC = ("fused-MoE µs + TFLOP/s & HBM GB/s (% roofline) at T=64 decode and "
          "T=4096 prefill")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def moe_bytes(cfg, stats):
    """Algorithmic bytes of one fused forward: packed weights + scales of the
    active local experts, bf16 activations in and out, routing in."""
    H, I = cfg.H, cfg.I
    per_expert = 2 * I * H // 2 + 2 * I * (H // 128) * 4 + H * I // 2 + H * (I // 128) * 4
    return stats["A"] * per_expert + cfg.T * H * 2 * 2 + cfg.T * cfg.topk * 8


def gate_up_bytes(cfg, stats):
    """Algorithmic bytes of the gate_up kernel: w13 + scales of the active
    experts, the fp8 activation rows and scales it reads, the fp8 intermediate
    and its scales it writes."""
    H, I = cfg.H, cfg.I
    w = stats["A"] * (2 * I * H // 2 + 2 * I * (H // 128) * 4)
    return w + cfg.T * (H + (H // 128) * 4) + stats["P"] * (I + (I // 128) * 4)


def down_bytes(cfg, stats):
    H, I = cfg.H, cfg.I
    w = stats["A"] * (H * I // 2 + H * (I // 128) * 4)
    return w + stats["P"] * (I + (I // 128) * 4) + stats["P"] * H * 4


def moe_flops(cfg, stats):
    return 2.0 * stats["P"] * (cfg.H * 2 * cfg.I + cfg.I * cfg.H)


def prefill_entry(cfg, stats, us):
    """Flat summary of one prefill workload: µs, TFLOP/s, GB/s, the fraction
    of the dense fp8 MFMA peak and the roofline fraction max(bytes / HBM peak,
    flops / fp8 peak) / t (whichever bound is the larger)."""
    fl, by = moe_flops(cfg, stats), moe_bytes(cfg, stats)
    t = us * 1e-6
    t_hbm, t_mfma = by / (HBM_PEAK_GBS * 1e9), fl / (FP8_PEAK_TFLOPS * 1e12)
    return {"workload": cfg.desc, "us": round(us, 1), "P": stats["P"], "A": stats["A"],
            "tflops": round(fl / t / 1e12, 2), "hbm_gbs": round(by / t / 1e9, 1),
            "frac_fp8_peak": round(fl / t / 1e12 / FP8_PEAK_TFLOPS, 4),
            "frac_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
            "bound": "mfma" if t_mfma >= t_hbm else "hbm",
            "roofline_frac": round(max(t_hbm, t_mfma) / t, 4)}


class Workload:
    def __init__(self, name, nsets, dev, prepack=True, fp4=False, recipe=0):
        import torch
        from w4a8_moe_grouped_amd import lib, synth
        self.cfg = cfg = synth.CONFIGS[name]
        self.fp4 = fp4
        self.recipe = recipe  # down-GEMM activation block (64 / 32), 0 = the plain call
        t0 = time.time()
        ids, w = synth.gen_routing(cfg)
        self.stats = synth.routing_stats(cfg, ids)
        put = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.hidden = put(synth.gen_hidden(cfg).view(np.int16)).view(torch.bfloat16)
        self.ids, self.w = put(ids), put(w)
        self.out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
        nbytes = lib.fused_moe_workspace_bytes(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        if fp4:
            # fp4 e2m1 weights with UE8M0 scales, prepacked once (not timed)
            self.psets = []
            for st in range(nsets):
                w13, s13, w2, s2 = (put(a) for a in synth.gen_expert_weights_fp4(cfg, seed=cfg.seed + st))
                self.psets.append(lib.prepack_weights_fp4(w13, s13, lib.FP4_GATE_UP) +
                                  lib.prepack_weights_fp4(w2, s2, lib.FP4_DOWN))
                del w13, s13, w2, s2
            self.sets = self.psets
            self.use_packed = True
            self.persistent = False
            self.ws_p = None
            log("[bench] %s fp4: T=%d P=%d A=%d, %d weight set(s), inputs in %.1fs"
                % (name, cfg.T, self.stats["P"], self.stats["A"], nsets, time.time() - t0))
            return
        self.sets = []
        for s in range(nsets):
            w13, s13, w2, s2 = synth.gen_expert_weights(cfg, seed=cfg.seed + s)
            self.sets.append(tuple(put(a) for a in (w13, s13, w2, s2)))
        # the load-time re-layout of the weights (w4a8_prepack_weights), done
        # once here, outside every timed region
        self.psets = [lib.prepack_weights(w13, s13) + lib.prepack_weights(w2, s2)
                      for (w13, s13, w2, s2) in self.sets] if prepack else None
        self.use_packed = prepack
        self.persistent = False  # w4a8_fused_moe_persistent (one launch after the align)
        self.ws_p = None
        log("[bench] %s: T=%d P=%d A=%d, %d weight set(s), inputs in %.1fs"
            % (name, cfg.T, self.stats["P"], self.stats["A"], nsets, time.time() - t0))

    def step(self, i):
        from w4a8_moe_grouped_amd import lib
        cfg = self.cfg
        if self.recipe:
            lib.fused_moe_recipe(self.hidden, self.ids, self.w, cfg.expert_begin, cfg.E_local, cfg.I,
                                 self.psets[i % len(self.psets)],
                                 lib.WEIGHTS_FP4_PACKED if self.fp4 else lib.WEIGHTS_INT4_PACKED,
                                 self.recipe, out=self.out, workspace=self.ws)
            return
        if self.persistent:
            if self.ws_p is None:
                import torch
                fmt = lib.WEIGHTS_FP4_PACKED if self.fp4 else lib.WEIGHTS_INT4_PACKED
                n = lib.fused_moe_persistent_workspace_bytes(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I, fmt)
                self.ws_p = torch.empty(n, dtype=torch.uint8, device=self.out.device)
            lib.fused_moe_persistent(self.hidden, self.ids, self.w, cfg.expert_begin, cfg.E_local, cfg.I,
                                     self.psets[i % len(self.psets)],
                                     lib.WEIGHTS_FP4_PACKED if self.fp4 else lib.WEIGHTS_INT4_PACKED,
                                     out=self.out, workspace=self.ws_p)
            return
        if self.fp4:
            lib.fused_moe_fp4(self.hidden, self.ids, self.w, cfg.expert_begin, cfg.E_local, cfg.I,
                              self.psets[i % len(self.psets)], out=self.out, workspace=self.ws)
            return
        j = i % len(self.sets)
        w13, s13, w2, s2 = self.sets[j]
        lib.fused_moe(self.hidden, self.ids, self.w, cfg.expert_begin, cfg.E_local, w13, s13,
                      w2, s2, out=self.out, workspace=self.ws,
                      prepacked=self.psets[j] if self.use_packed else None)


def time_steps(wl, steps, warmup, span=None):
    """Whole-step time: events + synchronize around exactly `steps` calls.
    With a SpanTimer, each timed call also records the two events of one
    stage on the library's stream; their mean span is returned too."""
    import torch
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        if span is not None:
            span.arm(i)
        wl.step(i)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / steps  # µs per step
    if span is None:
        return us
    return us, float(np.mean(span.read_ms())) * 1e3


def graph_steps(wl, steps, warmup):
    """The same steps replayed from HIP graphs (one captured call per weight
    set, torch.cuda.CUDAGraph): the host's launch overhead leaves the timed
    region, as in a serving decode loop.  Returns µs per step."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for j in range(len(wl.sets)):
            wl.step(j)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for j in range(len(wl.sets)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            wl.step(j)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / steps
    del graphs
    return us


def stage_breakdown(wl, steps):
    """Per-stage µs from HIP events the library records on its own stream."""
    import torch
    from w4a8_moe_grouped_amd import lib
    timer = lib.StageTimer()
    acc = {k: [] for k in lib.STAGES}
    for i in range(steps):
        timer.arm()
        wl.step(i)
        for k, v in timer.read_ms().items():
            acc[k].append(v * 1e3)
    torch.cuda.synchronize()
    timer.close()
    return {k: float(np.mean(v)) for k, v in acc.items()}


# Kernel sources whose HBM traffic the committed counter summary describes;
# the summary's figure is reported only while they are unchanged.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_T64_gate_up_traffic.md")
TRAFFIC_SOURCES = ("gemm_skinny.hip", "common.hpp", "internal.hpp", "lds_direct.hpp")


def kernel_source_digest(names=TRAFFIC_SOURCES):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "w4a8_moe_grouped_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the decode gate_up kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a device-copy
    calibration), or None if absent or taken on other kernel sources."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    d = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m or not d or d.group(1) != kernel_source_digest():
        return None
    return float(m.group(1))


def copy_calibration(nbytes=1 << 30, reps=4):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _oracle_slices(d, cfg, rows, threads):
    """The oracle on disjoint token slices, one thread each (the C library
    releases the GIL; every output row depends only on its own token, so the
    result equals one single-threaded call on the same rows)."""
    import concurrent.futures
    import oracle
    parts = [p for p in np.array_split(rows, threads) if p.size]

    def run(r):
        return oracle.fused_moe(d["hidden"][r], d["topk_ids"][r], d["topk_weights"][r],
                                cfg.expert_begin, cfg.E_local, d["w13"], d["s13"], d["w2"], d["s2"])
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, parts))
    return time.perf_counter() - t0, len(parts)


def gpu_warmup(seconds=0.3):
    """Plain device copies for a fixed time before anything is timed, so that
    the GPU's clocks have left their idle state (measured here: the first
    ~10 ms of work after idle run several percent slower).  No workload step
    runs here: the W warm-up steps and the K timed steps are untouched."""
    import torch
    src = torch.empty(64 << 20, dtype=torch.int32, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
    del src, dst


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """GB/s of a plain 1 GiB device-to-device copy (read + write bytes), the
    box's measured HBM figure printed beside the 8 TB/s datasheet peak."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    s = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / s / 1e9


def dense_linear(dev, steps):
    """The dense W4AFP8 linear (w4a8_gemm on w4a8_quantize_act's codes):
    µs of the GEMM and of the quantisation, TFLOP/s and GB/s of the GEMM."""
    import torch
    from w4a8_moe_grouped_amd import lib, synth
    cfg = synth.CONFIGS["dense"]
    x, w, sw = synth.gen_dense(cfg)
    put = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    xt = put(x.view(np.int16)).view(torch.bfloat16)
    wt, swt = put(w), put(sw)
    q, qs = lib.quantize_act(xt)
    gws = torch.empty(max(lib.gemm_workspace_bytes(cfg.M, cfg.K, cfg.N), 1), dtype=torch.uint8, device=dev)
    out = lib.gemm(q, qs, wt, swt, workspace=gws)
    for _ in range(200):  # ~4 ms of the same calls first (steady state)
        lib.gemm(q, qs, wt, swt, out=out, workspace=gws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        lib.gemm(q, qs, wt, swt, out=out, workspace=gws)
    b.record()
    torch.cuda.synchronize()
    g_us = a.elapsed_time(b) * 1e3 / steps
    a.record()
    for _ in range(steps):
        lib.quantize_act(xt, out_q=q, out_scales=qs)
    b.record()
    torch.cuda.synchronize()
    q_us = a.elapsed_time(b) * 1e3 / steps
    M, K, N = cfg.M, cfg.K, cfg.N
    byts = N * K // 2 + N * (K // 128) * 4 + M * K + M * (K // 128) * 4 + M * N * 2
    res = {"workload": cfg.desc, "gemm_us": round(g_us, 2), "quant_us": round(q_us, 2),
           "gemm_tflops": round(2.0 * M * N * K / (g_us * 1e-6) / 1e12, 2),
           "gemm_hbm_gbs": round(byts / (g_us * 1e-6) / 1e9, 1)}
    log("[bench] dense: %s" % res)
    return res


def extra_workloads(dev, steps):
    """The skewed-routing MoE configs and the dense linear: µs and rates."""
    import torch
    from w4a8_moe_grouped_amd import lib, synth
    res = {}
    for name in ("skew_perm", "skew_id"):
        q = Workload(name, nsets=2, dev=dev)
        us = time_steps(q, steps, 100)
        res[name] = {"workload": q.cfg.desc, "us": round(us, 2), "P": q.stats["P"], "A": q.stats["A"],
                     "hbm_gbs": round(moe_bytes(q.cfg, q.stats) / (us * 1e-6) / 1e9, 1),
                     "frac_hbm": round(moe_bytes(q.cfg, q.stats) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "stages_us": {k: round(v, 1) for k, v in stage_breakdown(q, 5).items()}}
        log("[bench] %s: %s" % (name, res[name]))
        del q
    res["dense"] = dense_linear(dev, steps)
    return res


def cpu_baseline(name):
    """The plain C oracle (fp64) on the host: the whole decode call on all the
    host's cores (token slices), the same call single-threaded, and the
    T=4096 prefill on every 16th token (extrapolated, labelled as such)."""
    import oracle
    from w4a8_moe_grouped_amd import synth
    oracle.lib()
    cfg = synth.CONFIGS[name]
    d = synth.gen_moe(cfg)
    # the machine's CPU share for one GPU is 16 threads, whatever os.cpu_count() says
    threads = max(1, min(16, os.cpu_count() or 1, cfg.T))
    rows = np.arange(cfg.T)
    t1, _ = _oracle_slices(d, cfg, rows, 1)
    tn, used = _oracle_slices(d, cfg, rows, threads)
    out = {"value": round(tn * 1e6, 1), "unit": "µs", "cores": used, "kind": "oracle",
           "sample": "the whole %s workload (T=%d, H=%d, I=%d, top-%d, experts 0..%d of %d), "
                     "one call, fp64 C, token slices over %d threads"
                     % (name, cfg.T, cfg.H, cfg.I, cfg.topk, cfg.E_local - 1, cfg.E_total, used),
           "single_thread_us": round(t1 * 1e6, 1)}
    try:
        import platform
        out["cpu"] = platform.processor() or platform.machine()
    except Exception:
        pass
    pc = synth.CONFIGS["prefill"]
    pd = synth.gen_moe(pc)
    sample = np.arange(0, pc.T, 16)
    tp, usedp = _oracle_slices(pd, pc, sample, threads)
    out["prefill_T4096_extrapolated_us"] = round(tp * 16 * 1e6, 1)
    out["prefill_sample"] = "every 16th token (%d of %d) on %d threads, time x16" % (sample.size, pc.T, usedp)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp4", action="store_true", help="skip the fp4-weight workloads")
    ap.add_argument("--only", default=None, help="time just this workload (decode/prefill/...)")
    ap.add_argument("--layout", choices=("prepacked", "canonical"), default="prepacked",
                    help="weight layout the timed calls read (prepacked once before timing)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs the fused MoE on one GPU's share of experts; "
              "multi-GPU runs are not part of it (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    from w4a8_moe_grouped_amd import lib
    if not os.path.exists(lib.LIB_PATH):
        from w4a8_moe_grouped_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    lib.load()

    if args.only == "dense":  # the dense linear alone (for profiling it)
        print(json.dumps({"dense": dense_linear(torch.device("cuda:0"), args.steps)}), flush=True)
        return
    primary = args.only or "decode"
    packed = args.layout == "prepacked"
    wl = Workload(primary, nsets=2, dev=dev, prepack=packed)
    cfg, st = wl.cfg, wl.stats
    gpu_warmup()  # the inputs were drawn on the host meanwhile: the GPU sat idle
    us = time_steps(wl, args.steps, args.warmup)
    graph_us = graph_steps(wl, args.steps, args.warmup)
    other_us = single_us = None
    if packed:  # the same calls on the canonical [E, N, K/2] weights, for comparison
        wl.use_packed = False
        other_us = time_steps(wl, args.steps, args.warmup)
        wl.use_packed = True
        # and through the single-launch export (block-tiled kernels at any size)
        wl.persistent = True
        single_us = time_steps(wl, args.steps, min(args.warmup, 50))
        wl.persistent = False
    # The dominant kernel of the decode step is gate_up (stage hook events
    # 2 -> 3).  Recording events costs GPU time of its own (a few µs each on
    # this stack), so its launches are timed in a second pass of the same
    # steps rather than inside the pass that gives `value`; the span includes
    # one event's overhead, so the achieved rate is a lower bound.
    span = lib.SpanTimer(2, 3, args.steps)
    _, dom_us = time_steps(wl, args.steps, 0, span=span)
    span.close()
    # per-call spread: one event pair around each whole call (stage hooks 0 -> 5)
    whole = lib.SpanTimer(0, 5, args.steps)
    time_steps(wl, args.steps, 0, span=whole)
    per_call = np.array(whole.read_ms()) * 1e3
    whole.close()
    stages = stage_breakdown(wl, max(5, min(args.steps, 20)))
    log("[bench] %s: %.1f us/call (%s weights; %.1f us/call replayed from HIP graphs), stages %s"
        % (primary, us, args.layout, graph_us, {k: round(v, 1) for k, v in stages.items()}))
    if other_us is not None:
        log("[bench] %s: %.1f us/call on the canonical weight layout, %.1f us/call as one launch "
            "after the align" % (primary, other_us, single_us))
    byts, flops = moe_bytes(cfg, st), moe_flops(cfg, st)
    gb_s = byts / (us * 1e-6) / 1e9
    tflops = flops / (us * 1e-6) / 1e12
    dom = "gate_up"
    dom_bytes = gate_up_bytes(cfg, st)
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic() if primary == "decode" else None

    result = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "µs",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 x fp8 (gate_up operands converted exactly to f16 for the MFMA, down on fp8 MFMA; fp32 accumulation and promotion)",
        "data": "synthetic (seeded; random int4 weights, N(0,1) activations and router logits)",
        "config": {"workload": "%s: %s" % (primary, cfg.desc), "T": cfg.T, "H": cfg.H, "I": cfg.I,
                   "experts_total": cfg.E_total, "experts_local": cfg.E_local, "topk": cfg.topk,
                   "local_pairs": st["P"], "active_experts": st["A"], "weight_sets": 2,
                   "weight_layout": args.layout},
        "timing": "value: K consecutive calls launched back to back between two events; graph_us: "
                  "the same calls replayed from HIP graphs (one captured call per weight set)",
        "graph_us": round(graph_us, 2),
        "canonical_layout_us": None if other_us is None else round(other_us, 2),
        "single_launch_us": None if single_us is None else round(single_us, 2),
        "tflops": round(tflops, 2),
        "hbm_gbs": round(gb_s, 1),
        "roofline_frac_call": round(gb_s / HBM_PEAK_GBS, 4),
        "stages_us": {k: round(v, 2) for k, v in stages.items()},
        "per_call_us": {"median": round(float(np.median(per_call)), 2),
                        "p10": round(float(np.percentile(per_call, 10)), 2),
                        "p90": round(float(np.percentile(per_call, 90)), 2), "calls": int(per_call.size)},
        "hbm_copy_gbs": round(copy_bandwidth(), 1),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 2)},
    }

    if not args.no_prefill and args.only is None:
        # steady state: ~30 ms of warm-up (the first ~20 ms of a workload's
        # calls run up to 9% slower) and two weight sets alternating, as for
        # decode, so no step reads the previous step's weights from cache.
        # Each workload is a flat object of scalars under its own key; its
        # per-stage µs sit beside it under <key>_stages_us.
        for name, steps, warm in (("prefill", 30, 60), ("prefill_ep8", 8, 10)):
            p = Workload(name, nsets=2, dev=dev, prepack=packed)
            pu = time_steps(p, steps, warm)
            pst = stage_breakdown(p, 2)
            ent = prefill_entry(p.cfg, p.stats, pu)
            p.persistent = True  # the same calls through the single-launch export
            ent["single_launch_us"] = round(time_steps(p, steps, warm), 2)
            p.persistent = False
            result[name] = ent
            result[name + "_stages_us"] = {k: round(v, 1) for k, v in pst.items()}
            log("[bench] %s: %s stages %s" % (name, ent, result[name + "_stages_us"]))
            del p
            torch.cuda.empty_cache()

    if not args.no_prefill and args.only is None:
        result["other_configs"] = extra_workloads(dev, args.steps)

    if not args.no_fp4 and args.only is None:
        # the same workloads on fp4 e2m1 weights with per-32-K UE8M0 scales
        # (weight and scale bytes equal the int4 path's, so the same roofline)
        fp4 = {}
        for name, steps, warm, nsets in (("decode", args.steps, args.warmup, 2), ("prefill", 30, 60, 2),
                                         ("prefill_ep8", 8, 10, 2)):
            if name != "decode" and args.no_prefill:
                continue
            q = Workload(name, nsets=nsets, dev=dev, fp4=True)
            qu = time_steps(q, steps, warm)
            qst = stage_breakdown(q, 5 if name == "decode" else 2)
            ent = {"workload": q.cfg.desc, "us": round(qu, 2), "P": q.stats["P"],
                   "tflops": round(moe_flops(q.cfg, q.stats) / (qu * 1e-6) / 1e12, 2),
                   "hbm_gbs": round(moe_bytes(q.cfg, q.stats) / (qu * 1e-6) / 1e9, 1),
                   "stages_us": {k: round(v, 2) for k, v in qst.items()}}
            if name == "decode":
                ent["gate_up_hbm_frac"] = round(gate_up_bytes(q.cfg, q.stats) / (qst["gate_up"] * 1e-6)
                                                / 1e9 / HBM_PEAK_GBS, 4)
            else:
                ent["frac_fp8_peak"] = round(moe_flops(q.cfg, q.stats) / (qu * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4)
            fp4[name] = ent
            log("[bench] fp4 %s: %s" % (name, ent))
            del q
            torch.cuda.empty_cache()
        result["fp4_weights"] = fp4

    if not args.no_fp4 and args.only is None:
        # the finer activation-scale recipes (down GEMM input per 64 / 32 K)
        rec = {}
        for fp4w in (False, True):
            for group in (64, 32):
                q = Workload("decode", nsets=2, dev=dev, fp4=fp4w, recipe=group)
                qu = time_steps(q, args.steps, args.warmup)
                rec["decode_%s_per%d" % ("fp4" if fp4w else "int4", group)] = round(qu, 2)
                del q
        log("[bench] recipes: %s" % rec)
        result["activation_recipes_us"] = rec

    if not args.no_cpu_baseline:
        cb = cpu_baseline(primary)
        result["cpu_baseline"] = cb
        log("[bench] cpu oracle: %.0f us" % cb["value"])

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
