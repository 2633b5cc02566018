"""Benchmark of the int4 group-quantized MoE SwitchGLU layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload moe_decode]

Default workload (the headline): one MoE SwitchGLU layer decoding one token — hidden 2048,
256 experts with int4 group-64 gate/up [512 x 2048] and down [2048 x 512], 8-bit router
and shared-expert gate, top-4 routing, a shared expert of intermediate 512 and unmerged
LoRA rank 16 (alpha 32) on its three projections.  A step is one complete layer forward
for one token.  Steps cycle through 40 independently seeded copies of the layer (18 GB of
packed experts resident in HBM, 70x the 256 MB last-level cache) and every step decodes a
different token, so expert weights come from HBM as they do in a deep decode loop.  All
inputs are resident before timing; the timed region is one HIP graph of exactly K steps.

Other workloads (--workload): gemv (one int4 linear, x [1 x 2048], W [512 x 2048]; --group
32 and --params bf16 select the port page's checkpoint format),
moe_prefill (512 tokens, top-4; --skew adds +2.0 to the logits of experts 0..15),
moe_stack (40 stacked layers, 16 tokens per step, top-8, 4 LoRA adapter sets),
supergroup (mixed ternary/4-bit GEMM, W [3072 x 1024], --batch 1 or 64), supergroup_a8
(the same GEMM with 8-bit activations and an integer dot product), prerouter (one prerouter
head forward per token).

Prints one JSON line: the metric, a roofline object for the dominant kernel (algorithmic
bytes per launch over its average launch time, measured here with HIP events on the stream
it runs on) and, at N = 1, the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA
INT8_MFMA_PEAK_TOPS = 5000.0    # dense int8 MFMA (TOP/s)

H, I, SI, E, LAYERS, RANK, ALPHA = 2048, 512, 512, 256, 40, 16, 32.0
MAT_BYTES_4BIT = lambda rows, cols: rows * cols // 2 + 2 * (rows * (cols // 64) * 2)
MAT_BYTES_8BIT = lambda rows, cols: rows * cols + 2 * (rows * (cols // 64) * 2)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def counter_entry(key):
    """A committed counter record (profiles/traffic.json) for `key` ("workload/kernel"), or
    None when it is absent or the kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        entry = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[key]
        h = hashlib.sha256()
        for src in entry["sources"]:
            h.update(open(os.path.join(ROOT, src), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    return entry if h.hexdigest() == entry["source_sha256"] else None


def measured_traffic(key):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE runs, or None."""
    e = counter_entry(key)
    return None if e is None else e.get("traffic_bytes_per_launch")


class CacheFlush:
    """Writes 1 GiB (4x the 256 MB last-level cache, 250x an XCD's L2) on the current stream,
    so that a timed region that follows starts with no benchmark data in any cache."""

    def __init__(self, torch):
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def __call__(self):
        self.buf.fill_(1)


# ------------------------------------------------------------------------------ device data

def make_layer(q, torch, gen, top_k=4, n_adapters=1, skew=False, residual=False):
    """One layer of the MoE model with fresh N(0, 0.02) weights quantized on the device."""
    dev = "cuda"

    def quant(rows, cols, bits):
        w = torch.randn((rows, cols), generator=gen, device=dev, dtype=torch.float32) * 0.02
        qw = q.quantize_affine(w, bits)
        del w
        return qw

    def stack(rows, cols):
        qw = quant(E * rows, cols, 4)
        qw.rows, qw.n_experts = rows, E
        return qw

    def lora(din, dout):
        A = (torch.randn((n_adapters, RANK, din), generator=gen, device=dev) * 0.01).half()
        B = (torch.randn((n_adapters, dout, RANK), generator=gen, device=dev) * 0.01).half()
        return q.Lora(A, B, ALPHA / RANK)

    bias = None
    if skew:
        bias = torch.zeros(E, device=dev)
        bias[:16] = 2.0
    return q.MoELayer(hidden=H, inter=I, shared_inter=SI, n_experts=E, top_k=top_k,
                      router=quant(E, H, 8), shared_gate=quant(1, H, 8),
                      exp_gate=stack(I, H), exp_up=stack(I, H), exp_down=stack(H, I),
                      sh_gate=quant(SI, H, 4), sh_up=quant(SI, H, 4), sh_down=quant(H, SI, 4),
                      lora_gate=lora(H, SI), lora_up=lora(H, SI), lora_down=lora(SI, H),
                      router_bias=bias, add_residual=residual)


def graph_of(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # one eager pass on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def chunked_graphs(torch, step, n, chunk):
    """Graphs that together run exactly n repetitions of `step` (which must do the same work
    each time): one of `chunk` steps with its replay count, and one of the remainder.  Keeps
    every graph at a bounded node count (a 40-layer step is 240 launches)."""
    full, rem = divmod(n, chunk)
    parts = []
    if full:
        parts.append((graph_of(torch, lambda: [step() for _ in range(chunk)]), full))
    if rem:
        parts.append((graph_of(torch, lambda: [step() for _ in range(rem)]), 1))
    return parts


def replay_chunks(parts):
    for g, reps in parts:
        for _ in range(reps):
            g.replay()


def time_chunks(torch, parts, flush=None):
    """ms of one pass over `parts` (every graph replayed its count, in order), HIP events on
    the stream they run on; with `flush`, the caches are flushed first, outside the span."""
    st = torch.cuda.current_stream()
    torch.cuda.synchronize()
    if flush is not None:
        flush()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    replay_chunks(parts)
    b.record(st)
    b.synchronize()
    return a.elapsed_time(b)


def time_graph(torch, g, reps=1, flush=None):
    """Average ms of one replay: HIP events on the stream the graph runs on.  With `flush`,
    the caches are flushed before each replay, outside the timed span."""
    st = torch.cuda.current_stream()
    torch.cuda.synchronize()
    total = 0.0
    if flush is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            g.replay()
        b.record(st)
        b.synchronize()
        return a.elapsed_time(b) / reps
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        g.replay()
        b.record(st)
        b.synchronize()
        total += a.elapsed_time(b)
    return total / reps


# ------------------------------------------------------------------------------ CPU baseline

def host_desc():
    """The host CPU model and the number of CPUs this process may run on."""
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{model}, {len(os.sched_getaffinity(0))} CPUs available"


def cpu_baseline_moe_decode(n_tokens=600, budget_s=20.0):
    """The oracle (float64 numpy) on a bounded sample: n_tokens single-token decodes of one
    seeded layer of the same shapes; only the experts those tokens reach are quantized."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import synth
    from layers import Shape, build_layer, routed_experts
    from oracle import moe
    from threadpoolctl import threadpool_info

    S = Shape(top_k=4)
    wl = synth.Workload.MOE_DECODE
    xs = synth.activations(n_tokens, H, wl, 0, 99)
    L = build_layer(wl, 0, S, only_experts=routed_experts(xs, wl, 0, S, margin=0))
    t0 = time.perf_counter()
    done = 0
    for i in range(n_tokens):
        moe.moe_layer(xs[i:i + 1], L)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    return {"value": done / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle", "host": host_desc(),
            "sample": f"{done} single-token decodes of one layer (hidden 2048, 256 experts, "
                      f"top-4, shared expert, LoRA r16), float64 numpy, {dt:.1f} s"}


# ------------------------------------------------------------------------------ workloads

def kernel_row(name, key, us, nbytes=None, flops=None, peak=HBM_PEAK_GBS):
    """One per-kernel entry: average launch time and its algorithmic rate against the peak."""
    r = {"kernel": name, "us_per_launch": us}
    if nbytes is not None:
        gbs = nbytes / (us * 1e-6) / 1e9
        r.update(bytes_per_launch=nbytes, gbps=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                 traffic=measured_traffic(key))
    if flops is not None:
        tf = flops / (us * 1e-6) / 1e12
        r.update(flops_per_launch=flops, tflops=tf, mfma_frac=tf / FP16_MFMA_PEAK_TFLOPS)
    return r


def roofline_of(row, bound="hbm"):
    """The bench line's roofline object for one per-kernel entry."""
    if bound == "hbm":
        return {"kernel": row["kernel"], "bound": "hbm", "achieved": row["gbps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": row["gbps"] / HBM_PEAK_GBS, "traffic": row.get("traffic"),
                "bytes_per_launch": row["bytes_per_launch"], "us_per_launch": row["us_per_launch"]}
    return {"kernel": row["kernel"], "bound": "mfma", "achieved": row["tflops"],
            "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": row["tflops"] / FP16_MFMA_PEAK_TFLOPS,
            "traffic": row.get("traffic"), "flops_per_launch": row["flops_per_launch"],
            "us_per_launch": row["us_per_launch"]}


# algorithmic bytes of the decode layer at one token (config 1 shapes, top-4, LoRA r16)
DEC_XSIDE_BYTES = (MAT_BYTES_8BIT(E, H) + MAT_BYTES_8BIT(1, H) + 2 * MAT_BYTES_4BIT(SI, H)
                   + 2 * RANK * H * 2 + H * 2 + (E + 1 + 2 * SI + 2 * RANK) * 4)
DEC_GATE_UP_BYTES = (4 * 2 * MAT_BYTES_4BIT(I, H) + H * 2 + 2 * SI * RANK * 2 + 2 * SI * 4
                     + (4 * I + SI) * 2)
DEC_DOWN_BYTES = (4 * MAT_BYTES_4BIT(H, I) + MAT_BYTES_4BIT(H, SI) + RANK * SI * 2 + H * RANK * 2
                  + (4 * I + SI) * 2 + H * 2)
DEC_STEP_BYTES = (MAT_BYTES_8BIT(E, H) + MAT_BYTES_8BIT(1, H) + 4 * 3 * MAT_BYTES_4BIT(I, H)
                  + 3 * MAT_BYTES_4BIT(SI, H) + 3 * RANK * (H + SI) * 2 + 2 * H * 2)


def bench_moe_decode(args, q, torch):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    t0 = time.perf_counter()
    layers = [make_layer(q, torch, gen) for _ in range(LAYERS)]
    flush = CacheFlush(torch)
    torch.cuda.synchronize()
    log(f"built {LAYERS} layers in {time.perf_counter() - t0:.1f} s")
    K, W = args.steps, args.warmup
    n_tok = K + W
    xs = (torch.randn((n_tok, 1, H), generator=gen, device="cuda")).half()
    ys = torch.empty_like(xs)
    ws_bytes = q.moe_workspace_bytes(layers[0], 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    calls = [q.MoECall(layers[i % LAYERS], xs[i], ys[i], ws) for i in range(n_tok)]

    def run(lo, hi):
        def f():
            for i in range(lo, hi):
                calls[i]()
        return f

    g_warm = graph_of(torch, run(K, K + W)) if W else None
    g_main = graph_of(torch, run(0, K))
    if g_warm is not None:
        g_warm.replay()
    t_wall = time.perf_counter()
    ms_total = time_graph(torch, g_main, flush=flush)
    t_wall = time.perf_counter() - t_wall
    log(f"main: {K} steps in {ms_total:.3f} ms (wall {t_wall * 1e3:.3f} ms, caches flushed first)")

    # each launch alone, over R (layer, token) pairs routed beforehand, caches flushed first
    R = 512
    wss = torch.empty((R, ws_bytes), dtype=torch.uint8, device="cuda")
    rx = (torch.randn((R, 1, H), generator=gen, device="cuda")).half()
    ry = torch.empty_like(rx)
    rcalls = [q.MoECall(layers[r % LAYERS], rx[r], ry[r], wss[r]) for r in range(R)]
    for c in rcalls:
        c()
    torch.cuda.synchronize()
    rows = []
    for name, st, nbytes in (("k_dec_xside", q.STAGE_ROUTE, DEC_XSIDE_BYTES),
                             ("k_dec_gate_up", q.STAGE_GATE_UP, DEC_GATE_UP_BYTES),
                             ("k_dec_down", q.STAGE_DOWN, DEC_DOWN_BYTES)):
        g = graph_of(torch, lambda st=st: [c(st) for c in rcalls])
        us = time_graph(torch, g, reps=3, flush=flush) / R * 1e3
        rows.append(kernel_row(name, f"moe_decode/{name}", us, nbytes))
    dom = max(rows, key=lambda r: r["us_per_launch"])
    ms_step = ms_total / K
    res = {
        "metric": "int4 MoE layer tokens/s (decode, 1 token per step)",
        "value": K / (ms_total * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "moe_switchglu_int4 decode: 1 token/step, hidden 2048, 256 "
                               "experts int4 g64, top-4, shared expert + 8-bit gate, LoRA r16 "
                               "a32, 40 independently seeded layers rotated, caches flushed "
                               "before the timed region",
                   "global_batch": 1, "layers_rotated": LAYERS,
                   "step_algorithmic_bytes": DEC_STEP_BYTES,
                   "step_hbm_gbps": DEC_STEP_BYTES / (ms_step * 1e-3) / 1e9,
                   "step_hbm_frac": DEC_STEP_BYTES / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "kernels": rows},
        "roofline": roofline_of(dom),
    }
    return res, cpu_baseline_moe_decode


def cpu_baseline_moe_routed(n_tokens=600, budget_s=20.0):
    """The oracle on a bounded sample: single-token layer forwards under a given routing
    (the layer evaluated on the stated selection, as the routed call computes it)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import synth
    from layers import Shape, build_layer
    from oracle import moe

    S = Shape(top_k=4)
    wl = synth.Workload.MOE_DECODE
    xs = synth.activations(n_tokens, H, wl, 0, 98)
    route = synth.expert_choices(n_tokens, 4, E, wl, 0, 98)
    L = build_layer(wl, 0, S, only_experts=set(route.ravel().tolist()))
    t0 = time.perf_counter()
    done = 0
    for i in range(n_tokens):
        moe.moe_layer(xs[i:i + 1], L, idx=route[i:i + 1])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": _threads(), "kind": "oracle", "host": host_desc(),
            "sample": f"{done} single-token decodes of one layer under a given top-4 routing (hidden 2048, "
                      f"256 experts, shared expert, LoRA r16), float64 numpy, {dt:.1f} s"}


def bench_moe_decode_routed(args, q, torch):
    """Decode with the prerouter head's prediction as the route ("double shift"): layer l at
    token i runs the experts that the head of layer l-1 predicted from token i's input, the
    routing layer l-1 executed for token i and the one it executed for token i-1.  The routes
    are predicted (and the executed routings taken) before the timed region; the timed steps
    are the routed layer calls alone, and the head's own forward is timed on its own."""
    D, F, TOPK = H, 512, 4
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1235)
    layers = [make_layer(q, torch, gen) for _ in range(LAYERS)]
    n_in = D + 2 * E
    rnd = lambda *sh: (torch.randn(sh, generator=gen, device="cuda") * 0.02).half()
    heads = [q.PrerouterHead(rnd(E, n_in), rnd(E), rnd(F, n_in), rnd(F), rnd(E, F), rnd(E))
             for _ in range(LAYERS)]
    flush = CacheFlush(torch)
    K, W = args.steps, args.warmup
    n_tok = K + W
    xs = torch.randn((n_tok, 1, H), generator=gen, device="cuda").half()
    ys = torch.empty_like(xs)
    ws = torch.empty(q.moe_workspace_bytes(layers[0], 1), dtype=torch.uint8, device="cuda")
    # executed routing of layer l-1 for every token, then the head's prediction for layer l
    execd = torch.empty((n_tok, 1, TOPK), dtype=torch.int32, device="cuda")
    for i in range(n_tok):
        lp = (i - 1) % LAYERS
        q.MoECall(layers[lp], xs[i], ys[i], ws, idx_out=execd[i])()
    routes = torch.empty((n_tok, 1, TOPK), dtype=torch.int32, device="cuda")
    for i in range(n_tok):
        _, _, pred, _ = q.prerouter_forward(heads[(i - 1) % LAYERS], xs[i], execd[i], execd[max(i - 1, 0)])
        routes[i].copy_(pred)
    torch.cuda.synchronize()
    wts = torch.empty((n_tok, 1, TOPK), dtype=torch.float32, device="cuda")

    def run(lo, hi):
        def f():
            for i in range(lo, hi):
                q.moe_switchglu_int4_routed(layers[i % LAYERS], xs[i], routes[i], ws=ws, out=ys[i], w_out=wts[i])
        return f
    if W:
        graph_of(torch, run(K, K + W)).replay()
    g_main = graph_of(torch, run(0, K))
    ms_total = time_graph(torch, g_main, flush=flush)
    ms_step = ms_total / K

    def heads_run():
        for i in range(K):
            q.prerouter_forward(heads[(i - 1) % LAYERS], xs[i], execd[i], execd[max(i - 1, 0)])
    ms_head = time_graph(torch, graph_of(torch, heads_run), flush=flush) / K
    row = kernel_row("routed layer call (k_dec_rt_gate_up + k_dec_down<routed>)", "moe_decode_routed/step",
                     ms_step * 1e3, DEC_STEP_BYTES)
    res = {
        "metric": "int4 MoE layer tokens/s (decode, 1 token per step, routed by the prerouter's prediction)",
        "value": K / (ms_total * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "moe_switchglu_int4_routed decode: 1 token/step, hidden 2048, 256 experts "
                               "int4 g64, top-4 given by the prerouter head's prediction (synthetic head "
                               "weights), shared expert + 8-bit gate, LoRA r16 a32, 40 layers rotated, "
                               "caches flushed before the timed region",
                   "global_batch": 1, "layers_rotated": LAYERS,
                   "step_algorithmic_bytes": DEC_STEP_BYTES,
                   "head_us_per_call": ms_head * 1e3,
                   "layer_plus_head_us_per_step": (ms_step + ms_head) * 1e3,
                   "kernels": [row]},
        "roofline": roofline_of(row),
    }
    return res, cpu_baseline_moe_routed


def cpu_baseline_moe_prefill(n_tokens=448, budget_s=20.0):
    """The oracle (float64 numpy) on a bounded sample: batches of 16 prefill tokens through
    one seeded layer of the same shapes (every expert the sample reaches is quantized)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import synth
    from layers import Shape, build_layer, routed_experts
    from oracle import moe
    from threadpoolctl import threadpool_info

    S = Shape(top_k=4)
    wl = synth.Workload.MOE_PREFILL
    xs = synth.activations(n_tokens, H, wl, 0, 99)
    L = build_layer(wl, 0, S, only_experts=routed_experts(xs, wl, 0, S, margin=0))
    t0 = time.perf_counter()
    done = 0
    for i in range(0, n_tokens, 16):
        moe.moe_layer(xs[i:i + 16], L)
        done += 16
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    return {"value": done / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle", "host": host_desc(),
            "sample": f"{done} prefill tokens in batches of 16 through one layer (hidden 2048, "
                      f"256 experts, top-4, shared expert, LoRA r16), float64 numpy, {dt:.1f} s"}


def bench_moe_prefill(args, q, torch):
    """512 tokens per step through one layer; 8 seeded layers rotated (3.6 GB of experts).
    --tokens sets another count (a sweep outside the workload: at thousands of tokens per
    step the experts see enough tokens for the GEMMs to be bound by MFMA, not HBM)."""
    T, NL, NX = args.tokens, 8, 8
    sweep = T != 512
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    t0 = time.perf_counter()
    layers = [make_layer(q, torch, gen, skew=args.skew) for _ in range(NL)]
    flush = CacheFlush(torch)
    xs = torch.randn((NX, T, H), generator=gen, device="cuda").half()
    ys = torch.empty_like(xs)
    ws_bytes = q.moe_workspace_bytes(layers[0], T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"built {NL} layers in {time.perf_counter() - t0:.1f} s; workspace {ws_bytes / 2**20:.1f} MiB")
    K, W = args.steps, args.warmup
    calls = [q.MoECall(layers[i % NL], xs[i % NX], ys[i % NX], ws) for i in range(K + W)]

    def run(lo, hi):
        def f():
            for i in range(lo, hi):
                calls[i]()
        return f
    if W:
        graph_of(torch, run(K, K + W)).replay()
    g_main = graph_of(torch, run(0, K))
    ms_total = time_graph(torch, g_main, flush=flush)
    ms_step = ms_total / K
    log(f"main: {K} steps in {ms_total:.3f} ms (caches flushed first)")

    # stages over NL routed workspaces (one per layer, distinct inputs)
    wss = torch.empty((NL, ws_bytes), dtype=torch.uint8, device="cuda")
    idx = torch.empty((NL, T, 4), dtype=torch.int32, device="cuda")
    scalls = [q.MoECall(layers[i], xs[i % NX], ys[i % NX], wss[i], idx_out=idx[i]) for i in range(NL)]
    for c in scalls:
        c(q.STAGE_ROUTE)
    torch.cuda.synchronize()
    stage_us = {}
    for name, st in (("route", q.STAGE_ROUTE), ("gate_up", q.STAGE_GATE_UP), ("down", q.STAGE_DOWN)):
        def f(st=st):
            for c in scalls:
                c(st)
        stage_us[name] = time_graph(torch, graph_of(torch, f), reps=5, flush=flush) / NL * 1e3
    ih = idx.cpu().numpy()
    used = np.mean([len(np.unique(ih[i])) for i in range(NL)])
    pairs = T * 4
    gu_bytes = used * 2 * MAT_BYTES_4BIT(I, H) + T * H * 2 + pairs * I * 2
    gu_flops = 2 * 2 * pairs * I * H
    us = stage_us["gate_up"]
    achieved = gu_bytes / (us * 1e-6) / 1e9
    tflops = gu_flops / (us * 1e-6) / 1e12
    step_bytes = (MAT_BYTES_8BIT(E, H) + MAT_BYTES_8BIT(1, H) + used * 3 * MAT_BYTES_4BIT(I, H)
                  + 3 * MAT_BYTES_4BIT(SI, H) + 3 * RANK * (H + SI) * 2 + 2 * T * H * 2)
    step_flops = 2 * T * (E * H + H + 3 * SI * H + 4 * 3 * I * H)
    # the gate/up kernel: the large-item GEMM once experts average more than 64 pairs
    big = pairs > 64 * E
    gu_kernel = "k_pf_big" if big else "k_pf_gemm"
    gu_name = (f"{gu_kernel} grouped gate/up ({'128-pair items, 32x32x16 MFMA' if big else 'small items'}; "
               "silu*up epilogue)")
    key = f"moe_prefill_{T}{'_skew' if args.skew else ''}/{gu_kernel}"
    ctr = counter_entry(key) or {}
    counted = {k: ctr[k] for k in ("traffic_bytes_per_launch", "mfma_flops_per_launch",
                                   "mfma_busy_frac") if k in ctr}
    if sweep:
        roofline = {"kernel": gu_name,
                    "bound": "mfma", "achieved": tflops, "peak": FP16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": tflops / FP16_MFMA_PEAK_TFLOPS,
                    "traffic": ctr.get("traffic_bytes_per_launch"),
                    "flops_per_launch": gu_flops, "us_per_launch": us,
                    "hbm_gbps": achieved, "hbm_frac": achieved / HBM_PEAK_GBS, "counters": counted}
    else:
        roofline = {"kernel": gu_name,
                    "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": ctr.get("traffic_bytes_per_launch"),
                    "bytes_per_launch": gu_bytes, "us_per_launch": us,
                    "mfma_tflops": tflops, "mfma_frac": tflops / FP16_MFMA_PEAK_TFLOPS, "counters": counted}
    res = {
        "metric": f"int4 MoE layer tokens/s (prefill, {T} tokens per step)",
        "value": T * K / (ms_total * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"moe_switchglu_int4 prefill: {T} tokens/step, hidden 2048, 256 "
                               "experts int4 g64, top-4, shared expert + 8-bit gate, LoRA r16 "
                               "a32, 8 independently seeded layers rotated"
                               + (", logits +2.0 on experts 0..15" if args.skew else "")
                               + (" (token-count sweep outside the 512-token workload)" if sweep else ""),
                   "global_batch": T, "experts_used_per_layer": used,
                   "step_algorithmic_bytes": step_bytes,
                   "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
                   "step_mfma_tflops": step_flops / (ms_step * 1e-3) / 1e12,
                   "stage_us": stage_us},
        "roofline": roofline,
    }
    return res, cpu_baseline_moe_prefill


def cpu_baseline_moe_stack(n_layers=2, budget_s=25.0):
    """The oracle (float64 numpy) on a bounded sample: the 16 multi-tenant tokens through the
    first layers of the stack (only the experts they reach are quantized); the rate is
    scaled to the 40-layer step."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import synth
    from layers import Shape, build_layer, routed_experts
    from oracle import moe
    from threadpoolctl import threadpool_info

    S = Shape(top_k=8, n_adapters=4)
    wl = synth.Workload.MOE_STACK
    x = synth.activations(16, H, wl, 0)
    ad = synth.adapter_index(16, 4)
    spent, done = 0.0, 0
    for layer in range(n_layers):
        L = build_layer(wl, layer, S, only_experts=routed_experts(x, wl, layer, S, margin=0))
        t0 = time.perf_counter()
        out = moe.moe_layer(x, L, ad)
        spent += time.perf_counter() - t0
        x = moe.residual(x, out["y"])
        done += 1
        if spent > budget_s:
            break
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    per_step = spent / done * LAYERS
    return {"value": 16 / per_step, "unit": "tokens/s", "cores": int(cores), "kind": "oracle", "host": host_desc(),
            "sample": f"16 tokens (4 adapters) through {done} of the 40 layers, float64 numpy, "
                      f"{spent:.1f} s, scaled to 40 layers"}


def bench_moe_stack(args, q, torch):
    """40 stacked layers, 16 tokens per step (4 LoRA adapter sets x 4 tokens), top-8."""
    T, TOPK, NAD = 16, 8, 4
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2468)
    t0 = time.perf_counter()
    layers = [make_layer(q, torch, gen, top_k=TOPK, n_adapters=NAD, residual=True)
              for _ in range(LAYERS)]
    torch.cuda.synchronize()
    log(f"built {LAYERS} layers in {time.perf_counter() - t0:.1f} s")
    K, W = args.steps, args.warmup
    ad = (torch.arange(T, device="cuda", dtype=torch.int32) // (T // NAD)).contiguous()
    x0 = torch.randn((T, H), generator=gen, device="cuda").half()
    acts = torch.empty((LAYERS + 1, T, H), dtype=torch.float16, device="cuda")
    ws = torch.empty(q.moe_workspace_bytes(layers[0], T), dtype=torch.uint8, device="cuda")
    calls = [q.MoECall(layers[l], acts[l], acts[l + 1], ws, adapter_idx=ad) for l in range(LAYERS)]

    def step():
        for c in calls:
            c()
    acts[0].copy_(x0)
    flush = CacheFlush(torch)
    # graphs of at most 25 steps (6,000 launches), replayed to make exactly W, then K steps
    CH = 25
    if W:
        replay_chunks(chunked_graphs(torch, step, W, CH))
    parts = chunked_graphs(torch, step, K, CH)
    ms = time_chunks(torch, parts, flush=flush)
    ms_step = ms / K

    # dominant kernel: gate/up of one layer over routed workspaces (one per layer)
    wss = torch.empty((LAYERS, ws.numel()), dtype=torch.uint8, device="cuda")
    idx = torch.empty((LAYERS, T, TOPK), dtype=torch.int32, device="cuda")
    rcalls = [q.MoECall(layers[l], acts[l], acts[l + 1], wss[l], adapter_idx=ad, idx_out=idx[l])
              for l in range(LAYERS)]
    for c in rcalls:
        c(q.STAGE_ROUTE)
    torch.cuda.synchronize()
    g_gu = graph_of(torch, lambda: [c(q.STAGE_GATE_UP) for c in rcalls])
    us_gu = time_graph(torch, g_gu, reps=3, flush=flush) / LAYERS * 1e3
    ih = idx.cpu().numpy()
    used = float(np.mean([len(np.unique(ih[l])) for l in range(LAYERS)]))
    # 128 (token, k) pairs take the token-sorted path: the grouped gate/up GEMM reads each
    # used expert's gate and up once, the tokens' x, and writes h per pair
    gu_bytes = used * 2 * MAT_BYTES_4BIT(I, H) + T * H * 2 + T * TOPK * I * 2
    step_bytes = LAYERS * (MAT_BYTES_8BIT(E, H) + MAT_BYTES_8BIT(1, H) + used * 3 * MAT_BYTES_4BIT(I, H)
                           + 3 * MAT_BYTES_4BIT(SI, H) + 3 * NAD * RANK * (H + SI) * 2 + 2 * T * H * 2)
    achieved = gu_bytes / (us_gu * 1e-6) / 1e9
    res = {
        "metric": "int4 MoE stack tokens/s (multi-tenant decode, 40 layers, 16 tokens per step)",
        "value": T * K / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "moe_switchglu_int4 x 40 stacked layers with residual, 16 tokens/step, "
                               "top-8 of 256 experts, 4 LoRA adapter sets (adapter = token // 4), "
                               "hidden 2048, int4 g64, shared expert + 8-bit gate",
                   "global_batch": T, "layers": LAYERS, "experts_used_per_layer": used,
                   "step_algorithmic_bytes": step_bytes,
                   "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9},
        "roofline": {"kernel": "k_pf_gemm grouped gate/up (16 tokens, top-8; silu*up epilogue)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("moe_stack/k_pf_gemm"),
                     "bytes_per_launch": gu_bytes, "us_per_launch": us_gu},
    }
    return res, cpu_baseline_moe_stack


def sg_bytes(rows, cols, period=4):
    n4 = rows // period
    return n4 * cols // 2 + (rows - n4) * cols // 4 + rows * 2


def cpu_baseline_supergroup(batch, budget_s=15.0, a8=False):
    """The oracle on a bounded sample: the super-group GEMM of one seeded 3072 x 1024 weight
    against `batch` inputs (weight-only, or with 8-bit activations), repeated until the budget
    is spent."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import synth
    from oracle import supergroup
    from threadpoolctl import threadpool_info

    w = synth.normal_f32((3072, 1024), synth.WEIGHT_SIGMA, synth.Workload.SUPERGROUP, 0,
                         synth.Role.SUPERGROUP)
    W, _ = supergroup.quantize(w, 4)
    x = synth.activations(batch, 1024, synth.Workload.SUPERGROUP, 0)
    t0 = time.perf_counter()
    n = 0
    gemm = supergroup.gemm_a8 if a8 else supergroup.gemm
    while True:
        gemm(x, W)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"value": n * batch / dt, "unit": "tokens/s", "cores": int(max(blas) if blas else 1),
            "kind": "oracle", "host": host_desc(), "sample": f"{n} {'8-bit activation ' if a8 else ''}GEMMs of W[3072x1024] "
                                        f"with {batch} inputs, float64/int64 numpy, {dt:.1f} s"}


def bench_supergroup(args, q, torch, a8=False):
    """Mixed ternary/4-bit super-group GEMM, W [3072 x 1024], B inputs per call (with a8: the
    weight-activation integer path, activations quantized to 8 bits inside the call)."""
    gemm = q.qlinear_supergroup_a8 if a8 else q.qlinear_supergroup
    B, N, Kc = args.batch, 3072, 1024
    COPIES = 1024                            # 1 GB of weights rotated, 4x the last-level cache
    gen = torch.Generator(device="cuda")
    gen.manual_seed(97)
    mats = []
    for _ in range(COPIES):
        w = torch.randn((N, Kc), generator=gen, device="cuda") * 0.02
        mats.append(q.quantize_supergroup(w, 4))
    del w
    K, W = args.steps, args.warmup
    xs = torch.randn((16, B, Kc), generator=gen, device="cuda").half()
    ys = torch.empty((16, B, N), dtype=torch.float16, device="cuda")

    def run(lo, hi):
        def f():
            for i in range(lo, hi):
                gemm(xs[i % 16], mats[i % COPIES], out=ys[i % 16])
        return f
    if W:
        graph_of(torch, run(K, K + W)).replay()
    g = graph_of(torch, run(0, K))
    ms = time_graph(torch, g, flush=CacheFlush(torch))
    us = ms / K * 1e3
    wbytes = sg_bytes(N, Kc)
    bytes_ = wbytes + B * Kc * 2 + B * N * 2
    flops = 2 * B * N * Kc
    ach = bytes_ / (us * 1e-6) / 1e9
    mfma_peak = INT8_MFMA_PEAK_TOPS if a8 else FP16_MFMA_PEAK_TFLOPS
    name = "k_sg_a8" if a8 else "k_sg"
    res = {"metric": f"super-group GEMM{' (8-bit activations)' if a8 else ''} tokens/s (B={B})",
           "value": B * K / (ms * 1e-3),
           "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms / K,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "i8/i32" if a8 else "f16", "data": "synthetic",
           "config": {"workload": f"{'qlinear_supergroup_a8' if a8 else 'qlinear_supergroup'} W[3072x1024] "
                                  f"(1 in 4 channels 4-bit, 3 ternary), x[{B}x1024], {COPIES} weight "
                                  f"copies rotated", "global_batch": B,
                      "tflops": flops / (us * 1e-6) / 1e12},
           "roofline": {"kernel": f"{name}_gemv" if B <= 8 else f"{name}_mfma", "bound": "hbm",
                        "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": ach / HBM_PEAK_GBS,
                        "traffic": measured_traffic(f"supergroup{'_a8' if a8 else ''}_b{B}/{name}"),
                        "bytes_per_launch": bytes_,
                        "us_per_launch": us, "mfma_tflops": flops / (us * 1e-6) / 1e12,
                        "mfma_frac": flops / (us * 1e-6) / 1e12 / mfma_peak}}
    return res, (lambda: cpu_baseline_supergroup(B, a8=a8))


def _threads():
    from threadpoolctl import threadpool_info
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return int(max(blas) if blas else 1)


def cpu_baseline_gemv(group=64, bf16=False, budget_s=10.0):
    """The oracle (float64 numpy) on a bounded sample: int4 linears x[1x2048] W[512x2048] of one
    seeded weight, repeated until the budget is spent."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import synth
    from oracle import affine, moe

    w = synth.normal_f32((512, 2048), synth.WEIGHT_SIGMA, synth.Workload.GEMV, 0, synth.Role.DENSE)
    W_ = affine.quantize(w, 4, group, "bf16" if bf16 else "f16")
    x = synth.activations(1, 2048, synth.Workload.GEMV)
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < budget_s:
        moe.to_f16(moe.qlinear(x, W_))
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "calls/s", "cores": _threads(), "kind": "oracle", "host": host_desc(),
            "sample": f"{n} calls of x[1x2048] W[512x2048] int4 g{group}, float64 numpy, {dt:.1f} s"}


def cpu_baseline_prerouter(budget_s=10.0):
    """The oracle on a bounded sample: prerouter head forwards of one token (hidden 2048, 256
    experts, head width 512, top-4) with one seeded head."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np
    import synth
    from oracle import moe
    from oracle import prerouter as pr

    D, E, F, k = 2048, 256, 512, 4
    R_ = synth.Role.MISC
    W_ = synth.Workload.TEST
    n_in = D + 2 * E
    P = pr.PrerouterHead(synth.normal_f16((E, n_in), 0.02, W_, 0, R_, 0), synth.normal_f16((E,), 0.02, W_, 0, R_, 1),
                         synth.normal_f16((F, n_in), 0.02, W_, 0, R_, 2), synth.normal_f16((F,), 0.02, W_, 0, R_, 3),
                         synth.normal_f16((E, F), 0.05, W_, 0, R_, 4), synth.normal_f16((E,), 0.02, W_, 0, R_, 5))
    h = synth.activations(1, D, W_, 0)
    g = np.random.default_rng(0)
    now, prev = g.choice(E, (1, k), replace=False), g.choice(E, (1, k), replace=False)
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < budget_s:
        _, lg = pr.forward(P, h, now, prev)
        moe.topk(lg.astype(np.float64), k)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "calls/s", "cores": _threads(), "kind": "oracle", "host": host_desc(),
            "sample": f"{n} one-token head forwards + top-4, float64 numpy, {dt:.1f} s"}


def bench_gemv(args, q, torch):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    N, Kc, COPIES = 512, 2048, 2048      # 2048 weight copies = 1.2 GB > 4x the 256 MB cache
    G, bf = args.group, args.params == "bf16"
    w = torch.randn((COPIES * N, Kc), generator=gen, device="cuda") * 0.02
    big = q.quantize_affine(w, 4, group=G)
    del w
    if bf:   # the port page's format: bf16 parameters (here the fp16 ones re-rounded to bf16)
        big.scales = big.scales.float().to(torch.bfloat16).view(torch.int16)
        big.biases = big.biases.float().to(torch.bfloat16).view(torch.int16)
    mats = []
    for c in range(COPIES):
        m = q.QWeight(big.packed[c * N:(c + 1) * N], big.scales[c * N:(c + 1) * N],
                      big.biases[c * N:(c + 1) * N], 4, N, Kc, 1, G,
                      q.PARAM_BF16 if bf else q.PARAM_F16)
        mats.append(m)
    K, W = args.steps, args.warmup
    xs = torch.randn((K + W, 1, Kc), generator=gen, device="cuda").half()
    ys = torch.empty((K + W, 1, N), dtype=torch.float16, device="cuda")

    def run(lo, hi):
        def f():
            for i in range(lo, hi):
                q.qlinear_int4(xs[i], mats[i % COPIES], out=ys[i])
        return f
    if W:
        graph_of(torch, run(K, K + W)).replay()
    g = graph_of(torch, run(0, K))
    ms = time_graph(torch, g, flush=CacheFlush(torch))
    bytes_ = N * Kc // 2 + 2 * (N * (Kc // G) * 2) + Kc * 2 + N * 2
    ach = bytes_ / (ms / K * 1e-3) / 1e9
    fmt = f"int4 g{G}{' bf16 parameters' if bf else ''}"
    res = {"metric": "int4 linear GEMV calls/s (decode)", "value": K / (ms * 1e-3),
           "unit": "calls/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms / K,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic",
           "config": {"workload": f"qlinear_int4 x[1x2048] W[512x2048] {fmt}, 2048 weight copies rotated"},
           "roofline": {"kernel": f"k_qgemv_fast<4,{G},{'bf16' if bf else 'f16'}>", "bound": "hbm", "achieved": ach,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                        "traffic": measured_traffic(f"gemv_g{G}{'_bf16' if bf else ''}/k_qgemv_fast"),
                        "bytes_per_launch": bytes_, "us_per_launch": ms / K * 1e3}}
    return res, (lambda: cpu_baseline_gemv(G, bf))


def bench_prerouter(args, q, torch):
    """One prerouter head forward per decode token (hidden 2048, 256 experts, head width 512,
    top-4), rotating over 128 independently drawn heads (540 MB, twice the 256 MB cache)."""
    D, E, F, k, HEADS = 2048, 256, 512, 4, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    n = D + 2 * E
    rnd = lambda *s: (torch.randn(s, generator=gen, device="cuda") * 0.02).half()
    heads = [q.PrerouterHead(rnd(E, n), rnd(E), rnd(F, n), rnd(F), rnd(E, F), rnd(E)) for _ in range(HEADS)]
    K, W = args.steps, args.warmup
    hs = torch.randn((K + W, 1, D), generator=gen, device="cuda").half()
    rt = torch.stack([torch.randperm(E, generator=gen, device="cuda")[:2 * k] for _ in range(K + W)]).int()
    now, prev = rt[:, None, :k].contiguous(), rt[:, None, k:].contiguous()
    cs = [heads[i % HEADS].c() for i in range(HEADS)]
    act = torch.empty((K + W, 1, F), dtype=torch.float16, device="cuda")
    logits = torch.empty((K + W, 1, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((K + W, 1, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((K + W, 1, k), dtype=torch.float32, device="cuda")
    import ctypes
    from int4_group_quantized_amd._lib import check

    def run(lo, hi):
        def f():
            st = torch.cuda.current_stream().cuda_stream
            for i in range(lo, hi):
                check(q.lib.prerouter_forward(ctypes.byref(cs[i % HEADS]), hs[i].data_ptr(), 1, k,
                                              now[i].data_ptr(), prev[i].data_ptr(), act[i].data_ptr(),
                                              logits[i].data_ptr(), idx[i].data_ptr(), wts[i].data_ptr(),
                                              st), "prerouter_forward")
        return f
    if W:
        graph_of(torch, run(K, K + W)).replay()
    g = graph_of(torch, run(0, K))
    ms = time_graph(torch, g, flush=CacheFlush(torch))
    us = ms / K * 1e3
    # algorithmic bytes: the dense parts of the fc1 and linear_init rows, the 2k gathered
    # one-hot columns of each, fc2, the biases, h in, act out and in, logits out and in, the
    # routing in and out
    bytes_ = ((F + E) * D * 2 + (F + E) * 2 * k * 2 + E * F * 2 + (F + 2 * E) * 2 + D * 2
              + 2 * F * 2 + 3 * E * 4 + 2 * k * 4 + 2 * k * 4)
    ach = bytes_ / (us * 1e-6) / 1e9
    res = {"metric": "prerouter head forwards/s (decode, 1 token)", "value": K / (ms * 1e-3),
           "unit": "calls/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms / K,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic",
           "config": {"workload": f"prerouter_forward h[1x{D}], {E} experts, head width {F}, top-{k}, "
                                  f"{HEADS} heads rotated"},
           "roofline": {"kernel": "whole call (k_pr_fc1, k_pr_fc2, k_router_topk)", "bound": "hbm",
                        "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic("prerouter/call"),
                        "bytes_per_launch": bytes_, "us_per_launch": us}}
    return res, cpu_baseline_prerouter


WORKLOADS = {"moe_decode": bench_moe_decode, "moe_decode_routed": bench_moe_decode_routed,
             "moe_prefill": bench_moe_prefill,
             "moe_stack": bench_moe_stack, "supergroup": bench_supergroup,
             "supergroup_a8": lambda args, q, torch: bench_supergroup(args, q, torch, a8=True),
             "gemv": bench_gemv, "prerouter": bench_prerouter}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="moe_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--skew", action="store_true", help="moe_prefill: +2.0 on experts 0..15")
    ap.add_argument("--batch", type=int, default=1, choices=(1, 64), help="supergroup: inputs per call")
    ap.add_argument("--group", type=int, default=64, choices=(32, 64), help="gemv: inputs per group")
    ap.add_argument("--params", default="f16", choices=("f16", "bf16"), help="gemv: scale/bias type")
    ap.add_argument("--tokens", type=int, default=512,
                    help="moe_prefill: tokens per step (512 is the workload; others are a sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note, not built)"}))
        sys.exit(2)
    import torch
    import int4_group_quantized_amd as q
    if not torch.cuda.is_available():
        raise SystemExit("no ROCm GPU visible")
    res, cpu_fn = WORKLOADS[args.workload](args, q, torch)
    if cpu_fn is not None and not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_fn()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
