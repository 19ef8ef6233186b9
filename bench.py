"""Benchmark of the routed-expert hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--activation swiglu|situ]

A step is one pass of the whole path over one batch: the router (when the workload has one)
and the expert forward (sort, fused W1/W3 + SwiGLU (or SiTU-GLU with --activation situ), W2,
combine); with a router both run as one k3x_route_moe_forward call.  The default workload is
one decode token through one layer of 896 experts with the router (E = 896, H = 3584,
I = 3072, top-16).  Inputs are synthetic and seeded (k3x_synth); pools are generated in
device memory and resident before timing.  Successive steps rotate over 64 different
tokens, so each step reads a different set of 16 experts and the 256 MB Infinity Cache
cannot serve them from a previous step.  `--workload chain12_t1_e896` runs one decode token
through 12 layers of 896 experts, all resident (about 188 GB): RMSNorm, router, experts and
residual add per layer, one graph per starting token.

Two helper modes support `roofline.traffic` (HBM bytes from rocprofv3 counters):
    python bench.py --copy-probe                 # a plain device copy of 1 GiB, run under
                                                 # rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE)
    python bench.py --traffic-from F W CF CW     # counter CSVs of the workload (F, W) and of
                                                 # the copy (CF, CW) -> profiles/traffic_<workload>.txt
The copy's readings give the scale of each counter (bytes moved / bytes counted); the
summary records the hash of the kernel sources, and a normal run reports the traffic only
while those sources are unchanged.  Two more turn profiler output into the summaries kept
with the code:
    python bench.py --workload W --stats-from STATS_CSV --profile-cmd "..."
        # rocprofv3 --kernel-trace --stats -> profiles/kernel_trace_<W>.md
    python bench.py --workload W --counters-from PASS1_CSV PASS2_CSV ... --profile-cmd "..."
        # rocprofv3 --pmc passes -> profiles/counters_<W>.txt (MFMA use, LDS conflicts, waits)

Prints ONE JSON line.  The timed region replays HIP graphs that run the rotated batches one
after another (a graph of min(steps, 64) batches, replayed steps // that many times, then a
graph of the remainder; every replay checked bit for bit against the eager results first),
so `value` and `ms_per_step` are the path's throughput without host launch gaps, as when the
layers of a model run inside one graph, for any --steps; `path.timed_mode` says how the steps
were split, and `path.ms_per_step_one_graph_per_step` is the same steps with one graph per
step (each graph launch adds a gap of several microseconds).  Kernel durations for the
roofline come from HIP events the library records around each of its launches
(k3x_profiler_*) in a second timed pass over the same steps, launched eagerly.

The default run (decode_t1_e896_router) also measures the 4096-token prefill
(prefill_t4096_e896: 896 experts, uniform routing, no router) and reports it in the same line
under "prefill", with its TFLOP/s against the bf16 MFMA peak (--no-prefill skips it) and,
as context, the TFLOP/s of the same FLOPs as two dense bf16 torch.matmul GEMMs on this GPU
("dense_bf16_reference"; `--dense-reference` runs only that), and a
decode batch of 32 tokens through the router with Zipf-skewed expert popularity
(decode_t32_e896_zipf) under "decode_batch" (--no-batch skips it).
`cpu_baseline` is the oracle on this host: the median of 3 runs on all of its threads
(`value`, `cores`) and of 3 on one thread (`value_1core`), with the CPU model.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode), TFLOP/s (prefill)"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
ROTATE = 64
TIMED_REGION = ("HIP graph replay: one graph runs the rotated batches in order, as a model's "
                "layers run inside one graph")
DEFAULT_WORKLOAD = "decode_t1_e896_router"
PREFILL_WORKLOAD = "prefill_t4096_e896"
BATCH_WORKLOAD = "decode_t32_e896_zipf"
ORACLE_ACT = {"swiglu": "swiglu", "situ": ("situ", 4.0, 25.0)}
COPY_PROBE_BYTES = 1 << 30
# the kernel sources of the routed path, with the headers they include
KERNEL_SOURCES = ("k3x_internal.h", "k3x_select.h", "k3x_decode.hip", "k3x_moe.hip", "k3x_prefill.hip",
                  "k3x_router.hip")
LATENT_SOURCES = KERNEL_SOURCES + ("k3x_dense.hip",)
# rocprofv3 kernel names of the library's launch names
KERNEL_SYMBOLS = {"w13_decode": "decode_w13", "w2_combine_decode": "decode_w2_combine",
                  "moe_combine": "moe_combine",
                  "w13_prefill": "gemm_prefill<true>", "w2_prefill": "gemm_prefill<false>",
                  "w13_grouped": "gemm_decode<true>", "w2_grouped": "gemm_decode<false>",
                  "route_scores": "route_scores", "route_select": "route_select",
                  "latent_in": "latent_in", "latent_out": "latent_out",
                  "w13_contract": "contract_rows<true>", "w2_contract": "contract_rows<false>"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_tensor_bytes(H, I):
    w13 = 2 * (I * H // 2 + I * H // 32)
    w2 = H * I // 2 + H * I // 32
    return w13, w2


def per_kernel_work(name, H, I, E, T, topk, U):
    """Algorithmic (bytes, flops) of one launch: U distinct experts, T tokens, T*topk slots."""
    w13, w2 = expert_tensor_bytes(H, I)
    slots = T * topk
    if name in ("w13_decode", "w13_grouped", "w13_prefill"):
        return U * w13 + T * H * 2 + slots * I * 2, slots * 4.0 * I * H
    if name == "w13_contract":  # h kept in fp32
        return U * w13 + T * H * 2 + slots * I * 4, slots * 4.0 * I * H
    if name == "w2_contract":
        return U * w2 + slots * I * 4 + slots * H * 4, slots * 2.0 * H * I
    if name == "combine_contract":
        return slots * H * 4 + T * H * 4 + slots * 8, 2.0 * slots * H
    if name in ("w2_grouped", "w2_prefill"):
        return U * w2 + slots * I * 2 + slots * H * 4, slots * 2.0 * H * I
    if name == "w2_combine_decode":
        return (U * w2 + slots * I * 2 + slots * 8 + T * H * 4,
                slots * 2.0 * H * I + 2.0 * slots * H)
    if name == "route_scores":
        return E * H * 2 + T * H * 2 + T * E * 4, 2.0 * T * E * H
    if name == "route_select":
        return T * E * 4 + E * 4 + T * topk * 8, 0.0
    if name == "moe_combine":
        return slots * H * 4 + T * H * 4 + slots * 8, 2.0 * slots * H
    if name == "moe_sort":
        return slots * 4 * 2, 0.0
    if name in ("sort_count", "sort_scatter"):
        return slots * 4 * (1 if name == "sort_count" else 3), 0.0
    if name == "sort_scan":
        return 64 * E * 4 * 2, 0.0
    if name == "rmsnorm_bf16":
        return T * H * 4, 3.0 * T * H
    if name == "residual_add_bf16":
        return T * H * 8, 1.0 * T * H
    if name == "residual_rmsnorm_bf16":
        return T * H * 10, 4.0 * T * H
    return 0, 0.0


def latent_kernel_work(name, sh, T):
    """Algorithmic (bytes, flops) of one launch of the latent block's dense kernels (sh: a
    k3x_synth.LatentShape), T tokens in the launch."""
    D, L, Sx = sh.D, sh.L, sh.S
    E = sh.E
    if name == "latent_in":  # router, down, sh1, sh3 rows; x in; scores, z, s out
        return ((E + L + 2 * Sx) * D * 2 + T * D * 2 + T * (E * 4 + L * 2 + Sx * 2),
                2.0 * T * D * (E + L + 2 * Sx))
    if name == "latent_out":  # up, sh2 rows; acc, s, norm weight in; out (fp32)
        return (D * (L + Sx) * 2 + T * (L * 4 + Sx * 2) + L * 4 + T * D * 4,
                2.0 * T * D * (L + Sx))
    return per_kernel_work(name, L, sh.I, sh.E, T, sh.topk, min(sh.E, T * sh.topk))


def graph_timing(torch, step, R, outs, eager, steps, warmup):
    """Times `steps` steps inside HIP graphs, the way a model's layers run back to back inside
    one graph.  The sequence graph runs Rs = min(steps, R) rotated batches in order; the timed
    region replays it steps // Rs times, then a graph of the first steps % Rs batches, so
    every timed step runs inside a multi-step graph whatever `steps` is.  Also captures one
    graph per batch and times the same steps with one graph launch per step.  Every replay
    is first checked bit for bit against the eager outputs (each output overwritten before,
    eager steps between replays).  outs(r) gives the output tensors of batch r, eager[r]
    their eager values.  Returns (wall seconds in the sequence mode, wall seconds with one
    graph per step, a description of the sequence mode)."""
    Rs = max(1, min(steps, R))
    rem = steps % Rs
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    singles = []
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        singles.append(g)

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(n):
                step(r)
        return g

    seq = capture(Rs)
    tail = capture(rem) if rem else None

    def spoil(r):
        for o in outs(r):
            o.fill_(-1)

    def check(what, r):
        if not all(torch.equal(o, e) for o, e in zip(outs(r), eager[r])):
            sys.exit(f"{what} differs from the eager result at batch {r}")

    for r in range(R):
        spoil(r)
        singles[r].replay()
        torch.cuda.synchronize()
        check("graph replay", r)
        step((r + 1) % R)
        torch.cuda.synchronize()
    for what, g, n in (("sequence graph", seq, Rs), ("tail graph", tail, rem)):
        if g is None:
            continue
        for rep_ in range(2):
            for r in range(n):
                spoil(r)
            g.replay()
            torch.cuda.synchronize()
            for r in range(n):
                check(f"{what} replay {rep_}", r)
            step((rep_ + 1) % R)
            torch.cuda.synchronize()

    def run(n, use_seq):
        if use_seq:
            for _ in range(n // Rs):
                seq.replay()
            if n % Rs:
                # the timed run ends with the tail graph; a warm-up remainder replays singles
                if n % Rs == rem and tail is not None:
                    tail.replay()
                else:
                    for j in range(n % Rs):
                        singles[j].replay()
        else:
            for j in range(n):
                singles[j % R].replay()

    walls = []
    for use_seq in (True, False):
        run(warmup, use_seq)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(steps, use_seq)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    mode = f"{steps // Rs} replay(s) of one graph of {Rs} rotated batch(es) in order"
    if rem:
        mode += f", then one graph of the first {rem}"
    return walls[0], walls[1], mode


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and its CPU counts."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def timed_oracle(run, n_all, n_one, units, unit, runs=3):
    """Times run(n) -> oracle seconds for the first n items of a sample: the median of `runs`
    runs over n_all items on all of the oracle's threads, then over n_one items on one
    thread.  units(n) is the work of n items in the unit of the rate."""
    import oracle

    threads = oracle.threads()
    all_t = [run(n_all) for _ in range(runs)]
    oracle.set_threads(1)
    try:
        one_t = [run(n_one) for _ in range(runs)]
    finally:
        oracle.set_threads(threads)
    med_all, med_one = float(np.median(all_t)), float(np.median(one_t))
    return {"value": units(n_all) / med_all, "unit": unit, "cores": threads,
            "value_1core": units(n_one) / med_one, "runs": runs,
            "seconds_all_cores": [round(v, 3) for v in all_t],
            "seconds_1core": [round(v, 3) for v in one_t],
            **host_cpu()}


def cpu_baseline(w, x, W, b, dev_idx, dev_gates, pool_dev, act="swiglu", seconds=3.0):
    """The oracle as it stands, on this host's cores, over a bounded sample of the same
    workload's tokens (each: the router when the workload has one, the token's experts, the
    slot-order combine).  Each token's expert bytes are copied from the generator's device
    pool (k3x_synth writes the same bytes on the device and the host) outside the timing.
    Median of three runs on all of the oracle's threads and three on one thread, each about
    `seconds` of oracle time."""
    import k3x_synth as S
    import oracle

    toks = []

    def token(i):
        while len(toks) <= i:
            t = len(toks) % len(x)
            xt = x[t:t + 1]
            if w.router:
                idx, gates = oracle.route(xt, W, b, w.topk)
            else:
                idx, gates = dev_idx[t:t + 1], dev_gates[t:t + 1]
            exps = [S.ExpertBytes(*[pool_dev[nm][int(e)].cpu().numpy() for nm in S.TENSOR_NAMES])
                    for e in idx[0]]
            toks.append((xt, gates, exps))
        return toks[i]

    def run(n):
        used = 0.0
        for i in range(n):
            xt, gates, exps = token(i)
            t0 = time.perf_counter()
            if w.router:
                _, gates = oracle.route(xt, W, b, w.topk)
            d = np.stack([oracle.expert_forward(xt[0], ex, act=act) for ex in exps])[None]
            oracle.combine(gates, d)
            used += time.perf_counter() - t0
        return used

    one = run(1)  # calibration (also fetches the first token's experts)
    n_all = max(1, int(round(seconds / one)))
    n_one = max(1, int(round(seconds / (one * oracle.threads()))))
    res = timed_oracle(run, n_all, n_one, lambda n: n, "tokens/s")
    res["kind"] = "oracle"
    res["sample"] = (f"the first {n_all} token(s) of the workload on all threads, {n_one} on one "
                     f"({'router + ' if w.router else ''}{w.topk} experts each + combine), median "
                     f"of 3 runs each; expert bytes copied to the host outside the timing")
    return res


def prefill_cpu_baseline(w, x, idx, gates, pool_dev, act="swiglu", seconds=3.0):
    """The oracle on a prefill batch, walking the experts one by one as a prefill does (each
    expert applied to every slot routed to it, oracle.expert_forward_many): a bounded sample
    of the experts in ascending order, timed as tokens/s = slots / topk per second (the
    slot-order combine, about 0.01 % of the work, is not in the sample).  Expert bytes are
    copied from the device pool outside the timing.  Median of three runs on all threads
    and three on one thread."""
    import k3x_synth as S
    import oracle

    k = idx.shape[1]
    flat = idx.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    experts, starts = np.unique(flat[order], return_index=True)
    bounds = list(starts) + [len(order)]
    cache = {}

    def expert(i):
        if i not in cache:
            e = int(experts[i])
            cache[i] = S.ExpertBytes(*[pool_dev[nm][e].cpu().numpy() for nm in S.TENSOR_NAMES])
        return cache[i]

    def run(n):
        used = 0.0
        for i in range(n):
            ex = expert(i)
            sl = order[bounds[i]:bounds[i + 1]]
            xs_ = x[sl // k]
            t0 = time.perf_counter()
            oracle.expert_forward_many(xs_, ex, act=act)
            used += time.perf_counter() - t0
        return used

    def tokens(n):
        return (bounds[n] - bounds[0]) / k

    one = run(1)
    n_all = max(1, min(len(experts), int(round(seconds / one))))
    n_one = max(1, min(len(experts), int(round(seconds / (one * oracle.threads())))))
    res = timed_oracle(run, n_all, n_one, tokens, "tokens/s")
    res["kind"] = "oracle"
    res["sample"] = (f"the first {n_all} of the batch's {len(experts)} experts with all their "
                     f"slots ({bounds[n_all]} slots = {tokens(n_all):.1f} tokens' worth) on all "
                     f"threads, {n_one} expert(s) on one, expert-major, median of 3 runs each; "
                     f"expert bytes copied to the host outside the timing")
    return res


def chain_cpu_baseline(w, x, layers, budget_s=12.0, act="swiglu"):
    """The oracle through the chained layers (RMSNorm, router, 16 experts, combine, residual)
    for a bounded sample of starting tokens, on this host's cores.  Expert bytes are copied
    from the device pools outside the timing."""
    import k3x_synth as S
    import oracle

    n_tok, t_used, i = 0, 0.0, 0
    while t_used < budget_s:
        xt = x[i % len(x):i % len(x) + 1].copy()
        i += 1
        for lay in layers:
            t0 = time.perf_counter()
            xn = oracle.rmsnorm_bf16(xt, 1e-6)
            idx, gates = oracle.route(xn, lay["W"], lay["b"], w.topk)
            t_used += time.perf_counter() - t0
            exps = [S.ExpertBytes(*[lay["pool"][nm][int(e)].cpu().numpy() for nm in S.TENSOR_NAMES])
                    for e in idx[0]]
            t0 = time.perf_counter()
            d = np.stack([oracle.expert_forward(xn[0], ex, act=act) for ex in exps])[None]
            y = oracle.combine(gates, d)
            xt = oracle.residual_add_bf16(xt, y)
            t_used += time.perf_counter() - t0
        n_tok += 1
    return {
        "value": n_tok / t_used,
        "unit": "tokens/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{n_tok} token(s) through {len(layers)} layers (RMSNorm + router + {w.topk} "
                  f"experts + combine + residual each), {t_used:.1f} s of oracle time; expert "
                  f"bytes copied to the host outside the timing",
    }


def bench_chain(w, args, torch, S, k3x):
    """One decode token through w.layers MoE layers, every layer's experts resident in HBM:
    RMSNorm -> router -> experts -> residual add per layer, one HIP graph per starting token.
    Each layer is one k3x_residual_route_moe_forward call (the previous layer's residual
    update and this layer's RMSNorm run inside the router's scores launch)."""
    steps = args.steps if args.steps is not None else 50
    warmup = args.warmup if args.warmup is not None else 5
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    free, _ = torch.cuda.mem_get_info(dev)
    need = w.layers * w.E * S.expert_bytes_per_expert(w.H, w.I)
    if free < need + (2 << 30):
        sys.exit(f"the chained workload needs {need / 1e9:.1f} GB of device memory, "
                 f"{free / 1e9:.1f} GB free")
    log(f"generating {w.layers} layers: E={w.E} H={w.H} I={w.I} ({need / 1e9:.1f} GB)")
    layers = []
    for layer in range(w.layers):
        pool_dev = S.device_pool(w.seed, layer, w.E, w.H, w.I)
        W, b = S.router_inputs(w, layer)
        Wd = torch.from_numpy(W.view(np.int16)).to(dev)
        bd = torch.from_numpy(b).to(dev)
        layers.append({"pool_dev": pool_dev, "W": W, "b": b, "Wd": Wd, "bd": bd,
                       "pool": k3x.k3x_expert_pool_create(pool_dev, hidden=w.H, inter=w.I,
                                                          n_experts=w.E,
                                                          activation=args.activation),
                       "rdesc": k3x.router_desc(Wd, bd, w.topk)})
    R = ROTATE
    x = S.normal_bf16(w.seed, S.P_X, 0, (R, w.H))
    xs = [torch.from_numpy(x[r:r + 1].view(np.int16)).to(dev) for r in range(R)]
    # the residual stream takes turns between two buffers (a layer's update must not write
    # the x it reads); y is both the previous layer's output and this layer's
    xbuf = [torch.empty((1, w.H), dtype=torch.int16, device=dev) for _ in range(2)]
    xn = torch.empty_like(xbuf[0])
    idx = torch.empty((1, w.topk), dtype=torch.int32, device=dev)
    gates = torch.empty((1, w.topk), dtype=torch.float32, device=dev)
    y = torch.empty((1, w.H), dtype=torch.float32, device=dev)
    ws = k3x.alloc_workspace(
        k3x.k3x_route_moe_workspace_size(layers[0]["rdesc"], layers[0]["pool"], 1), dev)

    def step(r):
        x_cur = xs[r]
        for li, lay in enumerate(layers):
            x_next = xbuf[0] if x_cur is not xbuf[0] else xbuf[1]
            k3x.k3x_residual_route_moe_forward(lay["rdesc"], lay["pool"], x_cur,
                                               y if li else None, 1e-6,
                                               x_next if li else None, xn, 1, idx, gates, y, ws)
            if li:
                x_cur = x_next
        k3x.k3x_residual_add_bf16(x_cur, y, 1, w.H)
        return x_cur

    out_eager = []
    for r in range(R):
        xb = step(r)
        torch.cuda.synchronize()
        out_eager.append(xb.clone())
    if k3x.k3x_fetch_drops(ws):
        sys.exit("run invalid: dropped slots")
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    for r in range(R):
        graphs[r].replay()
        torch.cuda.synchronize()
        if not torch.equal(xb, out_eager[r]):
            sys.exit(f"graph replay of token {r} differs from the eager result")
        step((r + 1) % R)
        torch.cuda.synchronize()

    for i in range(warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    prof = k3x.k3x_profiler_create(steps * w.layers * 8 + 16)
    torch.cuda.synchronize()
    k3x.k3x_profiler_attach(prof)
    for i in range(steps):
        step(i % R)
    torch.cuda.synchronize()
    k3x.k3x_profiler_attach(None)
    durs = k3x.profiler_durations(prof)
    k3x.k3x_profiler_destroy(prof)

    kernels = {}
    for name, ms in durs.items():
        nbytes, flops = per_kernel_work(name, w.H, w.I, w.E, 1, w.topk, w.topk)
        avg_s = float(np.mean(ms)) * 1e-3
        kernels[name] = {"launches": len(ms), "avg_us": round(avg_s * 1e6, 3),
                         "alg_bytes": int(nbytes), "gbps": round(nbytes / avg_s / 1e9, 1),
                         "tflops": round(flops / avg_s / 1e12, 2)}
    dominant = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches"])
    dk = kernels[dominant]
    traffic = traffic_for(w.name, dominant)
    roof = {"bound": "hbm", "achieved": dk["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(dk["gbps"] / PEAK_HBM_GBS, 4),
            "traffic": int(traffic) if traffic is not None else None, "kernel": dominant,
            "alg_bytes": dk["alg_bytes"]}
    w13, w2 = expert_tensor_bytes(w.H, w.I)
    layer_bytes = w.topk * (w13 + w2) + w.E * w.H * 2 + w.E * 4 + w.H * (2 + 4)
    path_bytes = w.layers * layer_bytes
    ksum = sum(k["avg_us"] * k["launches"] for k in kernels.values()) / steps * 1e-6
    out = {
        "metric": METRIC,
        "value": round(steps / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "activation": args.activation, "tokens": 1,
                   "layers": w.layers, "experts": w.E,
                   "hidden": w.H, "inter": w.I, "topk": w.topk, "router": True,
                   "zipf_bias": w.zipf, "weights": "mxfp4 (e2m1 + e8m0 per 32)",
                   "resident_expert_gb": round(need / 1e9, 1), "rotated_batches": R},
        "roofline": roof,
        "path": {"kernel_sum_us": round(ksum * 1e6, 3),
                 "alg_bytes_per_step": int(path_bytes),
                 "hbm_gbps_kernel_sum": round(path_bytes / ksum / 1e9, 1),
                 "hbm_frac_kernel_sum": round(path_bytes / ksum / 1e9 / PEAK_HBM_GBS, 4),
                 "hbm_gbps_wall": round(path_bytes / (wall / steps) / 1e9, 1),
                 "timed_region": "HIP graph replay, one graph per starting token"},
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)")
        out["cpu_baseline"] = chain_cpu_baseline(
            w, x, [{"W": l_["W"], "b": l_["b"], "pool": l_["pool_dev"]} for l_ in layers],
            act=ORACLE_ACT[args.activation])
    print(json.dumps(out), flush=True)


LATENT_WORKLOADS = {"latent_t1_e896": 1, "latent_t8_e896": 8}
# expert arena: (layers, slots) -- one decode token through the chained layers, the experts in
# pinned host memory (about 36 GB can be pinned here: two layers, 31.4 GB), n slots in HBM
ARENA_WORKLOADS = {"arena_chain2_t1_e896_s512": (2, 512)}
PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def bench_arena(args, torch, S, k3x):
    """Decode tokens through L chained layers of 896 experts whose bytes live in pinned host
    memory (L * 15.7 GB), with an HBM arena of n slots: RMSNorm -> router -> arena expert
    forward (misses copied in from the host) -> residual per layer.  Every step is a fresh
    token (steady-state decode, no graph: the arena waits for each layer's routing)."""
    L, n_slots = ARENA_WORKLOADS[args.workload]
    w = S.WORKLOADS[5]  # the chained workload's shape, router and Zipf bias per layer
    H, I, E, k = w.H, w.I, w.E, w.topk
    steps = args.steps if args.steps is not None else 100
    warmup = args.warmup if args.warmup is not None else 50
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    log(f"backing store: {L} layers x {E} experts in pinned host memory "
        f"({L * E * S.expert_bytes_per_expert(H, I) / 1e9:.1f} GB); arena {n_slots} slots")
    host = {}
    for t, n in enumerate(S.TENSOR_NAMES):
        rows, cols = S.tensor_shape(t, H, I)
        host[n] = torch.empty((L * E, rows, cols), dtype=torch.uint8, pin_memory=True)
    layers = []
    for l in range(L):  # generated on the device, one layer at a time, then copied out
        pool_dev = S.device_pool(w.seed, l, E, H, I)
        for n in S.TENSOR_NAMES:
            host[n][l * E:(l + 1) * E].copy_(pool_dev[n])
        del pool_dev
        W, b = S.router_inputs(w, l)
        Wd = torch.from_numpy(W.view(np.int16)).to(dev)
        bd = torch.from_numpy(b).to(dev)
        layers.append({"W": W, "b": b, "rdesc": k3x.router_desc(Wd, bd, k), "keep": (Wd, bd)})
        log(f"layer {l} in the backing store")
    torch.cuda.synchronize()
    arena = k3x.k3x_arena_create(host, n_slots, L, E, H, I, max_slots_per_call=64)
    n_tok = warmup + steps
    x = S.normal_bf16(w.seed, S.P_X, 0, (n_tok, H))
    xb = torch.empty((1, H), dtype=torch.int16, device=dev)
    xn = torch.empty_like(xb)
    idx = torch.empty((1, k), dtype=torch.int32, device=dev)
    gates = torch.empty((1, k), dtype=torch.float32, device=dev)
    y = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = k3x.alloc_workspace(k3x.k3x_moe_workspace_size(arena.pool, 1, k), dev)
    rws = k3x.alloc_workspace(k3x.k3x_route_workspace_size(layers[0]["rdesc"], 1), dev)
    xs = torch.from_numpy(x.view(np.int16)).to(dev)
    idx_log = torch.empty((n_tok, L, k), dtype=torch.int32, device=dev)  # the routing trace

    def step(i):
        xb.copy_(xs[i:i + 1])
        k3x.k3x_rmsnorm_bf16(xb, 1, H, 1e-6, xn)
        for li, lay in enumerate(layers):
            k3x.k3x_route_topk(lay["rdesc"], xn, 1, idx, gates, rws)
            k3x.k3x_arena_moe_forward(arena, li, xn, 1, idx, gates, k, y, ws)
            idx_log[i, li].copy_(idx[0])
            if li + 1 < L:
                k3x.k3x_residual_add_rmsnorm_bf16(xb, y, 1, H, 1e-6, xn)
            else:
                k3x.k3x_residual_add_bf16(xb, y, 1, H)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    h0, m0, b0 = k3x.k3x_arena_stats(arena)
    t0 = time.perf_counter()
    for i in range(warmup, n_tok):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    h1, m1, b1 = k3x.k3x_arena_stats(arena)
    if k3x.k3x_fetch_drops(ws):
        sys.exit("run invalid: dropped slots")

    # kernel times of a few more steps, event-timed
    prof = k3x.k3x_profiler_create(20 * L * 8 + 16)
    k3x.k3x_profiler_attach(prof)
    for i in range(min(20, n_tok)):
        step(i)
    torch.cuda.synchronize()
    k3x.k3x_profiler_attach(None)
    durs = k3x.profiler_durations(prof)
    k3x.k3x_profiler_destroy(prof)
    kernels = {}
    for name, ms in durs.items():
        nbytes, flops = per_kernel_work(name, H, I, E, 1, k, k)
        avg_s = float(np.mean(ms)) * 1e-3
        kernels[name] = {"launches": len(ms), "avg_us": round(avg_s * 1e6, 3),
                         "alg_bytes": int(nbytes), "gbps": round(nbytes / avg_s / 1e9, 1)}
    dk = kernels["w13_decode"]
    traffic = traffic_for("decode_t1_e896_router", "w13_decode")
    roof = {"bound": "hbm", "achieved": dk["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(dk["gbps"] / PEAK_HBM_GBS, 4),
            "traffic": int(traffic) if traffic is not None else None, "kernel": "w13_decode",
            "alg_bytes": dk["alg_bytes"]}
    # sizing by trace replay: the recorded routing of the timed steps, keys layer * E + expert
    log_np = idx_log.cpu().numpy()[warmup:warmup + steps]
    tr = [int(li * E + e) for row in log_np for li in range(L) for e in row[li]]
    counts = np.bincount(np.asarray(tr, dtype=np.int64), minlength=L * E)
    by_count = np.lexsort((np.arange(L * E), -counts))  # most requested first, ties by key
    sizes = sorted({128, 256, n_slots, 1024, 1536})
    replay = {}
    for cap in sizes:
        pins = [int(v) for v in by_count[:cap // 2] if counts[v] > 0]
        replay[str(cap)] = {
            "lru": round(k3x.k3x_cache_replay(tr, cap, k3x.K3X_CACHE_LRU) / len(tr), 4),
            "belady": round(k3x.k3x_cache_replay(tr, cap, k3x.K3X_CACHE_BELADY) / len(tr), 4),
            "pin_lru": round(k3x.k3x_cache_replay(tr, cap, k3x.K3X_CACHE_PIN_LRU, pins) / len(tr), 4)}
    dh, dm, db = h1 - h0, m1 - m0, b1 - b0
    res = {
        "metric": METRIC,
        "value": round(steps / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": 1, "layers": L, "experts": E,
                   "hidden": H, "inter": I, "topk": k, "router": True, "zipf_bias": True,
                   "arena_slots": n_slots, "arena_gb": round(n_slots * k3x.k3x_expert_bytes(H, I) / 1e9, 1),
                   "backing_gb_pinned_host": round(L * E * k3x.k3x_expert_bytes(H, I) / 1e9, 1),
                   "timed_region": "eager: every layer waits for its routing on the host"},
        "roofline": roof,
        "arena": {"hit_rate": round(dh / max(dh + dm, 1), 4), "hits": dh, "misses": dm,
                  "h2d_bytes_per_token": int(db / steps),
                  "h2d_gbps": round(db / wall / 1e9, 2), "h2d_peak_gbps": PCIE_PEAK_GBS,
                  "replay_hit_rate_by_slots": replay,
                  "distinct_in_trace": len(set(tr)), "requests_in_trace": len(tr)},
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)")
        pools = [{n: host[n][l * E:(l + 1) * E] for n in S.TENSOR_NAMES} for l in range(L)]
        res["cpu_baseline"] = chain_cpu_baseline(
            w, x, [{"W": lay["W"], "b": lay["b"], "pool": pools[l]} for l, lay in enumerate(layers)])
    arena.close()
    print(json.dumps(res), flush=True)


def latent_cpu_baseline(sh, x, w, pool_dev, topk, budget_s=12.0):
    """The oracle's latent block, one token at a time, for a bounded sample of the rotated
    tokens, on this host's cores.  The bytes of the experts each token routes to are copied
    from the device pool outside the timing (the others stay untouched zero pages)."""
    import k3x_synth as S
    import oracle

    shapes = {n: tuple(pool_dev[n].shape) for n in S.TENSOR_NAMES}
    n_tok, t_used, i = 0, 0.0, 0
    while t_used < budget_s:
        xt = x[i % len(x):i % len(x) + 1].copy()
        i += 1
        idx, _ = oracle.route(xt, w["Wr"], w["bias"], topk)
        host = {n: np.zeros(shapes[n], dtype=np.uint8) for n in S.TENSOR_NAMES}
        for e in set(int(v) for v in idx.ravel()):
            for n in S.TENSOR_NAMES:
                host[n][e] = pool_dev[n][e].cpu().numpy()
        t0 = time.perf_counter()
        oracle.latent_block(xt, w["Wr"], w["bias"], topk, w["down"], w["up"], w["sh1"],
                            w["sh3"], w["sh2"], w["norm_w"], 1e-6, host, act="swiglu",
                            act_shared=("situ", 4.0, 25.0))
        t_used += time.perf_counter() - t0
        n_tok += 1
    return {
        "value": n_tok / t_used,
        "unit": "tokens/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{n_tok} token(s) through the whole latent block (router on {sh.D}, down, "
                  f"{topk} of {sh.E} experts, latent RMSNorm, up, 2 shared experts), "
                  f"{t_used:.1f} s of oracle time; expert bytes copied to the host outside the "
                  f"timing",
    }


def bench_latent(args, torch, S, k3x):
    """The latent MoE block (router on the full width, down-projection, the routed experts
    on the latent, RMSNorm of the aggregate, up-projection, two shared experts) on T decode
    tokens, one HIP graph per rotated batch."""
    T = LATENT_WORKLOADS[args.workload]
    sh = S.LATENT_K3
    steps = args.steps if args.steps is not None else 4 * ROTATE
    warmup = args.warmup if args.warmup is not None else ROTATE
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    seed = S.LATENT_SEED
    log(f"generating the latent block: D={sh.D} L={sh.L} S={sh.S} E={sh.E} I={sh.I}")
    pool_dev = S.device_pool(seed, 0, sh.E, sh.L, sh.I)
    pool = k3x.k3x_expert_pool_create(pool_dev, hidden=sh.L, inter=sh.I, n_experts=sh.E)
    w = S.latent_inputs(seed, 0, sh.D, sh.L, sh.S, sh.E)
    dv = {n: torch.from_numpy(w[n].view(np.int16) if w[n].dtype == np.uint16 else w[n]).to(dev)
          for n in w}
    d = k3x.latent_desc(dv["down"], dv["up"], dv["sh1"], dv["sh3"], dv["sh2"], dv["norm_w"],
                        eps=1e-6, latent_norm=1, shared_activation="situ")
    r = k3x.router_desc(dv["Wr"], dv["bias"], sh.topk)
    R = ROTATE
    x = S.normal_bf16(seed, S.P_X, 0, (R * T, sh.D))
    xs = [torch.from_numpy(x[i * T:(i + 1) * T].view(np.int16)).to(dev) for i in range(R)]
    outs_ = [torch.empty((T, sh.D), dtype=torch.float32, device=dev) for _ in range(R)]
    ws = k3x.alloc_workspace(k3x.k3x_latent_workspace_size(d, pool, r, T), dev)
    moe_off = k3x.k3x_latent_ws_layout(d, pool, r, T)["moe"]

    def step(i):
        k3x.k3x_latent_forward(d, pool, r, xs[i], T, outs_[i], ws)

    eager = []
    for i in range(R):
        step(i)
        torch.cuda.synchronize()
        eager.append([outs_[i].clone()])
    if k3x.k3x_fetch_drops(ws[moe_off:]):
        sys.exit("run invalid: dropped slots")
    wall, wall_single, mode = graph_timing(torch, step, R, lambda i: (outs_[i],), eager, steps,
                                           warmup)

    prof = k3x.k3x_profiler_create(steps * 16 + 16)
    torch.cuda.synchronize()
    k3x.k3x_profiler_attach(prof)
    for i in range(steps):
        step(i % R)
    torch.cuda.synchronize()
    k3x.k3x_profiler_attach(None)
    durs = k3x.profiler_durations(prof)
    k3x.k3x_profiler_destroy(prof)

    kernels = {}
    for name, ms in durs.items():
        nbytes, flops = latent_kernel_work(name, sh, T)
        avg_s = float(np.mean(ms)) * 1e-3
        kernels[name] = {"launches": len(ms), "avg_us": round(avg_s * 1e6, 3),
                         "alg_bytes": int(nbytes), "gbps": round(nbytes / avg_s / 1e9, 1),
                         "tflops": round(flops / avg_s / 1e12, 2)}
    dominant = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches"])
    dk = kernels[dominant]
    traffic = traffic_for(args.workload, dominant)
    roof = {"bound": "hbm", "achieved": dk["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(dk["gbps"] / PEAK_HBM_GBS, 4),
            "traffic": int(traffic) if traffic is not None else None, "kernel": dominant,
            "alg_bytes": dk["alg_bytes"]}
    w13, w2 = expert_tensor_bytes(sh.L, sh.I)
    dense = (sh.L * sh.D * 2 + sh.S * sh.D * 2) * 2 + sh.E * sh.D * 2
    U = min(sh.E, T * sh.topk)
    path_bytes = dense + U * (w13 + w2)
    ksum = sum(k["avg_us"] * k["launches"] for k in kernels.values()) / steps * 1e-6
    res = {
        "metric": METRIC,
        "value": round(steps * T / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "hidden": sh.D, "latent": sh.L,
                   "shared_inter": sh.S, "experts": sh.E, "inter": sh.I, "topk": sh.topk,
                   "router": True, "routed_activation": "swiglu", "shared_activation": "situ",
                   "weights": "routed mxfp4 (e2m1 + e8m0 per 32), dense bf16",
                   "rotated_batches": R},
        "roofline": roof,
        "path": {"kernel_sum_us": round(ksum * 1e6, 3),
                 "alg_bytes_per_step": int(path_bytes),
                 "hbm_gbps_kernel_sum": round(path_bytes / ksum / 1e9, 1),
                 "hbm_frac_kernel_sum": round(path_bytes / ksum / 1e9 / PEAK_HBM_GBS, 4),
                 "hbm_gbps_wall": round(path_bytes / (wall / steps) / 1e9, 1),
                 "timed_region": TIMED_REGION, "timed_mode": mode,
                 "ms_per_step_one_graph_per_step": round(wall_single / steps * 1e3, 5)},
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)")
        res["cpu_baseline"] = latent_cpu_baseline(sh, x, w, pool_dev, sh.topk)
    print(json.dumps(res), flush=True)


def code_only(text):
    """C++ source text without its comments and blank space: what the compiler sees, so that
    editing a comment does not orphan counters taken on the same code."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_hash(workload=None, read=None):
    """Hash of the code of the kernel sources a workload runs (the routed path's, plus the
    dense kernels for the latent block), comments and spacing left out.  read(name) returns a
    source's text (default: the file in the tree)."""
    import hashlib
    if read is None:
        def read(f):
            with open(os.path.join(ROOT, "mxfp4_routed_expert_k3x_amd", "csrc", f)) as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in LATENT_SOURCES if workload in LATENT_WORKLOADS else KERNEL_SOURCES:
        h.update(code_only(read(f)).encode())
    return h.hexdigest()[:16]


def dense_reference(torch, T, H, I, topk, reps=10):
    """The prefill's FLOPs as two plain dense bf16 GEMMs through torch.matmul (hipBLASLt):
    [T*topk, H] x [H, 2I] (W1 and W3 side by side) and [T*topk, I] x [I, H] (W2), event-timed
    on the current stream.  Context for the prefill's TFLOP/s: what the vendor's tuned dense
    GEMM reaches on this GPU for the same work without grouping by expert or decoding FP4."""
    M = T * topk
    g = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    total_flops, total_ms = 0.0, 0.0
    for name, (k, n) in (("w13", (H, 2 * I)), ("w2", (I, H))):
        a = torch.randn(M, k, dtype=torch.bfloat16, device="cuda", generator=g)
        b = torch.randn(k, n, dtype=torch.bfloat16, device="cuda", generator=g)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = 2.0 * M * k * n
        res[name] = {"shape": [M, n, k], "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
        total_flops += flops
        total_ms += ms
        del a, b, c
    torch.cuda.empty_cache()
    res["tflops"] = round(total_flops / total_ms / 1e9, 1)
    res["kind"] = "torch.matmul bf16 (hipBLASLt), the prefill's FLOPs as two dense GEMMs"
    return res


def copy_probe():
    import torch
    a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "dispatches": 3}))


def _counter_rows(path, counter):
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def traffic_from(f_csv, w_csv, cf_csv, cw_csv, workload):
    """Per-launch HBM bytes of the library's kernels from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by bytes / counted bytes of the plain copy."""
    def copy_scale(path, counter):
        vals = [v for k, v in _counter_rows(path, counter) if "copy" in k.lower()]
        vals = [v for v in vals if v > 0.5 * COPY_PROBE_BYTES / 1024]  # the 1 GiB copies
        return COPY_PROBE_BYTES / (1024.0 * float(np.median(vals))), len(vals)
    sf, nf = copy_scale(cf_csv, "FETCH_SIZE")
    sw, nw = copy_scale(cw_csv, "WRITE_SIZE")
    lines = [f"# HBM traffic of {workload} from rocprofv3 counters",
             f"sources_hash={sources_hash(workload)}",
             f"copy_fetch_scale={sf:.4f} (from {nf} copies of {COPY_PROBE_BYTES} B)",
             f"copy_write_scale={sw:.4f} (from {nw} copies)"]
    fetch = _counter_rows(f_csv, "FETCH_SIZE")
    write = _counter_rows(w_csv, "WRITE_SIZE")
    for name, sym in KERNEL_SYMBOLS.items():
        fv = [v for k, v in fetch if sym in k]
        wv = [v for k, v in write if sym in k]
        if not fv or not wv:
            continue
        b = 1024.0 * (float(np.mean(fv)) * sf + float(np.mean(wv)) * sw)
        lines.append(f"traffic {name} {b:.0f} fetch_kib={np.mean(fv):.0f} write_kib={np.mean(wv):.0f} "
                     f"dispatches={len(fv)}/{len(wv)}")
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _kernel_label(name):
    """The library's launch name of a kernel symbol (or the symbol, shortened)."""
    for label, sym in KERNEL_SYMBOLS.items():
        if sym in name:
            return label
    for sym in ("moe_combine", "moe_sort", "sort_count", "sort_scan", "sort_scatter",
                "residual_rmsnorm", "rmsnorm", "residual", "latent_in", "latent_out", "w13_contract",
                "w2_contract", "fill_packed", "fill_scale", "combine_contract"):
        if sym in name:
            return sym
    return name[:60]


def stats_from(path, workload, command, steps):
    """profiles/kernel_trace_<workload>.md from a rocprofv3 --stats kernel CSV, with the
    per-dispatch trace beside it (run_kernel_trace.csv): the average of the last `steps`
    dispatches of each kernel is that of bench.py's event-timed eager pass, the figure the
    bench line's roofline uses; the trace also gives each kernel's registers and LDS."""
    import csv
    rows = list(csv.DictReader(open(path)))
    trace = os.path.join(os.path.dirname(path), "run_kernel_trace.csv")
    per = {}
    res = {}
    if os.path.exists(trace):
        for r in csv.DictReader(open(trace)):
            lab = _kernel_label(r["Kernel_Name"])
            per.setdefault(lab, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
            res[lab] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["SGPR_Count"], r["LDS_Block_Size"],
                        r["Scratch_Size"], r["Workgroup_Size_X"], r["Grid_Size_X"])
    out = [f"# rocprofv3 kernel trace: {workload}", "",
           "Command (from /tmp with TMPDIR=/tmp, repository at $R):", "", f"    {command}", "",
           "Calls include the warm-up, graph-check and eager passes of bench.py; `last N avg` is",
           f"the mean of each kernel's last N = {steps} dispatches, bench.py's event-timed eager pass.", "",
           "| kernel | calls | avg us | last N avg us | min us | max us | % of GPU time | VGPR | AGPR | SGPR | LDS B | scratch B | WG | grid |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lab = _kernel_label(r["Name"])
        d = sorted(per.get(lab, []))[-steps:]
        last = f"{np.mean([(b - a) for a, b in d]) / 1e3:.2f}" if d else "-"
        rs = res.get(lab, ("-",) * 7)
        out.append(f"| {lab} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {last} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} | " + " | ".join(rs) + " |")
    dst = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.md")
    with open(dst, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def counters_from(paths, workload, command, n_xcd=8, n_simd=1024):
    """profiles/counters_<workload>.txt from rocprofv3 --pmc CSVs (one per counter pass):
    per library kernel the average of each counter per dispatch and the figures derived
    from them.  SQ counters are summed over the chip; GRBM_GUI_ACTIVE is summed over the
    n_xcd dies, so the kernel's clock cycles are GRBM_GUI_ACTIVE / n_xcd."""
    import csv
    acc = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            lab = _kernel_label(r["Kernel_Name"])
            if lab not in KERNEL_SYMBOLS and lab not in ("moe_combine",):
                continue
            d = acc.setdefault(lab, {"dur": []})
            d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            d["dur"].append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9)
    lines = [f"# rocprofv3 counters of {workload} (averages per dispatch)", "",
             "Commands (from /tmp with TMPDIR=/tmp, repository at $R), one pass per counter set:", "",
             f"    {command}", "",
             f"Derived: mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {n_xcd} * {n_simd} SIMDs);",
             "mfma_tflops = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 / duration; lds_conflict = SQ_LDS_BANK_CONFLICT /",
             "SQ_LDS_IDX_ACTIVE; valu_per_mfma = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA; wait_frac =",
             "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; clock_ghz = GRBM_GUI_ACTIVE / n_xcd / duration (clock and",
             "MFMA use only for dispatches of 100 us or more: GRBM_GUI_ACTIVE spans the counter window, a few",
             "microseconds more than the dispatch).  duration = the counter run's own dispatch times.", ""]
    for lab in sorted(acc):
        d = {k: float(np.mean(v)) for k, v in acc[lab].items()}
        dur = d.pop("dur")
        lines.append(f"kernel {lab} duration_us={dur * 1e6:.1f}")
        for k in sorted(d):
            lines.append(f"  {k} {d[k]:.6g}")
        der = []
        g = d.get("GRBM_GUI_ACTIVE")
        # GRBM_GUI_ACTIVE spans the counter window, a few microseconds more than a dispatch, so
        # the clock and the MFMA use are derived only for dispatches of 100 us or more
        if g and dur >= 100e-6:
            der.append(f"clock_ghz={g / n_xcd / dur / 1e9:.3f}")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in d:
                der.append(f"mfma_util={d['SQ_VALU_MFMA_BUSY_CYCLES'] / (g / n_xcd * n_simd):.3f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in d:
            der.append(f"mfma_tflops={d['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / dur / 1e12:.1f}")
        if d.get("SQ_LDS_IDX_ACTIVE"):
            der.append(f"lds_conflict={d.get('SQ_LDS_BANK_CONFLICT', 0) / d['SQ_LDS_IDX_ACTIVE']:.3f}")
        if d.get("SQ_INSTS_MFMA"):
            der.append(f"valu_per_mfma={(d.get('SQ_INSTS_VALU', 0) - d['SQ_INSTS_MFMA']) / d['SQ_INSTS_MFMA']:.2f}")
        if d.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in d:
            der.append(f"wait_frac={d['SQ_WAIT_INST_ANY'] / d['SQ_WAVE_CYCLES']:.3f}")
        if der:
            lines.append("  derived " + " ".join(der))
    dst = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    with open(dst, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_for(workload, kernel):
    """Calibrated HBM bytes per launch of `kernel`, or None (no summary, or kernels changed)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals, ok = {}, False
    for line in open(path):
        if line.startswith("sources_hash="):
            ok = line.strip().split("=", 1)[1] == sources_hash(workload)
        elif line.startswith("traffic "):
            parts = line.split()
            vals[parts[1]] = float(parts[2])
    return vals.get(kernel) if ok else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-batch", action="store_true",
                    help="skip the 32-token decode batch leg of the default run")
    ap.add_argument("--no-prefill", action="store_true",
                    help="the default run skips its prefill leg (prefill_t4096_e896)")
    ap.add_argument("--prefill-steps", type=int, default=None,
                    help="timed steps of the default run's prefill leg (default 20)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--activation", choices=("swiglu", "situ"), default="swiglu",
                    help="gated activation of the expert pool (situ: SiTU-GLU, caps 4 and 25)")
    ap.add_argument("--contract", action="store_true",
                    help="the floating point contract's arithmetic (double sums in the listing's "
                         "order, h in fp32); one token per call")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--dense-reference", action="store_true",
                    help="time only the prefill's FLOPs as dense bf16 torch.matmul GEMMs")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"))
    ap.add_argument("--stats-from", metavar="KERNEL_STATS_CSV",
                    help="write profiles/kernel_trace_<workload>.md from a rocprofv3 --stats CSV")
    ap.add_argument("--counters-from", nargs="+", metavar="COUNTER_CSV",
                    help="write profiles/counters_<workload>.txt from rocprofv3 --pmc CSVs")
    ap.add_argument("--profile-cmd", default="",
                    help="the profiling command, recorded in the summary")
    args = ap.parse_args()
    if args.copy_probe:
        return copy_probe()
    if args.dense_reference:
        import torch
        import k3x_synth as S
        pw = {w.name: w for w in S.WORKLOADS.values()}[PREFILL_WORKLOAD]
        print(json.dumps(dense_reference(torch, pw.T, pw.H, pw.I, pw.topk)), flush=True)
        return
    if args.traffic_from:
        return traffic_from(*args.traffic_from, args.workload)
    if args.stats_from:
        steps = args.steps or (20 if args.workload.startswith("prefill") else 4 * ROTATE)
        return stats_from(args.stats_from, args.workload, args.profile_cmd, steps)
    if args.counters_from:
        return counters_from(args.counters_from, args.workload, args.profile_cmd)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              f"built and measured for a single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch

    import k3x_synth as S
    import mxfp4_routed_expert_k3x_amd as k3x

    k3x.load_library()
    if args.workload in LATENT_WORKLOADS:
        return bench_latent(args, torch, S, k3x)
    if args.workload in ARENA_WORKLOADS:
        return bench_arena(args, torch, S, k3x)
    wl = {w.name: w for w in S.WORKLOADS.values()}
    if args.workload not in wl:
        sys.exit(f"unknown workload {args.workload}; one of "
                 f"{sorted(wl) + sorted(LATENT_WORKLOADS) + sorted(ARENA_WORKLOADS)}")
    w = wl[args.workload]
    if w.layers != 1:
        return bench_chain(w, args, torch, S, k3x)
    out = bench_single(w, args, torch, S, k3x, args.steps, args.warmup)
    if args.workload == DEFAULT_WORKLOAD and not args.no_prefill and not args.contract:
        # the prefill half of the metric, in the same line
        torch.cuda.empty_cache()
        pw = wl[PREFILL_WORKLOAD]
        pre = bench_single(pw, args, torch, S, k3x, args.prefill_steps, None)
        out["prefill"] = {k_: pre[k_] for k_ in ("value", "unit", "steps", "warmup", "ms_per_step",
                                                 "config", "roofline", "path", "kernels",
                                                 "cpu_baseline")}
        out["prefill"]["tflops"] = pre["path"]["tflops_wall"]
        ref = dense_reference(torch, pw.T, pw.H, pw.I, pw.topk)
        ref["prefill_over_reference"] = round(pre["path"]["tflops_wall"] / ref["tflops"], 4)
        out["prefill"]["dense_bf16_reference"] = ref
    if args.workload == DEFAULT_WORKLOAD and not args.no_batch and not args.contract:
        # a decode batch of 32 tokens through the router, experts shared Zipf-fashion
        torch.cuda.empty_cache()
        bt = bench_single(wl[BATCH_WORKLOAD], args, torch, S, k3x, None, None)
        out["decode_batch"] = {k_: bt[k_] for k_ in ("value", "unit", "steps", "warmup",
                                                     "ms_per_step", "config", "roofline", "path",
                                                     "kernels", "cpu_baseline")}
    print(json.dumps(out), flush=True)


def bench_single(w, args, torch, S, k3x, steps, warmup):
    """One layer of w.E experts, w.T tokens per step (decode rotates over ROTATE batches;
    prefill repeats one batch of 4096 tokens).  Returns the result record."""
    prefill = w.T > 64
    if steps is None:
        steps = 20 if prefill else 4 * ROTATE
    if warmup is None:
        warmup = 3 if prefill else ROTATE
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    log(f"{w.name}: generating pool E={w.E} H={w.H} I={w.I}")
    pool_dev = S.device_pool(w.seed, 0, w.E, w.H, w.I)
    if args.contract and w.T != 1:
        sys.exit("--contract runs one token per call: use a decode workload")
    pool = k3x.k3x_expert_pool_create(pool_dev, hidden=w.H, inter=w.I, n_experts=w.E,
                                      activation=args.activation, contract=args.contract)
    R = 1 if prefill else ROTATE
    x = S.normal_bf16(w.seed, S.P_X, 0, (R * w.T, w.H))
    xs = [torch.from_numpy(x[r * w.T:(r + 1) * w.T].view(np.int16)).to(dev) for r in range(R)]
    W = b = Wd = bd = None
    if w.router:
        W, b = S.router_inputs(w)
        Wd = torch.from_numpy(W.view(np.int16)).to(dev)
        bd = torch.from_numpy(b).to(dev)
    routes, routes_np = [], []
    if not w.router:
        for r in range(R):
            i_, g_ = S.uniform_routing(w.seed + r, w.T, w.E, w.topk)
            routes_np.append((i_, g_))
            routes.append((torch.from_numpy(i_).to(dev), torch.from_numpy(g_).to(dev)))
    # outputs of each rotated batch
    idxs = [torch.empty((w.T, w.topk), dtype=torch.int32, device=dev) for _ in range(R)]
    gatess = [torch.empty((w.T, w.topk), dtype=torch.float32, device=dev) for _ in range(R)]
    ys = [torch.empty((w.T, w.H), dtype=torch.float32, device=dev) for _ in range(R)]
    rdesc = k3x.router_desc(Wd, bd, w.topk) if w.router else None
    # with a router: router + experts in one call
    ws = k3x.alloc_workspace(k3x.k3x_route_moe_workspace_size(rdesc, pool, w.T) if w.router
                             else k3x.k3x_moe_workspace_size(pool, w.T, w.topk), dev)

    def step(r):
        if w.router:
            k3x.k3x_route_moe_forward(rdesc, pool, xs[r], w.T, idxs[r], gatess[r], ys[r], ws)
        else:
            i_, g_ = routes[r]
            k3x.k3x_moe_forward(pool, xs[r], w.T, i_, g_, w.topk, ys[r], ws)

    def outs(r):
        return (idxs[r], gatess[r], ys[r]) if w.router else (ys[r],)

    # distinct experts per rotated batch (from the GPU's own routing), eager results kept
    U, eager = [], []
    for r in range(R):
        step(r)
        torch.cuda.synchronize()
        ids = (idxs[r] if w.router else routes[r][0]).cpu().numpy()
        U.append(len(np.unique(ids)))
        eager.append([o.clone() for o in outs(r)])
    drops = k3x.k3x_fetch_drops(ws)
    if drops:
        sys.exit(f"run invalid: {drops} dropped slots")

    wall, wall_single, mode = graph_timing(torch, step, R, outs, eager, steps, warmup)

    # kernel durations: the same steps launched eagerly, HIP events around each launch
    prof = k3x.k3x_profiler_create(steps * 16 + 16)
    torch.cuda.synchronize()
    k3x.k3x_profiler_attach(prof)
    t1 = time.perf_counter()
    for i in range(steps):
        step(i % R)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t1
    k3x.k3x_profiler_attach(None)
    durs = k3x.profiler_durations(prof)
    k3x.k3x_profiler_destroy(prof)

    mean_U = float(np.mean([U[i % R] for i in range(steps)]))
    kernels = {}
    for name, ms in durs.items():
        if len(ms) != steps:
            sys.exit(f"profiler recorded {len(ms)} launches of {name} over {steps} steps")
        nbytes, flops = per_kernel_work(name, w.H, w.I, w.E, w.T, w.topk, mean_U)
        avg_s = float(np.mean(ms)) * 1e-3
        kernels[name] = {
            "launches": len(ms),
            "avg_us": round(avg_s * 1e6, 3),
            "alg_bytes": int(nbytes),
            "alg_flops": float(flops),
            "gbps": round(nbytes / avg_s / 1e9, 1),
            "tflops": round(flops / avg_s / 1e12, 2),
        }
    dominant = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches"])
    dk = kernels[dominant]
    traffic = traffic_for(w.name, dominant)
    traffic = int(traffic) if traffic is not None else None
    if prefill:
        # The prefill metric is TFLOP/s against the bf16 MFMA peak.  With ~73 slots per
        # expert every expert's weights are still streamed once per launch, so the kernel's
        # arithmetic intensity (FLOPs per algorithmic byte) sits near the chip's ridge point
        # (bf16 peak / HBM peak); the HBM view is reported beside it.
        roof = {"bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dk["tflops"] / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": dominant, "alg_bytes": dk["alg_bytes"],
                "intensity_flop_per_byte": round(dk["alg_flops"] / dk["alg_bytes"], 1),
                "ridge_flop_per_byte": round(PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
                "hbm": {"achieved": dk["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(dk["gbps"] / PEAK_HBM_GBS, 4)}}
    else:
        roof = {"bound": "hbm", "achieved": dk["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dk["gbps"] / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": dominant,
                "alg_bytes": dk["alg_bytes"]}

    w13, w2 = expert_tensor_bytes(w.H, w.I)
    path_bytes = mean_U * (w13 + w2) + w.T * (w.H * 2 + w.H * 4)
    if w.router:
        path_bytes += w.E * w.H * 2 + w.E * 4
    path_flops = w.T * w.topk * 6.0 * w.H * w.I
    ksum = sum(k["avg_us"] * k["launches"] for k in kernels.values()) / steps * 1e-6
    ms_per_step = wall / steps * 1e3
    out = {
        "metric": METRIC,
        "value": round(w.T * steps / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "activation": args.activation, "tokens": w.T,
                   "arithmetic": "contract (fp64 sums, h fp32)" if args.contract else "routed (fp32 sums, h bf16)",
                   "experts": w.E, "hidden": w.H,
                   "inter": w.I, "topk": w.topk, "router": w.router, "zipf_bias": w.zipf,
                   "weights": "mxfp4 (e2m1 + e8m0 per 32)", "rotated_batches": R,
                   "distinct_experts_per_step": round(mean_U, 2)},
        "roofline": roof,
        "path": {"kernel_sum_us": round(ksum * 1e6, 3),
                 "alg_bytes_per_step": int(path_bytes),
                 "alg_flops_per_step": path_flops,
                 "hbm_gbps_kernel_sum": round(path_bytes / ksum / 1e9, 1),
                 "hbm_frac_kernel_sum": round(path_bytes / ksum / 1e9 / PEAK_HBM_GBS, 4),
                 "tflops_kernel_sum": round(path_flops / ksum / 1e12, 2),
                 "hbm_gbps_wall": round(path_bytes / (wall / steps) / 1e9, 1),
                 "tflops_wall": round(path_flops / (wall / steps) / 1e12, 2),
                 "timed_region": TIMED_REGION, "timed_mode": mode,
                 "ms_per_step_one_graph_per_step": round(wall_single / steps * 1e3, 5),
                 "eager_ms_per_step": round(wall_eager / steps * 1e3, 5)},
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"{w.name}: timing the oracle on the host (bounded sample)")
        act = ORACLE_ACT[args.activation]
        if prefill:
            i_, g_ = routes_np[0]
            out["cpu_baseline"] = prefill_cpu_baseline(w, x, i_, g_, pool_dev, act=act)
        else:
            di = np.concatenate([r_[0] for r_ in routes_np]) if routes_np else None
            dg = np.concatenate([r_[1] for r_ in routes_np]) if routes_np else None
            out["cpu_baseline"] = cpu_baseline(w, x, W, b, di, dg, pool_dev, act=act)
    del pool, pool_dev, ws, ys
    return out


if __name__ == "__main__":
    main()
