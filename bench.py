"""Benchmark: one decode step of the quantised MoE layer on one MI355X.

Default workload (layer4): a step is one MoE layer forward for one token
(router GEMV -> softmax/top-4 of 512 -> shared expert -> gathered dequant
gate/up -> SwiGLU -> down -> weighted combine + sigmoid-gated shared expert +
residual -> RMSNorm) at hidden 4096, 512 routed experts + 1 shared, expert
intermediate 1024, 4-bit codes in groups of 64 with bf16 scale/bias.  Inputs
are seeded synthetic data resident in HBM.  layer2 is the same layer with
2-bit codes.

Cold-cache protocol: the steps rotate over R distinct layer replicas (default
32, ~116 GB of expert slabs) and a pool of 64 activation vectors, so that the
per-layer router (8 MB) and shared expert (7 MB) do not stay in the 256 MB
Infinity Cache.  Steps are captured in HIP graphs of 64 layers and replayed;
HIP events on the capture/replay stream time exactly --steps steps.

Other workloads (not the default line):
  expert   one expert's fused gate/up -> SwiGLU -> down (fmoe_expert_ffn) at
           [1024 x 4096] / [4096 x 1024], rotating over 128 experts; the gate
           GEMV and the down GEMV (fmoe_dequant_gemv) are timed alone beside it.
  stack60  60 distinct 4-bit layers (217.8 GB of slabs) chained on the device
           (x_{l+1} = y_l, r_{l+1} = h_l) for a batch of 32 independent tokens;
           a step is the whole 60-layer pass, captured in one HIP graph.

Prints one JSON line.  `value` is the achieved HBM throughput (algorithmic
bytes / time); per-layer microseconds and tokens/s are reported beside it.
--gpus N with N > 1 is rejected (single-GPU build).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = ("µs per MoE layer & achieved HBM GB/s (% of peak), 4-bit, hidden 4096, "
          "512 experts")
GRAPH_LEN = 64
XPOOL = 64
DEFAULT_STEPS = {"layer4": (6400, 640), "layer2": (6400, 640), "expert": (4096, 640),
                 "stack60": (40, 4)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 6400 layers; 64 expert passes x 64; 40 stacks)")
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="layer4",
                   choices=["layer4", "layer2", "expert", "stack60"],
                   help="layer4/layer2: one batch-1 layer per step; expert: one expert's "
                        "gate/up/down per step; stack60: 60 chained layers x 32 tokens per step")
    p.add_argument("--replicas", type=int, default=32)
    p.add_argument("--cpu-sample", type=int, default=40, help="tokens timed on the oracle")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-steps", type=int, default=0,
                   help="launch only this many plain (non-graph) steps, for profilers")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="run only a plain device copy of this many bytes (calibrates the HBM "
                        "byte counters of a profiler) and exit")
    p.add_argument("--no-stream-probe", action="store_true",
                   help="skip measuring the streaming-read ceiling")
    return p.parse_args()


def layer_bytes(cfg):
    """Algorithmic bytes of one batch-1 layer: the k+1 active expert slabs, the
    fp32 router, the shared-gate vector and gamma read, x and r read, h and y
    written."""
    off, slab = cfg.spec.layout()
    experts = (cfg.k + 1) * slab
    router = cfg.E * cfg.H * 4
    vectors = 6 * cfg.H * 4
    return experts + router + vectors, experts


# The pages' own figures, for context only: whole-system numbers of an Apple
# M3 Max laptop (unified memory ~400 GB/s, experts streamed from SSD, the
# attention and state layers included), not this metric on this workload, so
# vs_baseline stays null.
PAGES_CONTEXT = {
    "hardware": "Apple M3 Max, 40-core GPU, ~400 GB/s unified memory, experts streamed from SSD",
    "ms_per_layer_whole_model_4bit": 4.28,
    "decode_tokens_per_s_whole_model_4bit": 4.36,
    "dequant_matvec_kernel_gib_per_s": 418,
    "comparable": False,
}


def source_hash():
    """Hash of the kernel sources with comments and white space removed, so
    that a profile stays matched to code whose comments were edited since."""
    import re
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_dequant_expert_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = re.sub(r"\s+", " ", text).strip()
        h.update(name.encode() + text.encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_hash, workload):
    """HBM bytes per launch of the layer kernel, from the rocprofv3 counter
    summary profiles/k_layer1_<workload>_traffic.txt when it was taken on this
    exact kernel source (its `source_hash:` line), else None."""
    path = os.path.join(ROOT, "profiles", f"k_layer1_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_hash") != kernel_hash:
        return None
    try:
        return int(float(rec["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def stack_traffic_from_profiles(kernel_hash, n_layers):
    """HBM bytes of one 60-layer step: the per-dispatch bytes of every layer kernel in
    profiles/k_moe_mfma_stack60_batch32_traffic.txt (rocprofv3 counters, copy-calibrated)
    times the layer count, when the profile was taken on this exact source, else None."""
    path = os.path.join(ROOT, "profiles", "k_moe_mfma_stack60_batch32_traffic.txt")
    if not os.path.exists(path):
        return None
    total, hsh = 0.0, None
    for line in open(path):
        if line.startswith("source_hash:"):
            hsh = line.split(":", 1)[1].strip()
        elif line.startswith("| ") and "fmoe::" in line:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            try:
                total += float(cells[-1])
            except ValueError:
                pass
    if hsh != kernel_hash or total <= 0:
        return None
    return int(total * n_layers)


def cpu_baseline(cfg, n_tokens):
    """The CPU oracle (single-threaded C, fp64) on a bounded sample of tokens of
    the same workload: routing over all 512 experts plus the 5 active experts'
    dequantise-and-multiply, combine, residual and RMSNorm."""
    import numpy as np
    import oracle
    import synth
    sp = cfg.spec
    Wr, wsg, gamma = synth.router(cfg, 0), synth.shared_gate(cfg, 0), synth.gamma(cfg, 0)
    x = synth.activations(cfg, n_tokens, pool=9)
    shared = synth.slab(sp, cfg.seed, 0, cfg.E)
    total = 0.0
    for t in range(n_tokens):
        t0 = time.perf_counter()
        idx, w, _, _, _ = oracle.route(Wr, x[t:t + 1], cfg.k)
        total += time.perf_counter() - t0
        slabs = [synth.slab(sp, cfg.seed, 0, int(e)) for e in idx[0]]     # untimed input prep
        t0 = time.perf_counter()
        oracle.moe_token(slabs, w[0], shared, cfg.H, cfg.I, sp.bits, sp.group, sp.sbytes, wsg,
                         gamma, cfg.eps, x[t], x[t])
        total += time.perf_counter() - t0
    us = total / n_tokens * 1e6
    nbytes, _ = layer_bytes(cfg)
    return us, nbytes / (us * 1e-6) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    dsteps, dwarm = DEFAULT_STEPS[args.workload]
    args.steps = dsteps if args.steps is None else args.steps
    args.warmup = dwarm if args.warmup is None else args.warmup
    if args.workload != "stack60" and (args.steps % GRAPH_LEN or args.warmup % GRAPH_LEN):
        sys.exit(f"--steps and --warmup must be multiples of {GRAPH_LEN}")

    import torch

    if args.copy_bytes:
        # Plain copy of known size: a profiler's FETCH/WRITE counters over this
        # dispatch give the scale from counter units to bytes.
        n = args.copy_bytes
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "dispatches": 3}))
        return

    if args.workload == "expert":
        out = bench_expert(args, torch)
    elif args.workload == "stack60":
        out = bench_stack(args, torch)
    else:
        out = bench_layer(args, torch)
    if out is not None:
        print(json.dumps(out), flush=True)


def stream_probe(args, torch):
    if args.no_stream_probe:
        return None
    try:
        import probes
        return round(probes.stream_read_gbps(torch), 1)
    except Exception as exc:  # the probe is context only
        print(f"[bench] stream probe skipped: {exc}", file=sys.stderr)
        return None


def time_replays(torch, graphs, reps, warmup_reps, stream):
    """Replay graphs[i % len] warmup_reps times untimed, then reps times between
    two HIP events on `stream`; then up to 20 single replays for the spread.
    Returns (total ms, sorted per-replay ms)."""
    with torch.cuda.stream(stream):
        for i in range(warmup_reps):
            graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(reps):
            graphs[i % len(graphs)].replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    per = []
    with torch.cuda.stream(stream):
        for i in range(min(reps, 20)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graphs[i % len(graphs)].replay()
            b.record(stream)
            per.append((a, b))
    torch.cuda.synchronize()
    return total_ms, sorted(a.elapsed_time(b) for a, b in per)


def spread(vals):
    return [round(vals[0], 3), round(vals[len(vals) // 2], 3), round(vals[int(len(vals) * 0.9)], 3)]


def bench_layer(args, torch):
    import numpy as np
    import bit_dequant_expert_amd as fm
    import synth

    cfg = synth.CONFIGS[args.workload]
    sp = cfg.spec
    dev = torch.device("cuda:0")
    off, stride = sp.layout()
    R = args.replicas
    print(f"[bench] generating {R} layer replicas ({R * stride * (cfg.E + 1) / 1e9:.1f} GB)",
          file=sys.stderr, flush=True)
    fmt = fm.qformat(sp.bits, sp.group, sp.sbytes == 2)
    layers = []
    for r in range(R):
        slabs = torch.empty(stride * (cfg.E + 1), dtype=torch.uint8, device=dev)
        synth.fill_device_slabs(slabs.data_ptr(), sp, cfg.seed, r, 0, cfg.E + 1, stride)
        Wr = torch.from_numpy(synth.router(cfg, r)).to(dev)
        wsg = torch.from_numpy(synth.shared_gate(cfg, r)).to(dev)
        gam = torch.from_numpy(synth.gamma(cfg, r)).to(dev)
        layers.append(fm.fmoe_layer_desc(cfg.H, cfg.I, cfg.E, cfg.k, fmt, Wr, slabs, stride,
                                         wsg, gam, cfg.eps))
    xpool = torch.from_numpy(synth.activations(cfg, XPOOL, pool=0)).to(dev)
    h = torch.empty(XPOOL, cfg.H, device=dev)
    y = torch.empty(XPOOL, cfg.H, device=dev)
    ws_bytes = fm.fmoe_workspace_size(layers[0], 1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    import ctypes as C
    Lp = [C.addressof(L) for L in layers]
    xb, hb, yb = xpool.data_ptr(), h.data_ptr(), y.data_ptr()
    row = cfg.H * 4

    def step(i, stream):
        r, j = i % R, i % XPOOL
        xi = xb + j * row
        rc = fm.fmoe_moe_layer_forward_raw(Lp[r], 1, xi, xi, hb + j * row, yb + j * row, None,
                                           None, None, ws.data_ptr(), ws_bytes, stream)
        if rc != 0:
            raise fm.FmoeError(rc, fm.fmoe_last_error())

    s = torch.cuda.Stream()
    if args.kernel_steps:
        # Plain launches (no graph), for kernel-level profilers.
        with torch.cuda.stream(s):
            for i in range(args.kernel_steps):
                step(i, s.cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_steps": args.kernel_steps, "workload": args.workload}))
        return

    # Graphs: one per 64-step window, so a replay sweeps every replica pairing.
    n_graphs = max(1, (R * XPOOL // GRAPH_LEN) // max(1, np.gcd(R, XPOOL)))
    n_graphs = min(n_graphs, 8)
    graphs = []
    with torch.cuda.stream(s):
        for i in range(8):                      # eager warm-up before capture
            step(i, s.cuda_stream)
    torch.cuda.synchronize()
    for gi in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(GRAPH_LEN):
                step(gi * GRAPH_LEN + i, cs)
        graphs.append(g)
    torch.cuda.synchronize()

    total_ms, rep_ms = time_replays(torch, graphs, args.steps // GRAPH_LEN,
                                    args.warmup // GRAPH_LEN, s)
    rep_us = [v * 1000.0 / GRAPH_LEN for v in rep_ms]

    ms_per_step = total_ms / args.steps
    us = ms_per_step * 1000.0
    nbytes, ebytes = layer_bytes(cfg)
    gbps = nbytes / (us * 1e-6) / 1e9
    khash = source_hash()
    traffic = traffic_from_profiles(khash, args.workload)
    stream = stream_probe(args, torch)
    out = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 codes x f16 activations, f32 accumulation (router f64)",
        "data": "synthetic",
        "config": {"workload": f"moe_layer_{args.workload}_h{cfg.H}_e{cfg.E}_i{cfg.I}"
                               f"_top{cfg.k}+1_batch1",
                   "hidden": cfg.H, "experts": cfg.E, "inter": cfg.I, "top_k": cfg.k,
                   "bits": sp.bits, "group": sp.group, "scale_dtype": "bf16",
                   "batch": 1, "replicas": R, "graph_len": GRAPH_LEN},
        "us_per_layer": round(us, 3),
        "us_per_layer_min_median_p90": spread(rep_us),
        "moe_layer_tokens_per_s": round(1e6 / us, 1),
        "pct_of_peak_hbm": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "algorithmic_bytes_per_layer": nbytes,
        "expert_bytes_per_layer": ebytes,
        "roofline": {"bound": "hbm", "kernel": "k_layer1 (whole layer, one launch)",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "kernel_source_hash": khash,
        "context": {"hbm_stream_read_gbps_measured": stream,
                    "note": "best of 10 passes of a plain 4 GiB streaming read on this GPU"},
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        import multiprocessing
        cus, cgb = cpu_baseline(cfg, args.cpu_sample)
        out["cpu_baseline"] = {"value": round(cgb, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{args.cpu_sample} tokens of the same layer "
                                         f"(route over 512 + 5 experts), {cus:.0f} us/token, "
                                         f"1 thread of {multiprocessing.cpu_count()} host "
                                         f"logical cores"}
    return out



def _fmt_and_layers(torch, fm, synth, cfg, layer_ids, dev):
    sp = cfg.spec
    off, stride = sp.layout()
    fmt = fm.qformat(sp.bits, sp.group, sp.sbytes == 2)
    layers = []
    for l in layer_ids:
        slabs = torch.empty(stride * (cfg.E + 1), dtype=torch.uint8, device=dev)
        synth.fill_device_slabs(slabs.data_ptr(), sp, cfg.seed, l, 0, cfg.E + 1, stride)
        Wr = torch.from_numpy(synth.router(cfg, l)).to(dev)
        wsg = torch.from_numpy(synth.shared_gate(cfg, l)).to(dev)
        gam = torch.from_numpy(synth.gamma(cfg, l)).to(dev)
        layers.append(fm.fmoe_layer_desc(cfg.H, cfg.I, cfg.E, cfg.k, fmt, Wr, slabs, stride,
                                         wsg, gam, cfg.eps))
    return fmt, layers


def bench_expert(args, torch):
    """One expert at hidden 4096 / inter 1024, 4-bit G64 bf16: the fused FFN
    (fmoe_expert_ffn) per step, and the gate and down GEMVs (fmoe_dequant_gemv)
    alone.  Steps rotate over 128 experts (906 MB of slabs, more than the
    Infinity Cache) and 64 input vectors."""
    import ctypes as C
    import bit_dequant_expert_amd as fm
    import synth

    cfg = synth.CONFIGS["layer4"]
    sp = cfg.spec
    H, I = cfg.H, cfg.I
    dev = torch.device("cuda:0")
    off, stride = sp.layout()
    NE = 128
    slabs = torch.empty(stride * NE, dtype=torch.uint8, device=dev)
    synth.fill_device_slabs(slabs.data_ptr(), sp, cfg.seed, 0, 0, NE, stride)
    fmt = fm.qformat(sp.bits, sp.group, sp.sbytes == 2)
    base = slabs.data_ptr()
    exps = []
    for e in range(NE):
        b = base + e * stride
        exps.append(fm.fmoe_expert(fm.qmat(b + off[0], b + off[1], b + off[2], I, H),
                                   fm.qmat(b + off[3], b + off[4], b + off[5], I, H),
                                   fm.qmat(b + off[6], b + off[7], b + off[8], H, I)))
    xpool = torch.from_numpy(synth.activations(cfg, XPOOL, pool=1)).to(dev)
    hpool = torch.from_numpy(synth.normal(cfg.seed, 20_000, 9, (XPOOL, I))).to(dev)
    y = torch.empty(XPOOL, H, device=dev)
    yi = torch.empty(XPOOL, I, device=dev)
    ws_bytes = fm.fmoe_expert_ffn_workspace_size(exps[0], fmt)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    L = fm.lib()
    xb, hb, yb, yib = xpool.data_ptr(), hpool.data_ptr(), y.data_ptr(), yi.data_ptr()

    def call(kind, i, stream):
        e, j = exps[i % NE], i % XPOOL
        if kind == "ffn":
            rc = L.fmoe_expert_ffn(C.byref(e), C.byref(fmt), xb + j * H * 4, yb + j * H * 4,
                                   ws.data_ptr(), ws_bytes, stream)
        elif kind == "gate":
            rc = L.fmoe_dequant_gemv(C.byref(e.gate), C.byref(fmt), xb + j * H * 4,
                                     yib + j * I * 4, stream)
        else:
            rc = L.fmoe_dequant_gemv(C.byref(e.down), C.byref(fmt), hb + j * I * 4,
                                     yb + j * H * 4, stream)
        if rc != 0:
            raise fm.FmoeError(rc, fm.fmoe_last_error())

    s = torch.cuda.Stream()
    if args.kernel_steps:
        with torch.cuda.stream(s):
            for kind in ("ffn", "gate", "down"):
                for i in range(args.kernel_steps):
                    call(kind, i, s.cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_steps": args.kernel_steps, "workload": args.workload}))
        return None

    qb = I * H * sp.bits // 8
    sb = 2 * I * (H // sp.group) * sp.sbytes
    nbytes = {"ffn": stride + 2 * H * 4, "gate": qb + sb + H * 4 + I * 4,
              "down": qb + sb + I * 4 + H * 4}
    res = {}
    for kind in ("ffn", "gate", "down"):
        with torch.cuda.stream(s):
            for i in range(8):
                call(kind, i, s.cuda_stream)
        torch.cuda.synchronize()
        graphs = []
        for gi in range(NE // GRAPH_LEN):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(GRAPH_LEN):
                    call(kind, gi * GRAPH_LEN + i, cs)
            graphs.append(g)
        torch.cuda.synchronize()
        total_ms, rep_ms = time_replays(torch, graphs, args.steps // GRAPH_LEN,
                                        args.warmup // GRAPH_LEN, s)
        us = total_ms * 1000.0 / args.steps
        res[kind] = {"us": round(us, 3), "gbps": round(nbytes[kind] / (us * 1e-6) / 1e9, 1),
                     "bytes": nbytes[kind],
                     "us_min_median_p90": spread([v * 1000.0 / GRAPH_LEN for v in rep_ms])}
    us = res["ffn"]["us"]
    gbps = res["ffn"]["gbps"]
    out = {
        "metric": METRIC,
        "value": gbps,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 codes x f16 activations, f32 accumulation",
        "data": "synthetic",
        "config": {"workload": f"expert_ffn_h{H}_i{I}_4bit_g{sp.group}_bf16_batch1",
                   "hidden": H, "inter": I, "bits": sp.bits, "group": sp.group,
                   "scale_dtype": "bf16", "batch": 1, "experts_rotated": NE,
                   "graph_len": GRAPH_LEN},
        "us_per_expert": us,
        "parts": res,
        "pct_of_peak_hbm": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "roofline": {"bound": "hbm", "kernel": "fmoe_expert_ffn (all launches of one call)",
                     "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None},
        "kernel_source_hash": source_hash(),
        "context": {"hbm_stream_read_gbps_measured": stream_probe(args, torch)},
    }
    if not args.no_cpu_baseline:
        import multiprocessing
        import oracle
        n = max(1, args.cpu_sample // 2)
        x = synth.activations(cfg, n, pool=1)
        total = 0.0
        for t in range(n):
            slab = synth.slab(sp, cfg.seed, 0, t)
            t0 = time.perf_counter()
            oracle.expert_ffn(slab, H, I, sp.bits, sp.group, sp.sbytes, x[t])
            total += time.perf_counter() - t0
        cus = total / n * 1e6
        out["cpu_baseline"] = {"value": round(nbytes["ffn"] / (cus * 1e-6) / 1e9, 4),
                               "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} experts' gate/up/down on the host, "
                                         f"{cus:.0f} us/expert, 1 thread of "
                                         f"{multiprocessing.cpu_count()} host logical cores"}
    return out


def bench_stack(args, torch):
    """60 distinct 4-bit layers chained on the device for 32 independent tokens
    (each layer's y and h are the next layer's x and residual); a step is the
    whole 60-layer pass, captured in one HIP graph.  The algorithmic bytes of a
    step count each distinct expert a layer touches once (its slab is read once
    for all the tokens routed to it), plus the shared expert, the router and the
    vectors; the distinct counts are read back from the run's own routing."""
    import ctypes as C
    import numpy as np
    import bit_dequant_expert_amd as fm
    import synth

    cfg = synth.CONFIGS["layer4"]
    sp = cfg.spec
    NL, T = 60, 32
    MODES = ("independent", "chained")
    dev = torch.device("cuda:0")
    off, stride = sp.layout()
    print(f"[bench] generating {NL} layers ({NL * stride * (cfg.E + 1) / 1e9:.1f} GB)",
          file=sys.stderr, flush=True)
    fmt, layers = _fmt_and_layers(torch, fm, synth, cfg, range(NL), dev)
    xs = torch.from_numpy(synth.activations(cfg, NL * T, pool=4)).to(dev).view(NL, T, cfg.H)
    hbuf = [torch.empty(T, cfg.H, device=dev) for _ in range(2)]
    ybuf = [torch.empty(T, cfg.H, device=dev) for _ in range(2)]
    idx = {m: torch.empty(NL, T, cfg.k, dtype=torch.int32, device=dev) for m in MODES}
    wts = torch.empty(NL, T, cfg.k, device=dev)
    ws_bytes = fm.fmoe_workspace_size(layers[0], T)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print("[bench] layers ready", file=sys.stderr, flush=True)
    Lp = [C.addressof(L) for L in layers]

    def step(mode, stream):
        x = r = xs[0].data_ptr()
        for l in range(NL):
            if mode == "independent":
                x = r = xs[l].data_ptr()
            h, y = hbuf[l % 2].data_ptr(), ybuf[l % 2].data_ptr()
            rc = fm.fmoe_moe_layer_forward_raw(Lp[l], T, x, r, h, y, idx[mode][l].data_ptr(),
                                               wts[l].data_ptr(), None, ws.data_ptr(),
                                               ws_bytes, stream)
            if rc != 0:
                raise fm.FmoeError(rc, fm.fmoe_last_error())
            x, r = y, h

    s = torch.cuda.Stream()
    if args.kernel_steps:
        with torch.cuda.stream(s):
            for i in range(args.kernel_steps):
                step("independent", s.cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_steps": args.kernel_steps, "workload": args.workload}))
        return None

    res = {}
    for mode in MODES:
        with torch.cuda.stream(s):
            step(mode, s.cuda_stream)                 # eager warm-up before capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step(mode, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        total_ms, rep_ms = time_replays(torch, [g], args.steps, args.warmup, s)
        ms = total_ms / args.steps
        sel = idx[mode].cpu().numpy()
        distinct = [int(np.unique(sel[l]).size) for l in range(NL)]
        counts = [np.bincount(sel[l].ravel(), minlength=cfg.E) for l in range(NL)]
        nbytes = (sum(distinct) + NL) * stride + NL * cfg.E * cfg.H * 4 \
            + NL * (4 * T + 2) * cfg.H * 4
        res[mode] = {"ms_per_step": round(ms, 6), "ms_min_median_p90": spread(rep_ms),
                     "tokens_per_s": round(T / (ms * 1e-3), 1),
                     "us_per_layer": round(ms * 1000.0 / NL, 3),
                     "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "algorithmic_bytes_per_step": nbytes,
                     "distinct_routed_experts_per_layer": {
                         "mean": round(float(np.mean(distinct)), 2), "min": min(distinct),
                         "max": max(distinct)},
                     "routed_experts_on_matrix_cores_per_layer": round(
                         float(np.mean([int((c >= 16).sum()) for c in counts])), 3)}
        del g
    main_res = res["independent"]
    ms, gbps = main_res["ms_per_step"], main_res["gbps"]
    out = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 codes x f16 activations, f32 accumulation (router f64)",
        "data": "synthetic",
        "config": {"workload": f"moe_stack60_h{cfg.H}_e{cfg.E}_i{cfg.I}_top{cfg.k}+1_batch{T}",
                   "layers": NL, "batch": T, "hidden": cfg.H, "experts": cfg.E,
                   "inter": cfg.I, "top_k": cfg.k, "bits": sp.bits, "group": sp.group,
                   "scale_dtype": "bf16", "resident_slab_gb": round(
                       NL * stride * (cfg.E + 1) / 1e9, 1)},
        "tokens_per_s": main_res["tokens_per_s"],
        "us_per_layer": main_res["us_per_layer"],
        "routing": "independent: every layer takes a fresh N(0,1) batch (x = r), so routing "
                   "is independent across tokens and layers; chained: y and h of each layer "
                   "are the next layer's x and residual",
        "modes": res,
        "pct_of_peak_hbm": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "roofline": {"bound": "hbm", "kernel": "all launches of the 60 layers (one graph)",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": stack_traffic_from_profiles(source_hash(), NL)},
        "kernel_source_hash": source_hash(),
        "context": {"hbm_stream_read_gbps_measured": stream_probe(args, torch)},
    }
    if not args.no_cpu_baseline:
        import multiprocessing
        n = max(1, args.cpu_sample // 2)
        cus, _ = cpu_baseline(cfg, n)
        out["cpu_baseline"] = {"value": round(1e6 / (NL * cus), 4), "unit": "tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{n} layer-tokens of a 4-bit layer (route over 512 + "
                                         f"5 experts), {cus:.0f} us per layer-token, scaled to "
                                         f"60 layers; 1 thread of "
                                         f"{multiprocessing.cpu_count()} host logical cores"}
    return out


if __name__ == "__main__":
    main()
