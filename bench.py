"""Benchmark: one decode step of the quantised MoE layer on one MI355X.

A step is one MoE layer forward for one token (router GEMV -> softmax/top-4 of
512 -> shared expert -> gathered dequant gate/up -> SwiGLU -> down -> weighted
combine + sigmoid-gated shared expert + residual -> RMSNorm) at hidden 4096,
512 routed experts + 1 shared, expert intermediate 1024, 4-bit codes in groups
of 64 with bf16 scale/bias.  Inputs are seeded synthetic data resident in HBM.

Cold-cache protocol: the steps rotate over R distinct layer replicas (default
32, ~116 GB of expert slabs) and a pool of 64 activation vectors, so that the
per-layer router (8 MB) and shared expert (7 MB) do not stay in the 256 MB
Infinity Cache.  Steps are captured in HIP graphs of 64 layers and replayed;
HIP events on the capture/replay stream time exactly --steps steps.

Prints one JSON line.  `value` is the achieved HBM throughput of the whole
layer (algorithmic bytes / time); us_per_layer and MoE-layer tokens/s are
reported beside it.  --gpus N with N > 1 is rejected (single-GPU build).
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=6400)
    p.add_argument("--warmup", type=int, default=640)
    p.add_argument("--workload", default="layer4", choices=["layer4", "layer2"])
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


def source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_dequant_expert_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + f.read())
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
    if args.steps % GRAPH_LEN or args.warmup % GRAPH_LEN:
        sys.exit(f"--steps and --warmup must be multiples of {GRAPH_LEN}")

    import numpy as np
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

    with torch.cuda.stream(s):
        for i in range(args.warmup // GRAPH_LEN):
            graphs[i % n_graphs].replay()
    torch.cuda.synchronize()

    reps = args.steps // GRAPH_LEN
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_replay = []
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        ev0.record(s)
        for i in range(reps):
            graphs[i % n_graphs].replay()
        ev1.record(s)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    # per-replay spread (separate pass, same protocol)
    with torch.cuda.stream(s):
        for i in range(min(reps, 20)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            graphs[i % n_graphs].replay()
            b.record(s)
            per_replay.append((a, b))
    torch.cuda.synchronize()
    rep_us = sorted(a.elapsed_time(b) * 1000.0 / GRAPH_LEN for a, b in per_replay)

    ms_per_step = total_ms / args.steps
    us = ms_per_step * 1000.0
    nbytes, ebytes = layer_bytes(cfg)
    gbps = nbytes / (us * 1e-6) / 1e9
    khash = source_hash()
    traffic = traffic_from_profiles(khash, args.workload)
    stream = None
    if not args.no_stream_probe:
        try:
            import probes
            stream = round(probes.stream_read_gbps(torch), 1)
        except Exception as exc:  # the probe is context only
            print(f"[bench] stream probe skipped: {exc}", file=sys.stderr)
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
        "us_per_layer_min_median_p90": [round(rep_us[0], 3), round(rep_us[len(rep_us) // 2], 3),
                                        round(rep_us[int(len(rep_us) * 0.9)], 3)],
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
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
