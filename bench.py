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
Infinity Cache.  The timed steps are launched one per layer forward behind a
GPU busy-wait that outlasts their queueing; HIP events on the launch stream
time exactly --steps steps.  Replays of a 64-layer HIP graph give the spread.

Other workloads (not the default line):
  expert   one expert's fused gate/up -> SwiGLU -> down (fmoe_expert_ffn) at
           [1024 x 4096] / [4096 x 1024], rotating over 128 experts; the gate
           GEMV and the down GEMV (fmoe_dequant_gemv) are timed alone beside it.
  stack60  60 distinct 4-bit layers (217.8 GB of slabs) chained on the device
           (x_{l+1} = y_l, r_{l+1} = h_l) for a batch of 32 independent tokens;
           a step is the whole 60-layer pass, captured in one HIP graph.
  chain60  the same 60 layers for one token (batch-1 decode through the whole
           MoE stack): a step is the 60-layer pass, one fmoe_moe_stack_forward
           call (the chained one-token kernel, one launch for all 60 layers);
           one HIP graph of 60 one-token layer launches is timed beside it.
  deltanet one Gated DeltaNet decode step (fmoe_deltanet_step) of one
           linear-attention layer for 32 sequences x 64 heads of 128 x 128 fp32
           state (268 MB), rotating over 8 layers' states so that no step finds
           its state in the Infinity Cache.
  attention decode attention of one new token (fmoe_attention_decode) for 32
           sequences, 32 query heads over 2 KV heads of dimension 256, a bf16
           cache of up to 8192 positions with lengths drawn in [2048, 8192],
           rotating over 4 layers' caches.
  stream   batch-1 layers whose experts live in pinned host memory (two full
           4-bit layers, 7.3 GB, alternating): a step routes the token on the
           GPU, fetches its 4 routed experts and the shared one into the HBM
           slab array (fmoe_fetch_experts, no host round trip) and runs the
           layer on it.

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
HOST_LINK_GBPS = 64.0     # the GPU's host link, PCIe 5.0 x16, one direction
METRIC = ("µs per MoE layer & achieved HBM GB/s (% of peak), 4-bit, hidden 4096, "
          "512 experts")
GRAPH_LEN = 64
XPOOL = 64
DEFAULT_STEPS = {"layer4": (640, 64), "layer2": (640, 64), "expert": (640, 64),
                 "stack60": (20, 2), "chain60": (20, 2), "deltanet": (640, 64),
                 "attention": (640, 64), "stream": (64, 8)}
SPIN_US = 2000          # GPU busy-wait queued ahead of a timed region
EAGER_SPIN_PER_STEP_US = 25   # and at least this per eagerly launched step (host queueing)


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps, any positive count (default 640 layers / expert passes, "
                        "20 stacks)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps before (>= 0)")
    p.add_argument("--workload", default="layer4",
                   choices=["layer4", "layer2", "expert", "stack60", "chain60", "deltanet",
                            "attention", "stream"],
                   help="layer4/layer2: one batch-1 layer per step; expert: one expert's "
                        "gate/up/down per step; stack60: 60 chained layers x 32 tokens per step; "
                        "chain60: 60 chained layers x 1 token per step")
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
    p.add_argument("--phase-trace", type=int, default=0,
                   help="run this many calls on the phase-trace build and print the timeline of "
                        "the one-token kernel's phases (layer workloads; chain60: its second "
                        "layer)")
    return p.parse_args(argv)


def resolve_steps(args):
    """Fill in the workload's default step counts; any positive --steps and any
    --warmup >= 0 is valid."""
    dsteps, dwarm = DEFAULT_STEPS[args.workload]
    args.steps = dsteps if args.steps is None else args.steps
    args.warmup = dwarm if args.warmup is None else args.warmup
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")
    return args


def step_chunks(n, start=0, size=GRAPH_LEN):
    """(first step, count) pieces of at most `size` steps that cover steps
    start .. start+n-1 in order: full graphs, then one shorter graph for the
    remainder."""
    return [(start + i, min(size, n - i)) for i in range(0, n, size)]


class GraphRunner:
    """HIP graphs of consecutive steps, keyed by (first step mod period, count):
    steps whose inputs repeat with `period` share one captured graph."""

    def __init__(self, torch, stream, step, period):
        self.torch, self.stream, self.step, self.period = torch, stream, step, period
        self.graphs = {}

    def graph(self, first, count):
        key = (first % self.period, count)
        if key not in self.graphs:
            torch = self.torch
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(first, first + count):
                    self.step(i, cs)
            self.graphs[key] = g
        return self.graphs[key]

    def prepare(self, chunks):
        for f, c in chunks:
            self.graph(f, c)
        self.torch.cuda.synchronize()

    def run(self, chunks):
        with self.torch.cuda.stream(self.stream):
            for f, c in chunks:
                self.graph(f, c).replay()

    def timed(self, chunks):
        """Exactly the steps of `chunks` between two HIP events on the stream the
        kernels run on.  A bounded busy-wait is queued first so that the GPU is
        still busy while the host queues the start event and the graphs, and the
        region holds no host launch latency.  Returns (event ms, host wall ms of
        the synchronised region)."""
        torch = self.torch
        import probes
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.stream):
            probes.spin(SPIN_US, self.stream.cuda_stream)
            ev0.record(self.stream)
            for f, c in chunks:
                self.graph(f, c).replay()
            ev1.record(self.stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        return ev0.elapsed_time(ev1), wall

    def timed_eager(self, first, n):
        """Steps first .. first+n-1 launched one by one (no graph) between two HIP
        events.  The busy-wait queued ahead lasts long enough (SPIN_US, and at
        least EAGER_SPIN_PER_STEP_US per step) for the host to queue every launch
        before the GPU reaches the start event, so the region holds the GPU's work
        and its launch gaps only, none of the host's launch latency nor a graph's
        first-replay cost.  Returns (event ms, host wall ms)."""
        torch = self.torch
        import probes
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.stream):
            probes.spin(max(SPIN_US, EAGER_SPIN_PER_STEP_US * n), self.stream.cuda_stream)
            ev0.record(self.stream)
            cs = self.stream.cuda_stream
            for i in range(first, first + n):
                self.step(i, cs)
            ev1.record(self.stream)
        queued = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        self.last_queue_ms = queued
        return ev0.elapsed_time(ev1), wall

    def spread(self, first, count, reps=20):
        """Per-replay ms of `reps` single replays of one graph (context only)."""
        torch = self.torch
        g = self.graph(first, count)
        per = []
        with torch.cuda.stream(self.stream):
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(self.stream)
                g.replay()
                b.record(self.stream)
                per.append((a, b))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in per)


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def traffic_from_profiles(kernel_hash, workload, kernel="k_layer1t"):
    """HBM bytes per launch of a kernel, from the rocprofv3 counter summary
    profiles/<kernel>_<workload>_traffic.txt when it was taken on this exact
    kernel source (its `source_hash:` line), else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
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


def _rel(a, ref):
    import numpy as np
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    d = np.linalg.norm(a - ref)
    return float(d if n == 0 else d / n)


def cpu_baseline(cfg, sample, xhost, gpu=None):
    """The CPU oracle (single-threaded C, fp64) on a bounded sample of steps of the
    timed workload: step t is (replica r, input j) -- routing over all E experts,
    then the k routed and the shared expert's dequantise-and-multiply, combine,
    residual and RMSNorm.  Only the oracle calls are timed.

    When `gpu` holds the library's outputs (idx, w, moe, h, y) for the first
    steps of the sample, they are compared with the oracle's: routing sets
    exactly (a step whose k-th/(k+1)-th logit gap is under 1e-6 is counted as
    excluded and checked with the GPU's own selection), weights to 1e-5 and
    moe/h/y by rel-L2 against 2e-3.  Returns (us per token, GB/s, parity)."""
    import numpy as np
    import oracle
    import synth
    sp = cfg.spec
    gpu = gpu or []
    per_layer = {}
    total = 0.0
    parity = {"tokens": len(gpu), "index_mismatch": 0, "excluded_near_ties": 0,
              "max_w_abs_err": 0.0, "max_rel_l2": {"moe": 0.0, "h": 0.0, "y": 0.0}}
    for t, (r, j) in enumerate(sample):
        if r not in per_layer:
            per_layer[r] = (synth.router(cfg, r), synth.shared_gate(cfg, r), synth.gamma(cfg, r),
                            synth.slab(sp, cfg.seed, r, cfg.E))
        Wr, wsg, gamma, shared = per_layer[r]
        x = xhost[j]
        t0 = time.perf_counter()
        idx, w, lg, gap, _ = oracle.route(Wr, x[None, :], cfg.k)
        total += time.perf_counter() - t0
        sel, wsel = idx[0], w[0]
        if t < len(gpu):
            gidx, gw, gmoe, gh, gy = gpu[t]
            if gap[0] < 1e-6:
                parity["excluded_near_ties"] += 1
                sel = np.asarray(gidx, np.int32)
                z = lg[0][sel] - lg[0][sel].max()
                wsel = np.exp(z) / np.exp(z).sum()
            elif sorted(gidx.tolist()) != sorted(sel.tolist()):
                parity["index_mismatch"] += 1
        slabs = [synth.slab(sp, cfg.seed, r, int(e)) for e in sel]     # untimed input prep
        t0 = time.perf_counter()
        ref = oracle.moe_token(slabs, wsel, shared, cfg.H, cfg.I, sp.bits, sp.group, sp.sbytes,
                               wsg, gamma, cfg.eps, x, x)
        total += time.perf_counter() - t0
        if t < len(gpu):
            order = {int(e): i for i, e in enumerate(gidx)}
            werr = max(abs(float(gw[order[int(e)]]) - float(wv)) for e, wv in zip(sel, wsel)
                       if int(e) in order) if order else 0.0
            parity["max_w_abs_err"] = max(parity["max_w_abs_err"], werr)
            for name, got in (("moe", gmoe), ("h", gh), ("y", gy)):
                parity["max_rel_l2"][name] = max(parity["max_rel_l2"][name],
                                                 _rel(got, ref[name]))
    us = total / len(sample) * 1e6
    nbytes, _ = layer_bytes(cfg)
    if gpu:
        parity["max_w_abs_err"] = float(f"{parity['max_w_abs_err']:.3e}")
        parity["max_rel_l2"] = {k: float(f"{v:.3e}") for k, v in parity["max_rel_l2"].items()}
        parity["pass"] = (parity["index_mismatch"] == 0 and parity["max_w_abs_err"] <= 1e-5
                          and max(parity["max_rel_l2"].values()) <= 2e-3)
    return us, nbytes / (us * 1e-6) / 1e9, parity


def main():
    args = parse()
    if args.gpus != 1:
        msg = (f"--gpus {args.gpus}: this build runs the layer on one GPU only (no multi-GPU "
               "path; the expert-sharded design is described, not built); use --gpus 1")
        print(json.dumps({"error": msg}))
        print(msg, file=sys.stderr)
        sys.exit(2)
    resolve_steps(args)

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
    elif args.workload == "chain60":
        out = bench_chain(args, torch)
    elif args.workload == "deltanet":
        out = bench_deltanet(args, torch)
    elif args.workload == "attention":
        out = bench_attention(args, torch)
    elif args.workload == "stream":
        out = bench_stream(args, torch)
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


def handoff(args, torch):
    if args.no_stream_probe:
        return None
    try:
        import probes
        v = probes.handoff_us(torch)
        return None if v is None else round(v, 3)
    except Exception as exc:  # context only
        print(f"[bench] hand-off probe skipped: {exc}", file=sys.stderr)
        return None


def empty_gap(args, torch):
    if args.no_stream_probe:
        return None
    try:
        import probes
        return round(probes.empty_gap_us(torch), 3)
    except Exception as exc:  # context only
        print(f"[bench] gap probe skipped: {exc}", file=sys.stderr)
        return None


def spread(vals):
    return [round(vals[0], 3), round(vals[len(vals) // 2], 3), round(vals[int(len(vals) * 0.9)], 3)]


TRACE_EVENTS = ["entry", "x staged", "logits stored", "shared SwiGLU published", "top-k known",
                "routed SwiGLU published", "first images in LDS", "sum of squares published",
                "every sum in", "exit", "(unused)", "wave 0 gate/up dots done",
                "wave 3 gate/up dots done", "wave 3 down rows requested", "phase A loads issued",
                "x in registers"]


CHAIN_TRACE_EVENTS = ["layer start", "logits stored", "shared SwiGLU published", "top-k known",
                      "routed SwiGLU published", "first images in LDS", "part published",
                      "every part polled", "next x complete", "down rows requested",
                      "down rows computed"]


def phase_trace(args, torch, fm, step, R, names=TRACE_EVENTS):
    """Wall-clock stamps of a one-token kernel's phase boundaries (trace
    build): per call, each workgroup's time of each event after the first
    workgroup's first event (entry; the traced layer's start in a chain);
    reported as the min / median / max over workgroups, each the median over
    calls."""
    import ctypes as C
    import numpy as np
    nwg, nev = 1024, 16
    buf = torch.zeros(nwg * nev, dtype=torch.int64, device="cuda")
    fm.lib().fmoe_trace_set.argtypes = [C.c_void_p]
    fm.lib().fmoe_trace_set(buf.data_ptr())
    s = torch.cuda.Stream()
    per = []
    for i in range(args.phase_trace + 8):
        buf.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            step(i, s.cuda_stream)
        torch.cuda.synchronize()
        if i < 8:
            continue
        t = buf.view(nwg, nev).cpu().numpy().astype(np.float64)
        live = t[:, 0] > 0
        t0 = t[live, 0].min()
        rows = []
        for e in range(len(names)):
            v = t[live, e]
            v = (v[v > 0] - t0) / 100.0          # 100 MHz ticks -> us
            rows.append((v.min(), np.median(v), v.max()) if v.size else (np.nan,) * 3)
        per.append(rows)
    arr = np.median(np.array(per), axis=0)
    return {"calls": args.phase_trace, "unit": "us after the first workgroup's entry",
            "events": {name: {"min": round(float(a[0]), 3), "median": round(float(a[1]), 3),
                              "max": round(float(a[2]), 3)}
                       for name, a in zip(names, arr) if not np.isnan(a[1])}}


def bench_layer(args, torch):
    import math
    import bit_dequant_expert_amd as fm
    import synth
    if args.phase_trace:
        fm.use_trace_library()

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
    xhost = synth.activations(cfg, XPOOL, pool=0)
    xpool = torch.from_numpy(xhost).to(dev)
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
        # step i: replica i mod R, input vector i mod XPOOL (x is also the residual)
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
    if args.phase_trace:
        print(json.dumps({"phase_trace": phase_trace(args, torch, fm, step, R),
                          "workload": args.workload, "kernel_source_hash": source_hash()}))
        return

    with torch.cuda.stream(s):
        for i in range(8):                      # eager warm-up before capture
            step(i, s.cuda_stream)
    torch.cuda.synchronize()
    period = R * XPOOL // math.gcd(R, XPOOL)
    runner = GraphRunner(torch, s, step, period)
    with torch.cuda.stream(s):
        for i in range(args.steps, args.steps + args.warmup):   # warm-up steps
            step(i, s.cuda_stream)
    torch.cuda.synchronize()
    total_ms, wall_ms = runner.timed_eager(0, args.steps)
    queue_ms = runner.last_queue_ms
    runner.prepare([(0, GRAPH_LEN)])
    rep_us = [v * 1000.0 / GRAPH_LEN for v in runner.spread(0, GRAPH_LEN)]
    timeout_word = int(ws[fm.fmoe_wait_timeout_offset():][:4].view(torch.int32).item())

    ms_per_step = total_ms / args.steps
    us = ms_per_step * 1000.0
    nbytes, ebytes = layer_bytes(cfg)
    gbps = nbytes / (us * 1e-6) / 1e9
    khash = source_hash()
    traffic = traffic_from_profiles(khash, args.workload)
    stream = stream_probe(args, torch)
    gap = empty_gap(args, torch)
    hand = handoff(args, torch)
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
        "dtype": "u4 codes x f16 activations, f32 accumulation (router f64)"
                 if sp.bits == 4 else "u2 codes x f16 activations, f32 accumulation (router f64)",
        "data": "synthetic",
        "config": {"workload": f"moe_layer_{args.workload}_h{cfg.H}_e{cfg.E}_i{cfg.I}"
                               f"_top{cfg.k}+1_batch1",
                   "hidden": cfg.H, "experts": cfg.E, "inter": cfg.I, "top_k": cfg.k,
                   "bits": sp.bits, "group": sp.group, "scale_dtype": "bf16",
                   "batch": 1, "replicas": R, "graph_len": GRAPH_LEN},
        "us_per_layer": round(us, 3),
        "timed_region": {"event_ms": round(total_ms, 4), "host_wall_ms": round(wall_ms, 4),
                         "host_queue_ms": round(queue_ms, 4),
                         "launches": "one per layer forward, queued behind a GPU busy-wait",
                         "note": f"exactly {args.steps} layer forwards between two HIP events on "
                                 f"the launch stream; the busy-wait queued first "
                                 f"({max(SPIN_US, EAGER_SPIN_PER_STEP_US * args.steps)} us) "
                                 "outlasts the host's queueing of every launch (host_queue_ms), "
                                 "so the region holds no host latency; host wall time includes "
                                 "that wait and both synchronisations"},
        "us_per_layer_min_median_p90": spread(rep_us),
        "spread_note": f"20 further replays of one {GRAPH_LEN}-layer HIP graph, outside the "
                       "timed region",
        "moe_layer_tokens_per_s": round(1e6 / us, 1),
        "pct_of_peak_hbm": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "pct_of_measured_stream_ceiling": None if not stream else round(100.0 * gbps / stream, 2),
        "algorithmic_bytes_per_layer": nbytes,
        "expert_bytes_per_layer": ebytes,
        "roofline": {"bound": "hbm", "kernel": "k_layer1t (whole layer, one launch per step)",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "wait_timeout_word": timeout_word,
        "kernel_source_hash": khash,
        "context": {"hbm_stream_read_gbps_measured": stream,
                    "stream_note": "best of 10 passes of a plain 4 GiB streaming read on this GPU",
                    "empty_kernel_gap_us": gap,
                    "gap_note": "per launch, 2000 empty one-wave kernels replayed from one graph",
                    "all_to_all_handoff_us": hand,
                    "handoff_note": "512 workgroups each store one 16-byte record, one wave of "
                                    "each polls all 512 (device-coherent loads and stores): "
                                    "median time until a workgroup has seen them all; the "
                                    "layer has three such hand-offs on its critical path"},
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        sample = [(t % R, t % XPOOL) for t in range(args.cpu_sample)]
        gpu = gpu_sample_outputs(torch, fm, layers, xpool, cfg, sample[:PARITY_TOKENS], ws)
        cus, cgb, parity = cpu_baseline(cfg, sample, xhost, gpu)
        out["cpu_baseline"] = {"value": round(cgb, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{len(sample)} steps of the timed workload (replica "
                                         f"t mod {R}, input t mod {XPOOL}; route over 512 + 5 "
                                         f"experts), {cus:.0f} us/token",
                               "threads": f"1 thread of {os.cpu_count()} host logical cores",
                               "cpu_model": host_cpu_model()}
        out["parity_vs_oracle"] = parity
    return out


PARITY_TOKENS = 4


def gpu_sample_outputs(torch, fm, layers, xpool, cfg, sample, ws):
    """Eager layer forwards on (replica, input) pairs of the timed workload, with
    the routing and moe outputs kept, for comparison with the oracle."""
    out = []
    for r, j in sample:
        x = xpool[j:j + 1]
        h = torch.empty(1, cfg.H, device=x.device)
        y = torch.empty(1, cfg.H, device=x.device)
        moe = torch.empty(1, cfg.H, device=x.device)
        idx = torch.empty(1, cfg.k, dtype=torch.int32, device=x.device)
        w = torch.empty(1, cfg.k, device=x.device)
        fm.fmoe_moe_layer_forward(layers[r], 1, x, x, h, y, idx, w, moe, ws)
        out.append((idx, w, moe, h, y))
    torch.cuda.synchronize()
    return [tuple(t.cpu().numpy()[0] for t in o) for o in out]


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
        runner = GraphRunner(torch, s, lambda i, cs, kind=kind: call(kind, i, cs), NE)
        timed = step_chunks(args.steps, 0)
        warm = step_chunks(args.warmup, args.steps)
        runner.prepare(warm + timed + [(0, GRAPH_LEN)])
        runner.run(warm)
        total_ms, wall_ms = runner.timed(timed)
        us = total_ms * 1000.0 / args.steps
        res[kind] = {"us": round(us, 3), "gbps": round(nbytes[kind] / (us * 1e-6) / 1e9, 1),
                     "bytes": nbytes[kind], "host_wall_ms": round(wall_ms, 4),
                     "us_min_median_p90": spread([v * 1000.0 / GRAPH_LEN
                                                  for v in runner.spread(0, GRAPH_LEN)])}
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
                                         f"{cus:.0f} us/expert",
                               "threads": f"1 thread of {os.cpu_count()} host logical cores",
                               "cpu_model": host_cpu_model()}
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

    import contextlib
    cfg = synth.CONFIGS["layer4"]
    sp = cfg.spec
    NL, T = 60, 32
    # the default (every expert of the batch on the matrix cores), and the
    # configuration's split (experts with >= 16 tokens on the matrix cores, the
    # rest on the multi-token GEMV kernels) beside it
    MODES = ("independent", "chained", "independent_split16", "chained_split16")
    dev = torch.device("cuda:0")
    off, stride = sp.layout()
    print(f"[bench] generating {NL} layers ({NL * stride * (cfg.E + 1) / 1e9:.1f} GB)",
          file=sys.stderr, flush=True)
    fmt, layers = _fmt_and_layers(torch, fm, synth, cfg, range(NL), dev)
    xs_host = synth.activations(cfg, NL * T, pool=4)
    xs = torch.from_numpy(xs_host).to(dev).view(NL, T, cfg.H)
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
            if mode.startswith("independent"):
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
        split = fm.paths(mfma_min_tokens=16) if mode.endswith("split16") else contextlib.nullcontext()
        with split:
            with torch.cuda.stream(s):
                step(mode, s.cuda_stream)                 # eager warm-up before capture
            torch.cuda.synchronize()
            # one graph holds one whole 60-layer step; a chunk of 1 step per graph
            runner = GraphRunner(torch, s, lambda i, cs, mode=mode: step(mode, cs), 1)
            runner.prepare([(0, 1)])                      # the kernels are chosen here
        timed = step_chunks(args.steps, 0, size=1)
        warm = step_chunks(args.warmup, 0, size=1)
        runner.run(warm)
        total_ms, wall_ms = runner.timed(timed)
        rep_ms = runner.spread(0, 1, reps=min(args.steps, 10))
        ms = total_ms / args.steps
        sel = idx[mode].cpu().numpy()
        distinct = [int(np.unique(sel[l]).size) for l in range(NL)]
        counts = [np.bincount(sel[l].ravel(), minlength=cfg.E) for l in range(NL)]
        nbytes = (sum(distinct) + NL) * stride + NL * cfg.E * cfg.H * 4 \
            + NL * (4 * T + 2) * cfg.H * 4
        res[mode] = {"ms_per_step": round(ms, 6), "ms_min_median_p90": spread(rep_ms),
                     "host_wall_ms": round(wall_ms, 3),
                     "tokens_per_s": round(T / (ms * 1e-3), 1),
                     "us_per_layer": round(ms * 1000.0 / NL, 3),
                     "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "algorithmic_bytes_per_step": nbytes,
                     "distinct_routed_experts_per_layer": {
                         "mean": round(float(np.mean(distinct)), 2), "min": min(distinct),
                         "max": max(distinct)},
                     "routed_experts_on_matrix_cores_per_layer": round(
                         float(np.mean([int((c >= 16).sum()) for c in counts])), 3)}
        del runner
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
                   "are the next layer's x and residual; _split16: experts with fewer than 16 "
                   "tokens on the multi-token GEMV kernels instead of the matrix cores",
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
        n = max(1, args.cpu_sample // 2)
        # layer-token t: layer t mod 60, token (7 t) mod 32 of that layer's independent batch
        sample = [(t % NL, (t % NL) * T + (7 * t) % T) for t in range(n)]
        cus, _, _ = cpu_baseline(cfg, sample, xs_host)
        out["cpu_baseline"] = {"value": round(1e6 / (NL * cus), 4), "unit": "tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{n} layer-tokens of the stack's independent-routing "
                                         f"pass (route over 512 + 5 experts), {cus:.0f} us per "
                                         f"layer-token, scaled to 60 layers",
                               "threads": f"1 thread of {os.cpu_count()} host logical cores",
                               "cpu_model": host_cpu_model()}
    return out


def bench_chain(args, torch):
    """Batch-1 decode through 60 distinct 4-bit layers chained on the device
    (each layer's y and h are the next layer's x and residual); a step is the
    whole 60-layer pass for one token: one fmoe_moe_stack_forward call, which
    runs the 60 layers in one launch of the chained one-token kernel.  Each
    layer writes its own h and y, so that sampled layers can be checked against
    the oracle fed the GPU's own layer inputs.  The same pass as 60 one-token
    layer launches in one HIP graph is timed beside it (context)."""
    import ctypes as C
    import numpy as np
    import bit_dequant_expert_amd as fm
    import oracle
    import synth

    if args.phase_trace:
        fm.use_trace_library()
    cfg = synth.CONFIGS["layer4"]
    sp = cfg.spec
    NL = 60
    dev = torch.device("cuda:0")
    off, stride = sp.layout()
    print(f"[bench] generating {NL} layers ({NL * stride * (cfg.E + 1) / 1e9:.1f} GB)",
          file=sys.stderr, flush=True)
    fmt, layers = _fmt_and_layers(torch, fm, synth, cfg, range(NL), dev)
    x0_host = synth.activations(cfg, 1, pool=40)
    x0 = torch.from_numpy(x0_host).to(dev)
    hs = torch.empty(NL, cfg.H, device=dev)
    ys = torch.empty(NL, cfg.H, device=dev)
    idx = torch.empty(NL, cfg.k, dtype=torch.int32, device=dev)
    wts = torch.empty(NL, cfg.k, device=dev)
    ws_bytes = fm.fmoe_workspace_size(layers[0], 1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print("[bench] layers ready", file=sys.stderr, flush=True)
    Lp = [C.addressof(L) for L in layers]
    arr = (fm.fmoe_layer * NL)(*layers)
    lib = fm.lib()

    def step(i, stream):
        rc = lib.fmoe_moe_stack_forward(arr, NL, 1, x0.data_ptr(), x0.data_ptr(), hs.data_ptr(),
                                        ys.data_ptr(), idx.data_ptr(), wts.data_ptr(),
                                        ws.data_ptr(), ws_bytes, stream)
        if rc != 0:
            raise fm.FmoeError(rc, fm.fmoe_last_error())

    def step_layers(i, stream):
        x = r = x0.data_ptr()
        for l in range(NL):
            h, y = hs[l].data_ptr(), ys[l].data_ptr()
            rc = fm.fmoe_moe_layer_forward_raw(Lp[l], 1, x, r, h, y, idx[l].data_ptr(),
                                               wts[l].data_ptr(), None, ws.data_ptr(),
                                               ws_bytes, stream)
            if rc != 0:
                raise fm.FmoeError(rc, fm.fmoe_last_error())
            x, r = y, h

    s = torch.cuda.Stream()
    if args.kernel_steps:
        with torch.cuda.stream(s):
            for i in range(args.kernel_steps):
                step(i, s.cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_steps": args.kernel_steps, "workload": args.workload}))
        return None
    if args.phase_trace:
        print(json.dumps({"phase_trace": phase_trace(args, torch, fm, step, 1,
                                                     names=CHAIN_TRACE_EVENTS),
                          "traced_layer": 1, "workload": args.workload,
                          "kernel_source_hash": source_hash()}))
        return None

    with torch.cuda.stream(s):
        step(0, s.cuda_stream)                  # eager warm-up before capture
    torch.cuda.synchronize()
    runner = GraphRunner(torch, s, lambda i, cs: step(i, cs), 1)
    timed = step_chunks(args.steps, 0, size=1)
    warm = step_chunks(args.warmup, 0, size=1)
    runner.prepare([(0, 1)])
    runner.run(warm)
    total_ms, wall_ms = runner.timed(timed)
    rep_ms = runner.spread(0, 1, reps=min(args.steps, 10))
    timeout_word = int(ws[fm.fmoe_wait_timeout_offset():][:4].view(torch.int32).item())
    # the outputs of the timed pass, for the parity check below
    hs_h, ys_h = hs.cpu().numpy(), ys.cpu().numpy()
    idx_h, w_h = idx.cpu().numpy(), wts.cpu().numpy()
    # context: the same pass as 60 one-token launches in one graph
    with torch.cuda.stream(s):
        step_layers(0, s.cuda_stream)
    torch.cuda.synchronize()
    same_bits = bool(np.array_equal(hs.cpu().numpy(), hs_h) and np.array_equal(ys.cpu().numpy(), ys_h))
    lrunner = GraphRunner(torch, s, lambda i, cs: step_layers(i, cs), 1)
    lrunner.prepare([(0, 1)])
    lrunner.run(warm)
    l_ms, _ = lrunner.timed(timed)
    l_ms /= args.steps
    timeout_word |= int(ws[fm.fmoe_wait_timeout_offset():][:4].view(torch.int32).item())
    ms = total_ms / args.steps
    us_layer = ms * 1000.0 / NL
    nbytes, ebytes = layer_bytes(cfg)
    gbps = nbytes / (us_layer * 1e-6) / 1e9
    khash = source_hash()
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
        "config": {"workload": f"moe_chain60_h{cfg.H}_e{cfg.E}_i{cfg.I}_top{cfg.k}+1_batch1",
                   "layers": NL, "batch": 1, "hidden": cfg.H, "experts": cfg.E,
                   "inter": cfg.I, "top_k": cfg.k, "bits": sp.bits, "group": sp.group,
                   "scale_dtype": "bf16", "resident_slab_gb": round(
                       NL * stride * (cfg.E + 1) / 1e9, 1)},
        "us_per_layer": round(us_layer, 3),
        "decode_tokens_per_s_moe_stack": round(1e3 / ms, 2),
        "ms_min_median_p90": spread(rep_ms),
        "timed_region": {"event_ms": round(total_ms, 4), "host_wall_ms": round(wall_ms, 4),
                         "note": f"exactly {args.steps} 60-layer passes (one graph each) between "
                                 "two HIP events on the launch stream"},
        "pct_of_peak_hbm": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "algorithmic_bytes_per_layer": nbytes,
        "roofline": {"bound": "hbm", "kernel": "k_chain1t (60 layers in one launch)",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_from_profiles(khash, "chain60", kernel="k_chain1t"),
                     "traffic_note": "HBM bytes of one launch (60 layers)"},
        "per_layer_launches": {"us_per_layer": round(l_ms * 1000.0 / NL, 3),
                               "ms_per_step": round(l_ms, 6),
                               "same_bits_as_one_launch": same_bits,
                               "note": "the same pass as 60 one-token layer launches in one "
                                       "HIP graph"},
        "wait_timeout_word": timeout_word,
        "kernel_source_hash": khash,
    }
    # Parity of the timed pass: sampled layers against the oracle on the GPU's
    # own inputs of that layer (teacher forcing); their oracle time is the CPU
    # baseline.
    sample = [0, 1, 29, 58, 59] if args.cpu_sample >= 5 else [0, NL - 1]
    parity = {"layers": sample, "index_mismatch": 0, "excluded_near_ties": 0,
              "max_rel_l2": {"h": 0.0, "y": 0.0}}
    t_oracle = 0.0
    for l in sample:
        x = x0_host[0] if l == 0 else ys_h[l - 1]
        r = x0_host[0] if l == 0 else hs_h[l - 1]
        Wr = synth.router(cfg, l)
        t0 = time.perf_counter()
        ridx, rw, rlg, gap, _ = oracle.route(Wr, x[None, :], cfg.k)
        t_oracle += time.perf_counter() - t0
        sel, wsel = ridx[0], rw[0]
        if gap[0] < 1e-6:
            parity["excluded_near_ties"] += 1
            sel = idx_h[l]
            z = rlg[0][sel] - rlg[0][sel].max()
            wsel = np.exp(z) / np.exp(z).sum()
        elif sorted(idx_h[l].tolist()) != sorted(sel.tolist()):
            parity["index_mismatch"] += 1
        slabs = [synth.slab(sp, cfg.seed, l, int(e)) for e in sel]
        shared = synth.slab(sp, cfg.seed, l, cfg.E)
        t0 = time.perf_counter()
        ref = oracle.moe_token(slabs, wsel, shared, cfg.H, cfg.I, sp.bits, sp.group, sp.sbytes,
                               synth.shared_gate(cfg, l), synth.gamma(cfg, l), cfg.eps, x, r)
        t_oracle += time.perf_counter() - t0
        parity["max_rel_l2"]["h"] = max(parity["max_rel_l2"]["h"], _rel(hs_h[l], ref["h"]))
        parity["max_rel_l2"]["y"] = max(parity["max_rel_l2"]["y"], _rel(ys_h[l], ref["y"]))
    parity["max_rel_l2"] = {k: float(f"{v:.3e}") for k, v in parity["max_rel_l2"].items()}
    parity["pass"] = parity["index_mismatch"] == 0 and max(parity["max_rel_l2"].values()) <= 2e-3
    out["parity_vs_oracle"] = parity
    if not args.no_cpu_baseline:
        cus = t_oracle / len(sample) * 1e6
        out["cpu_baseline"] = {"value": round(1e6 / (NL * cus), 4), "unit": "tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{len(sample)} layers of the timed pass ({sample}), "
                                         f"route over 512 + 5 experts each, {cus:.0f} us per "
                                         "layer, scaled to 60 layers",
                               "threads": f"1 thread of {os.cpu_count()} host logical cores",
                               "cpu_model": host_cpu_model()}
    return out


def bench_deltanet(args, torch):
    """One Gated DeltaNet decode step per timed step: 32 sequences x 64 heads of a
    128 x 128 fp32 state, updated in place; step i works on layer i mod 8's
    state and input set i mod 8.  Algorithmic bytes: the state read and written
    once, plus q, k, v, decay, beta read and the output written."""
    import numpy as np
    import bit_dequant_expert_amd as fm
    import oracle

    B, NH, DK, DV, NL = 32, 64, 128, 128, 8
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(2027)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    states = [(torch.randn(B, NH, DK, DV, generator=g) * 0.3).to(dev) for _ in range(NL)]
    ins = []
    for _ in range(NL):
        ins.append(dict(q=unit(torch.randn(B, NH, DK, generator=g)).to(dev),
                        k=unit(torch.randn(B, NH, DK, generator=g)).to(dev),
                        v=torch.randn(B, NH, DV, generator=g).to(dev),
                        a=torch.empty(B, NH).uniform_(0.5, 1.0, generator=g).to(dev),
                        b=torch.empty(B, NH).uniform_(0.0, 1.0, generator=g).to(dev)))
    out = torch.empty(B, NH, DV, device=dev)
    # a copy of layer 0's state before any step, for the parity check
    s0_host = states[0].cpu().numpy()
    torch.cuda.synchronize()
    lib = fm.lib()

    def step(i, stream):
        l = i % NL
        x = ins[l]
        rc = lib.fmoe_deltanet_step(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
                                    x["a"].data_ptr(), x["b"].data_ptr(), states[l].data_ptr(),
                                    out.data_ptr(), B, NH, DK, DV, stream)
        if rc != 0:
            raise fm.FmoeError(rc, fm.fmoe_last_error())

    s = torch.cuda.Stream()
    # parity first: one step on layer 0 against the oracle (sampled heads)
    with torch.cuda.stream(s):
        step(0, s.cuda_stream)
    torch.cuda.synchronize()
    got_s, got_o = states[0].cpu().numpy(), out.cpu().numpy()
    x0 = {k: v.cpu().numpy() for k, v in ins[0].items()}
    sample_b = [0, 7, 31]
    t0 = time.perf_counter()
    rs, ro = oracle.deltanet_step(x0["q"][sample_b], x0["k"][sample_b], x0["v"][sample_b],
                                  x0["a"][sample_b], x0["b"][sample_b], s0_host[sample_b])
    t_oracle = time.perf_counter() - t0
    worst = 0.0
    for j, b in enumerate(sample_b):
        for h in range(NH):
            worst = max(worst, _rel(got_o[b, h], ro[j, h]), _rel(got_s[b, h], rs[j, h]))
    if args.kernel_steps:
        with torch.cuda.stream(s):
            for i in range(args.kernel_steps):
                step(i, s.cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_steps": args.kernel_steps, "workload": args.workload}))
        return None

    runner = GraphRunner(torch, s, step, NL)
    timed = step_chunks(args.steps, 0)
    warm = step_chunks(args.warmup, args.steps)
    runner.prepare(warm + timed)
    runner.run(warm)
    torch.cuda.synchronize()
    total_ms, wall_ms = runner.timed(timed)
    ms = total_ms / args.steps
    state_bytes = B * NH * DK * DV * 4
    nbytes = 2 * state_bytes + B * NH * (2 * DK + 2 * DV + 2) * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "µs per Gated DeltaNet decode step (32 sequences x 64 heads) & achieved HBM GB/s",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"deltanet_step_b{B}_h{NH}_dk{DK}_dv{DV}", "sequences": B,
                   "heads": NH, "dk": DK, "dv": DV, "layers_rotated": NL},
        "us_per_step": round(ms * 1000.0, 3),
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": "k_deltanet_step",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None},
        "parity_vs_oracle": {"sequences": sample_b, "heads": NH, "max_rel_l2": float(f"{worst:.3e}"),
                             "pass": worst <= 2e-5},
        "timed_region": {"event_ms": round(total_ms, 4), "host_wall_ms": round(wall_ms, 4)},
        "context": {"hbm_stream_read_gbps_measured": stream_probe(args, torch)},
    }
    if not args.no_cpu_baseline:
        us_seq = t_oracle / len(sample_b) * 1e6
        res["cpu_baseline"] = {"value": round(nbytes / (us_seq * B * 1e-6) / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{len(sample_b)} sequences x {NH} heads of the first "
                                         f"step, {us_seq:.0f} us per sequence, scaled to {B}",
                               "threads": f"1 thread of {os.cpu_count()} host logical cores",
                               "cpu_model": host_cpu_model()}
    return res


def bench_attention(args, torch):
    """Decode attention per timed step: 32 sequences, 32 query heads over 2 KV
    heads of dimension 256, bf16 caches of capacity 8192 with lengths drawn in
    [2048, 8192]; step i uses layer i mod 4's caches.  Algorithmic bytes: the
    used part of K and V read once, q read, the output written."""
    import numpy as np
    import bit_dequant_expert_amd as fm
    import oracle
    import synth

    B, NQ, NKV, D, CAP, NL = 32, 32, 2, 256, 8192, 4
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(2028)
    lens_h = rng.integers(2048, CAP + 1, size=B).astype(np.int32)
    g = torch.Generator(device="cpu").manual_seed(2028)
    caches = []
    for _ in range(NL):
        k = torch.randn(B, NKV, CAP, D, generator=g).to(dev).to(torch.bfloat16).view(torch.int16)
        v = torch.randn(B, NKV, CAP, D, generator=g).to(dev).to(torch.bfloat16).view(torch.int16)
        caches.append((k, v))
    qs = [torch.randn(B, NQ, D, generator=g).to(dev) for _ in range(NL)]
    lens = torch.from_numpy(lens_h).to(dev)
    out = torch.empty(B, NQ, D, device=dev)
    wsb = fm.fmoe_attention_workspace_size(B, NKV, D, CAP)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    lib = fm.lib()

    def step(i, stream):
        l = i % NL
        kc, vc = caches[l]
        rc = lib.fmoe_attention_decode(qs[l].data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                       lens.data_ptr(), B, NQ, NKV, D, CAP, 10000.0,
                                       out.data_ptr(), ws.data_ptr(), wsb, stream)
        if rc != 0:
            raise fm.FmoeError(rc, fm.fmoe_last_error())

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(0, s.cuda_stream)
    torch.cuda.synchronize()
    # parity: sampled sequences of the first step against the oracle
    sample_b = [0, 13, 31]
    got = out.cpu().numpy()
    q0 = qs[0].cpu().numpy()
    k0 = caches[0][0].cpu().numpy().view(np.uint16)
    v0 = caches[0][1].cpu().numpy().view(np.uint16)
    t0 = time.perf_counter()
    ref = oracle.attention_decode(q0[sample_b], k0[sample_b], v0[sample_b], lens_h[sample_b])
    t_oracle = time.perf_counter() - t0
    worst = max(_rel(got[b, h], ref[j, h]) for j, b in enumerate(sample_b) for h in range(NQ))
    if args.kernel_steps:
        with torch.cuda.stream(s):
            for i in range(args.kernel_steps):
                step(i, s.cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_steps": args.kernel_steps, "workload": args.workload}))
        return None

    runner = GraphRunner(torch, s, step, NL)
    timed = step_chunks(args.steps, 0)
    warm = step_chunks(args.warmup, args.steps)
    runner.prepare(warm + timed)
    runner.run(warm)
    torch.cuda.synchronize()
    total_ms, wall_ms = runner.timed(timed)
    ms = total_ms / args.steps
    used = int(lens_h.sum())
    nbytes = 2 * NKV * used * D * 2 + 2 * B * NQ * D * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "µs per decode-attention step (32 sequences) & achieved HBM GB/s",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 cache x f32 query (matrix cores, query as two bf16 halves), f32 softmax",
        "data": "synthetic",
        "config": {"workload": f"attention_decode_b{B}_q{NQ}_kv{NKV}_d{D}_cap{CAP}",
                   "sequences": B, "q_heads": NQ, "kv_heads": NKV, "head_dim": D,
                   "cap": CAP, "lens": "uniform [2048, 8192], seed 2028",
                   "mean_len": round(float(lens_h.mean()), 1), "layers_rotated": NL},
        "us_per_step": round(ms * 1000.0, 3),
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": "k_attn_chunk + k_attn_merge",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None},
        "parity_vs_oracle": {"sequences": sample_b, "max_rel_l2": float(f"{worst:.3e}"),
                             "pass": worst <= 1e-4},
        "timed_region": {"event_ms": round(total_ms, 4), "host_wall_ms": round(wall_ms, 4)},
        "context": {"hbm_stream_read_gbps_measured": stream_probe(args, torch)},
    }
    if not args.no_cpu_baseline:
        frac = float(lens_h[sample_b].sum()) / used
        res["cpu_baseline"] = {"value": round(nbytes * frac / t_oracle / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"sequences {sample_b} of the first step "
                                         f"({int(lens_h[sample_b].sum())} positions), "
                                         f"{t_oracle * 1e3:.0f} ms",
                               "threads": f"1 thread of {os.cpu_count()} host logical cores",
                               "cpu_model": host_cpu_model()}
    return res


def bench_stream(args, torch):
    """Host-tier expert streaming at the full layer shape: two layers' 513 slabs
    each in pinned host memory, one HBM slab array shared by both (tags = the
    layer), step i runs layer i mod 2 on input vector i mod 64: route (device),
    fetch the 5 active experts' slabs host -> HBM, layer forward.  Every step
    misses (the other layer left its experts in the slots).  Reported: us per
    layer with streaming, and the host-link bytes of the fetches per second of
    fetch time."""
    import ctypes as C
    import numpy as np
    import bit_dequant_expert_amd as fm
    import synth

    cfg = synth.CONFIGS["layer4"]
    sp = cfg.spec
    off, stride = sp.layout()
    NL = 2
    dev = torch.device("cuda:0")
    nbytes_tier = stride * (cfg.E + 1)
    print(f"[bench] pinning {NL * nbytes_tier / 1e9:.1f} GB of host slabs", file=sys.stderr, flush=True)
    hosts = []
    hbm = torch.empty(nbytes_tier, dtype=torch.uint8, device=dev)
    for l in range(NL):
        synth.fill_device_slabs(hbm.data_ptr(), sp, cfg.seed, l, 0, cfg.E + 1, stride)
        h = torch.empty(nbytes_tier, dtype=torch.uint8, pin_memory=True)
        h.copy_(hbm)
        hosts.append(h)
    torch.cuda.synchronize()
    fmt = fm.qformat(sp.bits, sp.group, sp.sbytes == 2)
    layers, routers = [], []
    for l in range(NL):
        Wr = torch.from_numpy(synth.router(cfg, l)).to(dev)
        wsg = torch.from_numpy(synth.shared_gate(cfg, l)).to(dev)
        gam = torch.from_numpy(synth.gamma(cfg, l)).to(dev)
        routers.append(Wr)
        layers.append(fm.fmoe_layer_desc(cfg.H, cfg.I, cfg.E, cfg.k, fmt, Wr, hbm, stride, wsg,
                                         gam, cfg.eps))
    tags = torch.full((cfg.E + 1,), -1, dtype=torch.int32, device=dev)
    ncp = torch.zeros(1, dtype=torch.int32, device=dev)
    xhost = synth.activations(cfg, XPOOL, pool=0)
    xpool = torch.from_numpy(xhost).to(dev)
    hbuf = torch.empty(XPOOL, cfg.H, device=dev)
    ybuf = torch.empty(XPOOL, cfg.H, device=dev)
    idx = torch.empty(XPOOL, cfg.k, dtype=torch.int32, device=dev)
    wts = torch.empty(XPOOL, cfg.k, device=dev)
    rws_b = fm.fmoe_route_workspace_size(1, cfg.E)
    rws = torch.zeros(rws_b, dtype=torch.uint8, device=dev)
    lws_b = fm.fmoe_workspace_size(layers[0], 1)
    lws = torch.zeros(lws_b, dtype=torch.uint8, device=dev)
    lib = fm.lib()
    Lp = [C.addressof(L) for L in layers]
    row = cfg.H * 4

    def step(i, stream, fetch=True, layer_fwd=True):
        l, j = i % NL, i % XPOOL
        xi = xpool.data_ptr() + j * row
        ii = idx[j].data_ptr()
        rc = lib.fmoe_route_topk(routers[l].data_ptr(), xi, 1, cfg.H, cfg.E, cfg.k, ii,
                                 wts[j].data_ptr(), None, rws.data_ptr(), rws_b, stream)
        if rc == 0 and fetch:
            rc = lib.fmoe_fetch_experts(ii, cfg.k, cfg.E, hosts[l].data_ptr(), stride, stride,
                                        hbm.data_ptr(), tags.data_ptr(), cfg.E + 1, l,
                                        ncp.data_ptr(), stream)
        if rc == 0 and layer_fwd:
            rc = fm.fmoe_moe_layer_forward_raw(Lp[l], 1, xi, xi, hbuf.data_ptr() + j * row,
                                               ybuf.data_ptr() + j * row, None, None, None,
                                               lws.data_ptr(), lws_b, stream)
        if rc != 0:
            raise fm.FmoeError(rc, fm.fmoe_last_error())

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i in range(4):
            step(i, s.cuda_stream)
    torch.cuda.synchronize()
    # parity: a few steps eagerly, outputs against the oracle
    sample = [(i % NL, i % XPOOL) for i in range(4, 8)]
    got = []
    for i in range(4, 8):
        with torch.cuda.stream(s):
            step(i, s.cuda_stream)
        torch.cuda.synchronize()
        j = i % XPOOL
        got.append((idx[j].cpu().numpy(), wts[j].cpu().numpy(), np.zeros(cfg.H),
                    hbuf[j].cpu().numpy(), ybuf[j].cpu().numpy()))
    cus, _, parity = cpu_baseline(cfg, sample, xhost, got)
    parity["max_rel_l2"].pop("moe", None)
    parity["pass"] = (parity["index_mismatch"] == 0 and parity["max_w_abs_err"] <= 1e-5
                      and max(parity["max_rel_l2"].values()) <= 2e-3)
    n0 = int(ncp.item())
    runner = GraphRunner(torch, s, step, NL * XPOOL)
    timed = step_chunks(args.steps, 8)
    warm = step_chunks(args.warmup, 8 + args.steps)
    runner.prepare(warm + timed)
    runner.run(warm)
    torch.cuda.synchronize()
    n1 = int(ncp.item())
    total_ms, wall_ms = runner.timed(timed)
    n2 = int(ncp.item())
    ms = total_ms / args.steps
    # the same steps without the fetch (experts already in HBM for that layer
    # would be the all-hit case): route + layer only
    nofetch = GraphRunner(torch, s, lambda i, cs: step(i, cs, fetch=False), NL * XPOOL)
    nofetch.prepare(timed)
    nf_ms, _ = nofetch.timed(timed)
    copied = (n2 - n1) / args.steps
    link_gbps = copied * stride / max(1e-9, (ms - nf_ms / args.steps) * 1e-3) / 1e9
    nbytes, _ = layer_bytes(cfg)
    return {
        "metric": "µs per MoE layer with host-tier expert streaming (4-bit, hidden 4096, 512 experts)",
        "value": round(ms * 1000.0, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 codes x f16 activations, f32 accumulation (router f64)",
        "data": "synthetic",
        "config": {"workload": f"moe_stream_h{cfg.H}_e{cfg.E}_i{cfg.I}_top{cfg.k}+1_batch1",
                   "layers_alternating": NL, "host_tier_gb": round(NL * nbytes_tier / 1e9, 1),
                   "hbm_tier_gb": round(nbytes_tier / 1e9, 1)},
        "slabs_copied_per_layer": round(copied, 3),
        "us_per_layer_without_fetch": round(nf_ms / args.steps * 1000.0, 3),
        "host_link_gbps_during_fetch": round(link_gbps, 1),
        "fetch_note": "fetch time = step time minus the same steps without the fetch",
        "roofline": {"bound": "host link", "kernel": "k_fetch",
                     "achieved": round(link_gbps, 1), "peak": HOST_LINK_GBPS, "unit": "GB/s",
                     "frac": round(link_gbps / HOST_LINK_GBPS, 4), "traffic": None,
                     "peak_note": "PCIe 5.0 x16, one direction"},
        "parity_vs_oracle": parity,
        "timed_region": {"event_ms": round(total_ms, 4), "host_wall_ms": round(wall_ms, 4)},
        "warmup_copies": n1 - n0,
    }


if __name__ == "__main__":
    main()
