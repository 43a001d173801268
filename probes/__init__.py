"""Measurement probes used by bench.py: HBM streaming-read ceiling, empty-kernel
launch gap, the latency of an all-to-all hand-off through device-coherent
records, and a bounded spin that keeps the GPU busy while the host queues a
timed region.  Not part of the MoE layer."""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "probes.hip")
LIB = os.path.join(HERE, "libfmoe_probes.so")
_lib = None


def build():
    import subprocess
    from bit_dequant_expert_amd.build import DEVICE, hipcc
    tmp = LIB + ".tmp"
    res = subprocess.run([hipcc(), *DEVICE, "-O3", "-fPIC", "-shared", "-x", "hip", SRC, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(res.stdout + res.stderr)
    os.replace(tmp, LIB)


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(LIB)
        L.probe_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p]
        L.probe_empty.argtypes = [C.c_int, C.c_void_p]
        L.probe_spin.argtypes = [C.c_int, C.c_void_p]
        L.probe_handoff.argtypes = [C.c_void_p, C.c_int, C.c_uint32, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib


def stream_read_gbps(torch, nbytes=4 << 30, reps=10, grid=None):
    """Best-of-reps GB/s of one read pass over a fresh `nbytes` buffer."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    props = torch.cuda.get_device_properties(0)
    grid = grid or props.multi_processor_count * 8
    s = torch.cuda.current_stream()
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        lib().probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, s.cuda_stream)
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return best


def empty_gap_us(torch, n=2000):
    """Average time per launch of an empty one-wave kernel, n launches replayed
    from one HIP graph: the fixed cost of a kernel boundary on this GPU."""
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(n):
            lib().probe_empty(1, cs)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1000.0 / n


def handoff_us(torch, grid=512, reps=24):
    """All-to-all hand-off on `grid` workgroups (as many as the one-token layer
    runs): every workgroup stores one 16-byte record, one wave of each polls
    all of them.  Per launch, the median over workgroups of the time from the
    first workgroup's start until the workgroup has seen every record; the
    median of that over launches (the first 4 dropped).  None if a wait gave up."""
    rec = torch.zeros(grid * 16, dtype=torch.uint8, device="cuda")
    st = torch.zeros(grid * 2, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    meds = []
    for r in range(reps):
        rc = lib().probe_handoff(rec.data_ptr(), grid, r + 1, st.data_ptr(), s)
        if rc != 0:
            raise RuntimeError(f"probe_handoff launch failed: {rc}")
        torch.cuda.synchronize()
        h = st.view(grid, 2).cpu()
        if bool((h[:, 1] == 0).any()):
            return None
        if r >= 4:
            meds.append(float(((h[:, 1] - h[:, 0].min()).double() / 100.0).median()))
    meds.sort()
    return meds[len(meds) // 2]


def spin(us, stream):
    """Enqueue one wave that busy-waits about `us` microseconds on `stream` (an
    integer hipStream_t)."""
    rc = lib().probe_spin(int(us), stream)
    if rc != 0:
        raise RuntimeError(f"probe_spin launch failed: {rc}")
