"""Measurement probes used by bench.py: HBM streaming-read ceiling, empty-kernel
launch gap, and a bounded spin that keeps the GPU busy while the host queues a
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


def spin(us, stream):
    """Enqueue one wave that busy-waits about `us` microseconds on `stream` (an
    integer hipStream_t)."""
    rc = lib().probe_spin(int(us), stream)
    if rc != 0:
        raise RuntimeError(f"probe_spin launch failed: {rc}")
