"""Build libfmoe.so (the C ABI + HIP kernels) in-tree for gfx950.

    python -m bit_dequant_expert_amd.build

Device code is compiled with hipcc for gfx950 only, one object per
(bits, group) kernel variant plus the common kernels, in parallel; the C ABI
layer is host-only C++.  Packed-fp32 instruction selection is switched off for
device code (the compiler would otherwise form v_pk_*_f32 from ordinary float
code).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfmoe.so")
# Phase-trace variant (FMOE_TRACE): the one-token kernel stamps the wall clock
# at its phase boundaries into a buffer given by fmoe_trace_set (bench.py
# --phase-trace); same kernels otherwise.
TRACE_BUILD = os.path.join(PKG, "_build_trace")
TRACE_LIB = os.path.join(PKG, "libfmoe_trace.so")
INCLUDE = os.path.join(ROOT, "include")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=10"]
VARIANTS = [(4, 32), (4, 64), (2, 32), (2, 64)]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def jobs(trace=False):
    bdir = TRACE_BUILD if trace else BUILD
    os.makedirs(bdir, exist_ok=True)
    hc = hipcc()
    flags = [*COMMON, "-DFMOE_TRACE"] if trace else COMMON
    out = []
    for b, g in VARIANTS:
        obj = os.path.join(bdir, f"fmoe_inst_{b}_{g}.o")
        out.append((obj, [hc, *flags, *DEVICE, "-x", "hip", f"-DFMOE_BITS={b}",
                          f"-DFMOE_GROUP={g}", "-c", os.path.join(CSRC, "fmoe_inst.hip"),
                          "-o", obj]))
    obj = os.path.join(bdir, "fmoe_common.o")
    out.append((obj, [hc, *flags, *DEVICE, "-x", "hip", "-c",
                      os.path.join(CSRC, "fmoe_common.hip"), "-o", obj]))
    for name in ("fmoe_deltanet", "fmoe_attention", "fmoe_stream"):
        obj = os.path.join(bdir, f"{name}.o")
        out.append((obj, [hc, *flags, *DEVICE, "-x", "hip", "-c",
                          os.path.join(CSRC, f"{name}.hip"), "-o", obj]))
    obj = os.path.join(bdir, "fmoe_api.o")
    out.append((obj, [hc, *flags, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                      "-x", "c++", "-c", os.path.join(CSRC, "fmoe_api.cpp"),
                      "-o", obj]))
    return out


# Host-sanitizer variant: the C ABI layer (host-only C++) built by g++ with
# AddressSanitizer and UBSan and linked with the plain build's device objects
# into libfmoe_san.so; CPU use only (validation paths), with the sanitizer
# runtimes preloaded into the interpreter.
SAN_LIB = os.path.join(PKG, "libfmoe_san.so")
SANITIZE = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]


def build_sanitized() -> str:
    if not all(os.path.exists(o) for o, _ in jobs()):   # the plain build's objects
        build()
    obj = os.path.join(BUILD, "fmoe_api_san.o")
    _run(["g++", "-O1", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", *SANITIZE,
          "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC,
          "-c", os.path.join(CSRC, "fmoe_api.cpp"), "-o", obj])
    objs = [o for o, _ in jobs() if not o.endswith("fmoe_api.o")]
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-shared", *SANITIZE, "-o", tmp, obj, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def build(force: bool = True, verbose: bool = False, trace: bool = False) -> str:
    lib_path = TRACE_LIB if trace else LIB
    if not force and os.path.exists(lib_path):
        return lib_path
    js = jobs(trace)
    workers = min(len(js), max(1, (os.cpu_count() or 4)), 8)
    with cf.ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(lambda j: _run(j[1]), js))
    tmp = lib_path + ".tmp"
    logs.append(_run([hipcc(), "-shared", "-fPIC", "-o", tmp, *[o for o, _ in js]]))
    if verbose:
        txt = "\n".join(l for l in logs if l.strip())
        if txt:
            print(txt, file=sys.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose=True, trace="--trace" in sys.argv))
