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
INCLUDE = os.path.join(ROOT, "include")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
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


def jobs():
    os.makedirs(BUILD, exist_ok=True)
    hc = hipcc()
    out = []
    for b, g in VARIANTS:
        obj = os.path.join(BUILD, f"fmoe_inst_{b}_{g}.o")
        out.append((obj, [hc, *COMMON, *DEVICE, "-x", "hip", f"-DFMOE_BITS={b}",
                          f"-DFMOE_GROUP={g}", "-c", os.path.join(CSRC, "fmoe_inst.hip"),
                          "-o", obj]))
    obj = os.path.join(BUILD, "fmoe_common.o")
    out.append((obj, [hc, *COMMON, *DEVICE, "-x", "hip", "-c",
                      os.path.join(CSRC, "fmoe_common.hip"), "-o", obj]))
    obj = os.path.join(BUILD, "fmoe_api.o")
    out.append((obj, [hc, *COMMON, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                      "-x", "c++", "-c", os.path.join(CSRC, "fmoe_api.cpp"),
                      "-o", obj]))
    return out


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    js = jobs()
    workers = min(len(js), max(1, (os.cpu_count() or 4)), 8)
    with cf.ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(lambda j: _run(j[1]), js))
    tmp = LIB + ".tmp"
    logs.append(_run([hipcc(), "-shared", "-fPIC", "-o", tmp, *[o for o, _ in js]]))
    if verbose:
        txt = "\n".join(l for l in logs if l.strip())
        if txt:
            print(txt, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
