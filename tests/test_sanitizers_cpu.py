"""The oracle pins and the C ABI's host validation under AddressSanitizer and
UBSan (CPU only): the sanitizer builds of the oracle (oracle/liboracle_san.so)
and of the ABI layer (libfmoe_san.so, host code instrumented, device code as
built) are loaded in a child interpreter with the sanitizer runtimes
preloaded; any report aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_and_validation_under_sanitizers():
    import bit_dequant_expert_amd as fm
    import oracle.build as ob
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not found")
    if not (os.path.exists(fm.SAN_LIB_PATH) and os.path.exists(ob.SAN_LIB)):
        pytest.skip("sanitizer builds missing (built by __graft_entry__.build())")
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", FMOE_SANITIZER_BUILD="1",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import bit_dequant_expert_amd as fm, oracle; fm.lib(); oracle.lib(); "
             "m = open('/proc/self/maps').read(); "
             "assert 'libfmoe_san' in m and 'liboracle_san' in m and 'libasan' in m")
    subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, check=True, timeout=300)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py", "tests/test_oracle_next_pins.py",
                          "tests/test_abi_cpu.py"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
