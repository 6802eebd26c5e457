"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The HIP sources are compiled for the host only (no device code), with the
sanitizers on the host pass, and linked with a host-memory double of the
HIP runtime (tests/asan/hip_host_double.cpp) and a driver
(tests/asan/host_check.cpp) that exercises the C ABI: ring metadata, pin,
push, staging fences, capsules, the state word, capture refusals, argument
validation and launch planning for the long-history, shared-KV and stack
shapes. Kernel launches are recorded, not run. Runs on the CPU.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "partitioned_kv_cache_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "asan")
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    text = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{text}")
    return r.stdout


def _build():
    os.makedirs(OUT, exist_ok=True)
    objs = []
    procs = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip"):
            o = os.path.join(OUT, f[:-4] + ".o")
            procs.append(subprocess.Popen(
                [HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
                 "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, f), "-o", o],
                stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
            objs.append(o)
    for p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(out)
    for f in ("hip_host_double.cpp", "host_check.cpp"):
        o = os.path.join(OUT, f[:-4] + ".o")
        _run([HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
              "-I", os.path.join(ROOT, "include"), "-I", HERE, "-I", CSRC, "-c", os.path.join(HERE, f), "-o", o])
        objs.append(o)
    # each HIP translation unit names its (absent) device code object; point them all at the double's
    fatbins = sorted({l.split()[-1] for l in _run(["nm", "-u", *objs]).splitlines() if "__hip_fatbin_" in l})
    exe = os.path.join(OUT, "host_check")
    _run([CLANG, "-fsanitize=address,undefined", "-g", *objs, "-o", exe,
          *[f"-Wl,--defsym,{s}=hip_double_fatbin" for s in fatbins]])
    return exe


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and shutil.which("nm")),
                    reason="needs hipcc and the ROCm clang")
def test_host_code_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-6000:]
    assert "0 failure(s)" in report
