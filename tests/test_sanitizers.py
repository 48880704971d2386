"""AddressSanitizer and UndefinedBehaviorSanitizer builds, run on the CPU.

* The oracle (oracle/lora_oracle.c) under both sanitizers, with leak checks,
  driven by tests/sanitize/oracle_check.c over edge cases (no tokens, rank 1,
  empty slots, negative and too-large slot indices, ragged sizes, bf16 and
  fp32, bias and DoRA terms), each checked against a dense merge.
* The library's host-side argument checks (include/lora_mi355x.h) with the
  host code of the runtime built under both sanitizers (device code as
  usual), driven by tests/sanitize/runtime_check.cpp: every call there returns
  its documented status before any device work, so it runs without a GPU.

The hipcc build takes about a minute; it is kept under tests/sanitize/_build and
redone only when a source changes.
"""
import hashlib
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
BUILD = os.path.join(SAN, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               OMP_NUM_THREADS="2")


def _digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def _build(out, cmd, sources):
    os.makedirs(BUILD, exist_ok=True)
    stamp = out + ".sha256"
    d = _digest(sources, cmd)
    if os.path.exists(out) and os.path.exists(stamp) and open(stamp).read() == d:
        return out
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    assert res.returncode == 0, msgs
    open(stamp, "w").write(d)
    return out


def test_oracle_under_asan_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    srcs = [os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "lora_oracle.c")]
    out = os.path.join(BUILD, "oracle_check")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", "-fopenmp", "-o", out, *srcs, "-lm"]
    _build(out, cmd, srcs)
    res = subprocess.run([out], capture_output=True, text=True, timeout=300,
                         env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "failures: 0" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr


def test_runtime_host_checks_under_asan_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    csrc = os.path.join(ROOT, "lora_adapter_application_amd", "csrc")
    srcs = [os.path.join(csrc, "lora_kernels.hip"), os.path.join(csrc, "lora_saved.hip"),
            os.path.join(csrc, "lora_runtime.cpp"), os.path.join(SAN, "runtime_check.cpp")]
    out = os.path.join(BUILD, "runtime_check")
    # each -fsanitize= applies to the host pass only
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), *srcs, "-o", out]
    _build(out, cmd, srcs + [os.path.join(ROOT, "include", "lora_mi355x.h"),
                             os.path.join(csrc, "lora_internal.h")])
    # the HIP runtime keeps allocations to process exit: no leak report
    res = subprocess.run([out], capture_output=True, text=True, timeout=300,
                         env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "failures: 0" in res.stdout
    assert "runtime error" not in res.stderr
