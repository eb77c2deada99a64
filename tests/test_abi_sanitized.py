"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's own sources are compiled with both sanitizers on the host side
only (each -fsanitize= flag behind -Xarch_host; the device code is built as
usual and never runs here), linked against the shared sanitizer runtime, and
test_abi_cpu.py is run against that build in a child process with the runtime
preloaded.  Every check there goes through the entry points' argument
validation, workspace arithmetic and error reporting; a sanitizer report
(out-of-bounds access, use after free, signed overflow, an out-of-range enum
value, ...) halts the child with a non-zero status.  The build lands in
_build/sanitized/ next to the package and is reused while the sources are
unchanged (about two minutes the first time).
"""

import glob
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_delta_rule_diag_amd")
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "_build", "sanitized")
LIB = os.path.join(OUT, "libkda_sanitized.so")
HIPCC = "/opt/rocm/bin/hipcc"
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_prefill.hip", "kda_backward.hip"]
# host-side sanitizers only: each flag directly behind -Xarch_host
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()


def runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def sources_digest():
    h = hashlib.sha256()
    files = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, "kda_internal.h"),
                                                          os.path.join(INCLUDE, "kda.h")]
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def build():
    os.makedirs(OUT, exist_ok=True)
    stamp = os.path.join(OUT, "sources.sha256")
    digest = sources_digest()
    if os.path.exists(LIB) and os.path.exists(stamp) and open(stamp).read() == digest:
        return
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", *HOST_SANITIZE,
              "-I", INCLUDE, "-I", CSRC]
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        dev = []
        if src.endswith(".hip"):
            dev = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
        cmd = [HIPCC, *dev, *common, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    for src, p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, f"compiling {src} failed:\n{out[-4000:]}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *HOST_SANITIZE, *objs,
           "-o", LIB, "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    with open(stamp, "w") as f:
        f.write(digest)


@pytest.mark.skipif(not os.path.exists(HIPCC) or runtime() is None,
                    reason="hipcc or the sanitizer runtime is not installed")
def test_abi_checks_pass_under_address_and_undefined_behavior_sanitizers():
    build()
    env = dict(os.environ)
    env.update({
        "KDA_ABI_LIB": LIB,
        "LD_PRELOAD": runtime(),
        # Python itself is not instrumented: its allocations are not leaks of ours
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "Sanitizer" not in r.stdout + r.stderr, tail
