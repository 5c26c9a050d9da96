"""Host-side sanitizer runs (no GPU): the oracle built with AddressSanitizer
and UndefinedBehaviorSanitizer runs its pins, and libhc.so with its host code
(the C ABI's argument validation) built the same way runs the ABI tests.
Each runs in a child Python process with the ASan runtime preloaded (an
uninstrumented interpreter loads the instrumented libraries), leak checks
off (the interpreter's own allocations), and any report fatal.  Device code
is not instrumented (GPU sanitizers are not used here)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer"]


def runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        pytest.skip(f"{name} not found")
    return out


def child_env(extra):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime("libasan.so") + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_oracle_pins_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN,
                           "-Wall", "-o", so, os.path.join(ROOT, "oracle", "hc_oracle.c"), "-lm"])
    tests = [os.path.join(ROOT, "tests", f) for f in (
        "test_oracle_pre.py", "test_oracle_post.py", "test_oracle_storage.py",
        "test_oracle_weights.py", "test_oracle_sinkhorn.py", "test_oracle_backward.py",
        "test_oracle_weights_backward.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=child_env({"HC_ORACLE_SO": so, "OMP_NUM_THREADS": "4"}),
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_abi_validation_under_asan_ubsan(tmp_path):
    from hyper_connections_amd import build
    objdir = build.OBJDIR
    if not os.path.isdir(objdir) or not any(f.endswith(".hip.o") for f in os.listdir(objdir)):
        build.build()
    api_o = str(tmp_path / "hc_api_san.o")
    # host code only: each sanitizer flag follows -Xarch_host
    cmd = [HIPCC, "-x", "hip", *build.CFLAGS, "-g"]
    for f in SAN:
        cmd += ["-Xarch_host", f]
    cmd += ["-c", os.path.join(build.CSRC, "hc_api.cpp"), "-o", api_o]
    subprocess.check_call(cmd)
    objs = [os.path.join(objdir, f) for f in sorted(os.listdir(objdir))
            if f.endswith(".hip.o")]
    so = str(tmp_path / "libhc_san.so")
    subprocess.check_call(["g++", "-shared", "-fPIC", *SAN, "-o", so, *objs, api_o,
                           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=child_env({"HC_LIB": so}), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
