"""The CPU code built with the host compiler's address and undefined-behaviour sanitizers: the
oracle (oracle.c), the input generator (gen.c) and libmoe's host helpers (host.cpp) are compiled
with -fsanitize=address,undefined into a scratch directory, and the oracle pins and the host-helper
checks run against those builds in a child process (the sanitizer runtime preloaded).  Any report
of an out-of-bounds access, use after free or undefined behaviour fails the run."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fPIC", "-shared"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_oracle_generator_and_host_helpers_under_sanitizers():
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("the host compiler has no address-sanitizer runtime")
    with tempfile.TemporaryDirectory() as d:
        libs = {
            "MOE_ORACLE_LIB": (["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                                os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], "liboracle_san.so"),
            "MOE_SYNTH_LIB": (["gcc", "-std=c11", "-ffp-contract=off", "-fopenmp",
                               os.path.join(ROOT, "synth", "gen.c"), "-lm"], "libsynth_san.so"),
            "MOE_HOST_LIB": (["g++", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                              "-D__HIP_PLATFORM_AMD__",
                              os.path.join(ROOT, "quantized_moe_routed_amd", "csrc", "host.cpp")], "libmoehost_san.so"),
        }
        env = dict(os.environ)
        for var, (cmd, out) in libs.items():
            path = os.path.join(d, out)
            r = subprocess.run(cmd[:1] + SAN + cmd[1:] + ["-o", path], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr
            env[var] = path
        env["LD_PRELOAD"] = asan
        logs = os.path.join(d, "san")
        env["ASAN_OPTIONS"] = f"detect_leaks=0:abort_on_error=0:halt_on_error=1:log_path={logs}"
        env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}"
        env["OMP_NUM_THREADS"] = "4"
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                            os.path.join(ROOT, "tests", "asan_host_helpers.py")],
                           cwd=os.path.join(ROOT, "tests"), env=env, capture_output=True, text=True, timeout=900)
        out = r.stdout + r.stderr
        for f in sorted(os.listdir(d)):
            if f.startswith("san"):
                out += open(os.path.join(d, f)).read()
        assert r.returncode == 0, out[-4000:]
        assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
        assert " passed" in out and "skipped" not in out.split("\n")[-2], out[-2000:]
