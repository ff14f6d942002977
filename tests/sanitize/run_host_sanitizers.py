#!/usr/bin/env python3
"""Host sanitizer run: the C ABI validation layer, the oracle and the input
generator built with AddressSanitizer + UndefinedBehaviorSanitizer, then the
host-only part of the CPU suite run against those builds.

    python tests/sanitize/run_host_sanitizers.py

Builds (into tests/sanitize/_build/, not committed):
  * libcakv_hostsan.so  -- context_attention_kv_amd/csrc/api.cpp (argument
    checks, ring schedule, block classes, grid sizing, workspace sizes) with
    the kernel launchers replaced by host_stubs.cpp (every launcher returns
    an error, so nothing can pass silently);
  * liboracle_san.so    -- oracle/oracle.c;
  * libcakvsynth_san.so -- cakv_synth/synth.c.
Runs tests/test_abi_host.py, test_oracle_pins.py, test_oracle_tiles.py and
test_inputs_and_sizes.py with the sanitizer runtimes preloaded and every
report fatal (halt_on_error / abort_on_error). Leak detection is off: the
Python interpreter and torch keep allocations alive until exit by design.
Exit status: that of pytest (0 = clean).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def main():
    os.makedirs(OUT, exist_ok=True)
    csrc = os.path.join(ROOT, "context_attention_kv_amd", "csrc")
    cakv = os.path.join(OUT, "libcakv_hostsan.so")
    run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
         "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", csrc,
         os.path.join(csrc, "api.cpp"), os.path.join(HERE, "host_stubs.cpp"),
         "-L", "/opt/rocm/lib", "-lamdhip64", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib",
         "-o", cakv])
    orc = os.path.join(OUT, "liboracle_san.so")
    run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", *SAN,
         os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", orc])
    syn = os.path.join(OUT, "libcakvsynth_san.so")
    run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN,
         os.path.join(ROOT, "cakv_synth", "synth.c"), "-lm", "-o", syn])
    rt = [subprocess.run(["gcc", f"-print-file-name={lib}"], capture_output=True, text=True,
                         check=True).stdout.strip() for lib in ("libasan.so", "libubsan.so")]
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": ":".join(rt),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "CAKV_LIB_PATH": cakv, "CAKV_ORACLE_LIB": orc, "CAKV_SYNTH_LIB": syn,
    })
    tests = [os.path.join(ROOT, "tests", t) for t in (
        "test_abi_host.py", "test_oracle_pins.py", "test_oracle_tiles.py",
        "test_inputs_and_sizes.py")]
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
