"""The library's host code (argument validation, workspace planning, the
automatic chunk) built with AddressSanitizer and UndefinedBehaviorSanitizer,
driven by tests/sanitize/abi_host_checks.cpp.  CPU only: the driver makes no
call that reaches a kernel launch.  The device code is compiled as usual and
not instrumented (each -fsanitize flag applies to the host side only)."""
import os
import subprocess

import pytest

from grpo_policy_loss_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    try:
        hipcc = libbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clangxx = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = "/opt/rocm/llvm/bin/clang++"
    objs = []
    procs = []
    for src in libbuild.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        flags = [f for f in libbuild.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE
        cmd = [hipcc, *flags, "-c", os.path.join(libbuild.CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    for cmd, p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out.decode(errors="replace")[-3000:]
    exe = str(tmp_path / "abi_host_checks")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    cmd = [clangxx, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "sanitize", "abi_host_checks.cpp"),
           *objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "host checks passed" in r.stdout
