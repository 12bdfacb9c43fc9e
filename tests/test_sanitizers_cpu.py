"""Sanitizer builds of the host code, run on the CPU (no GPU):

  * the oracle (oracle.c) built with address and undefined-behaviour
    sanitizers, with the oracle's own pins run against that build;
  * the oracle's pthread row split built with the thread sanitizer, driven from
    1 to 24 threads (tests/sanitize/oracle_threads.c), which also checks that
    every thread count gives the same bits;
  * the library's host layer (argument validation, workspace sizing, status
    strings in abi.hip) with address and undefined-behaviour sanitizers on the
    host code only, driven by tests/sanitize/abi_host.cpp over valid and
    invalid arguments (every call returns before anything is enqueued).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# sanitizers on the host side of a HIP compile only
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
GCC_ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
REPORT_MARKS = ("AddressSanitizer", "runtime error:", "ThreadSanitizer", "LeakSanitizer")


def _gcc_lib(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout
    return p.strip()


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout, cwd=ROOT)
    out = r.stdout + r.stderr
    return r.returncode, out


def _clean(out):
    return not any(m in out for m in REPORT_MARKS)


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_asan.so")
    rc, out = _run(["gcc", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                    "-shared", "-fPIC", "-pthread", *GCC_ASAN, ORACLE_C, "-o", lib, "-lm"])
    assert rc == 0, out
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{_gcc_lib('libasan.so')}:{_gcc_lib('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               MTP_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    # the override really loads the sanitizer build
    rc, out = _run([sys.executable, "-c", "import oracle; print(oracle.lib()._name)"], env=env)
    assert rc == 0 and out.strip().endswith(lib), out
    rc, out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                    "tests/test_oracle_steps.py", "tests/test_oracle_formats.py",
                    "tests/test_oracle_chain.py", "tests/test_neartie_cpu.py",
                    "-k", "not torch"], env=env, timeout=900)
    assert rc == 0 and _clean(out), out[-4000:]


def test_oracle_threads_under_thread_sanitizer(tmp_path):
    exe = str(tmp_path / "oracle_threads")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fsanitize=thread",
                    os.path.join(SAN, "oracle_threads.c"), ORACLE_C, "-o", exe, "-lm"])
    assert rc == 0, out
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    rc, out = _run([exe], env=env)
    assert rc == 0 and _clean(out) and "threads ok" in out, out[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_layer_under_address_and_ub_sanitizers(tmp_path):
    from mtp_draft_head_embed_amd import build as hip_build
    others = [os.path.join(hip_build.BUILD_DIR, os.path.splitext(f)[0] + ".o")
              for f in hip_build.SOURCES if f != "abi.hip"]
    if not all(os.path.exists(o) for o in others):
        hip_build.build()
    abi_o = str(tmp_path / "abi_san.o")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    *HOST_SANITIZE, "-Xarch_host", "-fno-omit-frame-pointer",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c",
                    os.path.join(ROOT, "mtp_draft_head_embed_amd", "csrc", "abi.hip"),
                    "-o", abi_o])
    assert rc == 0, out
    exe = str(tmp_path / "abi_host")
    link = [CLANGXX if os.path.exists(CLANGXX) else shutil.which("clang++"),
            "-fsanitize=address,undefined", "-std=c++17", os.path.join(SAN, "abi_host.cpp"), abi_o,
            *others, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    rc, out = _run(link)
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    rc, out = _run([exe], env=env)
    assert rc == 0 and _clean(out) and "host layer ok" in out, out[-4000:]
