"""Host code of the C ABI under AddressSanitizer, UndefinedBehaviorSanitizer
and ThreadSanitizer.

Builds the library sources with the sanitizers on the host side only (the
device code is compiled as usual) together with a driver:
``abi_sanitize_main.cpp`` takes every entry point through its host-side
rejections, the empty batch and the workspace-size functions at the edges of
their argument ranges; ``abi_threads_main.cpp`` makes the same kind of calls
from eight threads at once.  Nothing is launched, so no GPU is needed; any
sanitizer report or unmet expectation fails the test.
"""
import os
import shutil
import subprocess

import pytest

from causal_prefill_attention_amd.build_lib import SOURCES  # the library's own list

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_prefill_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# every sanitizer flag applies to the host compilation only
ASAN_UBSAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all",
              "-Xarch_host", "-fno-omit-frame-pointer"]
TSAN = ["-Xarch_host", "-fsanitize=thread"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")),
                                reason="no hipcc")


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    """Builds both sanitizer drivers at the same time."""
    out = tmp_path_factory.mktemp("sanitize")
    jobs = {}
    for name, flags, main in (("asan", ASAN_UBSAN, "abi_sanitize_main.cpp"),
                              ("tsan", TSAN, "abi_threads_main.cpp")):
        exe = str(out / name)
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", *flags,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               *[os.path.join(CSRC, s) for s in SOURCES],
               os.path.join(ROOT, "tests", main), "-o", exe]
        jobs[name] = (exe, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.PIPE, text=True))
    built = {}
    for name, (exe, proc) in jobs.items():
        _, err = proc.communicate(timeout=900)
        built[name] = (exe, proc.returncode, err)
    return built


def test_host_abi_under_address_and_ub_sanitizers(drivers):
    exe, rc, err = drivers["asan"]
    assert rc == 0, err[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0 and "ok: 0 failure(s)" in run.stdout, out[-4000:]


def test_host_abi_under_thread_sanitizer(drivers):
    """All host state is thread-local, so ThreadSanitizer must stay silent
    and every thread must read its own error message."""
    exe, rc, err = drivers["tsan"]
    assert rc == 0, err[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    out = run.stdout + run.stderr
    assert "ThreadSanitizer" not in out, out[-4000:]
    assert run.returncode == 0 and "ok: 0 mismatch(es)" in run.stdout, out[-4000:]
