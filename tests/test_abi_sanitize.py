"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library sources with the sanitizers on the host side only (the
device code is compiled as usual) together with ``abi_sanitize_main.cpp``,
which drives every entry point through its host-side rejections, the empty
batch and the workspace-size functions at the edges of their argument
ranges.  Nothing is launched, so no GPU is needed; any sanitizer report or
unmet expectation fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_prefill_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["prefill_fwd.hip", "prefill_wide.hip", "prefill_d512.hip", "decode_fwd.hip",
           "attn_prefill.cpp"]
# every sanitizer flag applies to the host compilation only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="no hipcc")
def test_host_abi_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", *HOST_SANITIZE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES],
           os.path.join(ROOT, "tests", "abi_sanitize_main.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0 and "ok: 0 failure(s)" in run.stdout, out[-4000:]
