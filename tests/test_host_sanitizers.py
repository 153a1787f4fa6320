"""The host container codec (ternary_quantized_moe_amd/csrc/host_codec.cpp)
built with the host compiler alone under AddressSanitizer and
UndefinedBehaviorSanitizer, and driven by tests/asan/codec_asan.cpp: round
trips, every byte value of every block position, the block reorder and the
error paths, on buffers of exactly the documented sizes.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_codec_under_address_sanitizer(tmp_path):
    exe = tmp_path / "codec_asan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "ternary_quantized_moe_amd", "csrc", "host_codec.cpp"),
           os.path.join(ROOT, "tests", "asan", "codec_asan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    assert res.stdout.strip() == "ok"
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
