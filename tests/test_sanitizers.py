"""Host AddressSanitizer + UndefinedBehaviorSanitizer build of the block
allocator and the CPU oracle, driven by tests/sanitize/driver.cpp (random
allocator traces with exhaustion and bad ids; the oracle's attention,
scatter and copy on exactly sized buffers).  Host code only: no GPU code is
built with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_305_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_allocator_and_oracle_are_clean_under_asan_and_ubsan(tmp_path):
    oracle_o = str(tmp_path / "oracle.o")
    subprocess.run(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "oracle", "oracle.c"),
                    "-o", oracle_o], check=True)
    exe = str(tmp_path / "driver")
    subprocess.run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
                    os.path.join(CSRC, "pa_allocator.cpp"), os.path.join(CSRC, "pa_error.cpp"),
                    oracle_o, "-lpthread", "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitizer driver: ok" in r.stdout
