"""Host code under the sanitizers (CPU only): the oracle with AddressSanitizer
and UndefinedBehaviorSanitizer, and the host update of the optimizer offload
(zs_cpu.cpp) with those two and, separately, ThreadSanitizer.  Each is built
with g++ into a throwaway directory from its sources and a small driver in
tests/sanitize/, and must run clean (any finding aborts the driver)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
GXX = shutil.which("g++")
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-pthread"]


def _build_and_run(tmp_path, name, sources, flags, env_extra):
    exe = os.path.join(str(tmp_path), name)
    cmd = [GXX, *COMMON, *flags, "-I", os.path.join(ROOT, "include"), *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower() and "cannot find" in r.stderr:
        pytest.skip(f"sanitizer runtime not installed: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "WARNING: ThreadSanitizer" not in out, out[-4000:]
    return out


ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ASAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


@pytest.mark.skipif(GXX is None, reason="g++ not found")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "oracle_asan",
                         [os.path.join(SAN, "oracle_driver.cpp"),
                          os.path.join(ROOT, "oracle", "zs_oracle.cpp")],
                         ASAN_UBSAN, ASAN_ENV)
    assert "oracle driver: ok" in out


@pytest.mark.skipif(GXX is None, reason="g++ not found")
def test_host_update_under_address_and_undefined_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "cpu_asan",
                         [os.path.join(SAN, "cpu_update_driver.cpp"),
                          os.path.join(ROOT, "adam_zs_shard_amd", "csrc", "zs_cpu.cpp")],
                         ASAN_UBSAN, ASAN_ENV)
    assert "cpu update driver" in out


@pytest.mark.skipif(GXX is None, reason="g++ not found")
def test_host_update_under_thread_sanitizer(tmp_path):
    out = _build_and_run(tmp_path, "cpu_tsan",
                         [os.path.join(SAN, "cpu_update_driver.cpp"),
                          os.path.join(ROOT, "adam_zs_shard_amd", "csrc", "zs_cpu.cpp")],
                         ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"})
    assert "cpu update driver" in out
