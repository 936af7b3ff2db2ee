"""The library's host logic (plan validation and layout, the replay schedule,
the static schedule builder, status and error texts, the host-side progress
wait) built with the compiler's sanitizers and driven on the CPU:
AddressSanitizer + UndefinedBehaviorSanitizer (any report aborts the run) over
the plain-C ABI program and a seeded stress of random task tables and
schedules, and ThreadSanitizer over the same stress from 8 threads at once
(separate plans and schedules are documented as usable from different
threads). These sources contain no HIP code; the GPU part of the library is
not built here."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bf16_fp8_weight_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("plan.cpp", "schedule.cpp", "host_api.cpp")] + [
    os.path.join(SAN, "plan_error_stub.cpp")]
INC = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _build(tmp_path, name, flags, extra_sources=(), c_source=None):
    objs = []
    if c_source:
        obj = str(tmp_path / (name + "_c.o"))
        subprocess.run(["gcc", "-std=c99", "-g", "-O1", *flags, *INC, "-c", c_source, "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-g", "-O1", *flags, *INC, *extra_sources, *HOST_SOURCES, *objs, "-o", exe,
                    "-lpthread"], check=True)
    return exe


def _run(exe, args, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=env)
    return r


ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ASAN_ENV = {"ASAN_OPTIONS": "halt_on_error=1:detect_leaks=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def test_c_abi_program_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, "c_abi_asan", ASAN, c_source=os.path.join(ROOT, "tests", "c_abi", "c_abi_check.c"))
    r = _run(exe, [], ASAN_ENV)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]


def test_host_stress_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, "host_stress_asan", ASAN, extra_sources=[os.path.join(SAN, "host_stress.cpp")])
    r = _run(exe, ["2000", "2"], ASAN_ENV)
    assert r.returncode == 0 and "host stress ok" in r.stdout, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]


def test_host_stress_under_tsan_from_eight_threads(tmp_path):
    exe = _build(tmp_path, "host_stress_tsan", ["-fsanitize=thread"],
                 extra_sources=[os.path.join(SAN, "host_stress.cpp")])
    r = _run(exe, ["300", "8"], {"TSAN_OPTIONS": "halt_on_error=1"})
    if r.returncode != 0 and "FATAL: ThreadSanitizer: unexpected memory mapping" in r.stderr:
        pytest.skip("ThreadSanitizer cannot run in this process environment (memory layout)")
    assert r.returncode == 0 and "host stress ok" in r.stdout, r.stdout + r.stderr[-4000:]
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
