"""The library's host C++ under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

allocator.cpp, scheduler.cpp and planner.cpp (the block allocator and slot mapping, the slot
checks, the step builder and the work planner: everything on the host side of the ABI except
the HIP launches and the pinned staging ring) are built with g++ together with
tests/host_sanitize/host_fuzz.cpp and run on seeded random event traces. The sanitizers turn
any out-of-bounds access, use after free, leak or undefined arithmetic into a failure; the
driver checks the allocator books after every event, the step builder's own consistency check
and the planner's coverage invariants.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefill_slot_mapping_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "host_sanitize", "host_fuzz.cpp")] + [
    os.path.join(CSRC, f) for f in ("allocator.cpp", "scheduler.cpp", "planner.cpp")]


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    out = str(tmp_path_factory.mktemp("sanitize") / "host_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *SOURCES, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("the sanitizer runtimes are not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_is_clean_under_asan_and_ubsan(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzz_binary, str(seed), "15"], capture_output=True, text=True, env=env,
                       timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures=0" in r.stdout
    fields = dict(kv.split("=") for kv in r.stdout.split()[1:])
    # the traces reached the cases they are meant to reach
    assert int(fields["exhaustions"]) > 100 and int(fields["shared_admits"]) > 100
    assert int(fields["refusals"]) > 100 and int(fields["preemptions"]) > 0
    assert int(fields["group_items"]) > 100
