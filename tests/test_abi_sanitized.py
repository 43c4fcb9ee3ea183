"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is built a second time into a temporary directory with the sanitizers on its host
code only (device code is compiled as usual and never runs here), and the CPU ABI tests run
against that copy in a child process with the sanitizer runtime preloaded: every argument
check, the workspace and layout arithmetic, the alias checks and the timing bookkeeping then
execute instrumented, and any report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_FLAGS = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer")


@pytest.mark.timeout(900)
def test_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    sys.path.insert(0, ROOT)
    from latent_moe_expert_amd import build as B
    lib = B.build(verbose=False, out=str(tmp_path / "libmoe_latent_san.so"), build_dir=str(tmp_path / "obj"),
                  extra_flags=SAN_FLAGS)
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), rt
    env = dict(os.environ, MOE_LATENT_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " passed" in r.stdout, report
