"""The C ABI's host code (argument validation, workspace planning, error strings, the profiling
registry) under AddressSanitizer: api.cpp and profile.cpp are compiled with host-only
-fsanitize=address and run through tests/abi_asan_main.cpp. CPU only; nothing reaches a GPU."""
import os
import subprocess

from block_diffusion_drafting_concat_amd import build


def test_abi_host_code_under_address_sanitizer():
    exe = build.build_asan_driver()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "abi host checks passed" in out
