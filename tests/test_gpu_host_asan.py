"""The C ABI's host code under AddressSanitizer (host side only).

tests/host_asan/abi_driver is built by the repository's build entry point:
the library's *_api.cpp sources and a C++ driver compiled with the sanitizer,
linked with the regular kernel objects. The driver makes every call of
include/onela.h on valid and invalid arguments, with host output buffers of
exactly the documented size, and checks each documented status. Run as a
child process; a sanitizer report fails the test.
"""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_asan", "abi_driver")


def test_abi_host_code_under_address_sanitizer():
    assert os.path.exists(DRIVER), "tests/host_asan/abi_driver is missing: run __graft_entry__.build()"
    env = dict(os.environ)
    # leak checking is off: the HIP runtime's own allocations at exit are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:verify_asan_link_order=0"
    print("[host-asan] running the C-ABI driver", flush=True)
    r = subprocess.run([DRIVER], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout[-2000:])
    print(r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr
    assert r.returncode == 0
    assert ", 0 failed" in r.stdout
