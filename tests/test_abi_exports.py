"""The built C-ABI library loads on the CPU and exports every function onela.h declares."""
import ctypes
import os
import re

import pytest

from linear_attention_beam_gdn_amd.onela import EXPORTED, LIB_PATH

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "onela.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(onela_[a-z_]+)\s*\(", text)))


def test_header_declares_binding_surface():
    assert declared() == sorted(EXPORTED)


@pytest.mark.skipif(not os.path.exists(LIB_PATH), reason="libonela.so not built (run __graft_entry__.build())")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name
    # pure host functions are callable without a GPU
    lib.onela_status_string.restype = ctypes.c_char_p
    assert lib.onela_status_string(0) == b"ok"
    lib.onela_last_error.restype = ctypes.c_char_p
    assert lib.onela_last_error(None) == b""


PROBE_HEADER = os.path.join(os.path.dirname(HEADER), "onela_probes.h")


def test_probe_library_exports_every_declared_symbol():
    from linear_attention_beam_gdn_amd import probes

    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(onela_[a-z_]+)\s*\(", text)))
    assert names == sorted(probes.EXPORTED)
    if not os.path.exists(probes.PROBE_LIB_PATH):
        pytest.skip("libonela_probes.so not built")
    lib = ctypes.CDLL(probes.PROBE_LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
