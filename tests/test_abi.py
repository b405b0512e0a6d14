"""The C-ABI library loads and exports every entry point include/ckv.h
declares (CPU only: no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "ckv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ckv_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ["ckv_create", "ckv_destroy", "ckv_append_kv", "ckv_certified_decode_attention",
              "ckv_dense_decode_attention", "ckv_last_error"]:
        assert s in syms


def test_library_exports_every_declared_symbol():
    from certified_quantized_kv_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libckv.so not built")
    L = ctypes.CDLL(binding.LIB_PATH)
    for s in declared_symbols():
        assert hasattr(L, s), s
    assert sorted(binding.EXPORTED) == declared_symbols()


def test_last_error_is_empty_string_initially():
    from certified_quantized_kv_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libckv.so not built")
    assert binding.lib().ckv_last_error() == b""
