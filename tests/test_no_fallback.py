"""The product path has no fallback: without the HIP library every call fails
loudly, and the package never reaches for the CPU oracle."""
import os
import re

import pytest

import dynamic_lora_moe_amd as dlm

PKG = os.path.dirname(dlm.__file__)


def test_missing_library_raises():
    saved = dlm._lib
    try:
        dlm._lib = None
        with pytest.raises(ImportError):
            dlm.load(os.path.join(PKG, "no_such_libdlm.so"))
        assert dlm._lib is None
    finally:
        dlm._lib = saved


def test_package_does_not_use_the_oracle():
    pat = re.compile(r"^\s*(import|from)\s+oracle\b|\boracle\.", re.M)
    for root, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".c", ".h")):
                with open(os.path.join(root, f), encoding="utf-8", errors="replace") as fh:
                    assert not pat.search(fh.read()), f"{f} refers to the oracle"
