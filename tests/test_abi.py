"""The C-ABI library: it builds, loads, and exports every symbol the header declares.

No compute call is made here (no GPU in this environment)."""
import ctypes
import os
import re
import subprocess

import pytest

from lora_adapter_application_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib_path():
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.LIB_PATH


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("lora_slots_create", "lora_slot_load", "lora_apply", "lora_shrink",
                     "lora_expand", "lora_plan_prepare"):
        assert required in names
    assert sorted(binding.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lora_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(lib_path)
    for n in declared_functions():
        assert hasattr(lib, n)


def test_library_carries_gfx950_code(lib_path):
    data = open(lib_path, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings_without_a_device(lib_path):
    binding.load_library(lib_path)
    assert binding.lora_status_string(0) == "ok"
    assert "rank exceeds maximum" in binding.lora_status_string(binding.LORA_ERR_RANK_EXCEEDS_MAX)
    assert binding.lora_status_string(12345) == "unknown status"
