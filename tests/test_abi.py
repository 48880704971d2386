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


def _create(lib, max_loras=4, max_rank=16, shapes=((64, 64),), dtype=0, max_tokens=8, device=0,
            out=True):
    arr = (binding._ModuleShape * max(len(shapes), 1))(*[binding._ModuleShape(a, b) for a, b in shapes])
    ctx = ctypes.c_void_p()
    st = lib.lora_slots_create(ctypes.byref(ctx) if out else None, max_loras, max_rank,
                               arr if shapes else None, len(shapes), dtype, max_tokens, device)
    return st, ctx


def test_create_checks_its_arguments_on_the_host(lib_path):
    """lora_slots_create validates every argument before it touches a device, and says
    why in lora_last_error(NULL)."""
    lib = binding.load_library(lib_path)
    last = lambda: (lib.lora_last_error(None) or b"").decode()
    cases = [
        (dict(out=False), binding.LORA_ERR_INVALID_ARGUMENT, "out is NULL"),
        (dict(max_loras=0), binding.LORA_ERR_INVALID_ARGUMENT, "max_loras"),
        (dict(max_loras=257), binding.LORA_ERR_INVALID_ARGUMENT, "max_loras"),
        (dict(max_rank=0), binding.LORA_ERR_INVALID_ARGUMENT, "max_rank"),
        (dict(max_rank=129), binding.LORA_ERR_RANK_EXCEEDS_MAX, "max_rank"),
        (dict(shapes=()), binding.LORA_ERR_INVALID_ARGUMENT, "no modules"),
        (dict(dtype=7), binding.LORA_ERR_INVALID_ARGUMENT, "dtype"),
        (dict(max_tokens=0), binding.LORA_ERR_INVALID_ARGUMENT, "max_tokens"),
        (dict(shapes=((64, 60),)), binding.LORA_ERR_INVALID_ARGUMENT, "multiples of 8"),
        (dict(shapes=((64, 64), (4, 64))), binding.LORA_ERR_INVALID_ARGUMENT, "module 1"),
        (dict(device=-1), binding.LORA_ERR_INVALID_ARGUMENT, "device -1"),
    ]
    for kw, want, text in cases:
        st, ctx = _create(lib, **kw)
        assert st == want, (kw, st, last())
        assert text in last(), (kw, last())
        assert not ctx.value


def test_calls_on_a_null_ctx_fail_cleanly(lib_path):
    lib = binding.load_library(lib_path)
    E = binding.LORA_ERR_INVALID_ARGUMENT
    assert lib.lora_slots_destroy(None) == binding.LORA_OK
    assert lib.lora_slot_clear(None, 0) == E
    assert lib.lora_sync_loads(None) == E
    assert lib.lora_plan_prepare(None, None, 0, None) == E
    assert lib.lora_shrink(None, None, 0, None) == E
    assert lib.lora_expand(None, None, 0, None) == E
    assert lib.lora_apply(None, None, None, None, 0, 0, None) == E


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message, before any GPU use."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
