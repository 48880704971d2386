"""CPU oracle for the batched multi-adapter LoRA update.

TEST INFRASTRUCTURE ONLY.  The parity tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product library in
``lora_adapter_application_amd`` never imports this package, and this package
never imports the product library: the two share no code.

The arithmetic lives in ``lora_oracle.c`` (plain scalar C, fp64 accumulation,
one round-to-nearest-even into the output dtype).  This module only compiles it
and marshals numpy arrays into it.

What the oracle computes, and which passage of the pages each input follows, is
written at the top of ``lora_oracle.c``.  Every function here is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_pins.py`` (brute-force dense merge,
exact small-integer cases, closed forms, invariants, a library rounding routine
and the example adapter_config of the pages); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liblora_oracle.so")

BF16 = 0
FP32 = 1

# -ffp-contract=off: no fused multiply-add, so each product and sum is one
# rounding in double, in the order the source states.
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11",
          "-shared", "-fPIC", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/_build/liblora_oracle.so``."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.lora_oracle_scale.restype = ctypes.c_double
    lib.lora_oracle_scale.argtypes = [ctypes.c_double, ctypes.c_int32, ctypes.c_int32]
    lib.lora_oracle_adapter_bytes.restype = ctypes.c_int64
    lib.lora_oracle_adapter_bytes.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32]
    lib.lora_oracle_round_bf16.restype = ctypes.c_uint16
    lib.lora_oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.lora_oracle_apply.restype = ctypes.c_int64
    lib.lora_oracle_apply.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3 + [
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    lib.lora_oracle_apply_ex.restype = ctypes.c_int64
    lib.lora_oracle_apply_ex.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3 + [
        ctypes.c_int32] + [ctypes.c_void_p] * 7 + [ctypes.c_int32]
    lib.lora_oracle_apply_saved.restype = ctypes.c_int64
    lib.lora_oracle_apply_saved.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3 + [
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    lib.lora_oracle_max_threads.restype = ctypes.c_int32
    lib.lora_oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def scale(lora_alpha: float, r: int, use_rslora: bool) -> float:
    """The adapter scale in double: lora_alpha / r, or lora_alpha / sqrt(r)."""
    return float(_load().lora_oracle_scale(float(lora_alpha), int(r), int(bool(use_rslora))))


def adapter_bytes(shapes: Sequence[tuple], targeted: Sequence[bool], r: int,
                  bytes_per_param: int) -> int:
    """sum over targeted linears of (d_in + d_out) * r * bytes_per_param."""
    d_in = np.ascontiguousarray([s[0] for s in shapes], dtype=np.int32)
    d_out = np.ascontiguousarray([s[1] for s in shapes], dtype=np.int32)
    tg = np.ascontiguousarray([1 if t else 0 for t in targeted], dtype=np.int32)
    return int(_load().lora_oracle_adapter_bytes(d_in.ctypes.data, d_out.ctypes.data,
                                                 tg.ctypes.data, len(shapes), int(r),
                                                 int(bytes_per_param)))


def round_bf16(v: float) -> int:
    """bf16 bit pattern of the double v, round to nearest even (the oracle's own)."""
    return int(_load().lora_oracle_round_bf16(float(v)))


def max_threads() -> int:
    return int(_load().lora_oracle_max_threads())


def apply(dtype: int, x: np.ndarray, y: np.ndarray, idx: np.ndarray,
          adapters: Sequence[Optional[dict]], n_threads: int = 0) -> np.ndarray:
    """Return y after applying one module's LoRA update; y itself is not modified.

    dtype     BF16 (x, y, weights are uint16 bf16 bit patterns) or FP32 (float32)
    x         [T, d_in];  y  [T, d_out];  idx  int32 [T]
    adapters  one entry per slot (or per adapter id): None when the slot is empty
              or the module is not targeted, else a dict with keys
              ``r``, ``lora_alpha``, ``use_rslora``, ``At`` (r x d_in) and ``B`` (r x d_out),
              and optionally ``bias`` (d_out values of the data dtype) and
              ``dora_scale`` (d_out floats): y <- round(g * (y + s * x A B) + c)
    """
    lib = _load()
    elem = np.uint16 if dtype == BF16 else np.float32
    x = np.ascontiguousarray(x, dtype=elem)
    out = np.array(y, dtype=elem, copy=True, order="C")
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, d_in = x.shape
    d_out = out.shape[1]
    assert out.shape[0] == T and idx.shape == (T,)
    n = len(adapters)
    rank = np.zeros(n, dtype=np.int32)
    alpha = np.zeros(n, dtype=np.float64)
    rs = np.zeros(n, dtype=np.int32)
    keep = []
    At_ptrs = (ctypes.c_void_p * max(n, 1))()
    B_ptrs = (ctypes.c_void_p * max(n, 1))()
    c_ptrs = (ctypes.c_void_p * max(n, 1))()
    g_ptrs = (ctypes.c_void_p * max(n, 1))()
    extras = False
    for k, a in enumerate(adapters):
        if a is None:
            continue
        At = np.ascontiguousarray(a["At"], dtype=elem)
        B = np.ascontiguousarray(a["B"], dtype=elem)
        r = int(a["r"])
        assert At.shape == (r, d_in) and B.shape == (r, d_out), (At.shape, B.shape, r)
        rank[k] = r
        alpha[k] = float(a["lora_alpha"])
        rs[k] = 1 if a.get("use_rslora", False) else 0
        At_ptrs[k] = At.ctypes.data
        B_ptrs[k] = B.ctypes.data
        keep.append((At, B))
        if a.get("bias") is not None:
            c = np.ascontiguousarray(a["bias"], dtype=elem)
            assert c.shape == (d_out,), c.shape
            c_ptrs[k] = c.ctypes.data
            keep.append(c)
            extras = True
        if a.get("dora_scale") is not None:
            g = np.ascontiguousarray(a["dora_scale"], dtype=np.float64)
            assert g.shape == (d_out,), g.shape
            g_ptrs[k] = g.ctypes.data
            keep.append(g)
            extras = True
    if T == 0:
        return out
    if extras:
        lib.lora_oracle_apply_ex(dtype, T, d_in, d_out, x.ctypes.data, out.ctypes.data,
                                 idx.ctypes.data, n, rank.ctypes.data, alpha.ctypes.data,
                                 rs.ctypes.data, ctypes.cast(At_ptrs, ctypes.c_void_p),
                                 ctypes.cast(B_ptrs, ctypes.c_void_p),
                                 ctypes.cast(c_ptrs, ctypes.c_void_p),
                                 ctypes.cast(g_ptrs, ctypes.c_void_p), int(n_threads))
    else:
        lib.lora_oracle_apply(dtype, T, d_in, d_out, x.ctypes.data, out.ctypes.data,
                              idx.ctypes.data, n, rank.ctypes.data, alpha.ctypes.data,
                              rs.ctypes.data, ctypes.cast(At_ptrs, ctypes.c_void_p),
                              ctypes.cast(B_ptrs, ctypes.c_void_p), int(n_threads))
    del keep
    return out


def apply_saved(dtype: int, x: np.ndarray, y: np.ndarray, idx: np.ndarray,
                saved: Sequence[Optional[dict]], n_threads: int = 0) -> np.ndarray:
    """Return y after the saved modules ("modules_to_save") replace the base
    output of their adapters' tokens; y itself is not modified.

    saved  one entry per slot (or adapter id): None when it saves no copy of this
           module, else a dict with ``W`` (d_out x d_in, the data dtype) and
           optionally ``bias`` (d_out values): y[t] <- round(x[t] . W^T + bias)
    """
    lib = _load()
    elem = np.uint16 if dtype == BF16 else np.float32
    x = np.ascontiguousarray(x, dtype=elem)
    out = np.array(y, dtype=elem, copy=True, order="C")
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, d_in = x.shape
    d_out = out.shape[1]
    assert out.shape[0] == T and idx.shape == (T,)
    n = len(saved)
    W_ptrs = (ctypes.c_void_p * max(n, 1))()
    c_ptrs = (ctypes.c_void_p * max(n, 1))()
    keep = []
    for k, e in enumerate(saved):
        if e is None:
            continue
        W = np.ascontiguousarray(e["W"], dtype=elem)
        assert W.shape == (d_out, d_in), W.shape
        W_ptrs[k] = W.ctypes.data
        keep.append(W)
        if e.get("bias") is not None:
            c = np.ascontiguousarray(e["bias"], dtype=elem)
            assert c.shape == (d_out,), c.shape
            c_ptrs[k] = c.ctypes.data
            keep.append(c)
    if T == 0:
        return out
    lib.lora_oracle_apply_saved(dtype, T, d_in, d_out, x.ctypes.data, out.ctypes.data,
                                idx.ctypes.data, n, ctypes.cast(W_ptrs, ctypes.c_void_p),
                                ctypes.cast(c_ptrs, ctypes.c_void_p), int(n_threads))
    del keep
    return out
