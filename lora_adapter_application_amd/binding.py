"""ctypes binding of ``include/lora_mi355x.h`` (argument marshalling only).

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors (device memory and streams come from torch; torch does no
arithmetic here): their pointers and sizes are passed to the library, which
runs every step of the update in its own HIP kernels.  A non-zero status
raises ``LoraError`` carrying the status and the library's detail message.

The library must have been built (``python -m lora_adapter_application_amd.build``);
there is no fallback: a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build is the only library the binding loads.
LIB_PATH = os.path.join(PKG, "liblora_mi355x.so")

LORA_BF16 = 0
LORA_FP32 = 1

LORA_OK = 0
LORA_ERR_INVALID_ARGUMENT = -1
LORA_ERR_RANK_EXCEEDS_MAX = -2
LORA_ERR_SLOT_OUT_OF_RANGE = -3
LORA_ERR_BAD_MODULE = -4
LORA_ERR_TOO_MANY_TOKENS = -5
LORA_ERR_HOST_NOT_PINNED = -6
LORA_ERR_OUT_OF_MEMORY = -7
LORA_ERR_HIP = -8
LORA_ERR_NO_PLAN = -9

LORA_FLAG_SLOT_INDEX_TOO_LARGE = 0x1
LORA_FLAG_FUSED_TIMEOUT = 0x2

# Every symbol the header declares, for the export check.
EXPORTS = ("lora_slots_create", "lora_slots_destroy", "lora_slot_load", "lora_slot_load_ex",
           "lora_slot_load_saved", "lora_slot_clear",
           "lora_sync_loads", "lora_plan_prepare", "lora_plan_prepare_slots", "lora_shrink",
           "lora_expand", "lora_apply",
           "lora_shrink_group", "lora_expand_group", "lora_apply_group",
           "lora_apply_group_noalloc", "lora_apply_group_fused",
           "lora_get_device_flags", "lora_get_stats", "lora_profile_begin", "lora_profile_end",
           "lora_status_string", "lora_last_error")

LORA_MAX_GROUP = 8


class LoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class _ModuleShape(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32)]


class _Profile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 5), ("total_ms", ctypes.c_double * 5),
                ("untimed", ctypes.c_int64)]


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("loads", "clears", "bytes_loaded", "plans", "shrinks", "expands", "tokens")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m lora_adapter_application_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    P, I32, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    sig = {
        "lora_slots_create": ([ctypes.POINTER(P), I32, I32, ctypes.POINTER(_ModuleShape), I32,
                               I32, I32, I32], ctypes.c_int),
        "lora_slots_destroy": ([P], ctypes.c_int),
        "lora_slot_load_ex": ([P, I32, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P),
                               ctypes.POINTER(P), I32, D, I32], ctypes.c_int),
        "lora_slot_load": ([P, I32, ctypes.POINTER(P), ctypes.POINTER(P), I32, D, I32],
                           ctypes.c_int),
        "lora_slot_load_saved": ([P, I32, I32, P, P], ctypes.c_int),
        "lora_slot_clear": ([P, I32], ctypes.c_int),
        "lora_sync_loads": ([P], ctypes.c_int),
        "lora_plan_prepare": ([P, P, I32, P], ctypes.c_int),
        "lora_plan_prepare_slots": ([P, P, I32, P, I32, P], ctypes.c_int),
        "lora_shrink": ([P, P, I32, P], ctypes.c_int),
        "lora_expand": ([P, P, I32, P], ctypes.c_int),
        "lora_apply": ([P, P, P, P, I32, I32, P], ctypes.c_int),
        "lora_shrink_group": ([P, I32, ctypes.POINTER(I32), ctypes.POINTER(P), P], ctypes.c_int),
        "lora_expand_group": ([P, I32, ctypes.POINTER(I32), ctypes.POINTER(P), P], ctypes.c_int),
        "lora_apply_group": ([P, I32, ctypes.POINTER(I32), ctypes.POINTER(P), ctypes.POINTER(P),
                              P, I32, P], ctypes.c_int),
        "lora_apply_group_noalloc": ([P, I32, ctypes.POINTER(I32), ctypes.POINTER(P),
                                      ctypes.POINTER(P), P, I32, P], ctypes.c_int),
        "lora_apply_group_fused": ([P, I32, ctypes.POINTER(I32), ctypes.POINTER(P),
                                    ctypes.POINTER(P), P, I32, P], ctypes.c_int),
        "lora_get_device_flags": ([P, ctypes.POINTER(ctypes.c_uint32)], ctypes.c_int),
        "lora_get_stats": ([P, ctypes.POINTER(_Stats)], ctypes.c_int),
        "lora_profile_begin": ([P, I32], ctypes.c_int),
        "lora_profile_end": ([P, ctypes.POINTER(_Profile)], ctypes.c_int),
        "lora_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "lora_last_error": ([P], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, ctx=None):
    if status != LORA_OK:
        lib = load_library()
        detail = (lib.lora_last_error(ctx) or b"").decode()
        text = lib.lora_status_string(status).decode()
        raise LoraError(status, f"{text}: {detail}" if detail else text)
    return status


def _ptr(t) -> Optional[int]:
    """Device or host pointer of a tensor, or an int address passed through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:      # the raw handle, without building a Stream object
            return int(raw(torch.cuda.current_device())) or None
        return int(torch.cuda.current_stream().cuda_stream) or None
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _require_cuda(t, name, dtype=None, numel=None):
    if isinstance(t, int):
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)

def lora_status_string(status: int) -> str:
    return load_library().lora_status_string(int(status)).decode()


def lora_last_error(ctx=None) -> str:
    return (load_library().lora_last_error(ctx) or b"").decode()


def lora_slots_create(max_loras: int, max_rank: int, modules: Sequence[Sequence[int]],
                      dtype: int = LORA_BF16, max_tokens: int = 8192, device: int = 0):
    """Returns an opaque ctx handle (int)."""
    lib = load_library()
    arr = (_ModuleShape * len(modules))(*[_ModuleShape(int(a), int(b)) for a, b in modules])
    out = ctypes.c_void_p()
    st = lib.lora_slots_create(ctypes.byref(out), int(max_loras), int(max_rank), arr,
                               len(modules), int(dtype), int(max_tokens), int(device))
    _check(st, None)
    return out.value


def lora_slots_destroy(ctx) -> None:
    _check(load_library().lora_slots_destroy(ctx), ctx)


def lora_slot_load(ctx, slot: int, A_t: Sequence, B: Sequence, r: int, lora_alpha: float,
                   use_rslora: bool = False) -> None:
    """A_t[m] / B[m]: pinned host or device tensors (or int addresses), None = not targeted."""
    n = len(A_t)
    if len(B) != n:
        raise ValueError("A_t and B must have one entry per module")
    a_arr = (ctypes.c_void_p * n)(*[_ptr(a) for a in A_t])
    b_arr = (ctypes.c_void_p * n)(*[_ptr(b) for b in B])
    _check(load_library().lora_slot_load(ctx, int(slot), a_arr, b_arr, int(r), float(lora_alpha),
                                         int(bool(use_rslora))), ctx)


def lora_slot_load_ex(ctx, slot: int, A_t: Sequence, B: Sequence, bias: Optional[Sequence],
                      dora_scale: Optional[Sequence], r: int, lora_alpha: float,
                      use_rslora: bool = False) -> None:
    """lora_slot_load with per-module output bias (ctx dtype) and DoRA factors (float32),
    each a sequence with one entry per module, or None."""
    n = len(A_t)
    if len(B) != n or (bias is not None and len(bias) != n) or \
            (dora_scale is not None and len(dora_scale) != n):
        raise ValueError("one entry per module in A_t, B, bias and dora_scale")
    arr = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts]) if ts is not None else None
    _check(load_library().lora_slot_load_ex(ctx, int(slot), arr(A_t), arr(B), arr(bias),
                                            arr(dora_scale), int(r), float(lora_alpha),
                                            int(bool(use_rslora))), ctx)


def lora_slot_load_saved(ctx, slot: int, module: int, W, bias=None) -> None:
    """A whole saved copy of one module for the adapter in `slot`: W is d_out x d_in
    (pinned host or device tensor, ctx dtype), bias d_out values or None."""
    _check(load_library().lora_slot_load_saved(ctx, int(slot), int(module), _ptr(W), _ptr(bias)),
           ctx)


def lora_slot_clear(ctx, slot: int) -> None:
    _check(load_library().lora_slot_clear(ctx, int(slot)), ctx)


def lora_sync_loads(ctx) -> None:
    _check(load_library().lora_sync_loads(ctx), ctx)


def lora_plan_prepare(ctx, token_slot_idx, n_tokens: Optional[int] = None, stream=None) -> None:
    import torch
    if n_tokens is None:
        n_tokens = token_slot_idx.numel()
    if n_tokens:
        _require_cuda(token_slot_idx, "token_slot_idx", torch.int32, n_tokens)
    _check(load_library().lora_plan_prepare(ctx, _ptr(token_slot_idx) if n_tokens else None,
                                            int(n_tokens), _stream(stream)), ctx)


def lora_plan_prepare_slots(ctx, token_slot_idx, used_slots: Sequence[int],
                            n_tokens: Optional[int] = None, stream=None) -> None:
    """lora_plan_prepare, declaring the (host) list of slots the batch reads."""
    import torch
    if n_tokens is None:
        n_tokens = token_slot_idx.numel()
    if n_tokens:
        _require_cuda(token_slot_idx, "token_slot_idx", torch.int32, n_tokens)
    used = [int(k) for k in used_slots]
    arr = (ctypes.c_int32 * max(len(used), 1))(*used)
    _check(load_library().lora_plan_prepare_slots(ctx, _ptr(token_slot_idx) if n_tokens else None,
                                                  int(n_tokens), arr, len(used), _stream(stream)), ctx)


def lora_shrink(ctx, x, module: int, stream=None) -> None:
    if x is not None:
        _require_cuda(x, "x")
    _check(load_library().lora_shrink(ctx, _ptr(x), int(module), _stream(stream)), ctx)


def lora_expand(ctx, y, module: int, stream=None) -> None:
    if y is not None:
        _require_cuda(y, "y")
    _check(load_library().lora_expand(ctx, _ptr(y), int(module), _stream(stream)), ctx)


def lora_apply(ctx, x, y, token_slot_idx, module: int, n_tokens: Optional[int] = None,
               stream=None) -> None:
    import torch
    if n_tokens is None:
        n_tokens = token_slot_idx.numel() if token_slot_idx is not None else 0
    if n_tokens:
        _require_cuda(token_slot_idx, "token_slot_idx", torch.int32, n_tokens)
        _require_cuda(x, "x")
        _require_cuda(y, "y")
    _check(load_library().lora_apply(ctx, _ptr(x), _ptr(y), _ptr(token_slot_idx), int(n_tokens),
                                     int(module), _stream(stream)), ctx)


def _group(modules, tensors, name):
    n = len(modules)
    if len(tensors) != n:
        raise ValueError(f"{name}: one tensor per module")
    for t in tensors:
        if t is not None:
            _require_cuda(t, name)
    mods = (ctypes.c_int32 * max(n, 1))(*[int(m) for m in modules])
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in tensors])
    return n, mods, ptrs


def lora_shrink_group(ctx, modules: Sequence[int], x: Sequence, stream=None) -> None:
    n, mods, xp = _group(modules, x, "x")
    _check(load_library().lora_shrink_group(ctx, n, mods, xp, _stream(stream)), ctx)


def lora_expand_group(ctx, modules: Sequence[int], y: Sequence, stream=None) -> None:
    n, mods, yp = _group(modules, y, "y")
    _check(load_library().lora_expand_group(ctx, n, mods, yp, _stream(stream)), ctx)


def lora_apply_group(ctx, modules: Sequence[int], x: Sequence, y: Sequence, token_slot_idx,
                     n_tokens: Optional[int] = None, stream=None) -> None:
    import torch
    if n_tokens is None:
        n_tokens = token_slot_idx.numel() if token_slot_idx is not None else 0
    if n_tokens:
        _require_cuda(token_slot_idx, "token_slot_idx", torch.int32, n_tokens)
    n, mods, xp = _group(modules, x, "x")
    _, _, yp = _group(modules, y, "y")
    _check(load_library().lora_apply_group(ctx, n, mods, xp, yp, _ptr(token_slot_idx),
                                           int(n_tokens), _stream(stream)), ctx)


def lora_apply_group_noalloc(ctx, modules: Sequence[int], x: Sequence, y: Sequence,
                             token_slot_idx, n_tokens: Optional[int] = None, stream=None) -> None:
    """lora_apply_group with the batch's plan and partials in the library's static
    scratch array (no device memory is allocated)."""
    import torch
    if n_tokens is None:
        n_tokens = token_slot_idx.numel() if token_slot_idx is not None else 0
    if n_tokens:
        _require_cuda(token_slot_idx, "token_slot_idx", torch.int32, n_tokens)
    n, mods, xp = _group(modules, x, "x")
    _, _, yp = _group(modules, y, "y")
    _check(load_library().lora_apply_group_noalloc(ctx, n, mods, xp, yp, _ptr(token_slot_idx),
                                                   int(n_tokens), _stream(stream)), ctx)


def lora_apply_group_fused(ctx, modules: Sequence[int], x: Sequence, y: Sequence,
                           token_slot_idx, n_tokens: Optional[int] = None, stream=None) -> None:
    """lora_apply_group with the shrink and the expand of a decode batch in one launch."""
    import torch
    if n_tokens is None:
        n_tokens = token_slot_idx.numel() if token_slot_idx is not None else 0
    if n_tokens:
        _require_cuda(token_slot_idx, "token_slot_idx", torch.int32, n_tokens)
    n, mods, xp = _group(modules, x, "x")
    _, _, yp = _group(modules, y, "y")
    _check(load_library().lora_apply_group_fused(ctx, n, mods, xp, yp, _ptr(token_slot_idx),
                                                 int(n_tokens), _stream(stream)), ctx)


def lora_get_device_flags(ctx) -> int:
    v = ctypes.c_uint32(0)
    _check(load_library().lora_get_device_flags(ctx, ctypes.byref(v)), ctx)
    return int(v.value)


def lora_get_stats(ctx) -> dict:
    s = _Stats()
    _check(load_library().lora_get_stats(ctx, ctypes.byref(s)), ctx)
    return {name: int(getattr(s, name)) for name, _ in _Stats._fields_}


def lora_profile_begin(ctx, max_launches: int) -> None:
    _check(load_library().lora_profile_begin(ctx, int(max_launches)), ctx)


def lora_profile_end(ctx) -> dict:
    p = _Profile()
    _check(load_library().lora_profile_end(ctx, ctypes.byref(p)), ctx)
    kinds = ("plan", "shrink", "expand", "saved", "fused")
    return {"launches": {k: int(p.launches[i]) for i, k in enumerate(kinds)},
            "total_ms": {k: float(p.total_ms[i]) for i, k in enumerate(kinds)},
            "untimed": int(p.untimed)}


# ---------------------------------------------------------------------------
# convenience owner of a ctx

class Slots:
    """A slot pool for a list of (d_in, d_out) modules, in bf16 or fp32."""

    def __init__(self, max_loras: int, max_rank: int, modules: Sequence[Sequence[int]],
                 dtype: str = "bf16", max_tokens: int = 8192, device: int = 0):
        self.modules = [(int(a), int(b)) for a, b in modules]
        self.dtype = dtype
        self.max_loras, self.max_rank, self.max_tokens = max_loras, max_rank, max_tokens
        self.ctx = lora_slots_create(max_loras, max_rank, self.modules,
                                     LORA_BF16 if dtype == "bf16" else LORA_FP32, max_tokens,
                                     device)

    def load(self, slot, A_t, B, r, lora_alpha, use_rslora=False, bias=None, dora_scale=None):
        if bias is None and dora_scale is None:
            lora_slot_load(self.ctx, slot, A_t, B, r, lora_alpha, use_rslora)
        else:
            lora_slot_load_ex(self.ctx, slot, A_t, B, bias, dora_scale, r, lora_alpha, use_rslora)

    def load_saved(self, slot, module, W, bias=None):
        lora_slot_load_saved(self.ctx, slot, module, W, bias)

    def clear(self, slot):
        lora_slot_clear(self.ctx, slot)

    def sync_loads(self):
        lora_sync_loads(self.ctx)

    def prepare(self, idx, n_tokens=None, stream=None, used_slots=None):
        if used_slots is None:
            lora_plan_prepare(self.ctx, idx, n_tokens, stream)
        else:
            lora_plan_prepare_slots(self.ctx, idx, used_slots, n_tokens, stream)

    def shrink(self, x, module, stream=None):
        lora_shrink(self.ctx, x, module, stream)

    def expand(self, y, module, stream=None):
        lora_expand(self.ctx, y, module, stream)

    def apply(self, x, y, idx, module, n_tokens=None, stream=None):
        lora_apply(self.ctx, x, y, idx, module, n_tokens, stream)

    def shrink_group(self, modules, x, stream=None):
        lora_shrink_group(self.ctx, modules, x, stream)

    def expand_group(self, modules, y, stream=None):
        lora_expand_group(self.ctx, modules, y, stream)

    def apply_group(self, modules, x, y, idx, n_tokens=None, stream=None):
        lora_apply_group(self.ctx, modules, x, y, idx, n_tokens, stream)

    def apply_group_fused(self, modules, x, y, idx, n_tokens=None, stream=None):
        lora_apply_group_fused(self.ctx, modules, x, y, idx, n_tokens, stream)

    def apply_group_noalloc(self, modules, x, y, idx, n_tokens=None, stream=None):
        lora_apply_group_noalloc(self.ctx, modules, x, y, idx, n_tokens, stream)

    def bind_step(self, groups, idx, stream=None, prepare=True, fused=False):
        """One step with its arguments marshalled once: lora_plan_prepare of idx
        (unless prepare is False: then the step reuses the plan an earlier
        lora_plan_prepare of the same idx made, as the layers of a model share
        one batch), then lora_apply_group for each (modules, x, y) in `groups`.
        Returns a function that makes exactly those library calls.  The tensors
        are checked here and must stay alive, at the same addresses, while the
        function is used; the stream is taken now (default: the current one)."""
        import torch
        lib = load_library()
        n_tokens = idx.numel()
        _require_cuda(idx, "token_slot_idx", torch.int32, n_tokens)
        st = _stream(stream)
        pidx = _ptr(idx)
        calls = []
        for modules, x, y in groups:
            n, mods, xp = _group(modules, x, "x")
            _, _, yp = _group(modules, y, "y")
            calls.append((n, mods, xp, yp))
        ctx = self.ctx
        plan = lib.lora_plan_prepare
        apply_group = lib.lora_apply_group_fused if fused else lib.lora_apply_group
        refs = (idx, groups)

        def step():
            _ = refs
            if prepare:
                rc = plan(ctx, pidx, n_tokens, st)
                if rc:
                    _check(rc, ctx)
            for n, mods, xp, yp in calls:
                rc = apply_group(ctx, n, mods, xp, yp, pidx, n_tokens, st)
                if rc:
                    _check(rc, ctx)
        return step

    def profile_begin(self, max_launches):
        lora_profile_begin(self.ctx, max_launches)

    def profile_end(self):
        return lora_profile_end(self.ctx)

    def flags(self):
        return lora_get_device_flags(self.ctx)

    def stats(self):
        return lora_get_stats(self.ctx)

    def close(self):
        if self.ctx:
            lora_slots_destroy(self.ctx)
            self.ctx = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
