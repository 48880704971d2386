"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: max |gpu - oracle| <= 1e-5 * (1 + |oracle|) for fp32 data and
<= 2e-2 * (1 + |oracle|) for bf16 data with fp32 accumulation; bit-identical
rows wherever the update must not touch y; bit-identical results for exact
small-integer fp32 data.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (as_f64, check_close, from_dev, full_workload, log, make_slots, rel_l2,
                      run_gpu, run_oracle, to_dev, to_pinned, to_pinned_misaligned)
from lora_adapter_application_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


# ---------------------------------------------------------------------------
# the five workloads

def test_tiny_fp32_full():
    wl = synth.tiny_fp32()
    log("case tiny_fp32", wl.n_tokens)
    S = make_slots(wl)
    got = run_gpu(wl, S)
    ref = run_oracle(wl, "linear")
    check_close(got["linear"], ref, wl.dtype, "tiny_fp32")
    skipped = wl.idx < 0
    assert np.array_equal(got["linear"][skipped].view(np.uint32), wl.y["linear"][skipped].view(np.uint32))
    S.close()


def test_llama7b_decode_full():
    wl = synth.llama7b_decode()
    log("case llama7b_decode", wl.n_tokens)
    S = make_slots(wl)
    got = run_gpu(wl, S)
    for m in wl.modules:
        ref = run_oracle(wl, m.name)
        check_close(got[m.name], ref, wl.dtype, "llama7b_decode " + m.name)
        skipped = wl.idx < 0
        assert np.array_equal(got[m.name][skipped], wl.y[m.name][skipped])
    S.close()


def test_llama7b_decode_weak_signal_diagnostic():
    """With y = 0 the output is the update itself: relative L2 error of the delta."""
    wl = synth.llama7b_decode(y_zero=True)
    S = make_slots(wl)
    got = run_gpu(wl, S)
    for m in wl.modules:
        ref = run_oracle(wl, m.name)
        e = rel_l2(as_f64(got[m.name], wl.dtype), as_f64(ref, wl.dtype))
        log(f"llama7b_decode y=0 {m.name}: rel L2 {e:.2e}")
        assert e < 1e-2
    S.close()


def test_qwen32b_decode_full():
    wl = synth.qwen32b_decode()
    log("case qwen32b_decode", wl.n_tokens)
    S = make_slots(wl)
    got = run_gpu(wl, S)
    for m in wl.modules:
        ref = run_oracle(wl, m.name)
        check_close(got[m.name], ref, wl.dtype, "qwen32b_decode " + m.name)
        skipped = wl.idx < 0
        assert np.array_equal(got[m.name][skipped], wl.y[m.name][skipped])
    S.close()


def test_llama7b_prefill_full_size_every_row():
    """The prefill workload at full size through lora_apply per module (the
    grouped launches are checked in test_gpu_configs.py): every row of every
    module against the oracle."""
    wl = full_workload("llama7b_prefill")
    T = wl.n_tokens
    log("case llama7b_prefill", T)
    S = make_slots(wl)
    got = run_gpu(wl, S)
    S.close()
    for m in wl.modules:
        ref = run_oracle(wl, m.name)
        w = check_close(got[m.name], ref, wl.dtype, "llama7b_prefill " + m.name)
        log(f"llama7b_prefill per-module {m.name}: {T} rows, worst err/bound {w:.3f}")


# ---------------------------------------------------------------------------
# sweeps: ragged tiles and tails, mixed ranks, several tiles per slot

SWEEP = [
    # dtype, (d_in, d_out) list, max_loras, R, ranks, T, p_base_only
    (synth.BF16, [(136, 264)], 8, 64, [1, 3, 16, 17, 33, 64, 8, 2], 300, 0.1),
    (synth.BF16, [(4096, 1024), (1024, 4096)], 16, 32, [32] * 16, 1000, 0.05),
    (synth.BF16, [(256, 512)], 4, 128, [128, 100, 65, 7], 200, 0.0),
    (synth.BF16, [(512, 256)], 3, 16, [16, 5, 9], 1, 0.0),
    (synth.BF16, [(128, 128)], 256, 8, [(k % 8) + 1 for k in range(256)], 5000, 0.2),
    (synth.BF16, [(384, 392)], 5, 48, [48, 40, 30, 20, 10], 3077, 0.1),
    (synth.BF16, [(200, 328)], 3, 64, [64, 33, 5], 2500, 0.05),
    (synth.BF16, [(4096, 1024)], 3, 32, [32, 16, 8], 1100, 0.0),
    (synth.BF16, [(1024, 512)], 8, 128, [128, 120, 64, 17, 1, 96, 32, 8], 4000, 0.1),
    (synth.FP32, [(72, 40)], 6, 8, [8, 1, 2, 3, 5, 8], 130, 0.1),
    (synth.FP32, [(264, 136), (96, 200)], 4, 24, [24, 17, 1, 9], 700, 0.1),
]


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_sweep(case):
    dtype, shapes, S_, R, ranks, T, pb = SWEEP[case]
    mods = [synth.Module(f"m{i}", a, b) for i, (a, b) in enumerate(shapes)]
    wl = synth.random_case(100 + case, dtype, mods, T, S_, R, ranks, p_base_only=pb)
    log(f"case sweep {case}: {dtype} {shapes} S={S_} R={R} T={T}")
    Sl = make_slots(wl)
    got = run_gpu(wl, Sl)
    for m in mods:
        check_close(got[m.name], run_oracle(wl, m.name), dtype, f"sweep {case} {m.name}")
    Sl.close()


# lora_apply against the separate lora_shrink / lora_expand entry points and the
# oracle: K ranges that end in a partial K block, column counts that are not a
# multiple of a wave's 64 columns, tiles of every length 1..64, 256 slots, one
# token, the largest inline-planned batch, batches above it (plan kernels,
# segment path), every padded-rank class.
APPLY_SWEEP = [
    # (d_in, d_out) list, max_loras, R, ranks, T, p_base_only, zipf_s
    ([(136, 264)], 8, 32, [1, 3, 16, 17, 31, 32, 8, 2], 300, 0.1, 1.1),
    ([(8, 8), (24, 1000)], 4, 16, [16, 1, 9, 4], 257, 0.05, 0.5),
    ([(5120, 1024), (1024, 520)], 16, 32, [32] * 16, 1024, 0.05, 1.2),
    ([(4096, 4096)], 8, 16, [16] * 8, 1, 0.0, 1.1),
    ([(512, 1536)], 256, 16, [(k % 16) + 1 for k in range(256)], 1024, 0.02, 0.3),
    ([(1160, 648)], 3, 32, [32, 20, 12], 1000, 0.0, 0.01),
    ([(2048, 8192), (8192, 2048)], 16, 32, [32] * 16, 512, 0.05, 1.2),
    ([(384, 392), (200, 328)], 5, 64, [64, 40, 30, 20, 10], 1025, 0.1, 1.1),
    ([(1024, 512)], 8, 128, [128, 120, 64, 17, 1, 96, 32, 8], 2600, 0.1, 0.8),
    ([(256, 256)], 64, 8, [(k % 8) + 1 for k in range(64)], 4000, 0.2, 0.5),
]


@pytest.mark.parametrize("case", range(len(APPLY_SWEEP)))
def test_apply_matches_split_entry_points_and_oracle(case):
    shapes, S_, R, ranks, T, pb, zs = APPLY_SWEEP[case]
    mods = [synth.Module(f"m{i}", a, b) for i, (a, b) in enumerate(shapes)]
    wl = synth.random_case(200 + case, synth.BF16, mods, T, S_, R, ranks, p_base_only=pb,
                           zipf_s=zs)
    log(f"case apply sweep {case}: {shapes} S={S_} R={R} T={T}")
    Sl = make_slots(wl)
    applied = run_gpu(wl, Sl)
    split = run_gpu(wl, Sl, path="split")
    assert Sl.flags() == 0
    for m in mods:
        assert np.array_equal(applied[m.name], split[m.name]), m.name
        check_close(applied[m.name], run_oracle(wl, m.name), wl.dtype, f"apply sweep {case} {m.name}")
        skipped = np.ones(T, bool)
        for k, ad in enumerate(wl.adapters):
            if ad is not None and m.name in ad.At:
                skipped &= wl.idx != k
        assert np.array_equal(applied[m.name][skipped], wl.y[m.name][skipped])
    Sl.close()


def test_consecutive_batches_of_changing_size_on_one_ctx():
    """Batches of changing sizes on one ctx switch between the in-kernel plan and
    the plan kernels; every apply equals the separate entry points on its batch."""
    mods = [synth.Module("a", 640, 384)]
    wl = synth.random_case(31, synth.BF16, mods, 3000, 6, 32, [32, 16, 8, 4, 32, 1], p_base_only=0.05)
    S = make_slots(wl, max_tokens=3000)
    x = to_dev(wl.x["a"], wl.dtype)
    for T in (3000, 100, 1, 1024, 1025, 3000, 64, 700):
        idx = torch.from_numpy(wl.idx[:T]).cuda()
        y1 = to_dev(wl.y["a"][:T], wl.dtype)
        y2 = to_dev(wl.y["a"][:T], wl.dtype)
        S.apply(x[:T], y1, idx, 0)
        S.prepare(idx)
        S.shrink(x[:T], 0)
        S.expand(y2, 0)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(y1, wl.dtype), from_dev(y2, wl.dtype)), T
    assert S.flags() == 0
    S.close()


def test_fp32_large_rslora_scales_keep_the_fp32_bound():
    """rsLoRA at high rank with lora_alpha = 2r gives s = 2 sqrt(r), up to 22.6, which
    multiplies the rounding error of h.  A batch of this shape (2047 tokens, K = 2048,
    28 slots of ranks up to 128) once exceeded 1e-5 (1 + |ref|) in its tail with fp32 sums
    over K; the fp32 shrink sums in fp64."""
    mods = [synth.Module("m0", 2048, 1024), synth.Module("m1", 1024, 1536)]
    ranks = [53, 104, 123, 30, 91, 119, 104, 1, 48, 54, 15, 32, 49, 91, 27, 128, 106, 74, 84,
             10, 98, 60, 52, 1, 102, 7, 120, 72]
    wl = synth.random_case(200046, synth.FP32, mods, 2047, 28, 128, ranks, rslora=True,
                           p_base_only=0.05, zipf_s=0.5)
    log("case fp32 rslora: T 2047 S 28 R 128")
    S = make_slots(wl)
    got = run_gpu(wl, S)
    for m in mods:
        check_close(got[m.name], run_oracle(wl, m.name), wl.dtype, f"fp32 rslora {m.name}")
    S.close()


def test_exact_integers_fp32_bit_identical():
    mods = [synth.Module("a", 200, 136), synth.Module("b", 64, 520)]
    wl = synth.random_case(7, synth.FP32, mods, 333, 4, 16, [16, 9, 4, 1], integer=True)
    S = make_slots(wl)
    got = run_gpu(wl, S)
    for m in mods:
        ref = run_oracle(wl, m.name)
        assert np.array_equal(got[m.name].view(np.uint32), ref.view(np.uint32)), m.name
    S.close()


def test_exact_integers_bf16_bit_identical():
    # final |y| stays <= 256 so every value is exact in bf16
    mods = [synth.Module("a", 8, 24)]
    wl = synth.random_case(8, synth.BF16, mods, 100, 3, 16, [2, 1, 2], integer=True)
    for ad in wl.adapters:
        for k in ad.At:
            ad.At[k] = synth.to_bf16_bits(np.clip(synth.bf16_bits_to_f32(ad.At[k]), -1, 1))
            ad.B[k] = synth.to_bf16_bits(np.clip(synth.bf16_bits_to_f32(ad.B[k]), -1, 1))
    wl.x["a"] = synth.to_bf16_bits(np.clip(synth.bf16_bits_to_f32(wl.x["a"]), -1, 1))
    S = make_slots(wl)
    got = run_gpu(wl, S)
    ref = run_oracle(wl, "a")
    assert np.array_equal(got["a"], ref)
    S.close()


# ---------------------------------------------------------------------------
# skip semantics, padding, determinism

def test_skip_rows_bit_identical_and_flag():
    mods = [synth.Module("q", 256, 256), synth.Module("v", 256, 256)]
    wl = synth.random_case(9, synth.BF16, mods, 64, 4, 16, [16, 8, 4, 2],
                           targeted=[[True, True], [True, False], [False, True], [True, True]],
                           empty_slots=[3], p_base_only=0.0)
    wl.idx = np.array([-1, -5, 0, 1, 2, 3, 4, 1000] * 8, dtype=np.int32)
    S = make_slots(wl)
    assert S.flags() == 0
    got = run_gpu(wl, S)
    assert S.flags() & binding.LORA_FLAG_SLOT_INDEX_TOO_LARGE
    assert S.flags() == 0                                   # read clears
    for mi, m in enumerate(mods):
        active = np.isin(wl.idx, [0, 1] if m.name == "q" else [0, 2])
        assert np.array_equal(got[m.name][~active], wl.y[m.name][~active]), m.name
        assert not np.array_equal(got[m.name][active], wl.y[m.name][active])
        check_close(got[m.name], run_oracle(wl, m.name), wl.dtype, m.name)
    S.close()


@pytest.mark.parametrize("dtype,path,wide", [(synth.BF16, "apply", 64), (synth.BF16, "split", 128),
                                             (synth.FP32, "apply", 64)])
def test_padding_to_max_rank_changes_nothing(dtype, path, wide):
    """Zero ranks added up to max_rank leave the result bit-identical."""
    mods = [synth.Module("a", 512, 768)]
    wl = synth.random_case(10, dtype, mods, 400, 4, 16, [16, 13, 8, 1], p_base_only=0.1)
    S16 = make_slots(wl, max_rank=16)
    Sw = make_slots(wl, max_rank=wide)
    a = run_gpu(wl, S16, path=path)["a"]
    b = run_gpu(wl, Sw, path=path)["a"]
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    check_close(a, run_oracle(wl, "a"), dtype, "padding")
    S16.close()
    Sw.close()


@pytest.mark.parametrize("R", [32, 64])
def test_deterministic_and_prepared_plan_matches_unprepared(R):
    """Repeated runs are bit-identical, whether the plan is computed in the kernel
    or read from an earlier launch, and the separate shrink / expand entry points
    equal lora_apply."""
    wl = synth.random_case(11, synth.BF16, [synth.Module("a", 1024, 2048)], 700, 8, R,
                           [32, 16, 8, 4, 32, 16, 8, 4])
    S = make_slots(wl)
    a = run_gpu(wl, S, prepare=True)["a"]
    b = run_gpu(wl, S, prepare=False)["a"]
    assert np.array_equal(a, b)
    # a second apply on the same prepared plan reads the plan the first one published
    idx = torch.from_numpy(wl.idx).cuda()
    x = to_dev(wl.x["a"], wl.dtype)
    ys = [to_dev(wl.y["a"], wl.dtype) for _ in range(2)]
    S.prepare(idx)
    for y in ys:
        S.apply(x, y, idx, 0)
    torch.cuda.synchronize()
    for y in ys:
        assert np.array_equal(from_dev(y, wl.dtype), a)
    # shrink and expand as separate entry points on a prepared plan
    s1 = run_gpu(wl, S, path="split")["a"]
    s2 = run_gpu(wl, S, path="split")["a"]
    assert np.array_equal(s1, s2)
    assert np.array_equal(s1, a)
    check_close(s1, run_oracle(wl, "a"), wl.dtype, "split")
    check_close(a, run_oracle(wl, "a"), wl.dtype, "apply")
    S.close()


def test_empty_batch_is_a_noop():
    wl = synth.random_case(12, synth.BF16, [synth.Module("a", 128, 128)], 4, 2, 16, [16, 8])
    S = make_slots(wl)
    y = to_dev(wl.y["a"], wl.dtype)
    before = from_dev(y, wl.dtype)
    empty = torch.zeros(0, dtype=torch.int32, device="cuda")
    S.apply(to_dev(wl.x["a"], wl.dtype), y, empty, 0)
    S.prepare(empty)
    S.shrink(None, 0)
    S.expand(None, 0)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(y, wl.dtype), before)
    S.close()


# ---------------------------------------------------------------------------
# loads: byte count, ordering against in-flight work, errors

def test_bytes_loaded_follow_the_page_formula():
    wl = synth.qwen32b_decode(n_tokens=8)
    S = make_slots(wl)
    st = S.stats()
    shapes = [(m.d_in, m.d_out) for m in wl.modules]
    per = oracle.adapter_bytes(shapes, [True] * 4, 32, 2)
    assert st["loads"] == 16 and st["bytes_loaded"] == 16 * per
    S.close()


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP32])
def test_load_sources_read_in_place_staged_and_from_device_agree(dtype):
    """A load reads aligned pinned host weights and device weights in place, and
    copies other sources (here pinned views one element past a 16-byte boundary)
    to the stage first.  One adapter loaded the three ways into three slots must
    give bit-identical updates, each matching the oracle."""
    mods = [synth.Module("a", 264, 136), synth.Module("b", 512, 1040)]
    wl = synth.random_case(31, dtype, mods, 96, 3, 32, [24, 24, 24], p_base_only=0.0)
    ad = wl.adapters[0]
    wl.adapters[1] = wl.adapters[2] = ad
    S = binding.Slots(3, 32, [(m.d_in, m.d_out) for m in mods], dtype, 96)
    keep = []

    def pinned_off(arr):
        v = to_pinned_misaligned(arr, dtype, keep)
        assert v.data_ptr() % 16 != 0
        return v

    makers = [lambda a: to_pinned(a, dtype), pinned_off, lambda a: to_dev(a, dtype)]
    for slot, mk in enumerate(makers):
        A_t = [mk(ad.At[m.name]) for m in mods]
        B = [mk(ad.B[m.name]) for m in mods]
        keep += A_t + B
        S.load(slot, A_t, B, ad.r, ad.lora_alpha, ad.use_rslora)
    S.sync_loads()
    outs = []
    for slot in range(3):
        wl.idx[:] = slot
        log(f"case load sources: {dtype} slot {slot}")
        outs.append(run_gpu(wl, S))
    for m in mods:
        ref = run_oracle(wl, m.name)          # every slot holds the same adapter
        for slot in range(3):
            check_close(outs[slot][m.name], ref, dtype, f"slot {slot} {m.name}")
            assert np.array_equal(outs[slot][m.name], outs[0][m.name]), (slot, m.name)
    S.close()


def _reload(S, wl, slot, A_list, B_list, r, alpha, keep):
    A_t, B = [], []
    for a, b in zip(A_list, B_list):
        ta, tb = to_pinned(a, wl.dtype), to_pinned(b, wl.dtype)
        keep += [ta, tb]
        A_t.append(ta)
        B.append(tb)
    S.load(slot, A_t, B, r, alpha)


def test_load_waits_for_in_flight_applies_and_applies_wait_for_loads():
    """WAR: a load issued while applies are in flight must not change their result.
    RAW: an apply issued right after a load must see the new weights."""
    T = 8192
    mods = [synth.Module("a", 4096, 4096)]
    wl = synth.random_case(13, synth.BF16, mods, T, 2, 16, [16, 16], p_base_only=0.0,
                           zipf_s=0.01)
    S = make_slots(wl, max_tokens=T)
    idx = torch.from_numpy(wl.idx).cuda()
    x = to_dev(wl.x["a"], wl.dtype)
    ys = [to_dev(wl.y["a"], wl.dtype) for _ in range(12)]
    new = synth.random_case(14, synth.BF16, mods, 1, 2, 16, [16, 16])
    keep = []
    S.prepare(idx)
    for y in ys:                                   # ~a dozen large applies in flight
        S.apply(x, y, idx, 0)
    _reload(S, wl, 0, [new.adapters[0].At["a"]], [new.adapters[0].B["a"]], 16, 32.0, keep)
    y_after = to_dev(wl.y["a"], wl.dtype)
    S.apply(x, y_after, idx, 0)                    # must see the new slot 0
    torch.cuda.synchronize()
    old_ref = run_oracle(wl, "a")
    for y in ys:
        check_close(from_dev(y, wl.dtype), old_ref, wl.dtype, "in-flight apply")
    wl.adapters[0] = new.adapters[0]
    check_close(from_dev(y_after, wl.dtype), run_oracle(wl, "a"), wl.dtype, "apply after load")
    S.close()


def test_clear_makes_slot_a_noop():
    wl = synth.random_case(15, synth.BF16, [synth.Module("a", 256, 256)], 128, 3, 16, [16, 8, 4],
                           p_base_only=0.0)
    S = make_slots(wl)
    S.clear(1)
    got = run_gpu(wl, S)["a"]
    on1 = wl.idx == 1
    assert np.array_equal(got[on1], wl.y["a"][on1])
    wl.adapters[1] = None
    check_close(got, run_oracle(wl, "a"), wl.dtype, "after clear")
    S.close()


def test_error_codes():
    S = binding.Slots(4, 16, [(128, 256), (256, 128)], "bf16", max_tokens=32)
    a = torch.zeros(16, 128, dtype=torch.bfloat16).pin_memory()
    b = torch.zeros(16, 256, dtype=torch.bfloat16).pin_memory()
    unpinned = torch.zeros(16, 128, dtype=torch.bfloat16)

    def status(fn):
        with pytest.raises(binding.LoraError) as e:
            fn()
        return e.value.status

    assert status(lambda: S.load(4, [a, None], [b, None], 16, 32.0)) == binding.LORA_ERR_SLOT_OUT_OF_RANGE
    assert status(lambda: S.load(-1, [a, None], [b, None], 16, 32.0)) == binding.LORA_ERR_SLOT_OUT_OF_RANGE
    assert status(lambda: S.load(0, [a, None], [b, None], 17, 32.0)) == binding.LORA_ERR_RANK_EXCEEDS_MAX
    assert status(lambda: S.load(0, [a, None], [b, None], 0, 32.0)) == binding.LORA_ERR_INVALID_ARGUMENT
    assert status(lambda: S.load(0, [a, None], [None, None], 16, 32.0)) == binding.LORA_ERR_INVALID_ARGUMENT
    assert status(lambda: S.load(0, [unpinned, None], [b, None], 16, 32.0)) == binding.LORA_ERR_HOST_NOT_PINNED
    assert status(lambda: S.clear(9)) == binding.LORA_ERR_SLOT_OUT_OF_RANGE
    x = torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(64, 256, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(64, dtype=torch.int32, device="cuda")
    assert status(lambda: S.apply(x, y, idx, 0)) == binding.LORA_ERR_TOO_MANY_TOKENS
    assert status(lambda: S.apply(x[:8], y[:8], idx[:8], 2)) == binding.LORA_ERR_BAD_MODULE
    assert status(lambda: S.shrink(x, 0)) == binding.LORA_ERR_NO_PLAN
    S.prepare(idx[:8])
    assert status(lambda: S.expand(y, 1)) == binding.LORA_ERR_INVALID_ARGUMENT
    assert "max_rank" in binding.lora_status_string(binding.LORA_ERR_RANK_EXCEEDS_MAX)
    with pytest.raises(binding.LoraError) as e:
        binding.Slots(4, 200, [(128, 128)], "bf16")
    assert e.value.status == binding.LORA_ERR_RANK_EXCEEDS_MAX
    with pytest.raises(binding.LoraError):
        binding.Slots(4, 16, [(100, 128)], "bf16")          # d_in not a multiple of 8
    # nothing was loaded by the failed calls
    assert S.stats()["loads"] == 0
    S.close()


# ---------------------------------------------------------------------------
# grouped calls: one launch per phase for several modules

def test_group_calls_equal_single_module_calls():
    mods = [synth.Module("q", 512, 1024), synth.Module("k", 512, 256),
            synth.Module("v", 1024, 512), synth.Module("o", 1024, 1024)]
    wl = synth.random_case(16, synth.BF16, mods, 300, 6, 32, [32, 16, 8, 32, 1, 24],
                           targeted=[[True, True, True, True], [True, False, True, False],
                                     [False, True, True, True], [True, True, True, True],
                                     [True, True, False, False], [False, False, False, True]],
                           p_base_only=0.1)
    S = make_slots(wl)
    single = run_gpu(wl, S)
    single_split = run_gpu(wl, S, path="split")
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
    ys = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
    S.apply_group([0, 1, 2, 3], xs, ys, idx)
    torch.cuda.synchronize()
    for i, m in enumerate(mods):
        assert np.array_equal(from_dev(ys[i], wl.dtype), single[m.name]), m.name
        assert np.array_equal(single_split[m.name], single[m.name]), m.name
        check_close(single[m.name], run_oracle(wl, m.name), wl.dtype, m.name)
    # separate phases, a module listed twice with its own x and y, prepared plan
    y2 = [to_dev(wl.y[m.name], wl.dtype) for m in (mods[2], mods[0], mods[2])]
    x2 = [xs[2], xs[0], xs[2]]
    S.prepare(idx)
    S.shrink_group([2, 0, 2], x2)
    S.expand_group([2, 0, 2], y2)
    torch.cuda.synchronize()
    for yy, name in zip(y2, ("v", "q", "v")):
        assert np.array_equal(from_dev(yy, wl.dtype), single_split[name]), name
    # errors
    with pytest.raises(binding.LoraError) as e:
        S.expand_group([0, 2, 2], y2)                       # not the shrunk list
    assert e.value.status == binding.LORA_ERR_INVALID_ARGUMENT
    with pytest.raises(binding.LoraError) as e:
        S.apply_group([0, 0], [xs[0], xs[0]], [ys[0], ys[0]], idx)   # same y twice
    assert e.value.status == binding.LORA_ERR_INVALID_ARGUMENT
    with pytest.raises(binding.LoraError) as e:
        S.apply_group([0] * 9, [xs[0]] * 9, [to_dev(wl.y["q"], wl.dtype) for _ in range(9)], idx)
    assert e.value.status == binding.LORA_ERR_INVALID_ARGUMENT
    with pytest.raises(binding.LoraError) as e:
        S.apply_group([0, 7], [xs[0], xs[1]], [ys[0], ys[1]], idx)
    assert e.value.status == binding.LORA_ERR_BAD_MODULE
    S.close()


@pytest.mark.parametrize("T", [700, 3000])
def test_group_of_eight_modules(T):
    shapes = [(256, 512), (512, 256), (256, 256), (384, 640), (640, 384), (128, 1024),
              (1024, 128), (256, 768)]
    mods = [synth.Module(f"m{i}", a, b) for i, (a, b) in enumerate(shapes)]
    wl = synth.random_case(17 + T, synth.BF16, mods, T, 4, 64, [64, 16, 40, 8], p_base_only=0.05)
    S = make_slots(wl, max_tokens=T)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
    ys = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
    S.apply_group(list(range(8)), xs, ys, idx)
    torch.cuda.synchronize()
    for i, m in enumerate(mods):
        check_close(from_dev(ys[i], wl.dtype), run_oracle(wl, m.name), wl.dtype, m.name)
    S.close()


def test_profile_times_every_dispatch():
    wl = synth.random_case(18, synth.BF16, [synth.Module("a", 512, 512), synth.Module("b", 512, 256)],
                           200, 4, 16, [16, 8, 4, 16])
    S = make_slots(wl)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in wl.modules]
    ys = [to_dev(wl.y[m.name], wl.dtype) for m in wl.modules]
    S.profile_begin(16)
    for _ in range(3):
        S.prepare(idx)
        S.shrink_group([0, 1], xs)
        S.expand_group([0, 1], ys)
    p = S.profile_end()
    assert p["launches"]["shrink"] == 3 and p["launches"]["expand"] == 3
    assert p["launches"]["plan"] == 0                     # planned inside the shrink
    assert p["total_ms"]["shrink"] > 0 and p["total_ms"]["expand"] > 0 and p["untimed"] == 0
    S.profile_begin(1)
    S.apply(xs[0], ys[0], idx, 0)                        # shrink and expand dispatches
    S.apply(xs[0], ys[0], idx, 0)
    p = S.profile_end()
    assert p["launches"]["shrink"] == 1 and p["untimed"] == 3
    S.profile_begin(4)
    S.apply_group_fused([0], [xs[0]], [ys[0]], idx)      # one fused dispatch
    p = S.profile_end()
    assert p["launches"]["fused"] == 1 and p["untimed"] == 0
    # a batch above 1024 tokens: plan kernels, then two launches even when fused is asked for
    big = synth.random_case(19, synth.BF16, [synth.Module("a", 512, 512)], 1500, 4, 16, [16, 8, 4, 16])
    Sb = make_slots(big)
    Sb.profile_begin(8)
    Sb.apply_group_fused([0], [to_dev(big.x["a"], big.dtype)], [to_dev(big.y["a"], big.dtype)],
                         torch.from_numpy(big.idx).cuda())
    pb = Sb.profile_end()
    assert pb["launches"]["plan"] == 2 and pb["launches"]["shrink"] == 1 and pb["launches"]["expand"] == 1
    assert pb["launches"]["fused"] == 0
    Sb.close()
    S.close()
