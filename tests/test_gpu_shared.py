"""Groups whose members read one x buffer (q, k and v of a layer read its
hidden state; gate and up likewise).  The grouped shrink runs the members of a
(tile, K split) back to back on one XCD, so x comes from HBM once and from L2
for the other members.  These tests check that aliased inputs give the
oracle's results: mixed ranks and targets, a batch large enough for the plan
kernels, small-integer data bit-exactly, and a shared group next to an
unshared one on one plan.
"""
import numpy as np
import pytest
import torch

from gpu_util import check_close, from_dev, log, make_slots, run_oracle, to_dev
from lora_adapter_application_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _run(wl, S, groups, share):
    """Apply the groups; the members listed in `share` read one x buffer."""
    idx = torch.from_numpy(wl.idx).cuda()
    names = [m.name for m in wl.modules]
    x0 = to_dev(wl.x[names[share[0]]], wl.dtype) if share else None
    xs = [x0 if (share and i in share) else to_dev(wl.x[n], wl.dtype) for i, n in enumerate(names)]
    ys = [to_dev(wl.y[n], wl.dtype) for n in names]
    S.prepare(idx)
    for g in groups:
        S.apply_group(g, [xs[i] for i in g], [ys[i] for i in g], idx)
    torch.cuda.synchronize()
    return [from_dev(y, wl.dtype) for y in ys]


def _shared_case(seed, mods, T, R, ranks, targeted=None, integer=False):
    wl = synth.random_case(seed, synth.BF16, mods, T, len(ranks), R, ranks, targeted=targeted,
                           p_base_only=0.1, integer=integer)
    first = wl.x[mods[0].name]          # every member reads the first one's activations
    for m in mods[1:]:
        wl.x[m.name] = first
    return wl


QKV = [synth.Module("q_proj", 512, 512), synth.Module("k_proj", 512, 256),
       synth.Module("v_proj", 512, 768)]
GU = [synth.Module("gate_proj", 1024, 1536), synth.Module("up_proj", 1024, 1536)]

CASES = [
    # name, modules, tokens, max rank, ranks per slot, targets
    ("qkv_decode_r32", QKV, 200, 32, [32, 16, 8, 32, 24, 16],
     [[True, True, True], [True, False, True], [True, True, False], [False, True, True],
      [True, True, True], [True, True, True]]),
    ("qkv_large_r64", QKV, 1500, 64, [64, 8, 16, 32, 64, 40], None),
    ("gate_up_r16", GU, 300, 16, [16, 8, 16, 4], [[True, True], [True, False], [False, True], [True, True]]),
    ("qkv_r16_tail", QKV, 67, 16, [16, 16, 12], None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_group_reading_one_x_matches_oracle(case):
    name, mods, T, R, ranks, targeted = case
    wl = _shared_case(7000 + T, mods, T, R, ranks, targeted)
    log("case shared x", name, T, R)
    S = make_slots(wl)
    got = _run(wl, S, [list(range(len(mods)))], share=list(range(len(mods))))
    S.close()
    for i, m in enumerate(mods):
        ref = run_oracle(wl, m.name)
        check_close(got[i], ref, wl.dtype, f"{name} {m.name}")
        skipped = wl.idx < 0
        assert np.array_equal(got[i][skipped], wl.y[m.name][skipped])


def test_group_reading_one_x_integer_data_is_exact():
    wl = _shared_case(7100, QKV, 150, 32, [32, 16, 32, 8], integer=True)
    S = make_slots(wl)
    got = _run(wl, S, [[0, 1, 2]], share=[0, 1, 2])
    S.close()
    for i, m in enumerate(QKV):
        assert np.array_equal(got[i], run_oracle(wl, m.name)), f"{m.name}: integer data must be exact"


def test_partly_shared_group():
    wl = synth.random_case(7200, synth.BF16, QKV, 180, 4, 32, [32, 16, 8, 32], p_base_only=0.1)
    wl.x["k_proj"] = wl.x["q_proj"]          # k reads q's x, v has its own
    S = make_slots(wl)
    got = _run(wl, S, [[0, 1, 2]], share=[0, 1])
    S.close()
    for i, m in enumerate(QKV):
        check_close(got[i], run_oracle(wl, m.name), wl.dtype, f"partly shared {m.name}")


def test_shared_group_then_unshared_group_on_one_plan():
    """A {q,k,v} group reading one x and an {o} group with its own, on one plan."""
    mods = QKV + [synth.Module("o_proj", 768, 512)]
    wl = synth.random_case(7300, synth.BF16, mods, 400, 5, 32, [32, 16, 8, 32, 24], p_base_only=0.05)
    for m in QKV[1:]:
        wl.x[m.name] = wl.x["q_proj"]
    S = make_slots(wl)
    got = _run(wl, S, [[0, 1, 2], [3]], share=[0, 1, 2])
    S.close()
    for i, m in enumerate(mods):
        check_close(got[i], run_oracle(wl, m.name), wl.dtype, f"two groups {m.name}")
