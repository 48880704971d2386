"""Small batches whose K-split count is a multiple of 8: the shrink warms each
split's x rows (every token) and, when small, its A^T rows (every slot) in L2
while it forms or reads the plan.  These cases pin the edges of that path
against the oracle: an odd token count, group members with different split
counts (one of them with splits the other lacks), the x-only warm-up when the
A^T block is large, and a second group that reads the published plan.
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


def _run(wl, groups):
    S = make_slots(wl)
    idx = torch.from_numpy(wl.idx).cuda()
    names = [m.name for m in wl.modules]
    xs = [to_dev(wl.x[n], wl.dtype) for n in names]
    ys = [to_dev(wl.y[n], wl.dtype) for n in names]
    S.prepare(idx)
    for g in groups:
        S.apply_group(g, [xs[i] for i in g], [ys[i] for i in g], idx)
    torch.cuda.synchronize()
    got = [from_dev(y, wl.dtype) for y in ys]
    S.close()
    return got


CASES = [
    # name, modules (d_in, d_out), tokens, slots, max rank, ranks, groups
    # 8 and 4 splits in one group, A^T block warmed too, 77 tokens
    ("mixed_splits_odd_T", [(2048, 1024), (1024, 768)], 77, 6, 16, [16, 8, 16, 4, 12, 16], [[0, 1]]),
    # rank 32: 8 splits, A^T block above the warm-up limit (x only)
    ("x_only_r32", [(4096, 1024)], 300, 12, 32, [32, 16, 24, 32, 8, 32, 32, 16, 32, 32, 20, 32], [[0]]),
    # a second group reads the plan the first published, and warms as well
    ("two_groups", [(4096, 1024), (2048, 4096)], 200, 8, 16, [16, 8, 16, 16, 4, 16, 16, 12], [[0], [1]]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_warmed_small_batch_matches_oracle(case):
    name, shapes, T, S, R, ranks, groups = case
    mods = [synth.Module(f"m{i}", di, do) for i, (di, do) in enumerate(shapes)]
    wl = synth.random_case(9500 + T, synth.BF16, mods, T, S, R, ranks, p_base_only=0.1)
    log("case warm", name, T, S, R)
    got = _run(wl, groups)
    for i, m in enumerate(mods):
        check_close(got[i], run_oracle(wl, m.name), wl.dtype, f"{name} {m.name}")
        skipped = wl.idx < 0
        assert np.array_equal(got[i][skipped], wl.y[m.name][skipped])


def test_warmed_small_batch_integer_data_is_exact():
    mods = [synth.Module("a", 2048, 1024), synth.Module("b", 1024, 512)]
    wl = synth.random_case(9600, synth.BF16, mods, 131, 5, 16, [16, 8, 16, 4, 12], integer=True)
    got = _run(wl, [[0, 1]])
    for i, m in enumerate(mods):
        assert np.array_equal(got[i], run_oracle(wl, m.name)), f"{m.name}: integer data must be exact"
