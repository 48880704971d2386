"""Seeded random configurations over wide slot counts and batch sizes.

Up to 256 slots (the library's limit) and 8192 tokens (plan kernels above 1024
tokens), base-only shares up to one half, uniform to steep Zipf popularity,
empty slots, rsLoRA, slot indices past max_loras and negative ones other than
-1 (both skipped), and adapter weights from pinned memory, device memory and
misaligned pinned views in turn.  Every module must match the oracle and every
token the update does not apply to must keep its row bit-identical.
"""
import numpy as np
import pytest
import torch

from gpu_util import check_close, from_dev, log, make_slots, run_oracle, to_dev
from lora_adapter_application_amd import binding, synth

pytestmark = pytest.mark.gpu

N_CASES = 24
TOKENS = [1, 31, 64, 255, 1024, 1025, 2049, 4096, 5000, 8192]
DIMS = [64, 128, 256, 512, 1024]
SLOTS = [1, 2, 7, 64, 128, 200, 256]
SOURCES = ["pinned", "device", "staged"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _draw(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.choice(TOKENS))
    n_mod = int(rng.integers(1, 4))
    mods = [synth.Module(f"m{i}", int(rng.choice(DIMS)), int(rng.choice(DIMS))) for i in range(n_mod)]
    S = int(rng.choice(SLOTS))
    R = int(rng.choice([8, 16, 32, 64, 128]))
    ranks = [int(r) for r in rng.integers(1, R + 1, S)]
    wl = synth.random_case(int(rng.integers(1 << 30)), synth.BF16, mods, T, S, R, ranks,
                           p_base_only=float(rng.choice([0.0, 0.1, 0.5])),
                           zipf_s=float(rng.choice([0.0, 0.5, 1.1, 3.0])),
                           empty_slots=[k for k in range(S) if rng.random() < 0.05],
                           rslora=bool(rng.random() < 0.3))
    if rng.random() < 0.2 and T > 4:
        wl.idx[rng.integers(0, T, 3)] = S + int(rng.integers(0, 5))
        wl.idx[rng.integers(0, T, 2)] = -int(rng.integers(2, 100))
    return wl


@pytest.mark.parametrize("seed", range(N_CASES))
def test_wide_configuration_matches_oracle(seed):
    wl = _draw(52000 + seed)
    mods = wl.modules
    S = wl.max_loras
    source = SOURCES[seed % 3]
    log("case wide", seed, source, "T", wl.n_tokens, "S", S, "R", wl.max_rank,
        [(m.d_in, m.d_out) for m in mods])
    Sl = make_slots(wl, source=source)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
    ys = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
    Sl.prepare(idx)
    Sl.apply_group(list(range(len(mods))), xs, ys, idx)
    torch.cuda.synchronize()
    Sl.close()
    for i, m in enumerate(mods):
        got = from_dev(ys[i], wl.dtype)
        check_close(got, run_oracle(wl, m.name), wl.dtype, f"seed {seed} {m.name}")
        applied = np.array([0 <= k < S and wl.adapters[k] is not None and m.name in wl.adapters[k].At
                            for k in wl.idx])
        assert np.array_equal(got[~applied], wl.y[m.name][~applied]), f"seed {seed} {m.name}: untouched rows"
