"""Seeded random configurations against the oracle.

Each case draws module shapes (multiples of 8, 64..4096), group layout (one
group or two, members sharing one x buffer or not), slot count, padded and
per-slot ranks, target masks, empty slots, rsLoRA, output bias and DoRA
factors, a base-only share, and a token count around the boundaries the
kernels switch at (16 and 64 tokens per tile, 1024 tokens for the inline
plan).  The adapter weights come from pinned memory, device memory or
misaligned pinned views in turn, the three ways a load reads them.  Every module's output must match the oracle, and tokens the update
does not apply to must stay bit-identical.
"""
import numpy as np
import pytest
import torch

from gpu_util import check_close, from_dev, log, make_slots, run_oracle, to_dev
from lora_adapter_application_amd import binding, synth

pytestmark = pytest.mark.gpu

N_CASES = 120
DIMS = [64, 128, 256, 384, 512, 768, 1024, 1536, 2048, 4096]
TOKENS = [1, 7, 16, 17, 64, 65, 200, 513, 1023, 1024, 1025, 1500, 2047]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _draw(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.choice(TOKENS))
    dims = DIMS if T <= 1024 else DIMS[:-1]           # keeps the oracle to seconds
    n_mod = int(rng.integers(1, 5))
    shared = n_mod > 1 and rng.random() < 0.4
    d0 = int(rng.choice(dims))
    mods = [synth.Module(f"m{i}", d0 if shared or i == 0 else int(rng.choice(dims)), int(rng.choice(dims)))
            for i in range(n_mod)]
    S = int(rng.integers(1, 33))
    R = int(rng.choice([8, 16, 24, 32, 48, 64, 96, 128]))
    ranks = [int(r) for r in rng.integers(1, R + 1, S)]
    targeted = [[bool(rng.random() < 0.85) for _ in mods] for _ in range(S)]
    empty = [k for k in range(S) if rng.random() < 0.1]
    wl = synth.random_case(int(rng.integers(1 << 30)), synth.BF16, mods, T, S, R, ranks,
                           targeted=targeted, p_base_only=float(rng.choice([0.0, 0.05, 0.3])),
                           zipf_s=float(rng.choice([0.5, 1.1, 2.0])), empty_slots=empty,
                           rslora=bool(rng.random() < 0.3))
    if rng.random() < 0.25:
        synth.add_output_terms(wl, seed, bias_slots=[k for k in range(S) if rng.random() < 0.5],
                               dora_slots=[k for k in range(S) if rng.random() < 0.3])
    if shared:
        for m in mods[1:]:
            wl.x[m.name] = wl.x[mods[0].name]
    if n_mod > 1 and rng.random() < 0.5:
        cut = int(rng.integers(1, n_mod))
        groups = [list(range(cut)), list(range(cut, n_mod))]
    else:
        groups = [list(range(n_mod))]
    return wl, groups, shared


SOURCES = ["pinned", "device", "staged"]


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration_matches_oracle(seed):
    wl, groups, shared = _draw(31000 + seed)
    source = SOURCES[seed % 3]
    log("case random", seed, "T", wl.n_tokens, "S", wl.max_loras, "R", wl.max_rank,
        [(m.d_in, m.d_out) for m in wl.modules], "groups", groups, "shared", shared, "weights", source)
    S = make_slots(wl, source=source)
    idx = torch.from_numpy(wl.idx).cuda()
    names = [m.name for m in wl.modules]
    x0 = to_dev(wl.x[names[0]], wl.dtype)
    xs = [x0 if (shared or i == 0) else to_dev(wl.x[n], wl.dtype) for i, n in enumerate(names)]
    ys = [to_dev(wl.y[n], wl.dtype) for n in names]
    S.prepare(idx)
    for g in groups:
        S.apply_group(g, [xs[i] for i in g], [ys[i] for i in g], idx)
    torch.cuda.synchronize()
    S.close()
    for i, m in enumerate(wl.modules):
        got = from_dev(ys[i], wl.dtype)
        check_close(got, run_oracle(wl, m.name), wl.dtype, f"seed {seed} {m.name}")
        applied = np.array([k >= 0 and wl.adapters[k] is not None and m.name in wl.adapters[k].At
                            for k in wl.idx])
        assert np.array_equal(got[~applied], wl.y[m.name][~applied]), f"seed {seed} {m.name}: untouched rows"
