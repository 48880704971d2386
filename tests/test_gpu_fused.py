"""The fused decode launch (lora_apply_group_fused on bf16 batches of at most
1024 tokens: shrink and expand in one launch, every workgroup of a tile on the
tile's XCD, the expand workgroups waiting for their tile's K-split partials
through per-(tile, member) counts).

Its results must equal the two-launch path of the separate lora_shrink /
lora_expand entry points bit for bit, launch after launch (the counts return to
zero after every launch), inside a captured graph replayed several times with
eager work between the replays, with the inline plan and with published tiles,
and never set LORA_FLAG_FUSED_TIMEOUT; and match the oracle.
"""
import numpy as np
import pytest
import torch

from gpu_util import check_close, from_dev, log, make_slots, run_gpu, run_oracle, to_dev
from lora_adapter_application_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


CASES = [
    # modules, max_loras, R, ranks, T, p_base_only, zipf
    ([(4096, 4096), (4096, 4096)], 8, 16, [16] * 8, 256, 0.10, 1.1),
    ([(5120, 8192), (5120, 1024), (5120, 1024)], 16, 32, [32] * 16, 512, 0.05, 1.2),
    ([(1032, 520), (264, 392)], 6, 64, [64, 8, 33, 1, 17, 64], 1024, 0.1, 0.5),
    ([(512, 256)], 3, 128, [128, 100, 7], 1, 0.0, 1.1),
    ([(384, 1544)], 256, 16, [(k % 16) + 1 for k in range(256)], 700, 0.02, 0.3),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_equals_two_launches_repeatedly(case):
    shapes, S_, R, ranks, T, pb, zs = CASES[case]
    mods = [synth.Module(f"m{i}", a, b) for i, (a, b) in enumerate(shapes)]
    wl = synth.random_case(9600 + case, synth.BF16, mods, T, S_, R, ranks, p_base_only=pb, zipf_s=zs)
    log(f"case fused {case}: {shapes} S={S_} R={R} T={T}")
    S = make_slots(wl)
    split = run_gpu(wl, S, path="split")           # two launches per module
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
    mi = list(range(len(mods)))
    S.prepare(idx)
    S.profile_begin(64)
    for rep in range(12):                           # inline plan first, published tiles after
        ys = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
        S.apply_group_fused(mi, xs, ys, idx)
        torch.cuda.synchronize()
        for i, m in enumerate(mods):
            assert np.array_equal(from_dev(ys[i], wl.dtype), split[m.name]), (rep, m.name)
    launches = S.profile_end()["launches"]
    log(f"fused case {case}: launches {launches}")
    # one fused launch per call (this device places workgroup i on XCD i % 8,
    # else the calls would have taken the two launches)
    assert launches["fused"] == 12 and launches["shrink"] == 0 and launches["expand"] == 0, launches
    assert S.flags() == 0
    for m in mods:
        check_close(split[m.name], run_oracle(wl, m.name), wl.dtype, f"fused case {case} {m.name}")
    S.close()


TERMS_CASES = [
    # modules, max_loras, R, ranks, T, bias slots, DoRA slots
    ([(4096, 4096), (4096, 1024)], 8, 16, [16, 9, 16, 16, 4, 16, 16, 1], 256, {1, 3, 4}, {2, 3, 6}),
    ([(5120, 1032), (1000, 520)], 6, 32, [32, 17, 32, 5, 32, 32], 600, {0, 2, 5}, {1, 2}),
]


@pytest.mark.parametrize("case", range(len(TERMS_CASES)))
def test_fused_with_output_terms_equals_two_launches(case):
    # slots with an output bias and / or a DoRA factor take the fused kernel's
    # output-terms instances
    shapes, S_, R, ranks, T, bias, dora = TERMS_CASES[case]
    mods = [synth.Module(f"m{i}", a, b) for i, (a, b) in enumerate(shapes)]
    wl = synth.random_case(9800 + case, synth.BF16, mods, T, S_, R, ranks, p_base_only=0.1, zipf_s=1.0)
    synth.add_output_terms(wl, 9800 + case, bias_slots=bias, dora_slots=dora)
    log(f"case fused terms {case}: {shapes} S={S_} R={R} T={T} bias {sorted(bias)} dora {sorted(dora)}")
    S = make_slots(wl)
    split = run_gpu(wl, S, path="split")
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
    S.prepare(idx)
    S.profile_begin(16)
    for rep in range(3):
        ys = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
        S.apply_group_fused(list(range(len(mods))), xs, ys, idx)
        torch.cuda.synchronize()
        for i, m in enumerate(mods):
            assert np.array_equal(from_dev(ys[i], wl.dtype), split[m.name]), (rep, m.name)
    launches = S.profile_end()["launches"]
    assert launches["fused"] == 3 and launches["shrink"] == 0 and launches["expand"] == 0, launches
    assert S.flags() == 0
    for m in mods:
        check_close(split[m.name], run_oracle(wl, m.name), wl.dtype, f"fused terms case {case} {m.name}")
    S.close()


def test_fused_launches_on_two_streams_at_once():
    # two ctxs launching fused decodes on two streams with no synchronisation
    # between them, so their kernels run side by side: each launch's
    # workgroups must still meet on their tiles' XCDs
    mods = [synth.Module("q", 4096, 4096), synth.Module("v", 4096, 1024)]
    cases = []
    for c, (S_, R) in enumerate([(8, 16), (12, 32)]):
        wl = synth.random_case(9900 + c, synth.BF16, mods, 384, S_, R, [R] * S_, p_base_only=0.1)
        S = make_slots(wl)
        split = run_gpu(wl, S, path="split")
        idx = torch.from_numpy(wl.idx).cuda()
        xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
        cases.append((wl, S, split, idx, xs))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = [[], []]
    for rep in range(16):
        for c, (wl, S, split, idx, xs) in enumerate(cases):
            with torch.cuda.stream(streams[c]):
                ys = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
                S.apply_group_fused([0, 1], xs, ys, idx, stream=streams[c])
                outs[c].append(ys)
    torch.cuda.synchronize()
    for c, (wl, S, split, idx, xs) in enumerate(cases):
        for rep, ys in enumerate(outs[c]):
            for i, m in enumerate(mods):
                assert np.array_equal(from_dev(ys[i], wl.dtype), split[m.name]), (c, rep, m.name)
        assert S.flags() == 0
        S.close()


def test_fused_launches_beside_a_long_kernel():
    # fused decodes on one stream while another stream runs large matrix
    # products that hold most of the chip: the fused workgroups start as CUs
    # free up, in whatever order, and must still meet on their tiles' XCDs
    mods = [synth.Module("q", 4096, 4096), synth.Module("v", 4096, 4096)]
    wl = synth.random_case(9950, synth.BF16, mods, 256, 8, 16, [16] * 8, p_base_only=0.1)
    S = make_slots(wl)
    split = run_gpu(wl, S, path="split")
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda")
    busy, work = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    with torch.cuda.stream(busy):
        for _ in range(6):
            c = torch.mm(a, b)
    for rep in range(24):
        with torch.cuda.stream(work):
            ys = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
            S.apply_group_fused([0, 1], xs, ys, idx, stream=work)
            outs.append(ys)
    torch.cuda.synchronize()
    del c
    for rep, ys in enumerate(outs):
        for i, m in enumerate(mods):
            assert np.array_equal(from_dev(ys[i], wl.dtype), split[m.name]), (rep, m.name)
    assert S.flags() == 0
    S.close()


def test_fused_graph_replays():
    mods = [synth.Module("q", 4096, 4096), synth.Module("v", 4096, 4096)]
    wl = synth.random_case(9700, synth.BF16, mods, 256, 8, 16, [16] * 8, p_base_only=0.1)
    S = make_slots(wl)
    split = run_gpu(wl, S, path="split")
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in mods]
    y0 = [to_dev(wl.y[m.name], wl.dtype) for m in mods]
    yg = [y.clone() for y in y0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        S.prepare(idx)
        S.apply_group_fused([0, 1], xs, yg, idx)
    torch.cuda.synchronize()
    ye = [y.clone() for y in y0]
    for rep in range(5):
        for i in range(2):
            yg[i].copy_(y0[i])
            ye[i].copy_(y0[i])
        S.apply_group_fused([0, 1], xs, ye, idx)    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, m in enumerate(mods):
            assert np.array_equal(from_dev(yg[i], wl.dtype), split[m.name]), (rep, m.name)
            assert np.array_equal(from_dev(ye[i], wl.dtype), split[m.name]), (rep, m.name)
    assert S.flags() == 0
    S.close()
