"""Graph capture of the launching calls.

A sequence of lora_plan_prepare / lora_apply_group calls captured into a HIP
graph (through torch.cuda.graph, which captures the current stream) must
replay bit-identically to the same calls made eagerly, replay after replay,
with the program's own eager work and host synchronisation between replays;
the eager result itself matches the oracle.  Covers the inline plan (a batch of
at most 1024 tokens) and the plan kernels (a larger batch), grouped launches,
and the rule that loads must be complete before a capture starts.
"""
import numpy as np
import pytest
import torch

from gpu_util import check_close, from_dev, log, make_slots, run_oracle, to_dev, to_pinned
from lora_adapter_application_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


MODS = [synth.Module("q_proj", 512, 512), synth.Module("k_proj", 512, 256),
        synth.Module("v_proj", 512, 512)]
GROUPS = [[0, 1], [2]]


def _case(n_tokens, seed):
    return synth.random_case(seed, synth.BF16, MODS, n_tokens, 6, 32, [32, 16, 8, 32, 24, 16],
                             targeted=[[True, True, True], [True, False, True],
                                       [True, True, False], [False, True, True],
                                       [True, True, True], [True, True, True]],
                             p_base_only=0.1)


def _steps(S, idx, xs, ys):
    S.prepare(idx)
    for g in GROUPS:
        S.apply_group(g, [xs[i] for i in g], [ys[i] for i in g], idx)


@pytest.mark.parametrize("n_tokens", [200, 1500])
def test_graph_replay_matches_eager_and_oracle(n_tokens):
    wl = _case(n_tokens, 9100 + n_tokens)
    log("case graph replay", n_tokens)
    S = make_slots(wl)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in MODS]
    y0 = [to_dev(wl.y[m.name], wl.dtype) for m in MODS]

    # eager reference, checked against the oracle
    ye = [y.clone() for y in y0]
    _steps(S, idx, xs, ye)
    torch.cuda.synchronize()
    ref = [from_dev(y, wl.dtype) for y in ye]
    for mi, m in enumerate(MODS):
        check_close(ref[mi], run_oracle(wl, m.name), wl.dtype, f"eager {m.name}")

    # capture the same calls; capturing runs nothing
    yg = [y.clone() for y in y0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _steps(S, idx, xs, yg)
    torch.cuda.synchronize()
    for mi in range(len(MODS)):
        assert torch.equal(yg[mi], y0[mi]), "capture must not run the kernels"

    yo = [y.clone() for y in y0]
    for rep in range(3):
        for mi in range(len(MODS)):
            yg[mi].copy_(y0[mi])
            yo[mi].copy_(y0[mi])
        # eager work on the same ctx between replays
        _steps(S, idx, xs, yo)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for mi, m in enumerate(MODS):
            got = from_dev(yg[mi], wl.dtype)
            assert np.array_equal(got, ref[mi]), f"replay {rep} {m.name} differs from eager"
            assert np.array_equal(from_dev(yo[mi], wl.dtype), ref[mi]), f"eager {rep} {m.name}"
    S.close()


def test_capture_with_pending_load_is_rejected():
    wl = _case(64, 9200)
    S = make_slots(wl)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in MODS]
    ys = [to_dev(wl.y[m.name], wl.dtype) for m in MODS]
    # a load the host has not waited for
    ad = wl.adapters[0]
    keep = [to_pinned(ad.At[m.name], wl.dtype) for m in MODS] + \
           [to_pinned(ad.B[m.name], wl.dtype) for m in MODS]
    S.load(0, keep[:3], keep[3:], ad.r, ad.lora_alpha, ad.use_rslora)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with pytest.raises(binding.LoraError, match="lora_sync_loads"):
        with torch.cuda.graph(g, stream=s):
            _steps(S, idx, xs, ys)
    torch.cuda.synchronize()
    # after the loads are complete the same calls capture and replay
    S.sync_loads()
    before = [from_dev(y, wl.dtype) for y in ys]
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        _steps(S, idx, xs, ys)
    g2.replay()
    torch.cuda.synchronize()
    for mi, m in enumerate(MODS):
        ref = run_oracle(wl, m.name)
        check_close(from_dev(ys[mi], wl.dtype), ref, wl.dtype, f"after sync {m.name}")
        assert not np.array_equal(from_dev(ys[mi], wl.dtype), before[mi]) or \
            np.array_equal(ref, before[mi])
    S.close()


def test_bound_step_matches_direct_calls():
    """Slots.bind_step marshals the arguments once; its calls give the same bits."""
    wl = _case(300, 9300)
    S = make_slots(wl)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in MODS]
    y0 = [to_dev(wl.y[m.name], wl.dtype) for m in MODS]
    yd = [y.clone() for y in y0]
    _steps(S, idx, xs, yd)
    yb = [y.clone() for y in y0]
    step = S.bind_step([(g, [xs[i] for i in g], [yb[i] for i in g]) for g in GROUPS], idx)
    step()
    torch.cuda.synchronize()
    for mi in range(len(MODS)):
        assert torch.equal(yb[mi], yd[mi])
    S.close()


def test_load_during_capture_is_rejected():
    """A load while a stream the ctx launched on is being captured fails before it
    enqueues anything (its fences would record into the capture); the capture and
    later loads are unaffected."""
    wl = _case(64, 9201)
    S = make_slots(wl)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in MODS]
    ys = [to_dev(wl.y[m.name], wl.dtype) for m in MODS]
    ad = wl.adapters[0]
    keep = [to_pinned(ad.At[m.name], wl.dtype) for m in MODS] + \
           [to_pinned(ad.B[m.name], wl.dtype) for m in MODS]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _steps(S, idx, xs, ys)
        with pytest.raises(binding.LoraError, match="graph capture"):
            S.load(0, keep[:3], keep[3:], ad.r, ad.lora_alpha, ad.use_rslora)
    g.replay()
    torch.cuda.synchronize()
    for mi, m in enumerate(MODS):
        check_close(from_dev(ys[mi], wl.dtype), run_oracle(wl, m.name), wl.dtype, f"replay {m.name}")
    # after the capture, the same load goes through
    S.load(0, keep[:3], keep[3:], ad.r, ad.lora_alpha, ad.use_rslora)
    S.sync_loads()
    assert S.stats()["loads"] == len([a for a in wl.adapters if a is not None]) + 1
    S.close()


def test_reload_between_replays_follows_the_replay_contract():
    """A slot reloaded between two replays, under the rules the header states
    (no replay in flight at the load; lora_sync_loads before the next replay),
    with an adapter of the same rank, lora_alpha and target modules: the first
    replay gives the old adapter's update, the second the new one's, each
    checked against the oracle."""
    wl = _case(300, 9400)
    log("case reload between replays")
    S = make_slots(wl)
    idx = torch.from_numpy(wl.idx).cuda()
    xs = [to_dev(wl.x[m.name], wl.dtype) for m in MODS]
    y0 = [to_dev(wl.y[m.name], wl.dtype) for m in MODS]
    yg = [y.clone() for y in y0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _steps(S, idx, xs, yg)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()                     # rule 1: no replay in flight at the load
    for mi, m in enumerate(MODS):
        check_close(from_dev(yg[mi], wl.dtype), run_oracle(wl, m.name), wl.dtype,
                    f"replay before reload {m.name}")
    # a new adapter for slot 0: same rank, lora_alpha and targets, other weights
    old = wl.adapters[0]
    new = _case(8, 9401).adapters[0]
    assert new.r == old.r and set(new.At) == set(old.At)
    keep = [to_pinned(new.At[m.name], wl.dtype) for m in MODS] + \
           [to_pinned(new.B[m.name], wl.dtype) for m in MODS]
    S.load(0, keep[:3], keep[3:], new.r, old.lora_alpha, old.use_rslora)
    S.sync_loads()                               # rule 2: the load is complete before the replay
    for mi in range(len(MODS)):
        yg[mi].copy_(y0[mi])
    g.replay()
    torch.cuda.synchronize()
    new.lora_alpha, new.use_rslora = old.lora_alpha, old.use_rslora
    wl.adapters[0] = new
    for mi, m in enumerate(MODS):
        got = from_dev(yg[mi], wl.dtype)
        check_close(got, run_oracle(wl, m.name), wl.dtype, f"replay after reload {m.name}")
        on0 = wl.idx == 0
        assert on0.any()
    S.close()
