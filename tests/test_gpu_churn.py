"""The churn workload on the GPU: 128 slots, a 200-adapter pinned pool, LRU
residency, loads before every step, and parity on every step.

The oracle takes each sampled token's *adapter id* and reads the host pool
directly, so a wrong slot mapping, a stale slot or a load that landed in the
wrong place fails the comparison."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import as_f64, log, rel_l2
from lora_adapter_application_amd import binding, synth
from lora_adapter_application_amd.lru import SlotLRU

pytestmark = pytest.mark.gpu

GROUPS = [["q_proj", "v_proj"], ["gate_proj", "up_proj"], ["down_proj"]]
N_STEPS = 50


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def pool():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    return synth.churn_pool_device()


def check_rows(slots, rng, full):
    """Rows compared on one step: all of them (full), else the first and the last
    token of every resident slot's run and random rows, at least 512 in all."""
    T = slots.shape[0]
    if full:
        return np.arange(T)
    picked = set()
    for k in np.unique(slots[slots >= 0]):
        where = np.flatnonzero(slots == k)
        picked.update((int(where[0]), int(where[-1])))
    picked.update((0, 1023, 1024, T - 1))
    need = max(0, 512 - len(picked)) + 64
    picked.update(int(r) for r in rng.choice(T, size=need, replace=False))
    return np.array(sorted(picked))


def compare_rows(pool, names, ids, rows, x, y, y0, what):
    """Oracle on the given rows (by adapter id, from the host pool) against the
    device result; returns the worst err/bound."""
    rows_t = torch.from_numpy(rows).cuda()
    worst = 0.0
    for n in names:
        adapters = [None] * 200
        for a in np.unique(ids[rows]):
            adapters[int(a)] = pool.adapter(n, int(a))
        ref = oracle.apply(oracle.BF16, bits(x[n][rows_t]), y0[n], ids[rows], adapters)
        got = bits(y[n][rows_t])
        g64, r64 = as_f64(got, synth.BF16), as_f64(ref, synth.BF16)
        w = float((np.abs(g64 - r64) / (2e-2 * (1 + np.abs(r64)))).max())
        worst = max(worst, w)
        assert w <= 1.0, f"{what} {n}: err/bound {w:.3f}"
    return worst


FULL_STEPS = (0, N_STEPS - 1)


def test_churn_all_steps_match_oracle(pool):
    mods = synth.CHURN_MODULES
    names = [m.name for m in mods]
    S = binding.Slots(128, 64, [(m.d_in, m.d_out) for m in mods], "bf16", max_tokens=8192)
    lru = SlotLRU(128)
    rng = np.random.default_rng(0)
    worst = 0.0
    n_rows = 0
    for step in range(N_STEPS + 1):
        weak = step == N_STEPS                  # one more step with base y = 0
        ids, redraws, x, y = synth.churn_step_device(step)
        if weak:
            y = {n: torch.zeros_like(y[n]) for n in names}
        slots, loads = lru.plan_step(ids)
        assert len(np.unique(ids)) <= 128
        for slot, a in loads:
            S.load(slot, [pool.At[n][a] for n in names], [pool.B[n][a] for n in names], 64, 128.0)
        rows = check_rows(slots, rng, full=step in FULL_STEPS or weak)
        rows_t = torch.from_numpy(rows).cuda()
        y0 = {n: bits(y[n][rows_t]) for n in names}
        idx = torch.from_numpy(slots).cuda()
        S.prepare(idx)
        for g in GROUPS:
            mi = [names.index(n) for n in g]
            S.shrink_group(mi, [x[n] for n in g])
            S.expand_group(mi, [y[n] for n in g])
        torch.cuda.synchronize()
        if weak:
            for n in names:
                adapters = [None] * 200
                for a in np.unique(ids):
                    adapters[int(a)] = pool.adapter(n, int(a))
                ref = oracle.apply(oracle.BF16, bits(x[n]), y0[n], ids, adapters)
                e = rel_l2(as_f64(bits(y[n]), synth.BF16), as_f64(ref, synth.BF16))
                log(f"weak-signal churn {n}: rel L2 {e:.3e}")
                assert e < 1e-2, (n, e)
            continue
        worst = max(worst, compare_rows(pool, names, ids, rows, x, y, y0, f"step {step}"))
        n_rows += len(rows)
        if step % 10 == 0 or step in FULL_STEPS:
            log(f"churn step {step}: {len(loads)} loads, redraws {redraws}, {len(rows)} rows, "
                f"worst {worst:.3f}")
    st = lru.stats
    log(f"churn: hits {st.hits} misses {st.misses} evictions {st.evictions} "
        f"thrash {st.thrash_ratio:.3f} rows compared {n_rows} worst err/bound {worst:.3f}")
    assert S.stats()["loads"] == st.misses
    assert S.stats()["bytes_loaded"] == st.misses * oracle.adapter_bytes(
        [(m.d_in, m.d_out) for m in mods], [True] * 5, 64, 2)
    S.close()


def test_churn_pipelined_uploads_match_oracle(pool):
    """The churn as a pipeline: step s+1's misses are uploaded while step s runs
    (declared slots, 144 slots for a per-step cap of 128), with no host wait
    between steps; every step's rows (at least 512, every row of the first and
    the last step) must match the oracle."""
    mods = synth.CHURN_MODULES
    names = [m.name for m in mods]
    n_steps = 16
    S = binding.Slots(144, 64, [(m.d_in, m.d_out) for m in mods], "bf16", max_tokens=8192)
    lru = SlotLRU(144)
    rng = np.random.default_rng(1)
    sched, prev = [], set()
    for step in range(n_steps):
        ids, _, x, y = synth.churn_step_device(100 + step)
        slots, loads = lru.plan_step(ids, avoid=prev)
        used = sorted({int(v) for v in slots[slots >= 0]})
        prev = set(used)
        rows = check_rows(slots, rng, full=step in (0, n_steps - 1))
        rows_t = torch.from_numpy(rows).cuda()
        y0 = {n: bits(y[n][rows_t]) for n in names}
        sched.append((ids, torch.from_numpy(slots).cuda(), used, loads, x, y, rows, y0))
    torch.cuda.synchronize()

    def issue(loads):
        for slot, a in loads:
            S.load(slot, [pool.At[n][a] for n in names], [pool.B[n][a] for n in names], 64, 128.0)

    issue(sched[0][3])
    for step in range(n_steps):
        _, idx, used, _, x, y, _, _ = sched[step]
        S.prepare(idx, used_slots=used)
        for g in GROUPS:
            mi = [names.index(n) for n in g]
            S.apply_group(mi, [x[n] for n in g], [y[n] for n in g], idx)
        if step + 1 < n_steps:
            issue(sched[step + 1][3])
    torch.cuda.synchronize()
    worst = 0.0
    for step in range(n_steps):
        ids, _, _, _, x, y, rows, y0 = sched[step]
        worst = max(worst, compare_rows(pool, names, ids, rows, x, y, y0, f"pipelined step {step}"))
    log(f"pipelined churn: {lru.stats.misses} misses, worst err/bound {worst:.3f}")
    S.close()
