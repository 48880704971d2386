"""The seeded input generators: determinism and the shape of the draws."""
import numpy as np

from lora_adapter_application_amd import synth


def test_zipf_probs_finite_law():
    p = synth.zipf_probs(8, 1.1)
    k = np.arange(1, 9)
    assert abs(p.sum() - 1.0) < 1e-12
    assert np.allclose(p[0] / p, k ** 1.1)                      # P(k) ∝ k^-s
    assert np.all(np.diff(p) < 0)                               # slot 0 hottest
    # s < 1 is valid for the finite law (the churn workload uses 0.9)
    assert np.all(synth.zipf_probs(200, 0.9) > 0)


def test_draw_slots_base_only_share_and_zipf_frequencies():
    rng = np.random.default_rng(0)
    n = 200_000
    s = synth.draw_slots(rng, n, 8, 1.1, 0.10)
    assert s.dtype == np.int32 and s.min() == -1 and s.max() == 7
    assert abs((s == -1).mean() - 0.10) < 0.005
    act = s[s >= 0]
    freq = np.bincount(act, minlength=8) / act.size
    assert np.allclose(freq, synth.zipf_probs(8, 1.1), atol=0.005)


def test_workloads_are_deterministic():
    a = synth.llama7b_decode(n_tokens=64)
    b = synth.llama7b_decode(n_tokens=64)
    assert np.array_equal(a.idx, b.idx)
    for m in ("q_proj", "v_proj"):
        assert np.array_equal(a.x[m], b.x[m]) and np.array_equal(a.y[m], b.y[m])
        assert np.array_equal(a.adapters[3].At[m], b.adapters[3].At[m])
    c = synth.llama7b_decode(seed=77, n_tokens=64)
    assert not np.array_equal(a.x["q_proj"], c.x["q_proj"])


def test_tiny_fp32_workload():
    w = synth.tiny_fp32()
    assert w.dtype == synth.FP32 and w.n_tokens == 64 and w.max_loras == 4 and w.max_rank == 8
    assert set(np.unique(w.idx)) <= {-1, 0, 1, 2, 3}
    ad = w.adapters[0]
    assert ad.r == 8 and ad.lora_alpha == 16 and ad.At["linear"].shape == (8, 256)
    assert 0.015 < ad.At["linear"].std() < 0.025 and ad.B["linear"].dtype == np.float32


def test_decode_workload_values():
    w = synth.llama7b_decode()
    assert w.n_tokens == 256 and w.dtype == synth.BF16
    At = synth.bf16_bits_to_f32(w.adapters[0].At["q_proj"])
    assert At.shape == (16, 4096) and np.abs(At).max() <= 1 / 64 + 1e-6
    B = synth.bf16_bits_to_f32(w.adapters[0].B["q_proj"])
    assert 0.008 < B.std() < 0.012


def test_bf16_round_trip_is_torch_rne():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], np.float32)
    b = synth.to_bf16_bits(v)
    assert list(b) == [0x3F80, 0x3F82, 0xC020, 0x0000]
    assert np.array_equal(synth.bf16_bits_to_f32(b), np.array([1.0, 1.0 + 2 ** -6, -2.5, 0.0],
                                                               np.float32))


def test_prefill_segments_sorted_and_sized():
    rng = np.random.default_rng(1)
    lengths, slots = synth.prefill_lengths_and_slots(rng)
    assert lengths.shape == (32,) and lengths.min() >= 128 and lengths.max() <= 2048
    assert np.all(np.diff(slots) >= 0)
    # the default seed's batch: about 32 * 1088 tokens
    r_i = [np.random.default_rng(c) for c in
           np.random.SeedSequence(synth.SEEDS["llama7b_prefill"]).spawn(5)][0]
    L, _ = synth.prefill_lengths_and_slots(r_i)
    assert 20_000 < L.sum() < 50_000


def test_churn_step_respects_per_step_cap():
    rng = np.random.default_rng(5)
    ids, redraws = synth.churn_adapter_ids(rng)
    assert ids.shape == (8192,)
    assert len(np.unique(ids)) <= 128
    assert redraws > 0                                          # the cap binds at 7176 draws over 200
    pre = ids[:1024].reshape(8, 128)
    assert len(np.unique(pre[:, 0])) == 8 and np.all(pre == pre[:, :1])
    # a looser cap is never binding for a small step
    ids2, r2 = synth.churn_adapter_ids(np.random.default_rng(5), n_decode=16, cap=128)
    assert r2 == 0 and ids2.shape == (1024 + 16,)


def test_random_case_integer_values_and_targeting():
    mods = [synth.Module("a", 32, 16), synth.Module("b", 16, 48)]
    w = synth.random_case(3, synth.BF16, mods, 40, 4, 8, [8, 4, 2, 1],
                          targeted=[[True, False], [True, True], [False, True], [True, True]],
                          empty_slots=[3], integer=True)
    assert "b" not in w.adapters[0].At and "a" not in w.adapters[2].At
    assert w.adapters[3] is None
    vals = synth.bf16_bits_to_f32(w.x["a"])
    assert set(np.unique(vals)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
