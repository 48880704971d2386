"""Seeded synthetic inputs for the multi-adapter LoRA update.

This module draws inputs only; it contains none of the update's arithmetic.  It
is shared by the parity tests (which hand the same bits to the CPU oracle and to
the HIP path) and by ``bench.py``.  Values meant to be bf16 are drawn in fp32 and
rounded to bf16 by torch's own conversion (round to nearest even), so both sides
see identical input bits.

Workloads (shapes follow Llama-7B and Qwen3-32B projections; the pages show
adapters on q/k/v/o projections and MLP layers with ranks up to 64, the example
adapter_config in "vLLM LoRA Resolver plugins explained", section 3.2, and the
manifest in "Multi-LoRA adapter cache in production", section "adapter capacity
cannot be planned by count alone"):

  tiny_fp32        1 module 256->256, fp32, 4 slots rank 8, alpha 16, 64 tokens
  llama7b_decode   q,v 4096->4096, bf16, 8 slots rank 16, alpha 32, 256 tokens
  llama7b_prefill  q,k,v,o 4096->4096, bf16, 8 slots ranks {8,16,32,64} padded to 64,
                   alpha 2r, 32 requests of 128..2048 tokens sorted into segments
  qwen32b_decode   q 5120->8192, k,v 5120->1024, o 8192->5120, bf16, 16 slots
                   rank 32, alpha 64, rsLoRA, 512 tokens
  churn            gate,up 4096->11008, down 11008->4096, q,v 4096->4096, bf16,
                   128 slots rank 64, alpha 128, 200-adapter pool, 8192 tokens/step

Readings of points the workload descriptions leave open:
  * N(mu, sigma): sigma is the standard deviation; U(+-a) is uniform on [-a, a].
  * Zipf(s) over N slots is the finite law P(k) ∝ k^-s, k = 1..N, rank k -> slot
    k-1 (slot 0 hottest).  The "base only" share is drawn first, per token.
  * Unstated distributions reuse the decode workload's: x ~ N(0,1),
    At ~ U(+-1/sqrt(d_in)), B ~ N(0, 0.01), base y ~ N(0,1).
  * Churn steps: 8 prefill requests x 128 tokens with 8 distinct adapters drawn
    without replacement, then 7168 one-token decode requests; a decode draw
    that would be the 129th distinct adapter of the step is drawn again, since
    only 128 slots exist and adapters in use cannot be evicted ("max_loras"
    bounds the adapters of one batch, "Multi-LoRA adapter cache in production",
    parameter table and section "common misconceptions", item 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


@dataclass
class Module:
    name: str
    d_in: int
    d_out: int


@dataclass
class Adapter:
    """One adapter: per targeted module, At (r x d_in) and B (r x d_out); optionally
    an output bias (d_out, data dtype) and a DoRA factor (d_out, float32)."""
    r: int
    lora_alpha: float
    use_rslora: bool
    At: Dict[str, np.ndarray] = field(default_factory=dict)
    B: Dict[str, np.ndarray] = field(default_factory=dict)
    bias: Optional[Dict[str, np.ndarray]] = None
    dora_scale: Optional[Dict[str, np.ndarray]] = None


@dataclass
class Workload:
    name: str
    dtype: str
    modules: List[Module]
    max_loras: int
    max_rank: int
    adapters: List[Optional[Adapter]]          # per slot (None = empty slot)
    idx: np.ndarray                            # int32 [T]
    x: Dict[str, np.ndarray]                   # per module [T, d_in]
    y: Dict[str, np.ndarray]                   # per module [T, d_out]

    @property
    def n_tokens(self) -> int:
        return int(self.idx.shape[0])


# ----------------------------------------------------------------------------
# primitives

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, via torch's round-to-nearest-even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(a) if dtype == BF16 else np.ascontiguousarray(a, dtype=np.float32)


def zipf_probs(n: int, s: float) -> np.ndarray:
    k = np.arange(1, n + 1, dtype=np.float64)
    w = k ** (-float(s))
    return w / w.sum()


def draw_slots(rng: np.random.Generator, n_tokens: int, n_slots: int, s: float,
               p_base_only: float) -> np.ndarray:
    """Per-token slot: -1 with probability p_base_only, else Zipf(s) over n_slots."""
    base_only = rng.random(n_tokens) < p_base_only
    slots = rng.choice(n_slots, size=n_tokens, p=zipf_probs(n_slots, s)).astype(np.int32)
    slots[base_only] = -1
    return slots


def normal(rng, shape, std, dtype):
    return _cast(rng.standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)


def uniform(rng, shape, bound, dtype):
    return _cast(rng.uniform(-bound, bound, size=shape).astype(np.float32), dtype)


def _children(seed: int, n: int = 5):
    return [np.random.default_rng(c) for c in np.random.SeedSequence(seed).spawn(n)]


# ----------------------------------------------------------------------------
# workloads

WORKLOADS = ("tiny_fp32", "llama7b_decode", "llama7b_prefill", "qwen32b_decode", "churn")
SEEDS = {name: 1000 + i for i, name in enumerate(WORKLOADS)}

LLAMA7B_ATTN = [Module("q_proj", 4096, 4096), Module("k_proj", 4096, 4096),
                Module("v_proj", 4096, 4096), Module("o_proj", 4096, 4096)]
QWEN32B_ATTN = [Module("q_proj", 5120, 8192), Module("k_proj", 5120, 1024),
                Module("v_proj", 5120, 1024), Module("o_proj", 8192, 5120)]
CHURN_MODULES = [Module("gate_proj", 4096, 11008), Module("up_proj", 4096, 11008),
                 Module("down_proj", 11008, 4096), Module("q_proj", 4096, 4096),
                 Module("v_proj", 4096, 4096)]


def _make_adapters(rng_a, rng_b, modules, ranks, alphas, rslora, a_dist, b_std, dtype):
    adapters = []
    for r, alpha in zip(ranks, alphas):
        ad = Adapter(r=int(r), lora_alpha=float(alpha), use_rslora=bool(rslora))
        for m in modules:
            if a_dist == "normal":
                ad.At[m.name] = normal(rng_a, (r, m.d_in), 0.02, dtype)
            else:
                ad.At[m.name] = uniform(rng_a, (r, m.d_in), 1.0 / np.sqrt(m.d_in), dtype)
            ad.B[m.name] = normal(rng_b, (r, m.d_out), b_std, dtype)
        adapters.append(ad)
    return adapters


def _activations(rng_x, rng_y, modules, T, dtype, y_zero=False):
    x = {m.name: normal(rng_x, (T, m.d_in), 1.0, dtype) for m in modules}
    if y_zero:
        y = {m.name: _cast(np.zeros((T, m.d_out), np.float32), dtype) for m in modules}
    else:
        y = {m.name: normal(rng_y, (T, m.d_out), 1.0, dtype) for m in modules}
    return x, y


def tiny_fp32(seed: Optional[int] = None, y_zero: bool = False) -> Workload:
    r_i, r_x, r_a, r_b, r_y = _children(SEEDS["tiny_fp32"] if seed is None else seed)
    mods = [Module("linear", 256, 256)]
    idx = (r_i.integers(0, 5, size=64) - 1).astype(np.int32)     # uniform over {-1,0,1,2,3}
    adapters = _make_adapters(r_a, r_b, mods, [8] * 4, [16.0] * 4, False, "normal", 0.02, FP32)
    x, y = _activations(r_x, r_y, mods, 64, FP32, y_zero)
    return Workload("tiny_fp32", FP32, mods, 4, 8, adapters, idx, x, y)


def llama7b_decode(seed: Optional[int] = None, n_tokens: int = 256, y_zero: bool = False,
                   modules: Optional[Sequence[Module]] = None) -> Workload:
    r_i, r_x, r_a, r_b, r_y = _children(SEEDS["llama7b_decode"] if seed is None else seed)
    mods = list(modules) if modules is not None else [Module("q_proj", 4096, 4096),
                                                      Module("v_proj", 4096, 4096)]
    idx = draw_slots(r_i, n_tokens, 8, 1.1, 0.10)
    adapters = _make_adapters(r_a, r_b, mods, [16] * 8, [32.0] * 8, False, "uniform", 0.01, BF16)
    x, y = _activations(r_x, r_y, mods, n_tokens, BF16, y_zero)
    return Workload("llama7b_decode", BF16, mods, 8, 16, adapters, idx, x, y)


def prefill_lengths_and_slots(rng_i, n_requests=32, lo=128, hi=2048, n_slots=8, s=1.1):
    """Request lengths U{lo..hi}, one Zipf(s) adapter per request, stable-sorted by slot."""
    lengths = rng_i.integers(lo, hi + 1, size=n_requests)
    slots = rng_i.choice(n_slots, size=n_requests, p=zipf_probs(n_slots, s))
    order = np.argsort(slots, kind="stable")
    return lengths[order], slots[order]


def llama7b_prefill(seed: Optional[int] = None, n_requests: int = 32, lo: int = 128,
                    hi: int = 2048, y_zero: bool = False,
                    modules: Optional[Sequence[Module]] = None) -> Workload:
    r_i, r_x, r_a, r_b, r_y = _children(SEEDS["llama7b_prefill"] if seed is None else seed)
    mods = list(modules) if modules is not None else list(LLAMA7B_ATTN)
    lengths, slots = prefill_lengths_and_slots(r_i, n_requests, lo, hi)
    idx = np.repeat(slots, lengths).astype(np.int32)
    ranks = [[8, 16, 32, 64][k % 4] for k in range(8)]
    adapters = _make_adapters(r_a, r_b, mods, ranks, [2.0 * r for r in ranks], False,
                              "uniform", 0.01, BF16)
    x, y = _activations(r_x, r_y, mods, int(idx.shape[0]), BF16, y_zero)
    return Workload("llama7b_prefill", BF16, mods, 8, 64, adapters, idx, x, y)


def qwen32b_decode(seed: Optional[int] = None, n_tokens: int = 512, y_zero: bool = False,
                   modules: Optional[Sequence[Module]] = None) -> Workload:
    r_i, r_x, r_a, r_b, r_y = _children(SEEDS["qwen32b_decode"] if seed is None else seed)
    mods = list(modules) if modules is not None else list(QWEN32B_ATTN)
    idx = draw_slots(r_i, n_tokens, 16, 1.2, 0.05)
    adapters = _make_adapters(r_a, r_b, mods, [32] * 16, [64.0] * 16, True, "uniform", 0.01, BF16)
    x, y = _activations(r_x, r_y, mods, n_tokens, BF16, y_zero)
    return Workload("qwen32b_decode", BF16, mods, 16, 32, adapters, idx, x, y)


# ----------------------------------------------------------------------------
# churn workload: a pool of adapters in host memory and a stream of steps

def churn_adapter_ids(rng: np.random.Generator, n_adapters: int = 200, s: float = 0.9,
                      n_prefill: int = 8, prefill_len: int = 128, n_decode: int = 7168,
                      cap: int = 128):
    """Adapter id per token for one churn step, and the number of capped redraws."""
    p = zipf_probs(n_adapters, s)
    pre = rng.choice(n_adapters, size=n_prefill, replace=False, p=p)
    pre = np.sort(pre, kind="stable")
    seen = set(int(a) for a in pre)
    dec = rng.choice(n_adapters, size=n_decode, p=p)
    redraws = 0
    for i in range(n_decode):
        a = int(dec[i])
        while a not in seen and len(seen) >= cap:
            a = int(rng.choice(n_adapters, p=p))
            redraws += 1
        seen.add(a)
        dec[i] = a
    ids = np.concatenate([np.repeat(pre, prefill_len), dec]).astype(np.int32)
    return ids, redraws


# ----------------------------------------------------------------------------
# generic small random case for parity sweeps

def random_case(seed: int, dtype: str, modules: Sequence[Module], n_tokens: int,
                max_loras: int, max_rank: int, ranks: Sequence[int],
                targeted: Optional[Sequence[Sequence[bool]]] = None,
                p_base_only: float = 0.1, zipf_s: float = 1.1,
                empty_slots: Sequence[int] = (), rslora: bool = False,
                alpha_per_rank: float = 2.0, y_zero: bool = False,
                integer: bool = False) -> Workload:
    """A seeded case of any size; ranks[k] is slot k's rank.

    integer=True draws every value from {-2..2} (exact in bf16 and fp32), so
    all sums of a small case stay exact.
    """
    r_i, r_x, r_a, r_b, r_y = _children(seed)
    mods = list(modules)
    idx = draw_slots(r_i, n_tokens, max_loras, zipf_s, p_base_only)
    adapters: List[Optional[Adapter]] = []
    for k in range(max_loras):
        r = int(ranks[k])
        ad = Adapter(r=r, lora_alpha=alpha_per_rank * r, use_rslora=rslora)
        for mi, m in enumerate(mods):
            if targeted is not None and not targeted[k][mi]:
                continue
            if integer:
                ad.At[m.name] = _cast(r_a.integers(-2, 3, (r, m.d_in)).astype(np.float32), dtype)
                ad.B[m.name] = _cast(r_b.integers(-2, 3, (r, m.d_out)).astype(np.float32), dtype)
            else:
                ad.At[m.name] = uniform(r_a, (r, m.d_in), 1.0 / np.sqrt(m.d_in), dtype)
                ad.B[m.name] = normal(r_b, (r, m.d_out), 0.05, dtype)
        adapters.append(None if k in empty_slots else ad)
    if integer:
        x = {m.name: _cast(r_x.integers(-2, 3, (n_tokens, m.d_in)).astype(np.float32), dtype)
             for m in mods}
        y = {m.name: _cast(r_y.integers(-2, 3, (n_tokens, m.d_out)).astype(np.float32), dtype)
             for m in mods}
        if y_zero:
            y = {m.name: _cast(np.zeros((n_tokens, m.d_out), np.float32), dtype) for m in mods}
    else:
        x, y = _activations(r_x, r_y, mods, n_tokens, dtype, y_zero)
    return Workload("random_case", dtype, mods, max_loras, max_rank, adapters, idx, x, y)


def oracle_adapters(wl: Workload, module: str, adapters=None):
    """Per-slot adapter records for one module, in the form the oracle takes."""
    out = []
    for ad in (wl.adapters if adapters is None else adapters):
        if ad is None or module not in ad.At:
            out.append(None)
        else:
            rec = {"r": ad.r, "lora_alpha": ad.lora_alpha, "use_rslora": ad.use_rslora,
                   "At": ad.At[module], "B": ad.B[module]}
            if ad.bias is not None:
                rec["bias"] = ad.bias[module]
            if ad.dora_scale is not None:
                rec["dora_scale"] = ad.dora_scale[module].astype(np.float64)
            out.append(rec)
    return out


def add_output_terms(wl: Workload, seed: int, bias_slots=(), dora_slots=()) -> Workload:
    """Give the listed slots an output bias c ~ N(0, 0.05) and / or a DoRA factor
    g ~ U(0.5, 1.5) per targeted module (seeded; c in the workload's dtype)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 77]))
    for k, ad in enumerate(wl.adapters):
        if ad is None:
            continue
        if k in bias_slots:
            ad.bias = {m: _cast(rng.standard_normal(ad.B[m].shape[1]).astype(np.float32) * 0.05, wl.dtype)
                       for m in ad.At}
        if k in dora_slots:
            ad.dora_scale = {m: rng.uniform(0.5, 1.5, ad.B[m].shape[1]).astype(np.float32) for m in ad.At}
    return wl


# ----------------------------------------------------------------------------
# churn workload drawn on the device (the pool is 1.6 GB; numpy would take minutes)

@dataclass
class DevicePool:
    """Adapter pool in pinned host memory: At[name] is [n][r][d_in], B[name] [n][r][d_out] (bf16).

    Each adapter's weights are one contiguous block, module after module (A^T
    then B), the way an adapter file is read into one buffer; At and B are
    views into the blocks."""
    r: int
    lora_alpha: float
    At: Dict[str, "object"]
    B: Dict[str, "object"]

    def adapter(self, module: str, a: int) -> dict:
        """The oracle's record for adapter a on one module (views of the pinned pool)."""
        import torch
        At = self.At[module][a].view(torch.int16).numpy().view(np.uint16)
        B = self.B[module][a].view(torch.int16).numpy().view(np.uint16)
        return {"r": self.r, "lora_alpha": self.lora_alpha, "use_rslora": False, "At": At, "B": B}


def _dev_gen(seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) % (2 ** 63))
    return g


def churn_pool_device(n_adapters: int = 200, rank: int = 64, modules=None, seed: Optional[int] = None,
                      device="cuda") -> DevicePool:
    """A^T ~ U(+-1/sqrt(d_in)) and B ~ N(0, 0.01), drawn with a seeded torch generator on
    the device, rounded to bf16 (torch), copied to pinned host memory."""
    import torch
    mods = list(modules) if modules is not None else list(CHURN_MODULES)
    base = SEEDS["churn"] if seed is None else seed
    g = _dev_gen(base * 7919 + 11, device)
    At, B = {}, {}
    per = sum(rank * (m.d_in + m.d_out) for m in mods)      # elements per adapter block
    packed = torch.empty((n_adapters, per), dtype=torch.bfloat16, pin_memory=True)
    off = 0
    for m in mods:
        a = packed.as_strided((n_adapters, rank, m.d_in), (per, m.d_in, 1), off)
        off += rank * m.d_in
        b = packed.as_strided((n_adapters, rank, m.d_out), (per, m.d_out, 1), off)
        off += rank * m.d_out
        bound = 1.0 / np.sqrt(m.d_in)
        a.copy_(((torch.rand((n_adapters, rank, m.d_in), generator=g, device=device) * 2 - 1)
                 * bound).to(torch.bfloat16))
        b.copy_((torch.randn((n_adapters, rank, m.d_out), generator=g, device=device) * 0.01)
                .to(torch.bfloat16))
        At[m.name], B[m.name] = a, b
    return DevicePool(rank, 2.0 * rank, At, B)


def churn_step_device(step: int, modules=None, seed: Optional[int] = None, n_adapters: int = 200,
                      n_prefill: int = 8, prefill_len: int = 128, n_decode: int = 7168,
                      cap: int = 128, device="cuda"):
    """One churn step: adapter id per token (numpy), redraw count, and x, y per module
    as device bf16 tensors drawn with a seeded torch generator (N(0, 1))."""
    import torch
    mods = list(modules) if modules is not None else list(CHURN_MODULES)
    base = SEEDS["churn"] if seed is None else seed
    r_i = np.random.default_rng(np.random.SeedSequence([base, step]))
    ids, redraws = churn_adapter_ids(r_i, n_adapters, 0.9, n_prefill, prefill_len, n_decode, cap)
    g = _dev_gen(base * 1000003 + step, device)
    T = int(ids.shape[0])
    x = {m.name: torch.randn((T, m.d_in), generator=g, device=device).to(torch.bfloat16) for m in mods}
    y = {m.name: torch.randn((T, m.d_out), generator=g, device=device).to(torch.bfloat16) for m in mods}
    return ids, redraws, x, y
