"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

Both the HIP path and the oracle read the tensors made here: the tests copy
the very device tensors the kernels consumed back to the host and upcast them
exactly to float64 for the oracle.  The shapes and distributions follow the
workloads the pages' examples suggest (single-head FP64 check; bf16 heads of
width 128 drawn N(0,1)/sqrt(128); a scalar per-token gate sigmoid(g) with
g ~ N(mu, 1); a batch of decode states; a long sequence whose inputs are
scaled x4 on 10% of positions to widen the range of denominators).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    T: int
    d: int
    dv: int
    io: str            # "bf16" | "f32" | "f64"
    chunk: int
    eps: float
    gated: bool
    seed: int
    gate_mean: float = 3.0        # g ~ N(gate_mean, 1), alpha = sigmoid(g)
    spike_frac: float = 0.0       # fraction of (b, t) positions scaled by spike_scale
    spike_scale: float = 4.0
    scale: float = 1.0 / math.sqrt(128.0)
    note: str = ""


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    requests: int
    slots: int
    heads: int
    d: int
    dv: int
    seed_writes: int
    steps: int
    eps: float
    seed: int
    scale: float = 1.0 / math.sqrt(128.0)
    note: str = ""

    @property
    def n_states(self) -> int:
        return self.requests * self.slots * self.heads


SINGLE_HEAD_F64 = PrefillConfig(
    "single_head_f64", B=1, H=1, T=64, d=16, dv=16, io="f64", chunk=16, eps=1e-6, gated=False, seed=1,
    scale=1.0, note="iid N(0,1) float64 from numpy PCG64; chunk is not fixed by the workload, 16 spans 4 chunks")
PREFILL_UNGATED = PrefillConfig(
    "prefill_ungated_b4_h16_t4096", B=4, H=16, T=4096, d=128, dv=128, io="bf16", chunk=64, eps=1e-6,
    gated=False, seed=2)
# The fp32-input path on the ungated prefill shape (the fp32 bar of 1e-4 applies; not one of the
# five workloads, measured beside them)
PREFILL_UNGATED_F32 = PrefillConfig(
    "prefill_ungated_f32_b4_h16_t4096", B=4, H=16, T=4096, d=128, dv=128, io="f32", chunk=64, eps=1e-6,
    gated=False, seed=9)
PREFILL_GATED = PrefillConfig(
    "prefill_gated_b2_h16_t16384", B=2, H=16, T=16384, d=128, dv=128, io="bf16", chunk=64, eps=1e-6,
    gated=True, gate_mean=3.0, seed=3)
DECODE = DecodeConfig(
    "decode_65536_states", requests=128, slots=32, heads=16, d=128, dv=128, seed_writes=256, steps=1024,
    eps=1e-6, seed=4)
PREFILL_LONG = PrefillConfig(
    "prefill_long_gated_b1_h32_t131072", B=1, H=32, T=131072, d=128, dv=128, io="bf16", chunk=128,
    eps=1e-6, gated=True, gate_mean=4.0, spike_frac=0.1, spike_scale=4.0, seed=5)

# delta-rule decode on the decode workload's memory shape: 65,536 memories of 128 x 128
DELTA_DECODE = DecodeConfig(
    "delta_decode_65536_states", requests=128, slots=32, heads=16, d=128, dv=128, seed_writes=0, steps=256,
    eps=0.0, seed=6, note="unit-norm keys, beta = sigmoid(N(0,1)), memories drawn N(0,1)*0.05")



@dataclass(frozen=True)
class KvStateConfig:
    """An explicit K/V history against the fixed recurrent state, one layer: per step every
    head gets a new (q, k, v); the history path appends it to the K/V caches and attends
    over all L rows, the state path writes it into S and z and reads them."""
    name: str
    batch: int
    heads: int
    d: int
    lengths: tuple
    warmup: int
    repeats: int
    eps: float
    seed: int
    note: str = ""

    @property
    def n_heads(self) -> int:
        return self.batch * self.heads


# the datawhalechina chapter's Step 5 setting: 8 heads x 64, bf16, L in {512, 2048, 8192},
# warmup 10, repeats 100; and the same at 128 sequences, where the longer histories exceed
# the last-level cache and the history step is bound by HBM
KV_STATE = KvStateConfig(
    "kv_history_vs_fixed_state_h8_d64", batch=1, heads=8, d=64, lengths=(512, 2048, 8192), warmup=10, repeats=100,
    eps=1e-6, seed=7, note="N(0,1)/sqrt(64) bf16 q, k, v; the history holds L-1 earlier rows, the step adds row L-1")
KV_STATE_BATCHED = KvStateConfig(
    "kv_history_vs_fixed_state_b128_h8_d64", batch=128, heads=8, d=64, lengths=(512, 2048, 8192), warmup=10,
    repeats=100, eps=1e-6, seed=8, note="as above for 128 sequences (1,024 head-states)")

CONFIGS = {c.name: c for c in (SINGLE_HEAD_F64, PREFILL_UNGATED, PREFILL_GATED, DECODE, PREFILL_LONG)}


def _torch():
    import torch
    return torch


def torch_dtype(io: str):
    torch = _torch()
    return {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}[io]


def state_dtype(io: str):
    torch = _torch()
    return torch.float64 if io == "f64" else torch.float32


def generator(seed: int, device):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, scale: float, io: str, gen, device):
    """N(0,1) drawn in float32 (float64 for f64 io), times scale, rounded to the io dtype (RNE)."""
    torch = _torch()
    base = torch.float64 if io == "f64" else torch.float32
    x = torch.randn(shape, generator=gen, device=device, dtype=base)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(torch_dtype(io))


def gates(shape, mean: float, gen, device):
    """alpha = sigmoid(g), g ~ N(mean, 1), float32."""
    torch = _torch()
    g = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    g.add_(mean)
    return torch.sigmoid(g)


def prefill_inputs(cfg: PrefillConfig, device, B=None, H=None, T=None, seed=None):
    """Q, K, V ([B,H,T,d]/[B,H,T,dv], io dtype) and alpha ([B,H,T] state dtype, or None).

    B, H, T and seed may be overridden (smaller variants of the same recipe).
    Spikes: a Bernoulli(spike_frac) mask over (b, t) positions scales Q, K and V of
    every head at those positions by spike_scale before rounding.
    """
    torch = _torch()
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    T = cfg.T if T is None else T
    seed = cfg.seed if seed is None else seed
    if cfg.io == "f64" and cfg.name == SINGLE_HEAD_F64.name:
        rng = np.random.Generator(np.random.PCG64(seed))
        q = rng.standard_normal((B, H, T, cfg.d))
        k = rng.standard_normal((B, H, T, cfg.d))
        v = rng.standard_normal((B, H, T, cfg.dv))
        to = lambda a: torch.from_numpy(a).to(device)
        return to(q), to(k), to(v), None
    gen = generator(seed, device)
    base = torch.float64 if cfg.io == "f64" else torch.float32
    out = []
    for width in (cfg.d, cfg.d, cfg.dv):
        x = torch.randn((B, H, T, width), generator=gen, device=device, dtype=base)
        x.mul_(cfg.scale)
        out.append(x)
    if cfg.spike_frac > 0.0:
        mask = torch.rand((B, 1, T, 1), generator=gen, device=device) < cfg.spike_frac
        factor = torch.where(mask, torch.tensor(cfg.spike_scale, device=device, dtype=base),
                             torch.tensor(1.0, device=device, dtype=base))
        for x in out:
            x.mul_(factor)
    q, k, v = (x.to(torch_dtype(cfg.io)) for x in out)
    del out
    alpha = None
    if cfg.gated:
        alpha = gates((B, H, T), cfg.gate_mean, gen, device).to(state_dtype(cfg.io))
    return q, k, v, alpha


def decode_seed_inputs(cfg: DecodeConfig, device, n_states=None):
    """The (k, v) writes that seed each decode state: [n_states, 1, seed_writes, d|dv] bf16.

    Fed to la_prefill_chunked from a zero state (with a q whose outputs are discarded).
    """
    n = cfg.n_states if n_states is None else n_states
    gen = generator(cfg.seed, device)
    k = normal((n, 1, cfg.seed_writes, cfg.d), cfg.scale, "bf16", gen, device)
    v = normal((n, 1, cfg.seed_writes, cfg.dv), cfg.scale, "bf16", gen, device)
    return k, v


def decode_step_inputs(cfg: DecodeConfig, step: int, device, n_states=None):
    """q, k, v for one decode step: [n_states, d|dv] bf16, seeded by (seed, step)."""
    n = cfg.n_states if n_states is None else n_states
    gen = generator(cfg.seed * 1_000_003 + 7919 * (step + 1), device)
    q = normal((n, cfg.d), cfg.scale, "bf16", gen, device)
    k = normal((n, cfg.d), cfg.scale, "bf16", gen, device)
    v = normal((n, cfg.dv), cfg.scale, "bf16", gen, device)
    return q, k, v


def delta_seed_state(cfg: DecodeConfig, device, n_states=None):
    """Initial delta-rule memories: [n_states, d, dv] float32, N(0,1) * 0.05."""
    torch = _torch()
    n = cfg.n_states if n_states is None else n_states
    gen = generator(cfg.seed, device)
    return torch.randn((n, cfg.d, cfg.dv), generator=gen, device=device, dtype=torch.float32).mul_(0.05)


def delta_step_inputs(cfg: DecodeConfig, step: int, device, n_states=None):
    """q, k, v (bf16) and beta (float32) for one delta-rule step, seeded by (seed, step).

    Keys are normalised to unit length in float32 before rounding (the page notes that
    normalised keys keep beta's meaning stable); beta = sigmoid(N(0,1)) lies in (0, 1),
    so every step contracts the error along its key.
    """
    torch = _torch()
    n = cfg.n_states if n_states is None else n_states
    gen = generator(cfg.seed * 1_000_003 + 7919 * (step + 1), device)
    q = normal((n, cfg.d), cfg.scale, "bf16", gen, device)
    k = torch.randn((n, cfg.d), generator=gen, device=device, dtype=torch.float32)
    k = (k / k.norm(dim=1, keepdim=True)).to(torch.bfloat16)
    v = normal((n, cfg.dv), cfg.scale, "bf16", gen, device)
    beta = torch.sigmoid(torch.randn((n,), generator=gen, device=device, dtype=torch.float32))
    return q, k, v, beta


def sampled_states(cfg: DecodeConfig, count: int, seed: int = 12345):
    """Sorted distinct state indices including 0 and N-1 and every (slot, head) pair."""
    n = cfg.n_states
    rng = np.random.Generator(np.random.PCG64(seed))
    per_req = cfg.slots * cfg.heads
    must = {0, n - 1}
    # one state of every (slot, head) pair, spread over requests
    for j in range(per_req):
        must.add(int(rng.integers(0, cfg.requests)) * per_req + j)
    rest = rng.choice(n, size=count, replace=False)
    picks = list(sorted(must))
    for x in rest:
        if len(picks) >= count:
            break
        if int(x) not in must:
            picks.append(int(x))
    return np.array(sorted(set(picks))[:count], dtype=np.int64)


def kv_state_history(cfg: KvStateConfig, L: int, device):
    """The L-1 earlier rows of every head: K, V [n_heads, L-1, d] (bf16), seeded per L."""
    g = generator(cfg.seed * 100003 + L, device)
    sc = 1.0 / math.sqrt(cfg.d)
    return (normal((cfg.n_heads, L - 1, cfg.d), sc, "bf16", g, device),
            normal((cfg.n_heads, L - 1, cfg.d), sc, "bf16", g, device))


def kv_state_steps(cfg: KvStateConfig, L: int, n_steps: int, device):
    """Per step the new q, k, v of every head ([n_heads, d] bf16), seeded per (L, step)."""
    g = generator(cfg.seed * 100003 + L + 7919, device)
    sc = 1.0 / math.sqrt(cfg.d)
    return [tuple(normal((cfg.n_heads, cfg.d), sc, "bf16", g, device) for _ in range(3)) for _ in range(n_steps)]
