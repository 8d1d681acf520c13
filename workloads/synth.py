"""Seeded synthetic attention-layer inputs with sink / recency / needle structure.

This module only draws random inputs.  It holds none of the method's arithmetic
(no softmax, no scores, no selection): both the CPU oracle and the GPU tests /
bench take their Q, K, V from here and nowhere else.

Why the structure looks like this (CRISP paper, "mass cliff" discussion in §3-§4
and the routing section §3.2): concentrated attention heads put most of their
mass on the first block of keys (architectural sinks) and on the local recency
window, a few task-relevant "signal" blocks carry moderate mass, and the
background carries per-token mass of order 1/n.  Diffuse heads spread mass
almost uniformly.  The shapes follow the layers the paper evaluates
(Llama-3.1-8B: 32 query / 8 KV heads; Qwen2.5-7B: 28 / 4; head dim 128).

Recipe (all per-chunk draws are seeded by (config seed, tensor, head, chunk),
so any row range can be regenerated without generating the rest):

* s_g: a random unit vector per KV group g.
* concentrated query head h in group g:   Q_i = 0.5 z_i + 4 s_g
* diffuse query head:                      Q_i = qd * z_i   (qd = 0.3)
* keys of group g:                         K_j = z'_j
      + c_g s_g            for j < 128                     (sink block)
      + c_g s_g            for j in a needle block          (signal blocks)
      + rho_g Q^(h*)_j     for j in the last 128 positions (recency: key j is
                                                             aligned with the
                                                             query at j of the
                                                             group's first
                                                             concentrated head)
* values: V_j ~ N(0, 1).
* every value is rounded to bfloat16 (round-to-nearest-even) unless the
  configuration is fp32.

Length compensation (a stated reading, on by default): with fixed planted
coefficients the planted logit gap is fixed while the background mass grows
with n, so the anchor share of a concentrated head falls like 1/n and such
heads stop looking concentrated past ~32k tokens.  The paper's premise is that
concentrated heads keep their anchor share at every length, so each planted
coefficient is raised to widen its logit gap by ln(n/4096) nats: c_g gains
ln(n/4096)*sqrt(d)/4 (the gap per unit of c is 4/sqrt(d) because Q ~ 4 s_g)
and rho_g gains ln(n/4096)*sqrt(d)/16 (the gap per unit of rho is |Q|^2/sqrt(d)
~ 16/sqrt(d)).  At n = 4096 nothing changes.  ``compensate=False`` gives the
literal constants.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

D = 128
BLOCK = 128
CHUNK = 4096          # rows per independently seeded draw

# tensor ids in the seed tree
_T_PARAMS, _T_Q, _T_K, _T_V = 0, 1, 2, 3


@dataclass(frozen=True)
class LayerConfig:
    name: str
    n: int
    hq: int
    hkv: int
    dtype: str                 # "bf16" or "fp32"
    seed: int
    tau: float = 0.3
    alpha: float = 1.0
    gamma: float = 0.95
    conc_frac: float = 0.6     # fraction of query heads that are concentrated
    sink: tuple = (4.0, 8.0)   # U[lo, hi] sink / needle coefficient per KV group
    needles: tuple = (2, 8)    # U{lo..hi} needle blocks per KV group
    recency: float = 3.0
    q_diffuse: float = 0.3
    tiny: bool = False         # the two-head fp32 case: head 0 concentrated, head 1 diffuse

    @property
    def nb(self) -> int:
        return self.n // BLOCK


TINY_FP32_4K = LayerConfig("tiny-fp32-4k", 4096, 2, 2, "fp32", seed=0, tiny=True,
                           sink=(6.0, 6.0), needles=(3, 3))
LLAMA_32K = LayerConfig("llama3.1-8b-32k", 32768, 32, 8, "bf16", seed=1)
LLAMA_128K = LayerConfig("llama3.1-8b-128k", 131072, 32, 8, "bf16", seed=2)
QWEN_128K = LayerConfig("qwen2.5-7b-128k", 131072, 28, 4, "bf16", seed=3,
                        conc_frac=0.45, sink=(3.0, 6.0), recency=1.5)
LLAMA_512K = LayerConfig("llama3.1-8b-512k", 524288, 32, 8, "bf16", seed=4,
                         needles=(2, 16))

# the named layers, by name
WORKLOADS = {c.name: c for c in (TINY_FP32_4K, LLAMA_32K, LLAMA_128K, QWEN_128K, LLAMA_512K)}


def custom_config(name, n, hq, hkv, dtype="bf16", seed=0, **kw) -> LayerConfig:
    """A layer of arbitrary shape with the same generator (used for edge cases)."""
    return LayerConfig(name, n, hq, hkv, dtype, seed, **kw)


@dataclass
class LayerSpec:
    cfg: LayerConfig
    compensate: bool
    concentrated: np.ndarray          # [hq] bool
    s: np.ndarray                     # [hkv, d] float32 unit vectors
    c: np.ndarray                     # [hkv] sink / needle coefficient (after compensation)
    rho: np.ndarray                   # [hkv] recency coefficient (after compensation)
    needle_blocks: list = field(default_factory=list)   # per group: sorted block ids
    lead: np.ndarray = None           # [hkv] first concentrated query head of the group, -1 if none
    kv_scale: np.ndarray = None       # [hkv] scale of K and V noise (0.3 for the tiny diffuse head)
    q_scale: np.ndarray = None        # [hq] scale of the query noise


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def make_spec(cfg: LayerConfig, compensate: bool = True) -> LayerSpec:
    g_of = lambda h: h // (cfg.hq // cfg.hkv)
    nb = cfg.nb
    lam = math.log(cfg.n / 4096.0) if (compensate and cfg.n > 4096) else 0.0
    dc = lam * math.sqrt(D) / 4.0
    drho = lam * math.sqrt(D) / 16.0
    rng = _rng(cfg.seed, _T_PARAMS)
    s = rng.standard_normal((cfg.hkv, D))
    s /= np.linalg.norm(s, axis=1, keepdims=True)
    s = s.astype(np.float32)
    if cfg.tiny:
        conc = np.zeros(cfg.hq, bool)
        conc[0] = True
    else:
        k = int(round(cfg.conc_frac * cfg.hq))
        perm = rng.permutation(cfg.hq)
        conc = np.zeros(cfg.hq, bool)
        conc[perm[:k]] = True
    c = rng.uniform(cfg.sink[0], cfg.sink[1], size=cfg.hkv) + dc
    rho = np.full(cfg.hkv, cfg.recency) + drho
    needles = []
    for g in range(cfg.hkv):
        m = int(rng.integers(cfg.needles[0], cfg.needles[1] + 1))
        m = min(m, max(nb - 2, 0))
        blocks = np.sort(rng.choice(np.arange(1, nb - 1), size=m, replace=False)) if m > 0 else np.zeros(0, int)
        needles.append([int(x) for x in blocks])
    lead = np.full(cfg.hkv, -1, dtype=np.int64)
    for h in range(cfg.hq):
        if conc[h] and lead[g_of(h)] < 0:
            lead[g_of(h)] = h
    kv_scale = np.ones(cfg.hkv, np.float32)
    q_scale = np.where(conc, 0.5, cfg.q_diffuse).astype(np.float32)
    if cfg.tiny:
        # head 1 of the tiny case is diffuse in Q, K and V alike, with no planted structure
        kv_scale[1] = cfg.q_diffuse
    return LayerSpec(cfg, compensate, conc, s, c.astype(np.float32), rho.astype(np.float32),
                     needles, lead, kv_scale, q_scale)


# ---------------------------------------------------------------- row draws (fp32, unrounded)

def _noise(spec: LayerSpec, tensor: int, head: int, r0: int, r1: int) -> np.ndarray:
    """Standard normal rows [r0, r1) of (tensor, head), drawn chunk by chunk."""
    out = np.empty((r1 - r0, D), np.float32)
    c0, c1 = r0 // CHUNK, (r1 - 1) // CHUNK
    for ch in range(c0, c1 + 1):
        lo, hi = ch * CHUNK, min((ch + 1) * CHUNK, spec.cfg.n)
        z = _rng(spec.cfg.seed, tensor, head, ch).standard_normal((hi - lo, D), dtype=np.float32)
        a, b = max(lo, r0), min(hi, r1)
        out[a - r0:b - r0] = z[a - lo:b - lo]
    return out


def q_rows(spec: LayerSpec, h: int, r0: int, r1: int) -> np.ndarray:
    g = h // (spec.cfg.hq // spec.cfg.hkv)
    z = _noise(spec, _T_Q, h, r0, r1)
    if spec.concentrated[h]:
        return (np.float32(spec.q_scale[h]) * z + np.float32(4.0) * spec.s[g][None, :]).astype(np.float32)
    return (np.float32(spec.q_scale[h]) * z).astype(np.float32)


def k_rows(spec: LayerSpec, g: int, r0: int, r1: int) -> np.ndarray:
    cfg = spec.cfg
    k = np.float32(spec.kv_scale[g]) * _noise(spec, _T_K, g, r0, r1)
    if cfg.tiny and g == 1:
        return k
    pos = np.arange(r0, r1)
    planted = (pos < BLOCK)
    for nb_id in spec.needle_blocks[g]:
        planted |= (pos // BLOCK) == nb_id
    if planted.any():
        k[planted] += np.float32(spec.c[g]) * spec.s[g][None, :]
    h_lead = int(spec.lead[g])
    lo = max(r0, cfg.n - BLOCK)
    if h_lead >= 0 and lo < r1:
        qr = q_rows(spec, h_lead, lo, r1)
        k[lo - r0:] += np.float32(spec.rho[g]) * qr
    return k.astype(np.float32)


def v_rows(spec: LayerSpec, g: int, r0: int, r1: int) -> np.ndarray:
    return (np.float32(spec.kv_scale[g]) * _noise(spec, _T_V, g, r0, r1)).astype(np.float32)


# ---------------------------------------------------------------- rounding

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _finish(spec: LayerSpec, x: np.ndarray) -> np.ndarray:
    """Storage form: uint16 bf16 bits for bf16 layers, float32 for fp32 layers."""
    return to_bf16_bits(x) if spec.cfg.dtype == "bf16" else x


def as_f64(spec: LayerSpec, x: np.ndarray) -> np.ndarray:
    """Exact float64 values of a storage-form array."""
    if spec.cfg.dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def rows(spec: LayerSpec, which: str, head: int, r0: int, r1: int) -> np.ndarray:
    """Storage-form rows [r0, r1) of Q (query head) / K / V (KV head)."""
    f = {"q": q_rows, "k": k_rows, "v": v_rows}[which]
    return _finish(spec, f(spec, head, r0, r1))


def generate(spec: LayerSpec, threads: int | None = None, heads_q=None):
    """Whole layer in storage form: Q [hq, n, d], K [hkv, n, d], V [hkv, n, d].

    Work is split by (tensor, head, chunk) over a thread pool; numpy releases the
    GIL while drawing and rounding, so this scales with host cores.
    """
    cfg = spec.cfg
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    heads_q = list(range(cfg.hq)) if heads_q is None else list(heads_q)
    Q = np.empty((cfg.hq, cfg.n, D), dt)
    K = np.empty((cfg.hkv, cfg.n, D), dt)
    V = np.empty((cfg.hkv, cfg.n, D), dt)
    nch = (cfg.n + CHUNK - 1) // CHUNK
    tasks = []
    for h in heads_q:
        for ch in range(nch):
            tasks.append((Q, "q", h, ch))
    for g in range(cfg.hkv):
        for ch in range(nch):
            tasks.append((K, "k", g, ch))
            tasks.append((V, "v", g, ch))

    def run(t):
        arr, which, head, ch = t
        r0, r1 = ch * CHUNK, min((ch + 1) * CHUNK, cfg.n)
        arr[head, r0:r1] = rows(spec, which, head, r0, r1)

    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, tasks))
    return Q, K, V


def sample_blocks(nb: int, count: int, seed: int) -> list[int]:
    """Seeded sample of query blocks: first, last and `count` others."""
    rng = _rng(seed, 99)
    others = rng.choice(np.arange(1, max(nb - 1, 1)), size=min(count, max(nb - 2, 0)), replace=False) if nb > 2 else []
    return sorted(set([0, nb - 1] + [int(x) for x in others]))
