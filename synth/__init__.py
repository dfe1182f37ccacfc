"""Seeded synthetic workloads for the KV-cache eviction step.

This module only makes inputs: the shapes and parameters of the five
workloads, and the incoming fp16 key/value rows.  It holds none of the
eviction method's arithmetic and imports neither the GPU library nor the CPU
oracle, so both of them can be fed from it.

Two generators with the same distribution:

* ``token_kv`` -- exact and counter-based (numpy, float64).  Any
  (layer, cache row, token, attempt) can be produced on its own, so a cache
  whose trajectory is checked against the oracle gets identical inputs on
  both sides, and a single token can be redrawn (``attempt``) without
  touching the rest of the stream.
* ``bulk_kv_torch`` -- fast, on the device, from torch's seeded generator,
  for the caches nobody compares (benchmark fill and the unchecked rows of a
  parity launch).  Not bit-identical to ``token_kv``.

Recipe (both generators): raw key and value elements ~ N(0, 1); the key is
rotated at its absolute position t with the half-split rotary embedding
(element j paired with j + D/2, frequency base^(-2j/D), base 10000) in the
model's usual way, then, for the late-riser workload, a fixed unit direction
u is added: with scale 0.2 on a Bernoulli(0.05) subset R of positions, and
with scale 3 * t / (T - 1) on every other position (T = prompt + decode
tokens).  Everything is rounded once to fp16 (nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

DATA_SEED = 0

# purposes of the counter-based streams
_P_KEY, _P_VAL, _P_DIR, _P_RISER = 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload: B*H caches per layer, L layers."""
    name: str
    batch: int
    layers: int
    kv_heads: int
    d: int
    prompt: int
    decode: int
    budget: int                      # uniform budget, or the average for a pyramid
    n_sink: int
    kind: str                        # "keyformer", "pyramid" or "tova"
    tau_init: float = 0.0
    tau_end: float = 0.0
    anneal_steps: int = 0
    beta: float = 1.0                # pyramid steepness
    late_riser: bool = False
    rope_base: float = 10000.0
    gumbel_seed: int = 0
    recent: int = 0                  # trailing protected window (0 = off)
    extra: dict = field(default_factory=dict)

    @property
    def bh(self) -> int:
        return self.batch * self.kv_heads

    @property
    def tokens(self) -> int:
        return self.prompt + self.decode

    def budgets(self, pyramid_fn) -> list[int]:
        """Per-layer budgets; ``pyramid_fn(L, avg, n_sink, beta)`` supplies the taper."""
        if self.kind == "pyramid":
            return list(pyramid_fn(self.layers, self.budget, self.n_sink, self.beta))
        return [self.budget] * self.layers


# The five workloads.  Index 0 is the small case; 1-2 Llama-3.2-3B shaped;
# 3 an 8B-shaped batched decode with the late-riser geometry; 4 the
# long-context stress case.
WORKLOADS: list[Workload] = [
    Workload("tiny-h2o", 1, 1, 4, 64, 128, 0, 32, 4, "keyformer", 0.0, 0.0, 0),
    Workload("llama3.2-3b-keyformer", 1, 28, 8, 128, 2048, 1024, 512, 4, "keyformer",
             1.0, 2.0, 1024),
    Workload("llama3.2-3b-pyramidkv", 1, 28, 8, 128, 2048, 1024, 512, 4, "pyramid",
             beta=2.0),
    Workload("8b-batched-late-riser", 32, 32, 8, 128, 4096, 512, 1024, 4, "keyformer",
             1.0, 2.0, 512, late_riser=True),
    Workload("long-context-pyramidkv", 64, 32, 8, 128, 16384, 1024, 4096, 4, "pyramid",
             beta=1.5),
]

# the tiny case is also run with an annealed temperature
TINY_ANNEALED = Workload("tiny-keyformer", 1, 1, 4, 64, 128, 0, 32, 4, "keyformer",
                         1.0, 2.0, 64)


def workload(i: int) -> Workload:
    return WORKLOADS[i]


# --------------------------------------------------------------------------
# counter-based generator (MurmurHash3's 64-bit finaliser as the mixer)
# --------------------------------------------------------------------------

_U64 = np.uint64


def _fmix64(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> _U64(33))
    z = z * _U64(0xFF51AFD7ED558CCD)
    z = z ^ (z >> _U64(33))
    z = z * _U64(0xC4CEB9FE1A85EC53)
    z = z ^ (z >> _U64(33))
    return z


def _hash(*fields) -> np.ndarray:
    arrs = np.broadcast_arrays(*[np.asarray(f, dtype=np.int64) for f in fields])
    h = np.full(arrs[0].shape, 0x243F6A8885A308D3, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for a in arrs:
            h = _fmix64(h ^ a.astype(np.uint64))
            h = h + _U64(0x9E3779B97F4A7C15)
    return h


def _uniform(*fields) -> np.ndarray:
    h = _hash(*fields)
    return ((h >> _U64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def _normal(*fields) -> np.ndarray:
    """Box-Muller from two counter-based uniforms (fields broadcast)."""
    u1 = _uniform(*fields, 0)
    u2 = _uniform(*fields, 1)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def _rotate_at(x: np.ndarray, t: np.ndarray, base: float) -> np.ndarray:
    """Rotary embedding of raw keys x [T, D] at absolute positions t [T] (float64)."""
    D = x.shape[-1]
    half = D // 2
    j = np.arange(half, dtype=np.float64)
    freq = base ** (-(2.0 * j) / D)
    ang = t.astype(np.float64)[:, None] * freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[:, :half], x[:, half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


def late_riser_direction(d: int, seed: int = DATA_SEED) -> np.ndarray:
    u = _normal(seed, _P_DIR, 0, 0, 0, np.arange(d), 0)
    return u / np.linalg.norm(u)


def late_riser_scale(w: Workload, t: np.ndarray, seed: int = DATA_SEED) -> np.ndarray:
    """Scale of u added to the key at absolute position t (late-riser geometry)."""
    t = np.asarray(t, dtype=np.int64)
    in_r = _uniform(seed, _P_RISER, 0, 0, t, 0, 0) < 0.05
    ramp = 3.0 * t.astype(np.float64) / float(max(w.tokens - 1, 1))
    return np.where(in_r, 0.2, ramp)


def token_kv(w: Workload, layer: int, hh: int, t, attempt=0,
             seed: int = DATA_SEED) -> tuple[np.ndarray, np.ndarray]:
    """Incoming (key, value) rows of one cache at absolute positions ``t``.

    Returns two uint16 arrays [len(t), D] holding fp16 bit patterns.
    ``attempt`` (scalar or per-token array) selects an independent redraw.
    """
    t = np.atleast_1d(np.asarray(t, dtype=np.int64))
    att = np.broadcast_to(np.asarray(attempt, dtype=np.int64), t.shape)
    dd = np.arange(w.d, dtype=np.int64)[None, :]
    tt, aa = t[:, None], att[:, None]
    kraw = _normal(seed, _P_KEY, layer, hh, tt, dd, aa)
    vraw = _normal(seed, _P_VAL, layer, hh, tt, dd, aa)
    key = _rotate_at(kraw, t, w.rope_base)
    if w.late_riser:
        key = key + late_riser_scale(w, t, seed)[:, None] * late_riser_direction(w.d, seed)[None, :]
    kb = key.astype(np.float16).view(np.uint16)
    vb = vraw.astype(np.float16).view(np.uint16)
    return kb, vb


# --------------------------------------------------------------------------
# bulk device generator (torch)
# --------------------------------------------------------------------------

def bulk_kv_torch(w: Workload, t0: int, count: int, bh: int, gen, device,
                  out_k=None, out_v=None):
    """Incoming rows for ``count`` tokens starting at absolute position ``t0``.

    Returns fp16 tensors [count, bh, D] on ``device`` (or fills out_k/out_v).
    Same recipe as ``token_kv`` (rotation done in float32 here), drawn from
    the seeded torch generator ``gen``.
    """
    import torch
    D = w.d
    half = D // 2
    kraw = torch.randn((count, bh, D), generator=gen, device=device, dtype=torch.float32)
    vraw = torch.randn((count, bh, D), generator=gen, device=device, dtype=torch.float32)
    t = torch.arange(t0, t0 + count, device=device, dtype=torch.float64)
    j = torch.arange(half, device=device, dtype=torch.float64)
    freq = w.rope_base ** (-(2.0 * j) / D)
    ang = t[:, None] * freq[None, :]
    c = torch.cos(ang).to(torch.float32)[:, None, :]
    s = torch.sin(ang).to(torch.float32)[:, None, :]
    x1, x2 = kraw[..., :half], kraw[..., half:]
    key = torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)
    if w.late_riser:
        scale = torch.from_numpy(late_riser_scale(w, np.arange(t0, t0 + count))).to(
            device=device, dtype=torch.float32)
        u = torch.from_numpy(late_riser_direction(D)).to(device=device, dtype=torch.float32)
        key = key + scale[:, None, None] * u[None, None, :]
    if out_k is None:
        return key.to(torch.float16), vraw.to(torch.float16)
    out_k.copy_(key)
    out_v.copy_(vraw)
    return out_k, out_v


def bulk_state_torch(k, v, scores, gumbel, positions, n: int, w: Workload, gen) -> None:
    """Fill rows [0, n) of every cache with a plausible mid-run state.

    k, v: fp16 [bh, cap, d]; scores, gumbel: fp32 [bh, cap] (gumbel may be None);
    positions: int32 [bh, cap].  Keys and values follow the recipe above at
    positions 0..n-1; scores are positive (uniform in [1e-3, 3)); Gumbel values
    are standard Gumbel draws (minus the log of a unit exponential draw);
    positions equal the row index.
    """
    import torch
    if n == 0:
        return
    dev = k.device
    bh = k.shape[0]
    kk, vv = bulk_kv_torch(w, 0, n, bh, gen, dev)          # [n, bh, d]
    k[:, :n] = kk.transpose(0, 1)
    v[:, :n] = vv.transpose(0, 1)
    scores[:, :n] = torch.rand((bh, n), generator=gen, device=dev) * 3.0 + 1e-3
    if gumbel is not None:
        e = torch.empty((bh, n), device=dev, dtype=torch.float32).exponential_(generator=gen)
        gumbel[:, :n] = -torch.log(e)
    positions[:, :n] = torch.arange(n, device=dev, dtype=torch.int32)[None, :]
