"""Synthetic mid-run cache states for the oracle (test infrastructure).

Used by the GPU parity tests and the CPU-baseline leg of ``bench.py``: a
cache that has already absorbed ``n`` tokens without evicting, built directly
instead of stepped there (keys from the seeded generator at positions
0 .. n-1, positive scores, frozen Gumbel values, positions equal to the row
index, as KeyformerState keeps them on the "veloxquant_mlx.quantizers.keyformer
module" page).  It holds none of the method's arithmetic.
"""
from __future__ import annotations

import numpy as np

import synth
from oracle import OracleCache, gumbel


def random_state(w: synth.Workload, layer: int, hh: int, n: int, cap: int, next_pos: int,
                 seed: int = 1) -> OracleCache:
    """A plausible mid-run cache: n rows with keys at positions 0..n-1, positive
    scores, frozen Gumbel values, positions == index."""
    c = OracleCache(w.d, cap)
    if n > 0:
        ks, vs = synth.token_kv(w, layer, hh, np.arange(n), attempt=10_000 + seed)
        rng = np.random.default_rng([seed, layer, hh])
        c.k[:n], c.v[:n] = ks, vs
        c.s[:n] = rng.gamma(0.7, 1.5, n).astype(np.float32)
        c.g[:n] = np.array([gumbel(w.gumbel_seed, hh, 7_000_000 + i) for i in range(n)],
                           dtype=np.float32) if w.kind == "keyformer" else 0.0
        c.p[:n] = np.arange(n)
        c.tid[:n] = np.arange(n)
    c.set_counters(n, next_pos, next_pos)
    return c
