"""Margin-guarded input streams (test infrastructure).

Where floating point decides an index (the eviction argmin), the GPU path and
the oracle are compared only on inputs whose decisions are not near-ties.
``guarded_trajectory`` runs one cache through the oracle token by token; when
an eviction's two smallest keys are closer than ``min_margin_rel`` times the
magnitude of the terms that form them (|score| + |tau * gumbel|), the step is
rolled back and that token's key/value are redrawn with the next ``attempt``
of the counter-based generator.  The accepted stream and the oracle's result
are returned together, so the same stream can be replayed on the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import synth
from oracle import OracleCache, Params

MIN_MARGIN_REL = 1e-4
MAX_ATTEMPTS = 16


@dataclass
class Trajectory:
    ks: np.ndarray          # [T, D] uint16 accepted keys
    vs: np.ndarray          # [T, D] uint16 accepted values
    evicted: np.ndarray     # [T] evicted index per token (-1 = none)
    attempts: np.ndarray    # [T] attempt number used per token
    cache: OracleCache      # final oracle state
    params: Params
    min_margin: float       # smallest accepted eviction gap


def params_for(w: synth.Workload, budget: int, hh: int) -> Params:
    kf = w.kind == "keyformer"
    return Params(budget=budget, n_sink=w.n_sink, use_gumbel=kf,
                  tau_init=w.tau_init if kf else 0.0, tau_end=w.tau_end if kf else 0.0,
                  anneal_steps=w.anneal_steps if kf else 0, rope_base=w.rope_base,
                  seed=w.gumbel_seed, hh=hh, recent=w.recent,
                  current_score=w.kind == "tova")


def guarded_trajectory(w: synth.Workload, layer: int, hh: int, budget: int, T: int,
                       cap: int | None = None, min_margin_rel: float = MIN_MARGIN_REL,
                       params: Params | None = None, t0: int = 0,
                       cache: OracleCache | None = None,
                       max_attempts: int = MAX_ATTEMPTS) -> Trajectory:
    """Tokens t0 .. t0+T-1 of cache (layer, hh) through the oracle, guarded."""
    prm = params if params is not None else params_for(w, budget, hh)
    if cache is None:
        cache = OracleCache(w.d, cap if cap is not None else budget + 1)
    ts = np.arange(t0, t0 + T)
    ks, vs = synth.token_kv(w, layer, hh, ts)
    ev = np.full(T, -1, dtype=np.int32)
    att = np.zeros(T, dtype=np.int32)
    min_gap = np.inf
    for i in range(T):
        for a in range(max_attempts):
            if a > 0:
                k1, v1 = synth.token_kv(w, layer, hh, [ts[i]], a)
                ks[i], vs[i] = k1[0], v1[0]
            rc, e, m = cache.step(ks[i], vs[i], prm, min_margin_rel)
            if rc == 0:
                break
        else:
            raise RuntimeError(f"no draw with an eviction margin above the guard after "
                               f"{max_attempts} attempts (layer {layer}, hh {hh}, t {ts[i]})")
        ev[i], att[i] = e, a
        if e >= 0:
            min_gap = min(min_gap, m)
    return Trajectory(ks, vs, ev, att, cache, prm, float(min_gap))
