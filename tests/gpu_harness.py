"""Helpers shared by the GPU parity tests and the smoke entry point.

A parity case steps a whole layer launch (every cache of the B*H set) on the
GPU through the C ABI, while a few sampled caches also run through the CPU
oracle on identical inputs.  The sampled caches get margin-guarded input
streams (no eviction decided by a near-tie); the other caches get bulk random
inputs of the same distribution.
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import synth
from oracle import OracleCache
from oracle.guard import guarded_trajectory, params_for
from oracle.states import random_state  # noqa: F401  (re-exported for the tests)

# acceptance (per cache): kept rows and evicted indices bit-exact, values
# bit-exact, keys within 1 fp16 ULP, scores within 1e-5 relative, Gumbel
# values within 1 fp32 ULP
SCORE_RTOL = 1e-5
KEY_ULP = 1
GUMBEL_ULP = 1


@dataclass
class Sample:
    hh: int
    budget: int
    init: dict | None            # oracle snapshot of the initial state (None = empty)
    ks: np.ndarray               # [T, D] guarded inputs
    vs: np.ndarray
    evicted: np.ndarray          # [T] oracle eviction log
    final: dict                  # oracle snapshot after T tokens
    attempts: int


def _sample_job(args) -> Sample:
    w, layer, hh, budget, T, cap, init_n, next_pos = args
    if init_n is None:
        tr = guarded_trajectory(w, layer, hh, budget, T, cap=cap)
        init = None
    else:
        c = random_state(w, layer, hh, init_n, cap, next_pos)
        init = c.snapshot()
        tr = guarded_trajectory(w, layer, hh, budget, T, cap=cap, t0=next_pos, cache=c)
    return Sample(hh, budget, init, tr.ks, tr.vs, tr.evicted, tr.cache.snapshot(),
                  int(tr.attempts.sum()))


def oracle_samples(w: synth.Workload, layer: int, hhs, budget: int, T: int, cap: int,
                   init_n: int | None = None, next_pos: int = 0,
                   workers: int | None = None) -> list[Sample]:
    jobs = [(w, layer, hh, budget, T, cap, init_n, next_pos) for hh in hhs]
    workers = workers or min(len(jobs), max(1, min(16, (os.cpu_count() or 2) - 1)))
    if workers <= 1 or len(jobs) == 1:
        return [_sample_job(j) for j in jobs]
    with ProcessPoolExecutor(workers) as ex:
        return list(ex.map(_sample_job, jobs))


def _sample_job_next(args) -> Sample:
    """_sample_job for cache hh, or else for the first of the next `tries` - 1
    caches whose whole stream can be guarded: over a long stream, a near-tie
    between two stored rows may be one that no redraw of the incoming token
    moves past the margin, and such a cache has no unique answer to compare."""
    (w, layer, hh, *rest), tries = args[:-1], args[-1]
    for k in range(tries):
        try:
            return _sample_job((w, layer, (hh + k) % w.bh, *rest))
        except RuntimeError:
            if k == tries - 1:
                raise
    raise AssertionError("unreachable")


def oracle_samples_layers(w: synth.Workload, picks: dict, budgets, T: int, init_n: bool,
                          next_pos: int = 0, tries: int = 1) -> dict:
    """oracle_samples for several layers at once (one pool): picks[l] lists the
    sampled caches of layer l, budgets[l] its budget; init_n: start full.
    tries > 1: a pick whose stream cannot be guarded moves on to the next
    cache (up to tries - 1 times)."""
    jobs, keys = [], []
    for l, hhs in picks.items():
        for hh in hhs:
            jobs.append((w, l, hh, budgets[l], T, budgets[l] + 1,
                         budgets[l] if init_n else None, next_pos, tries))
            keys.append(l)
    workers = min(len(jobs), max(1, min(16, (os.cpu_count() or 2) - 1)))
    if workers <= 1:
        res = [_sample_job_next(j) for j in jobs]
    else:
        with ProcessPoolExecutor(workers) as ex:
            res = list(ex.map(_sample_job_next, jobs))
    out: dict = {}
    for l, smp in zip(keys, res):
        out.setdefault(l, []).append(smp)
    return out


def load_state_into(layer, hh: int, st: dict) -> None:
    """Copy an oracle snapshot into row hh of a GPU layer."""
    n = st["n"]
    dev = layer.k.device
    if n == 0:
        return
    layer.k[hh, :n] = torch.from_numpy(st["k"].view(np.float16)).to(dev)
    layer.v[hh, :n] = torch.from_numpy(st["v"].view(np.float16)).to(dev)
    layer.scores[hh, :n] = torch.from_numpy(st["s"]).to(dev)
    if layer.gumbel is not None:
        layer.gumbel[hh, :n] = torch.from_numpy(st["g"]).to(dev)
    layer.positions[hh, :n] = torch.from_numpy(st["p"]).to(dev)


def bulk_state(layer, n: int, w: synth.Workload, gen) -> None:
    """Fill rows [0, n) of every cache of a GPU layer with a random plausible state."""
    synth.bulk_state_torch(layer.k, layer.v, layer.scores, layer.gumbel, layer.positions, n, w,
                           gen)


def workspace_ready(ws) -> bool:
    """A kve_step_ws workspace left ready for the next call: its header's
    first words are the two reservation counters and the phase of the next
    call; the counter of the next call's phase is zero."""
    h = ws[:16].view(torch.int32).cpu().tolist()
    return h[h[2] & 1] == 0 and h[2] >= 0


def ulp16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


def ulp32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = x.view(np.int32).astype(np.int64)
        return np.where(x < 0, -(x & 0x7FFFFFFF), x)
    return np.abs(ordered(a.astype(np.float32)) - ordered(b.astype(np.float32)))


def kept_tids(init_n: int, first_tid: int, ev_log: np.ndarray) -> list[int]:
    """Replay an eviction log: the original token position of every kept row."""
    tids = list(range(init_n))
    for t, e in enumerate(ev_log):
        tids.append(first_tid + t)
        if e >= 0:
            tids.pop(int(e))
    return tids


def compare_cache(layer, hh: int, s: Sample, gpu_ev: np.ndarray, first_tid: int) -> list[str]:
    """Differences between GPU cache hh and oracle sample s (empty list = parity)."""
    errs = []
    o = s.final
    n = o["n"]
    if not np.array_equal(gpu_ev, s.evicted):
        bad = np.nonzero(gpu_ev != s.evicted)[0]
        errs.append(f"hh {hh}: evicted differs at {len(bad)} steps, first t={bad[0]}: "
                    f"gpu {gpu_ev[bad[0]]} oracle {s.evicted[bad[0]]}")
        return errs
    init_n = s.init["n"] if s.init else 0
    if kept_tids(init_n, first_tid, gpu_ev) != list(o["tid"]):
        errs.append(f"hh {hh}: kept token positions differ")
    gk = layer.k[hh, :n].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    gv = layer.v[hh, :n].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    gs = layer.scores[hh, :n].cpu().numpy()
    gp = layer.positions[hh, :n].cpu().numpy()
    if not np.array_equal(gv, o["v"]):
        errs.append(f"hh {hh}: values differ ({int((gv != o['v']).sum())} elements)")
    ku = ulp16(gk, o["k"])
    if ku.max(initial=0) > KEY_ULP:
        errs.append(f"hh {hh}: keys differ by up to {ku.max()} ulp")
    if not np.array_equal(gp, o["p"]):
        errs.append(f"hh {hh}: positions differ")
    rel = np.abs(gs.astype(np.float64) - o["s"]) / np.maximum(np.abs(o["s"].astype(np.float64)), 1e-30)
    rel[(gs == 0) & (o["s"] == 0)] = 0
    if rel.max(initial=0) > SCORE_RTOL:
        i = int(np.argmax(rel))
        errs.append(f"hh {hh}: score rel err {rel.max():.3g} at row {i} "
                    f"(gpu {gs[i]!r} oracle {o['s'][i]!r})")
    if layer.gumbel is not None:
        gg = layer.gumbel[hh, :n].cpu().numpy()
        gu = ulp32(gg, o["g"])
        if gu.max(initial=0) > GUMBEL_ULP:
            errs.append(f"hh {hh}: gumbel differs by up to {gu.max()} ulp")
    return errs


def policy_for(w: synth.Workload):
    """The kve_step policy of a workload (same parameters as params_for)."""
    import kv_cache_eviction_step_amd as kve
    prm = params_for(w, w.budget, 0)
    kind = {"keyformer": "keyformer", "pyramid": "pyramid", "tova": "tova"}[w.kind]
    return kve.policy(kind, w.n_sink, w.recent, prm.tau_init, prm.tau_end, prm.anneal_steps,
                      w.rope_base, w.gumbel_seed)


def run_layer(w: synth.Workload, layer_idx: int, budget: int, T: int, samples: list[Sample],
              init_n: int | None, next_pos: int, device, cap: int | None = None,
              bh: int | None = None, gen_seed: int = 1234, hh_base: int = 0,
              workspace: bool = False):
    """Step one layer launch T tokens on the GPU; sampled caches get the oracle's
    inputs and initial states.  workspace: one token per kve_step_ws call with
    a workspace sized for every move (long moves handed to the move kernel).
    Returns (layer, evicted log [T, bh] numpy, counters)."""
    import kv_cache_eviction_step_amd as kve
    bh = bh or w.bh
    cap = cap or budget + 1
    kf = w.kind == "keyformer"
    L = kve.Layer.empty(bh, cap, w.d, device, gumbel=kf, hh_base=hh_base)
    gen = torch.Generator(device=device)
    gen.manual_seed(gen_seed)
    n0 = init_n or 0
    bulk_state(L, n0, w, gen)
    for s in samples:
        if s.init is not None:
            load_state_into(L, s.hh, s.init)
    nk, nv = synth.bulk_kv_torch(w, next_pos, T, bh, gen, device)      # [T, bh, d]
    for s in samples:
        nk[:, s.hh] = torch.from_numpy(s.ks.view(np.float16)).to(device)
        nv[:, s.hh] = torch.from_numpy(s.vs.view(np.float16)).to(device)
    ev = torch.full((T, bh), -7, dtype=torch.int32, device=device)
    ctr = kve.Counters(n0, next_pos, next_pos)
    prm = params_for(w, budget, 0)
    if w.kind == "tova" or w.recent > 0 or workspace:
        # the extensions and the workspace form go through the general entry
        # points, one token per call
        batch = kve.LayerBatch([L], [budget], [ctr])
        pol = policy_for(w)
        ws = kve.workspace(bh, budget, w.d, device) if workspace else None
        for t in range(T):
            kve.step(batch, [nk[t]], [nv[t]], pol, [ev[t]], workspace=ws)
        torch.cuda.synchronize(device)
        if ws is not None:
            assert workspace_ready(ws), "workspace not ready for the next call"
        return L, ev.cpu().numpy(), batch.ctrs[0]
    cl = L.c_struct()
    for t in range(T):
        if kf:
            kve.keyformer_step(L, nk[t], nv[t], ctr, budget, w.n_sink, prm.tau_init, prm.tau_end,
                               prm.anneal_steps, w.rope_base, w.gumbel_seed, ev[t], c_layer=cl)
        else:
            kve.pyramid_step(L, nk[t], nv[t], ctr, budget, w.n_sink, w.rope_base, ev[t],
                             c_layer=cl)
    torch.cuda.synchronize(device)
    return L, ev.cpu().numpy(), ctr


def run_batched(w: synth.Workload, layer_ids, budgets, T: int, samples: dict, init_n, next_pos,
                device, gen_seed: int = 99, tokens_per_call: int = 1, workspace: bool = False,
                decode_from: int | None = None):
    """Step several layers together on the GPU: one batched launch per token,
    or per `tokens_per_call` tokens (*_step_layers_tokens).  samples[l] lists
    the oracle samples of layer position l.  workspace: single-token launches
    go through kve_step_ws with a workspace sized for every move.
    decode_from: tokens from this one on go one per launch (the decode form
    after a prompt ingested `tokens_per_call` at a time).  Returns (layers,
    evicted log [T, L, bh] numpy, batch)."""
    import kv_cache_eviction_step_amd as kve
    kf = w.kind == "keyformer"
    gen = torch.Generator(device=device)
    gen.manual_seed(gen_seed)
    layers = []
    for li, b in enumerate(budgets):
        L = kve.Layer.empty(w.bh, b + 1, w.d, device, gumbel=kf)
        n0 = b if init_n is not None else 0
        bulk_state(L, n0, w, gen)
        for s in samples.get(li, []):
            if s.init is not None:
                load_state_into(L, s.hh, s.init)
        layers.append(L)
    n0s = [b if init_n is not None else 0 for b in budgets]
    batch = kve.LayerBatch(layers, budgets, [kve.Counters(n, next_pos, next_pos) for n in n0s])
    nk = torch.empty((T, len(budgets), w.bh, w.d), dtype=torch.float16, device=device)
    nv = torch.empty_like(nk)
    for li in range(len(budgets)):
        k, v = synth.bulk_kv_torch(w, next_pos, T, w.bh, gen, device)
        nk[:, li], nv[:, li] = k, v
        for s in samples.get(li, []):
            nk[:, li, s.hh] = torch.from_numpy(s.ks.view(np.float16)).to(device)
            nv[:, li, s.hh] = torch.from_numpy(s.vs.view(np.float16)).to(device)
    ev = torch.full((T, len(budgets), w.bh), -7, dtype=torch.int32, device=device)
    prm = params_for(w, budgets[0], 0)
    S = tokens_per_call
    ws = kve.workspace(w.bh * len(budgets), max(budgets), w.d, device) if workspace else None
    pol = policy_for(w) if workspace else None
    T_multi = T if decode_from is None else decode_from
    if S > 1:
        # [L, T, bh, d]: each layer's run of tokens is one contiguous block
        nkl, nvl = nk.transpose(0, 1).contiguous(), nv.transpose(0, 1).contiguous()
        evl = torch.full((len(budgets), T, w.bh), -7, dtype=torch.int32, device=device)
        for t0 in range(0, T_multi, S):
            n = min(S, T_multi - t0)
            ks, vs, es = nkl[:, t0:t0 + n], nvl[:, t0:t0 + n], evl[:, t0:t0 + n]
            if kf:
                kve.keyformer_step_layers_tokens(batch, ks, vs, w.n_sink, prm.tau_init,
                                                 prm.tau_end, prm.anneal_steps, w.rope_base,
                                                 w.gumbel_seed, es, n_tokens=n)
            else:
                kve.pyramid_step_layers_tokens(batch, ks, vs, w.n_sink, w.rope_base, es,
                                               n_tokens=n)
        for t in range(T_multi, T):                 # the decode tokens, one per launch
            kve.step(batch, nkl[:, t], nvl[:, t], pol or policy_for(w), evl[:, t],
                     workspace=ws)
        ev = evl.transpose(0, 1)
    else:
        for t in range(T):
            if ws is not None:
                kve.step(batch, nk[t], nv[t], pol, ev[t], workspace=ws)
            elif kf:
                kve.keyformer_step_layers(batch, nk[t], nv[t], w.n_sink, prm.tau_init,
                                          prm.tau_end, prm.anneal_steps, w.rope_base,
                                          w.gumbel_seed, ev[t])
            else:
                kve.pyramid_step_layers(batch, nk[t], nv[t], w.n_sink, w.rope_base, ev[t])
    torch.cuda.synchronize(device)
    if ws is not None:
        assert workspace_ready(ws), "workspace not ready for the next call"
    _ = layer_ids
    return layers, ev.cpu().numpy(), batch
