"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a value printed on the pages, a closed
form, a textbook or library routine, an invariant the pages state, or an
independent brute-force formulation on tiny caches.  Pages cited:
  [KF] "veloxquant_mlx.quantizers.keyformer module"
  [PK] "PyramidKV -- Layer-Adaptive Budget Attention-Mass Eviction"
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import OracleCache, Params
from oracle.guard import guarded_trajectory

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


# ---------------------------------------------------------------------------
# pyramid_budgets: [PK] The budget schedule, Parameters, Evidence
# ---------------------------------------------------------------------------

def test_pyramid_budgets_page_example():
    g = _read_golden("pyramid_budgets_12L_avg512_sink4_beta2.txt")
    L, avg, ns, beta = int(g["n_layers"][0]), int(g["avg_budget"][0]), int(g["n_sink"][0]), float(g["beta"][0])
    want = [int(x) for x in g["budgets"]]
    got = oracle.pyramid_budgets(L, avg, ns, beta)
    assert got == want
    assert np.mean(got) == float(g["mean"][0])


@pytest.mark.parametrize("L,avg,ns,beta", [
    (28, 512, 4, 2.0), (32, 4096, 4, 1.5), (12, 512, 4, 1.5), (7, 100, 2, 1.3),
    (40, 64, 4, 3.0), (2, 10, 0, 1.9), (5, 5, 4, 2.0)])
def test_pyramid_budgets_properties(L, avg, ns, beta):
    b = oracle.pyramid_budgets(L, avg, ns, beta)
    assert len(b) == L                                     # one per layer
    assert all(x >= y for x, y in zip(b, b[1:]))           # monotone taper, deepest smallest
    assert all(x >= ns + 1 for x in b)                     # floor n_sink + 1
    assert abs(np.mean(b) - avg) <= 0.05 * avg             # mean within 5%
    assert abs(np.mean(b) - avg) <= 0.5 + 1e-9             # centred up to rounding


def test_pyramid_budgets_flat_and_steepness():
    assert oracle.pyramid_budgets(28, 512, 4, 1.0) == [512] * 28     # beta 1 is flat
    s15 = oracle.pyramid_budgets(12, 512, 4, 1.5)
    s20 = oracle.pyramid_budgets(12, 512, 4, 2.0)
    assert s20[0] - s20[-1] > s15[0] - s15[-1]                       # larger beta, wider spread
    assert s15[0] == 768 and s15[-1] == 256                          # ~1.5x / 0.5x of the average


def test_pyramid_budgets_edges():
    assert oracle.pyramid_budgets(0, 512, 4, 2.0) == []
    assert oracle.pyramid_budgets(1, 512, 4, 2.0) == [512]
    with pytest.raises(ValueError):
        oracle.pyramid_budgets(12, 512, 4, 0.99)                     # beta < 1 raises
    with pytest.raises(ValueError):
        oracle.pyramid_budgets(-1, 512, 4, 2.0)
    with pytest.raises(ValueError):
        oracle.pyramid_budgets(4, 4, 4, 2.0)                         # avg below the floor


# ---------------------------------------------------------------------------
# Gumbel noise: [KF] THE HONESTY CRUX item 2, KeyformerState (gumbel, seed)
# ---------------------------------------------------------------------------

def test_splitmix64_known_answer():
    g = _read_golden("splitmix64_state0.txt")
    want = [int(x, 16) for x in g["outputs"]]
    assert oracle.splitmix64_stream(int(g["state"][0]), len(want)) == want


def test_gumbel_inverse_cdf_identity():
    # the textbook Gumbel CDF F(x) = exp(-exp(-x)) must map each value back to its uniform
    for hh in range(3):
        for pos in range(0, 4000, 37):
            u = oracle.gumbel_uniform(7, hh, pos)
            assert 0.0 < u < 1.0
            gval = float(oracle.gumbel(7, hh, pos))
            assert abs(math.exp(-math.exp(-gval)) - u) <= 2e-6 * max(u, 1e-3) + 1e-9


def test_gumbel_distribution_moments_and_ks():
    from scipy import stats
    n = 60000
    vals = np.array([oracle.gumbel(0, hh, pos) for hh in range(3) for pos in range(n // 3)],
                    dtype=np.float64)
    assert abs(vals.mean() - 0.5772156649) < 0.02          # Euler-Mascheroni
    assert abs(vals.var() - math.pi ** 2 / 6) < 0.05         # pi^2 / 6
    assert stats.kstest(vals, stats.gumbel_r.cdf).pvalue > 1e-3
    # streams of different rows are not copies of each other
    a = np.array([oracle.gumbel(0, 0, p) for p in range(2000)])
    b = np.array([oracle.gumbel(0, 1, p) for p in range(2000)])
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.1


def test_gumbel_deterministic_and_frozen():
    assert oracle.gumbel(3, 5, 1234) == oracle.gumbel(3, 5, 1234)
    assert oracle.gumbel(3, 5, 1234) != oracle.gumbel(4, 5, 1234)


# ---------------------------------------------------------------------------
# temperature schedule: [KF] FIXED GAP #1, KeyformerState, init_keyformer_state
# ---------------------------------------------------------------------------

def test_tau_closed_forms():
    assert oracle.tau(1.0, 2.0, 64, 0) == np.float32(1.0)        # tau_init at pos 0
    assert oracle.tau(1.0, 2.0, 64, 32) == np.float32(1.5)       # linear ramp midpoint
    assert oracle.tau(1.0, 2.0, 64, 64) == np.float32(2.0)       # tau_end at T
    assert oracle.tau(1.0, 2.0, 64, 10 ** 6) == np.float32(2.0)  # held after T
    assert oracle.tau(1.0, 2.0, 0, 500) == np.float32(1.0)       # T = 0: constant tau_init
    assert oracle.tau(0.7, 0.7, 100, 50) == np.float32(0.7)      # equal ends: constant
    assert oracle.tau(0.0, 0.0, 64, 30) == np.float32(0.0)
    ts = [float(oracle.tau(1.0, 2.0, 1024, p)) for p in range(0, 1100, 10)]
    assert all(x <= y for x, y in zip(ts, ts[1:]))
    for p in (1, 3, 100, 777):
        assert abs(float(oracle.tau(1.0, 2.0, 1024, p)) - (1.0 + p / 1024)) <= 1.2e-7


# ---------------------------------------------------------------------------
# fp16 storage: IEEE binary16, against numpy's conversion routines
# ---------------------------------------------------------------------------

def test_f16_to_f32_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_f32_to_f16_round_to_nearest_even():
    rng = np.random.default_rng(0)
    grid = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)            # exact ties
    near = np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))
    rnd = rng.uniform(-70000, 70000, 4000).astype(np.float32)
    small = (rng.standard_normal(4000) * 1e-5).astype(np.float32)     # subnormal range
    edge = np.array([65504, 65519.996, 65520, 65535, 1e9, 6.1e-5, 5.96e-8, 2.98e-8,
                     2.99e-8, -0.0, 0.0], dtype=np.float32)
    sel = rng.choice(len(mids), 6000, replace=False)
    x = np.concatenate([mids[sel], near[0][sel], near[1][sel], -mids[sel], rnd, small, edge])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16(x)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# RoPE remap: [KF] FIXED GAP #2, KeyformerState (positions), FUSED METAL KERNEL
# ---------------------------------------------------------------------------

def _rope_complex(r: np.ndarray, pos: float, base: float = 10000.0) -> np.ndarray:
    """Rotary embedding as complex multiplication (x_j + i x_{j+D/2}) * e^{i pos f_j}."""
    D = r.shape[-1]
    h = D // 2
    f = base ** (-np.arange(h) * 2.0 / D)
    z = (r[:h] + 1j * r[h:]) * np.exp(1j * pos * f)
    return np.concatenate([z.real, z.imag])


def _pair_ulps(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """|a - b| in units of the fp16 spacing at the magnitude of each element's
    rotation pair (a rotation mixes the two members, so its rounding error is
    set by the pair's norm, not by the smaller member)."""
    a = a_bits.view(np.float16).astype(np.float64)
    b = b_bits.view(np.float16).astype(np.float64)
    h = a.shape[-1] // 2
    nrm = np.hypot(b[..., :h], b[..., h:])
    nrm = np.concatenate([nrm, nrm], axis=-1)
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(nrm, 2.0 ** -14))) - 10)
    return np.abs(a - b) / spacing


@pytest.mark.parametrize("D", [64, 128])
def test_rope_remap_matches_direct_rotation(D):
    rng = np.random.default_rng(D)
    for _ in range(40):
        r = rng.standard_normal(D)
        p = int(rng.integers(0, 20000))
        q = int(rng.integers(0, 8000))
        src = _rope_complex(r, p).astype(np.float16).view(np.uint16)
        want = _rope_complex(r, q).astype(np.float16).view(np.uint16)
        got = oracle.rope_rotate(src, q - p)
        assert _pair_ulps(got, want).max() <= 2.0


def test_rope_remap_direction_pairing_identity():
    D = 8
    for j in range(D // 2):
        e = np.zeros(D)
        e[j] = 1.0
        out = oracle.f16_to_f32(oracle.rope_rotate(e.astype(np.float16).view(np.uint16), 1))
        f = 10000.0 ** (-2.0 * j / D)
        want = np.zeros(D)
        want[j], want[j + D // 2] = math.cos(f), math.sin(f)     # positive angle, half-split pair
        assert np.allclose(out, want, atol=1e-3)
    rng = np.random.default_rng(1)
    bits = rng.standard_normal(128).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.rope_rotate(bits, 0), bits)     # delta 0 is the identity
    x = oracle.f16_to_f32(bits).astype(np.float64)
    y = oracle.f16_to_f32(oracle.rope_rotate(bits, -1234)).astype(np.float64)
    n0 = np.hypot(x[:64], x[64:])
    n1 = np.hypot(y[:64], y[64:])
    assert np.allclose(n0, n1, rtol=2e-3, atol=1e-3)               # pair norms preserved


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------

def _tiny(d=8, budget=6, n_sink=2, tau=(0.0, 0.0, 0), name="t"):
    return synth.Workload(name, 1, 1, 1, d, 40, 0, budget, n_sink, "keyformer",
                          tau[0], tau[1], tau[2])


def test_single_step_softmax_and_argmin_against_library_routines():
    """One scoring + eviction step from a random state, checked with torch.softmax
    (float64) for the mass and numpy.argmin for the eviction choice."""
    rng = np.random.default_rng(5)
    D, budget, ns = 64, 48, 4
    c = OracleCache(D, budget + 1)
    n = budget
    K = rng.standard_normal((n, D)).astype(np.float16)
    c.k[:n] = K.view(np.uint16)
    c.s[:n] = rng.uniform(0, 3, n).astype(np.float32)
    c.g[:n] = rng.gumbel(size=n).astype(np.float32)
    c.p[:n] = np.arange(n)
    c.tid[:n] = np.arange(n)
    c.set_counters(n, 900, 900)
    S0, G0 = c.s[:n].copy(), c.g[:n].copy()
    k = rng.standard_normal(D).astype(np.float16)
    v = rng.standard_normal(D).astype(np.float16)
    prm = Params(budget, ns, True, 1.0, 2.0, 1024, 10000.0, seed=3, hh=2)
    rc, e, m = c.step(k.view(np.uint16), v.view(np.uint16), prm)
    assert rc == 0
    logits = torch.from_numpy(K.astype(np.float64) @ k.astype(np.float64) / math.sqrt(D))
    p = torch.softmax(logits, dim=0).numpy()
    snew = S0 + p.astype(np.float32)
    tau = 1.0 + 900 / 1024
    g_new = float(oracle.gumbel(3, 2, 900))
    keys = np.concatenate([snew[ns:].astype(np.float64) + tau * G0[ns:], [tau * g_new]])
    assert e == ns + int(np.argmin(keys))
    # scores of the survivors: the rows before e in place, the rows after e moved down
    keep = np.concatenate([snew[:e], snew[e + 1:], [0.0]]) if e < n else snew
    assert np.allclose(c.s[:c.n], keep.astype(np.float32), rtol=2e-7, atol=0)
    assert c.n == budget


def test_exact_tie_goes_to_lowest_index():
    """Zero keys give every stored row the same increment (1/8, exact), so two
    rows with equal scores and equal noise tie exactly; the lowest index goes."""
    D, budget, ns = 16, 8, 2
    pos = next(p for p in range(1000) if oracle.gumbel(0, 0, p) > 3.0)   # new row not the min
    c = OracleCache(D, budget + 1)
    c.s[:budget] = np.array([5, 5, 3, 1, 1, 4, 4, 4], dtype=np.float32)
    c.g[:budget] = 0.0
    c.p[:budget] = np.arange(budget)
    c.tid[:budget] = np.arange(budget)
    c.set_counters(budget, pos, pos)
    z = np.zeros(D, dtype=np.uint16)
    rc, e, m = c.step(z, z, Params(budget, ns, True, 1.0, 1.0, 0, seed=0, hh=0))
    assert rc == 0 and e == 3 and m == 0.0
    assert list(c.tid[:c.n]) == [0, 1, 2, 4, 5, 6, 7, pos]


def test_identical_keys_closed_form_scores():
    """All keys equal -> every logit equal -> each row gets 1/n_prev per step,
    so the score of token i is the sum over later steps of 1/n (float32 adds)."""
    D, T = 16, 30
    c = OracleCache(D, T + 1)
    k = np.full(D, 0.5, dtype=np.float16).view(np.uint16)
    prm = Params(budget=T, n_sink=0, use_gumbel=False)
    for t in range(T):
        c.step(k, k, prm)
    want = np.zeros(T, dtype=np.float32)
    for t in range(1, T):                      # token t sees n_prev = t rows
        want[:t] = want[:t] + np.float32(1.0 / t)
    assert np.array_equal(c.s[:T], want)


def test_mass_conservation_and_h2o_corollary():
    """At tau = 0 the newest row (score 0) is always the one evicted: the kept
    tokens are the first `budget`, and no mass ever leaves the cache."""
    w = _tiny(d=64, budget=24, n_sink=4)
    tr = guarded_trajectory(w, 0, 0, 24, 100)
    c = tr.cache
    assert list(c.tid[:c.n]) == list(range(24))
    assert all(e == 24 for e in tr.evicted[24:])
    assert abs(float(c.s[:c.n].astype(np.float64).sum()) - 99.0) < 1e-4


@pytest.mark.parametrize("n_sink,budget,kind", [
    (0, 1, "kf"), (0, 5, "kf"), (4, 5, "kf"), (4, 32, "kf"), (2, 9, "h2o"), (0, 3, "h2o")])
def test_invariants(n_sink, budget, kind):
    tau = (1.0, 2.0, 64) if kind == "kf" else (0.0, 0.0, 0)
    w = _tiny(d=64, budget=budget, n_sink=n_sink, tau=tau)
    c = OracleCache(64, budget + 1)
    prm = Params(budget, n_sink, True, *tau, seed=1, hh=0)
    ks, vs = synth.token_kv(w, 0, 0, np.arange(120))
    for t in range(120):
        n_before = c.n
        rc, e, _ = c.step(ks[t], vs[t], prm)
        assert rc == 0
        assert c.n == min(n_before + 1, budget)                 # budget + 1 -> budget
        assert c.n <= budget                                    # never exceeded
        if e >= 0:
            assert n_sink <= e <= n_before                      # sinks never evicted
            assert np.array_equal(c.p[:c.n], np.arange(c.n))    # contiguous positions
        tid = c.tid[:c.n]
        assert np.all(np.diff(tid) > 0)                         # temporal order kept
        assert np.array_equal(c.v[:c.n], vs[tid])               # values travel with their token
        assert np.array_equal(c.g[:c.n], [oracle.gumbel(1, 0, x) for x in tid])  # frozen noise too
        assert list(tid[:min(n_sink, c.n)]) == list(range(min(n_sink, c.n)))
        assert np.all(c.s[:c.n] >= 0)                           # non-negative scores


def test_tau_zero_keyformer_equals_h2o_and_beta_one():
    """[KF] WHERE THIS SITS: tau_init = tau_end = 0 is H2O exactly; [PK] Relationship
    to H2O: beta = 1 gives every layer the average budget, i.e. uniform H2O."""
    w = synth.WORKLOADS[0]
    ks, vs = synth.token_kv(w, 0, 1, np.arange(128))
    budget = oracle.pyramid_budgets(4, 32, 4, 1.0)[2]
    a, b = OracleCache(64, 33), OracleCache(64, 33)
    ea = a.run(ks, vs, Params(32, 4, True, 0.0, 0.0, 64, seed=0, hh=1))
    eb = b.run(ks, vs, Params(budget, 4, False))
    assert np.array_equal(ea, eb)
    for name in ("k", "v", "s", "p", "tid"):
        assert np.array_equal(getattr(a, name)[:a.n], getattr(b, name)[:b.n])


def test_block_boundary_independence_and_determinism():
    """[KF] KeyformerState (pos): the draw and the schedule do not depend on how
    the token stream is split into calls."""
    w = synth.TINY_ANNEALED
    ks, vs = synth.token_kv(w, 0, 2, np.arange(128))
    prm = Params(32, 4, True, 1.0, 2.0, 64, seed=0, hh=2)
    a = OracleCache(64, 33)
    ea = a.run(ks, vs, prm)
    b = OracleCache(64, 33)
    eb1 = b.run(ks[:50], vs[:50], prm)
    c = OracleCache(64, 33)
    c.load(b.snapshot())
    eb2 = c.run(ks[50:], vs[50:], prm)
    assert np.array_equal(ea, np.concatenate([eb1, eb2]))
    sa, sc = a.snapshot(), c.snapshot()
    for key in ("k", "v", "s", "g", "p", "tid"):
        assert np.array_equal(sa[key], sc[key])


# ---------------------------------------------------------------------------
# brute force on tiny caches: an independent formulation of the same semantics
# ---------------------------------------------------------------------------

def _brute_force(ks_bits, budget, n_sink, tau_fn, gumbel_fn, base=10000.0, recent=0,
                 current=False):
    """Kept tokens as a list; each kept token's stored key is its incoming key
    rotated (complex form, float64) from its absolute position to its index in
    the list; each step's mass comes from torch.softmax (float64) and is kept as
    a per-token history whose sum is the score (its last entry, for the
    current-step score of TOVA); the eviction is numpy.argmin over the tokens
    after the first n_sink and before the last `recent`."""
    def score(tok):
        h = hist[tok]
        return (h[-1] if h else 0.0) if current else sum(h)

    D = ks_bits.shape[1]
    kin = ks_bits.view(np.float16).astype(np.float64)
    kept, hist, evicted = [], {}, []
    for t in range(len(kin)):
        if kept:
            K = np.stack([_rope_complex(kin[tok], idx - tok, base) for idx, tok in enumerate(kept)])
            p = torch.softmax(torch.from_numpy(K @ kin[t] / math.sqrt(D)), 0).numpy()
            for tok, pi in zip(kept, p):
                hist[tok].append(pi)
        kept.append(t)
        hist[t] = []
        if len(kept) > budget:
            tau = tau_fn(t)
            vals = [score(tok) + tau * gumbel_fn(tok)
                    for tok in kept[n_sink:len(kept) - recent]]
            e = n_sink + int(np.argmin(vals))
            evicted.append(e)
            kept.pop(e)
        else:
            evicted.append(-1)
    scores = np.array([score(tok) for tok in kept])
    keys = np.stack([_rope_complex(kin[tok], idx - tok, base) for idx, tok in enumerate(kept)])
    return kept, np.array(evicted), scores, keys


@pytest.mark.parametrize("D", [4, 8])
@pytest.mark.parametrize("tau", [(0.0, 0.0, 0), (0.5, 0.5, 0), (1.0, 2.0, 16)])
def test_brute_force_tiny_caches(D, tau):
    T = 40
    for n_sink in range(0, 4):
        for budget in range(n_sink + 1, 9):
            w = _tiny(d=D, budget=budget, n_sink=n_sink, tau=tau, name=f"bf{D}")
            hh = 3 * n_sink + budget
            # generous guard: the brute force keeps exact keys while the oracle
            # re-rounds moved keys to fp16, so their scores differ by ~1e-3
            tr = guarded_trajectory(w, 0, hh, budget, T, min_margin_rel=0.02,
                                    max_attempts=200)
            c = tr.cache
            tau_fn = (lambda t: tau[0] + min(t, tau[2]) * (tau[1] - tau[0]) / tau[2]) if tau[2] \
                else (lambda t: tau[0])
            kept, ev, sc, keys = _brute_force(tr.ks, budget, n_sink, tau_fn,
                                              lambda tok: float(oracle.gumbel(0, hh, tok)))
            assert list(c.tid[:c.n]) == kept
            assert np.array_equal(c.v[:c.n], tr.vs[kept])
            assert np.array_equal(tr.evicted, ev)
            assert np.allclose(c.s[:c.n], sc, rtol=5e-3, atol=1e-6)
            got = c.k[:c.n]
            want = keys.astype(np.float16).view(np.uint16)
            assert _pair_ulps(got, want).max() <= 8.0


# ---------------------------------------------------------------------------
# the recent window ([KF] KeyformerState, init_keyformer_state: trailing rows
# protected, an extension off by default) and TOVA-adapted scoring ([PK] table
# of eviction axes: the current step's attention weight is the score)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D", [4, 8])
@pytest.mark.parametrize("tau,current", [((0.0, 0.0, 0), False), ((1.0, 2.0, 16), False),
                                         ((0.0, 0.0, 0), True), ((0.5, 1.5, 8), True)])
@pytest.mark.parametrize("recent", [1, 3])
def test_brute_force_recent_and_tova(D, tau, current, recent):
    T = 40
    for n_sink in range(0, 3):
        for budget in range(n_sink + recent + 1, n_sink + recent + 6):
            kind = "tova" if current else "keyformer"
            w = synth.Workload(f"bfr{D}", 1, 1, 1, D, 40, 0, budget, n_sink, kind,
                               tau[0], tau[1], tau[2], recent=recent)
            hh = 5 * n_sink + budget
            prm = Params(budget, n_sink, True, *tau, seed=0, hh=hh, recent=recent,
                         current_score=current)
            tr = guarded_trajectory(w, 0, hh, budget, T, min_margin_rel=0.02,
                                    max_attempts=200, params=prm)
            c = tr.cache
            tau_fn = (lambda t: tau[0] + min(t, tau[2]) * (tau[1] - tau[0]) / tau[2]) if tau[2] \
                else (lambda t: tau[0])
            kept, ev, sc, keys = _brute_force(tr.ks, budget, n_sink, tau_fn,
                                              lambda tok: float(oracle.gumbel(0, hh, tok)),
                                              recent=recent, current=current)
            assert list(c.tid[:c.n]) == kept
            assert np.array_equal(tr.evicted, ev)
            assert np.array_equal(c.v[:c.n], tr.vs[kept])
            assert np.allclose(c.s[:c.n], sc, rtol=5e-3, atol=1e-6)
            assert _pair_ulps(c.k[:c.n], keys.astype(np.float16).view(np.uint16)).max() <= 8.0


@pytest.mark.parametrize("recent,kind", [(1, "kf"), (7, "kf"), (1, "h2o"), (20, "h2o"),
                                         (5, "tova")])
def test_recent_window_always_kept(recent, kind):
    """The last `recent` tokens and the sinks are present after every step, the
    newest token is never the one evicted, and positions stay contiguous."""
    budget, n_sink, T = 32, 4, 200
    tau = (1.0, 2.0, 64) if kind == "kf" else (0.0, 0.0, 0)
    w = synth.Workload("rw", 1, 1, 1, 64, T, 0, budget, n_sink, "keyformer", *tau)
    c = OracleCache(64, budget + 1)
    prm = Params(budget, n_sink, kind == "kf", *tau, seed=4, hh=1, recent=recent,
                 current_score=kind == "tova")
    ks, vs = synth.token_kv(w, 0, 1, np.arange(T))
    for t in range(T):
        n_before = c.n
        rc, e, _ = c.step(ks[t], vs[t], prm)
        assert rc == 0
        tid = list(c.tid[:c.n])
        assert tid[-min(recent, t + 1):] == list(range(max(0, t + 1 - recent), t + 1))
        assert tid[:min(n_sink, c.n)] == list(range(min(n_sink, c.n)))
        if e >= 0:
            assert n_sink <= e <= n_before - recent         # newest never evicted
            assert np.array_equal(c.p[:c.n], np.arange(c.n))


def test_recent_zero_is_the_plain_step():
    """recent = 0 reproduces the step without the window, bit for bit."""
    w = synth.TINY_ANNEALED
    ks, vs = synth.token_kv(w, 0, 3, np.arange(150))
    a, b = OracleCache(64, 33), OracleCache(64, 33)
    ea = a.run(ks, vs, Params(32, 4, True, 1.0, 2.0, 64, seed=0, hh=3))
    eb = b.run(ks, vs, Params(32, 4, True, 1.0, 2.0, 64, seed=0, hh=3, recent=0))
    assert np.array_equal(ea, eb)
    for name in ("k", "v", "s", "g", "p", "tid"):
        assert np.array_equal(getattr(a, name)[:a.n], getattr(b, name)[:b.n])


def test_tova_scores_are_the_current_softmax():
    """One TOVA step from two random states that differ only in their scores:
    both give the survivors torch.softmax (float64) of this step's logits,
    rounded to float32, whatever the scores were before; the new row has 0."""
    rng = np.random.default_rng(9)
    D, budget, ns, recent = 64, 40, 4, 3
    K = rng.standard_normal((budget, D)).astype(np.float16)
    k = rng.standard_normal(D).astype(np.float16)
    v = rng.standard_normal(D).astype(np.float16)
    logits = torch.from_numpy(K.astype(np.float64) @ k.astype(np.float64) / math.sqrt(D))
    p = torch.softmax(logits, dim=0).numpy().astype(np.float32)
    outs = []
    for seed in (1, 2):
        c = OracleCache(D, budget + 1)
        c.k[:budget] = K.view(np.uint16)
        c.s[:budget] = np.random.default_rng(seed).uniform(0, 9, budget).astype(np.float32)
        c.p[:budget] = np.arange(budget)
        c.tid[:budget] = np.arange(budget)
        c.set_counters(budget, 500, 500)
        rc, e, _ = c.step(k.view(np.uint16), v.view(np.uint16),
                          Params(budget, ns, False, recent=recent, current_score=True))
        assert rc == 0
        assert e == ns + int(np.argmin(p[ns:budget + 1 - recent]))
        want = np.concatenate([p[:e], p[e + 1:], [0.0]]).astype(np.float32)
        assert np.allclose(c.s[:c.n], want, rtol=2.5e-7, atol=0)
        assert c.s[c.n - 1] == 0.0
        outs.append((e, c.s[:c.n].copy()))
    assert outs[0][0] == outs[1][0] and np.array_equal(outs[0][1], outs[1][1])


def test_tova_without_window_evicts_the_newest():
    """Without a recent window the new row (score 0) is TOVA's minimum on every
    step, as for H2O: the first `budget` tokens are kept."""
    w = _tiny(d=64, budget=20, n_sink=4)
    ks, vs = synth.token_kv(w, 0, 0, np.arange(90))
    c = OracleCache(64, 21)
    ev = c.run(ks, vs, Params(20, 4, False, current_score=True))
    assert list(c.tid[:c.n]) == list(range(20))
    assert np.all(ev[20:] == 20) and np.all(ev[:20] == -1)


@pytest.mark.parametrize("budget,n_sink,recent,ok", [(10, 4, 5, True), (10, 4, 6, False),
                                                     (10, 0, 9, True), (10, 0, 10, False),
                                                     (10, 4, -1, False)])
def test_recent_validation(budget, n_sink, recent, ok):
    """[KF] init_keyformer_state: sinks plus the recent window must leave room
    to evict within the budget."""
    c = OracleCache(8, budget + 1)
    z = np.zeros(8, dtype=np.uint16)
    prm = Params(budget, n_sink, False, recent=recent)
    if ok:
        assert c.step(z, z, prm)[0] == 0
    else:
        with pytest.raises(ValueError):
            c.step(z, z, prm)
