"""GPU parity: the C-ABI library on gfx950 against the CPU oracle.

Every case steps a full launch (all B*H caches of a layer) through
keyformer_step / pyramid_step and compares sampled caches with the oracle on
identical, margin-guarded inputs: evicted indices, kept token positions,
values and positions bit-exact; keys within 1 fp16 ULP; scores within 1e-5
relative; Gumbel values within 1 fp32 ULP.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (Sample, compare_cache, load_state_into, oracle_samples,
                         oracle_samples_layers, policy_for,
                         random_state,
                         run_batched, run_layer, workspace_ready)
from oracle.guard import guarded_trajectory, params_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_eviction_step_amd as kve
    assert len(kve.hip_runtimes_mapped()) == 1, kve.hip_runtimes_mapped()
    return torch.device("cuda:0")


def _say(msg: str) -> None:
    print(msg, flush=True)


def _assert_parity(L, ev, samples, first_tid):
    errs = []
    for s in samples:
        errs += compare_cache(L, s.hh, s, ev[:, s.hh], first_tid)
    assert not errs, "\n".join(errs[:20])


# ---------------------------------------------------------------------------
# the tiny workload, both temperature runs, every cache, full trajectory
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w", [synth.WORKLOADS[0], synth.TINY_ANNEALED], ids=lambda w: w.name)
def test_tiny_full_trajectory(dev, w):
    _say(f"[tiny] {w.name} bh={w.bh} d={w.d} budget={w.budget} T={w.tokens}")
    samples = oracle_samples(w, 0, range(w.bh), w.budget, w.tokens, w.budget + 1, workers=1)
    L, ev, ctr = run_layer(w, 0, w.budget, w.tokens, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)
    assert (ctr.n_kept, ctr.next_pos, ctr.pos) == (w.budget, w.tokens, w.tokens)


# ---------------------------------------------------------------------------
# single steps from random states: edge cases of the eviction index
# ---------------------------------------------------------------------------

def _edge_workload(d, kind):
    if kind == "kf":
        return synth.Workload(f"edge{d}kf", 1, 1, 6, d, 64, 0, 32, 4, "keyformer", 1.0, 2.0, 64)
    return synth.Workload(f"edge{d}pk", 1, 1, 6, d, 64, 0, 32, 4, "pyramid")


def _forced(w, hh, n, cap, next_pos, target):
    """Random state whose eviction is steered to row `target`.

    Keyformer: the target gets score 0 and a Gumbel value far below any other.
    H2O / PyramidKV: every stored row gains mass, so the new row (score 0)
    always loses -- unless the target's key points so far away from the
    incoming key that its softmax weight underflows to exactly 0 in fp32 on
    both sides; then it ties the new row at 0 and the lower index goes."""
    c = random_state(w, 0, hh, n, cap, next_pos, seed=hh + 17)
    if target is not None and target < n:
        c.s[target] = 0.0
        if w.kind == "keyformer":
            c.g[target] = -12.0
        else:
            knew = synth.token_kv(w, 0, hh, [next_pos])[0][0].view(np.float16).astype(np.float32)
            c.k[target] = (-40.0 * knew).astype(np.float16).view(np.uint16)
    return c


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["kf", "pk"])
@pytest.mark.parametrize("n,budget,n_sink,target", [
    (0, 8, 2, None),          # bootstrap: first token only appended
    (5, 8, 2, None),          # under budget: score + append, no eviction
    (7, 8, 0, None),          # reaches budget exactly, no eviction
    (8, 8, 0, 0),             # n_sink 0: row 0 is evictable
    (8, 8, 3, 3),             # evict the first non-sink row
    (40, 40, 4, 20),          # middle row
    (40, 40, 4, 39),          # the newest stored row
    (40, 40, 4, None),        # whatever the keys decide (new row included)
    (300, 300, 4, 4),         # spans two score sweeps; every row after 4 moves
    (1000, 1000, 4, 517),     # several sweeps and move chunks, ragged tails
    (1000, 1000, 4, 998),
    # score slots per thread change at n = 1024 / 1025 and 4096 / 4097
    (1024, 1024, 4, 700),     # 2 slots, every slot used
    (1024, 1100, 4, None),    # 2 slots, under budget
    (1025, 1025, 4, 1000),    # 8 slots, the 1025th row in the first one
    (4096, 4096, 4, 3000),    # 8 slots, every slot used
    (4097, 4097, 4, 4096),    # 24 slots: evict the newest stored row
    (4097, 4200, 4, None),    # 24 slots, under budget
])
def test_single_step_edges(dev, d, kind, n, budget, n_sink, target):
    import kv_cache_eviction_step_amd as kve
    w = _edge_workload(d, kind)
    w = synth.Workload(w.name, 1, 1, 6, d, 64, 0, budget, n_sink, w.kind, w.tau_init,
                       w.tau_end, w.anneal_steps)
    cap = budget + 5                                  # rows past budget + 1 are sentinels
    next_pos = n if n < budget else 5000 + n
    _say(f"[edge] d={d} kind={kind} n={n} budget={budget} n_sink={n_sink} target={target}")
    bh = w.bh
    samples = []
    exact_tie = kind == "pk" and target is not None and n >= budget
    for hh in range(bh):
        c = _forced(w, hh, n, cap, next_pos, target)
        init = c.snapshot()
        tr = guarded_trajectory(w, 0, hh, budget, 1, cap=cap, t0=next_pos, cache=c,
                                params=params_for(w, budget, hh),
                                min_margin_rel=-1.0 if exact_tie else 1e-4)
        samples.append(Sample(hh, budget, init, tr.ks, tr.vs, tr.evicted, tr.cache.snapshot(),
                              int(tr.attempts.sum())))
        if target is not None and n >= budget:
            assert tr.evicted[0] == target
    L = kve.Layer.empty(bh, cap, d, dev, gumbel=(kind == "kf"))
    sentinel_k = torch.full((bh, cap, d), 12345.0, dtype=torch.float16, device=dev)
    L.k.copy_(sentinel_k)
    L.v.fill_(-7.0)
    L.scores.fill_(-3.0)
    L.positions.fill_(-99)
    if L.gumbel is not None:
        L.gumbel.fill_(99.0)
    for s in samples:
        load_state_into(L, s.hh, s.init)
    nk = torch.stack([torch.from_numpy(s.ks[0].view(np.float16)) for s in samples]).to(dev)
    nv = torch.stack([torch.from_numpy(s.vs[0].view(np.float16)) for s in samples]).to(dev)
    ev = torch.full((bh,), -7, dtype=torch.int32, device=dev)
    ctr = kve.Counters(n, next_pos, next_pos)
    prm = params_for(w, budget, 0)
    if kind == "kf":
        kve.keyformer_step(L, nk, nv, ctr, budget, n_sink, prm.tau_init, prm.tau_end,
                           prm.anneal_steps, w.rope_base, w.gumbel_seed, ev)
    else:
        kve.pyramid_step(L, nk, nv, ctr, budget, n_sink, w.rope_base, ev)
    torch.cuda.synchronize()
    evn = ev.cpu().numpy()[None, :]
    _assert_parity(L, evn, samples, next_pos)
    assert ctr.n_kept == min(n + 1, budget)
    # nothing written past row n (the slot the new row may take) in any cache
    assert torch.equal(L.k[:, n + 1:], sentinel_k[:, n + 1:])
    assert bool((L.v[:, n + 1:] == -7.0).all())
    assert bool((L.scores[:, n + 1:] == -3.0).all())
    assert bool((L.positions[:, n + 1:] == -99).all())
    if L.gumbel is not None:
        assert bool((L.gumbel[:, n + 1:] == 99.0).all())


# ---------------------------------------------------------------------------
# whole trajectories at the Llama-3.2-3B shapes (8 caches, D = 128)
# ---------------------------------------------------------------------------

def test_keyformer_trajectory_llama_shape(dev):
    w = synth.WORKLOADS[1]
    T = 760                                            # 512 appends, then 248 evicting steps
    _say(f"[traj] {w.name} layer 3 bh={w.bh} budget={w.budget} T={T}")
    samples = oracle_samples(w, 3, range(w.bh), w.budget, T, w.budget + 1)
    L, ev, _ = run_layer(w, 3, w.budget, T, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)
    assert (ev[w.budget:] < w.budget).any()            # interior evictions happened


@pytest.mark.parametrize("layer", [0, 27])
def test_pyramid_trajectory_llama_shape(dev, layer):
    w = synth.WORKLOADS[2]
    budget = oracle.pyramid_budgets(w.layers, w.budget, w.n_sink, w.beta)[layer]
    T = budget + 200
    _say(f"[traj] {w.name} layer {layer} budget={budget} T={T}")
    samples = oracle_samples(w, layer, range(w.bh), budget, T, budget + 1)
    L, ev, _ = run_layer(w, layer, budget, T, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)


def test_beta_one_pyramid_is_h2o_bit_for_bit(dev):
    """PyramidKV at beta = 1 (every layer the average budget) and Keyformer at
    tau = 0 are the same H2O step: identical GPU states, bit for bit."""
    import kv_cache_eviction_step_amd as kve
    w = synth.WORKLOADS[2]
    budget = kve.pyramid_budgets(w.layers, w.budget, w.n_sink, 1.0)[5]
    assert budget == w.budget
    T = 700
    _say(f"[beta1] bh={w.bh} budget={budget} T={T}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    nk, nv = synth.bulk_kv_torch(w, 0, T, w.bh, gen, dev)
    A = kve.Layer.empty(w.bh, budget + 1, w.d, dev, gumbel=False)
    B = kve.Layer.empty(w.bh, budget + 1, w.d, dev, gumbel=True)
    ca, cb = kve.Counters(0, 0, 0), kve.Counters(0, 0, 0)
    eva = torch.empty((T, w.bh), dtype=torch.int32, device=dev)
    evb = torch.empty_like(eva)
    for t in range(T):
        kve.pyramid_step(A, nk[t], nv[t], ca, budget, w.n_sink, w.rope_base, eva[t])
        kve.keyformer_step(B, nk[t], nv[t], cb, budget, w.n_sink, 0.0, 0.0, 0, w.rope_base,
                           123, evb[t])
    torch.cuda.synchronize()
    assert torch.equal(eva, evb)
    n = ca.n_kept
    for name in ("k", "v", "scores", "positions"):
        assert torch.equal(getattr(A, name)[:, :n], getattr(B, name)[:, :n]), name


# ---------------------------------------------------------------------------
# full launch sizes: every cache of the layer stepped, sampled caches checked
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ws", [False, True], ids=["in-place", "workspace"])
def test_full_size_batched_late_riser(dev, ws):
    """The 8B-shaped workload, one layer launch of 256 caches per token:
    keyformer_step (every cache compacts in place) and kve_step_ws (moves of
    more than 128 rows handed to the move kernel)."""
    w = synth.WORKLOADS[3]                             # B*H = 256, budget 1024, D = 128
    T, next_pos = 40, w.prompt
    hhs = [0, 37, 128, 255]
    _say(f"[full] {w.name} bh={w.bh} cap={w.budget + 1} sampled={hhs} T={T} ws={ws}")
    samples = oracle_samples(w, 9, hhs, w.budget, T, w.budget + 1, init_n=w.budget,
                             next_pos=next_pos)
    L, ev, _ = run_layer(w, 9, w.budget, T, samples, w.budget, next_pos, dev, workspace=ws)
    _assert_parity(L, ev, samples, next_pos)
    assert ((ev >= 0) & (ev < w.budget)).any()


@pytest.mark.parametrize("layer", [0, 31])
def test_full_size_long_context(dev, layer):
    w = synth.WORKLOADS[4]                             # B*H = 512, budgets 6144 .. 2048
    budget = oracle.pyramid_budgets(w.layers, w.budget, w.n_sink, w.beta)[layer]
    T, next_pos = 16, w.prompt
    hhs = [0, 311, 511]
    _say(f"[full] {w.name} layer {layer} bh={w.bh} budget={budget} sampled={hhs} T={T}")
    samples = oracle_samples(w, layer, hhs, budget, T, budget + 1, init_n=budget,
                             next_pos=next_pos)
    L, ev, _ = run_layer(w, layer, budget, T, samples, budget, next_pos, dev)
    _assert_parity(L, ev, samples, next_pos)


# ---------------------------------------------------------------------------
# determinism and split launches
# ---------------------------------------------------------------------------

def test_deterministic_and_split_bh_launches(dev):
    """Two identical runs give identical bits; splitting the B*H set into two
    launches (hh_base offsets the Gumbel streams) gives the same result."""
    import kv_cache_eviction_step_amd as kve
    w = synth.TINY_ANNEALED
    w = synth.Workload("split", 1, 1, 16, 128, 300, 0, 64, 4, "keyformer", 1.0, 2.0, 100)
    T = 300
    _say(f"[split] bh={w.bh} budget={w.budget} T={T}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    nk, nv = synth.bulk_kv_torch(w, 0, T, w.bh, gen, dev)

    def run_whole():
        L = kve.Layer.empty(w.bh, w.budget + 1, w.d, dev)
        c = kve.Counters(0, 0, 0)
        for t in range(T):
            kve.keyformer_step(L, nk[t], nv[t], c, w.budget, w.n_sink, 1.0, 2.0, 100, 1e4, 9)
        return L

    a, b = run_whole(), run_whole()
    halves = [kve.Layer.empty(8, w.budget + 1, w.d, dev, hh_base=8 * i) for i in range(2)]
    cs = [kve.Counters(0, 0, 0), kve.Counters(0, 0, 0)]
    for t in range(T):
        for i in range(2):
            kve.keyformer_step(halves[i], nk[t, 8 * i:8 * i + 8].contiguous(),
                               nv[t, 8 * i:8 * i + 8].contiguous(), cs[i], w.budget, w.n_sink,
                               1.0, 2.0, 100, 1e4, 9)
    torch.cuda.synchronize()
    for name in ("k", "v", "scores", "gumbel", "positions"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
        joined = torch.cat([getattr(halves[0], name), getattr(halves[1], name)])
        assert torch.equal(getattr(a, name), joined), name


# ---------------------------------------------------------------------------
# batched calls: several layers per launch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["kf", "pk"])
def test_batched_equals_per_layer_calls(dev, kind):
    """keyformer_step_layers / pyramid_step_layers give the same bits as one
    per-layer call per layer (layers of different B*H, cap and budget)."""
    import kv_cache_eviction_step_amd as kve
    kf = kind == "kf"
    shapes = [(8, 64, 65), (5, 40, 50), (12, 64, 67), (3, 9, 10)]     # (bh, budget, cap)
    T, d = 200, 128
    _say(f"[batched==per-layer] kind={kind} shapes={shapes} T={T}")
    w = synth.Workload("mix", 1, 1, 1, d, T, 0, 64, 4, "keyformer" if kf else "pyramid",
                       1.0 if kf else 0.0, 2.0 if kf else 0.0, 100 if kf else 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    ins = [synth.bulk_kv_torch(w, 0, T, bh, gen, dev) for bh, _, _ in shapes]
    A = [kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=7 * i)
         for i, (bh, _, cap) in enumerate(shapes)]
    B = [kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=7 * i)
         for i, (bh, _, cap) in enumerate(shapes)]
    ca = [kve.Counters(0, 0, 0) for _ in shapes]
    batch = kve.LayerBatch(B, [b for _, b, _ in shapes])
    eva = [torch.empty((T, bh), dtype=torch.int32, device=dev) for bh, _, _ in shapes]
    evb = [torch.empty((T, bh), dtype=torch.int32, device=dev) for bh, _, _ in shapes]
    for t in range(T):
        for i, (bh, budget, cap) in enumerate(shapes):
            if kf:
                kve.keyformer_step(A[i], ins[i][0][t], ins[i][1][t], ca[i], budget, 4, 1.0, 2.0,
                                   100, 1e4, 3, eva[i][t])
            else:
                kve.pyramid_step(A[i], ins[i][0][t], ins[i][1][t], ca[i], budget, 4, 1e4,
                                 eva[i][t])
        ks = [ins[i][0][t] for i in range(len(shapes))]
        vs = [ins[i][1][t] for i in range(len(shapes))]
        evs = [evb[i][t] for i in range(len(shapes))]
        if kf:
            kve.keyformer_step_layers(batch, ks, vs, 4, 1.0, 2.0, 100, 1e4, 3, evs)
        else:
            kve.pyramid_step_layers(batch, ks, vs, 4, 1e4, evs)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert (ca[i].n_kept, ca[i].next_pos, ca[i].pos) == \
            (batch.ctrs[i].n_kept, batch.ctrs[i].next_pos, batch.ctrs[i].pos)
        assert torch.equal(eva[i], evb[i])
        n = ca[i].n_kept
        for name in ("k", "v", "scores", "positions") + (("gumbel",) if kf else ()):
            assert torch.equal(getattr(A[i], name)[:, :n], getattr(B[i], name)[:, :n]), (i, name)
    if kf:
        assert any(bool(((e >= 0) & (e < b)).any()) for e, (_, b, _) in zip(eva, shapes))


@pytest.mark.parametrize("ws", [False, True], ids=["in-place", "workspace"])
def test_full_size_batched_all_layers_late_riser(dev, ws):
    """The 8B-shaped workload with all 32 layers in one launch per token:
    keyformer_step_layers (in place) and kve_step_ws (8192 caches, long moves
    handed over), the decode form the benchmark times."""
    w = synth.WORKLOADS[3]
    T, next_pos = 24, w.prompt
    picks = {0: [0, 255], 17: [100], 31: [31, 200]}
    _say(f"[full-batched] {w.name} layers={w.layers} bh={w.bh} sampled={picks} T={T} ws={ws}")
    samples = {l: oracle_samples(w, l, hhs, w.budget, T, w.budget + 1, init_n=w.budget,
                                 next_pos=next_pos) for l, hhs in picks.items()}
    layers, ev, _ = run_batched(w, list(range(w.layers)), [w.budget] * w.layers, T, samples,
                                w.budget, next_pos, dev, workspace=ws)
    errs = []
    for l, ss in samples.items():
        for s in ss:
            errs += compare_cache(layers[l], s.hh, s, ev[:, l, s.hh], next_pos)
    assert not errs, "\n".join(errs[:20])


def test_full_size_tokens_late_riser_every_layer(dev):
    """The 8B-shaped workload as the bench times it best: all 32 layers x 32
    tokens in one launch (keys cached between tokens, 1024-thread
    workgroups), one sampled cache per layer spread over batch and head."""
    w = synth.WORKLOADS[3]
    T, next_pos = 32, w.prompt
    picks = {l: [(7 + 37 * l) % w.bh] for l in range(w.layers)}
    _say(f"[full-tokens] {w.name} layers={w.layers} bh={w.bh} one cache per layer T={T} S={T}")
    samples = oracle_samples_layers(w, picks, [w.budget] * w.layers, T, True, next_pos)
    layers, ev, _ = run_batched(w, list(range(w.layers)), [w.budget] * w.layers, T, samples,
                                w.budget, next_pos, dev, tokens_per_call=T)
    errs = []
    for l, ss in samples.items():
        for s in ss:
            errs += compare_cache(layers[l], s.hh, s, ev[:, l, s.hh], next_pos)
    assert not errs, "\n".join(errs[:20])
    assert any(((ev[:, l] >= 0) & (ev[:, l] < w.budget)).any() for l in range(w.layers))


@pytest.mark.parametrize("decode", ["tokens32", "single_ws"])
def test_whole_run_late_riser_every_layer(dev, decode):
    """The 8B-shaped workload's whole run (4096 + 512 tokens from empty caches)
    through all 32 layers x 256 caches, one sampled cache per layer spread over
    batch and head, against the oracle.  The prompt goes 32 tokens per launch;
    the decode tokens go the same way (tokens32), or one per launch through
    kve_step_ws over all layers with long moves handed to the move kernel
    (single_ws: the decode form the benchmark times).  Over 4608 tokens about
    one cache in twenty meets a near-tie between two stored rows that no
    redraw of the incoming token clears; the sample then moves on to the next
    cache of the layer."""
    w = synth.WORKLOADS[3]
    T = w.tokens
    picks = {l: [(13 + 41 * l) % w.bh] for l in range(w.layers)}
    _say(f"[whole-run] {w.name} layers={w.layers} bh={w.bh} one cache per layer T={T} "
         f"decode={decode}: oracle")
    samples = oracle_samples_layers(w, picks, [w.budget] * w.layers, T, False, tries=4)
    _say(f"[whole-run] {w.name}: GPU, sampled {[s.hh for l in sorted(samples) for s in samples[l]]}")
    single = decode == "single_ws"
    layers, ev, batch = run_batched(w, list(range(w.layers)), [w.budget] * w.layers, T, samples,
                                    None, 0, dev, tokens_per_call=32, workspace=single,
                                    decode_from=w.prompt if single else None)
    errs = []
    for l, ss in samples.items():
        for s in ss:
            errs += compare_cache(layers[l], s.hh, s, ev[:, l, s.hh], 0)
    assert not errs, "\n".join(errs[:20])
    assert all(c.n_kept == w.budget for c in batch.ctrs)
    late = ev[w.budget:]
    assert ((late >= 0) & (late < w.budget)).mean() > 0.02       # interior evictions happened
    if single:                                  # some decode moves went to the move kernel
        dec = ev[w.prompt:]
        assert ((dec >= 0) & (w.budget - 1 - dec > 128)).any()


def test_full_size_tokens_long_context_every_layer(dev):
    """The long-context workload, all 32 layers (budgets 6144 .. 2048) x 16
    tokens per launch (keys streamed, 1024-thread workgroups), four launches,
    one sampled cache per layer."""
    w = synth.WORKLOADS[4]
    budgets = oracle.pyramid_budgets(w.layers, w.budget, w.n_sink, w.beta)
    T, next_pos = 64, w.prompt
    picks = {l: [(11 + 53 * l) % w.bh] for l in range(w.layers)}
    _say(f"[full-tokens] {w.name} layers={w.layers} bh={w.bh} one cache per layer T={T} S=16")
    samples = oracle_samples_layers(w, picks, budgets, T, True, next_pos)
    layers, ev, _ = run_batched(w, list(range(w.layers)), budgets, T, samples, 1, next_pos, dev,
                                tokens_per_call=16)
    errs = []
    for l, ss in samples.items():
        for s in ss:
            errs += compare_cache(layers[l], s.hh, s, ev[:, l, s.hh], next_pos)
    assert not errs, "\n".join(errs[:20])


def test_full_size_batched_long_context_pyramid(dev):
    """The long-context PyramidKV workload, 8 of its layers (budgets 6144 ..
    2048 spread) in one launch per token."""
    w = synth.WORKLOADS[4]
    allb = oracle.pyramid_budgets(w.layers, w.budget, w.n_sink, w.beta)
    lids = [0, 5, 10, 15, 20, 25, 30, 31]
    budgets = [allb[l] for l in lids]
    T, next_pos = 8, w.prompt
    picks = {0: [0, 511], 7: [77]}
    _say(f"[full-batched] {w.name} layers={lids} budgets={budgets} sampled={picks} T={T}")
    samples = {li: oracle_samples(w, lids[li], hhs, budgets[li], T, budgets[li] + 1,
                                  init_n=budgets[li], next_pos=next_pos)
               for li, hhs in picks.items()}
    layers, ev, _ = run_batched(w, lids, budgets, T, samples, 1, next_pos, dev)
    errs = []
    for li, ss in samples.items():
        for s in ss:
            errs += compare_cache(layers[li], s.hh, s, ev[:, li, s.hh], next_pos)
    assert not errs, "\n".join(errs[:20])


# ---------------------------------------------------------------------------
# limits and degenerate shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,kind", [(128, "kf"), (64, "kf"), (128, "pk")])
def test_maximum_budget_single_steps(dev, d, kind):
    """Budget 12288, the largest the library accepts (LDS past 64 KiB): a
    step whose eviction moves almost every row, and a bootstrap-free step."""
    budget, n_sink, bh = 12288, 4, 3
    w = synth.Workload(f"max{d}{kind}", 1, 1, bh, d, 64, 0, budget, n_sink,
                       "keyformer" if kind == "kf" else "pyramid",
                       1.0 if kind == "kf" else 0.0, 2.0 if kind == "kf" else 0.0,
                       64 if kind == "kf" else 0)
    cap, next_pos = budget + 1, 20000
    _say(f"[max] d={d} kind={kind} budget={budget} bh={bh}")
    samples = []
    for hh in range(bh):
        c = _forced(w, hh, budget, cap, next_pos, n_sink + 1 if hh == 0 else None)
        init = c.snapshot()
        tr = guarded_trajectory(w, 0, hh, budget, 2, cap=cap, t0=next_pos, cache=c,
                                params=params_for(w, budget, hh),
                                min_margin_rel=-1.0 if kind == "pk" and hh == 0 else 1e-4)
        samples.append(Sample(hh, budget, init, tr.ks, tr.vs, tr.evicted, tr.cache.snapshot(),
                              int(tr.attempts.sum())))
    if kind == "kf":
        assert samples[0].evicted[0] == n_sink + 1            # a move of ~12k rows
    L, ev, _ = run_layer(w, 0, budget, 2, samples, budget, next_pos, dev, bh=bh)
    _assert_parity(L, ev, samples, next_pos)


@pytest.mark.parametrize("kind", ["kf", "pk"])
def test_single_evictable_slot(dev, kind):
    """budget = n_sink + 1: one non-sink row competes with the incoming one."""
    w = synth.Workload(f"slot1{kind}", 1, 1, 8, 128, 300, 0, 5, 4,
                       "keyformer" if kind == "kf" else "pyramid",
                       0.5 if kind == "kf" else 0.0, 1.5 if kind == "kf" else 0.0,
                       100 if kind == "kf" else 0)
    T = 300
    _say(f"[slot1] kind={kind} budget=5 n_sink=4 T={T}")
    samples = oracle_samples(w, 0, range(w.bh), w.budget, T, w.budget + 1, workers=1)
    L, ev, _ = run_layer(w, 0, w.budget, T, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)


# ---------------------------------------------------------------------------
# whole trajectories through the prompt -> decode boundary
# ---------------------------------------------------------------------------

def test_full_trajectory_llama_keyformer(dev):
    """Llama-3.2-3B-shaped Keyformer: the full 2048 + 1024 tokens, every cache
    of one layer."""
    w = synth.WORKLOADS[1]
    _say(f"[full-traj] {w.name} layer 11 bh={w.bh} T={w.tokens}")
    samples = oracle_samples(w, 11, range(w.bh), w.budget, w.tokens, w.budget + 1)
    L, ev, ctr = run_layer(w, 11, w.budget, w.tokens, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)
    assert (ctr.n_kept, ctr.next_pos) == (w.budget, w.tokens)


@pytest.mark.parametrize("beta,layer", [(2.0, 3), (1.0, 20)])
def test_full_trajectory_llama_pyramid(dev, beta, layer):
    """Llama-3.2-3B-shaped PyramidKV: the full 3072 tokens at one layer's budget."""
    w = synth.Workload(f"pk-beta{beta}", 1, 28, 8, 128, 2048, 1024, 512, 4, "pyramid",
                       beta=beta)
    budget = oracle.pyramid_budgets(w.layers, w.budget, w.n_sink, beta)[layer]
    _say(f"[full-traj] pyramid beta={beta} layer {layer} budget={budget} T={w.tokens}")
    samples = oracle_samples(w, layer, range(w.bh), budget, w.tokens, budget + 1)
    L, ev, _ = run_layer(w, layer, budget, w.tokens, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)


def test_full_trajectory_8b_late_riser(dev):
    """8B-shaped late-riser Keyformer: 4096 + 512 tokens through one full
    256-cache layer launch, four caches checked."""
    w = synth.WORKLOADS[3]
    hhs = [0, 99, 200, 255]
    _say(f"[full-traj] {w.name} layer 7 bh={w.bh} sampled={hhs} T={w.tokens}")
    samples = oracle_samples(w, 7, hhs, w.budget, w.tokens, w.budget + 1)
    L, ev, _ = run_layer(w, 7, w.budget, w.tokens, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)
    moved = [(ev[w.budget:, s.hh] < w.budget).mean() for s in samples]
    assert max(moved) > 0.02                               # interior evictions happened



# ---------------------------------------------------------------------------
# multi-token calls: S tokens per launch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["kf", "pk"])
@pytest.mark.parametrize("d,S", [(128, 7), (64, 64), (128, 1)])
def test_multi_token_equals_single_calls(dev, kind, d, S):
    """keyformer_step_tokens / pyramid_step_tokens of S tokens give the same
    bits as S single-token calls, across the budget boundary and with interior
    evictions."""
    import kv_cache_eviction_step_amd as kve
    kf = kind == "kf"
    bh, budget, cap, T = 12, 48, 53, 200
    _say(f"[tokens==single] kind={kind} d={d} S={S} T={T}")
    w = synth.Workload("mt", 1, 1, 1, d, T, 0, budget, 4, "keyformer" if kf else "pyramid",
                       1.0 if kf else 0.0, 2.0 if kf else 0.0, 80 if kf else 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    nk, nv = synth.bulk_kv_torch(w, 0, T, bh, gen, dev)
    A = kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=3)
    B = kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=3)
    ca, cb = kve.Counters(0, 0, 0), kve.Counters(0, 0, 0)
    eva = torch.empty((T, bh), dtype=torch.int32, device=dev)
    evb = torch.empty((T, bh), dtype=torch.int32, device=dev)
    for t in range(T):
        if kf:
            kve.keyformer_step(A, nk[t], nv[t], ca, budget, 4, 1.0, 2.0, 80, 1e4, 5, eva[t])
        else:
            kve.pyramid_step(A, nk[t], nv[t], ca, budget, 4, 1e4, eva[t])
    for t0 in range(0, T, S):
        t1 = min(T, t0 + S)
        if kf:
            kve.keyformer_step_tokens(B, nk[t0:t1], nv[t0:t1], cb, budget, 4, 1.0, 2.0, 80, 1e4, 5,
                                      evb[t0:t1])
        else:
            kve.pyramid_step_tokens(B, nk[t0:t1], nv[t0:t1], cb, budget, 4, 1e4, evb[t0:t1])
    torch.cuda.synchronize()
    assert (ca.n_kept, ca.next_pos, ca.pos) == (cb.n_kept, cb.next_pos, cb.pos)
    assert torch.equal(eva, evb)
    n = ca.n_kept
    for name in ("k", "v", "scores", "positions") + (("gumbel",) if kf else ()):
        assert torch.equal(getattr(A, name)[:, :n], getattr(B, name)[:, :n]), name
    if kf:
        assert bool(((eva >= 0) & (eva < budget)).any())


def test_multi_token_full_trajectory_oracle(dev):
    """The Llama-3.2-3B-shaped Keyformer trajectory (3072 tokens) in calls of
    64 tokens, against the oracle for every cache of the layer."""
    import kv_cache_eviction_step_amd as kve
    w = synth.WORKLOADS[1]
    S, T = 64, w.tokens
    _say(f"[tokens-oracle] {w.name} layer 2 S={S} T={T}")
    samples = oracle_samples(w, 2, range(w.bh), w.budget, T, w.budget + 1)
    L = kve.Layer.empty(w.bh, w.budget + 1, w.d, dev)
    nk = torch.stack([torch.from_numpy(s.ks.view(np.float16)) for s in samples], 1).to(dev)
    nv = torch.stack([torch.from_numpy(s.vs.view(np.float16)) for s in samples], 1).to(dev)
    ev = torch.full((T, w.bh), -7, dtype=torch.int32, device=dev)
    ctr = kve.Counters(0, 0, 0)
    prm = params_for(w, w.budget, 0)
    for t0 in range(0, T, S):
        kve.keyformer_step_tokens(L, nk[t0:t0 + S].contiguous(), nv[t0:t0 + S].contiguous(), ctr,
                                  w.budget, w.n_sink, prm.tau_init, prm.tau_end,
                                  prm.anneal_steps, w.rope_base, w.gumbel_seed, ev[t0:t0 + S])
    torch.cuda.synchronize()
    evh = ev.cpu().numpy()
    _assert_parity(L, evh, samples, 0)
    # return_indices from the GPU's eviction log name the oracle's kept tokens
    for s in samples:
        assert kve.kept_indices(0, evh[:, s.hh]) == list(s.final["tid"])
    k, v = L.get_kv(ctr.n_kept)
    assert tuple(k.shape) == (w.bh, w.budget, w.d) and k.data_ptr() == L.k.data_ptr()


@pytest.mark.parametrize("kind", ["kf", "pk"])
@pytest.mark.parametrize("d,S", [(128, 7), (64, 64), (128, 128)])
def test_layers_tokens_equals_single_calls(dev, kind, d, S):
    """keyformer_step_layers_tokens / pyramid_step_layers_tokens over layers of
    different sizes, budgets and Gumbel streams give the same bits as one
    single-token call per layer and token; the layers cross their budgets at
    different tokens of one call."""
    import kv_cache_eviction_step_amd as kve
    kf = kind == "kf"
    shapes = [(5, 48, 53, 0), (12, 20, 21, 7), (9, 33, 40, 100)]   # bh, budget, cap, hh_base
    T = 180
    _say(f"[layers*tokens==single] kind={kind} d={d} S={S} T={T}")
    w = synth.Workload("lt", 1, 3, 1, d, T, 0, 48, 4, "keyformer" if kf else "pyramid",
                       1.0 if kf else 0.0, 2.0 if kf else 0.0, 80 if kf else 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(23)
    nks, nvs, As, Bs, evas, evbs, cas = [], [], [], [], [], [], []
    for bh, budget, cap, hb in shapes:
        k, v = synth.bulk_kv_torch(w, 0, T, bh, gen, dev)
        nks.append(k)
        nvs.append(v)
        As.append(kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=hb))
        Bs.append(kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=hb))
        evas.append(torch.empty((T, bh), dtype=torch.int32, device=dev))
        evbs.append(torch.full((T, bh), -9, dtype=torch.int32, device=dev))
        cas.append(kve.Counters(0, 0, 0))
    budgets = [s[1] for s in shapes]
    for t in range(T):
        for l in range(len(shapes)):
            if kf:
                kve.keyformer_step(As[l], nks[l][t], nvs[l][t], cas[l], budgets[l], 4, 1.0, 2.0,
                                   80, 1e4, 5, evas[l][t])
            else:
                kve.pyramid_step(As[l], nks[l][t], nvs[l][t], cas[l], budgets[l], 4, 1e4,
                                 evas[l][t])
    batch = kve.LayerBatch(Bs, budgets)
    for t0 in range(0, T, S):
        t1 = min(T, t0 + S)
        ks = [x[t0:t1] for x in nks]
        vs = [x[t0:t1] for x in nvs]
        es = [x[t0:t1] for x in evbs]
        if kf:
            kve.keyformer_step_layers_tokens(batch, ks, vs, 4, 1.0, 2.0, 80, 1e4, 5, es)
        else:
            kve.pyramid_step_layers_tokens(batch, ks, vs, 4, 1e4, es)
    torch.cuda.synchronize()
    for l in range(len(shapes)):
        cb = batch.ctrs[l]
        assert (cas[l].n_kept, cas[l].next_pos, cas[l].pos) == (cb.n_kept, cb.next_pos, cb.pos)
        assert torch.equal(evas[l], evbs[l]), l
        n = cas[l].n_kept
        for name in ("k", "v", "scores", "positions") + (("gumbel",) if kf else ()):
            assert torch.equal(getattr(As[l], name)[:, :n], getattr(Bs[l], name)[:, :n]), \
                (l, name)


@pytest.mark.parametrize("wi,layers", [(2, [0, 14, 27]), (1, [2, 20])],
                         ids=["pyramid-beta2", "keyformer"])
def test_layers_tokens_full_trajectory_oracle(dev, wi, layers):
    """Llama-3.2-3B-shaped layers (PyramidKV: budgets from the top, middle and
    bottom of the schedule; Keyformer: two layers) stepped together through
    the full 3072 tokens in calls of 64 tokens, against the oracle for every
    cache."""
    import kv_cache_eviction_step_amd as kve
    w = synth.WORKLOADS[wi]
    kf = w.kind == "keyformer"
    S, T = 64, w.tokens
    budgets = [w.budgets(oracle.pyramid_budgets)[l] for l in layers]
    _say(f"[layers*tokens-oracle] {w.name} layers={layers} budgets={budgets} S={S} T={T}")
    samples = [oracle_samples(w, l, range(w.bh), b, T, b + 1) for l, b in zip(layers, budgets)]
    Ls = [kve.Layer.empty(w.bh, b + 1, w.d, dev, gumbel=kf) for b in budgets]
    nk = [torch.stack([torch.from_numpy(s.ks.view(np.float16)) for s in ss], 1).to(dev)
          for ss in samples]
    nv = [torch.stack([torch.from_numpy(s.vs.view(np.float16)) for s in ss], 1).to(dev)
          for ss in samples]
    ev = torch.full((len(layers), T, w.bh), -7, dtype=torch.int32, device=dev)
    batch = kve.LayerBatch(Ls, budgets)
    prm = params_for(w, budgets[0], 0)
    for t0 in range(0, T, S):
        ks = [x[t0:t0 + S] for x in nk]
        vs = [x[t0:t0 + S] for x in nv]
        es = [ev[i, t0:t0 + S] for i in range(len(layers))]
        if kf:
            kve.keyformer_step_layers_tokens(batch, ks, vs, w.n_sink, prm.tau_init, prm.tau_end,
                                             prm.anneal_steps, w.rope_base, w.gumbel_seed, es)
        else:
            kve.pyramid_step_layers_tokens(batch, ks, vs, w.n_sink, w.rope_base, es)
    torch.cuda.synchronize()
    evh = ev.cpu().numpy()
    for i in range(len(layers)):
        _assert_parity(Ls[i], evh[i], samples[i], 0)
        assert batch.ctrs[i].n_kept == budgets[i]



@pytest.mark.parametrize("wi,beta", [(1, None), (2, None), (2, 1.0)],
                         ids=["keyformer", "pyramid-beta2", "pyramid-beta1"])
def test_every_cache_every_layer_llama_shapes(dev, wi, beta):
    """The Llama-3.2-3B-shaped workloads in full: all 28 layers x 8 caches
    (224 caches) through the whole 2048 + 1024-token stream, all layers in one
    launch per 64 tokens, every cache against the oracle.  PyramidKV runs at
    beta 2 (budgets 1019 ... 5) and at beta 1 (every layer 512)."""
    import dataclasses
    import kv_cache_eviction_step_amd as kve
    w = synth.WORKLOADS[wi]
    if beta is not None:
        w = dataclasses.replace(w, name=f"{w.name}-beta{beta:g}", beta=beta)
    kf = w.kind == "keyformer"
    S, T = 64, w.tokens
    budgets = w.budgets(oracle.pyramid_budgets)
    _say(f"[every cache] {w.name} layers={w.layers} bh={w.bh} budgets={budgets[0]}..{budgets[-1]} "
         f"T={T}: oracle")
    picks = {l: list(range(w.bh)) for l in range(w.layers)}
    samples = oracle_samples_layers(w, picks, budgets, T, init_n=False)
    _say(f"[every cache] {w.name}: GPU")
    Ls = [kve.Layer.empty(w.bh, b + 1, w.d, dev, gumbel=kf) for b in budgets]
    nk = [torch.stack([torch.from_numpy(s.ks.view(np.float16)) for s in samples[l]], 1).to(dev)
          for l in range(w.layers)]
    nv = [torch.stack([torch.from_numpy(s.vs.view(np.float16)) for s in samples[l]], 1).to(dev)
          for l in range(w.layers)]
    ev = torch.full((w.layers, T, w.bh), -7, dtype=torch.int32, device=dev)
    batch = kve.LayerBatch(Ls, budgets)
    prm = params_for(w, budgets[0], 0)
    for t0 in range(0, T, S):
        ks = [x[t0:t0 + S] for x in nk]
        vs = [x[t0:t0 + S] for x in nv]
        es = [ev[l, t0:t0 + S] for l in range(w.layers)]
        if kf:
            kve.keyformer_step_layers_tokens(batch, ks, vs, w.n_sink, prm.tau_init, prm.tau_end,
                                             prm.anneal_steps, w.rope_base, w.gumbel_seed, es)
        else:
            kve.pyramid_step_layers_tokens(batch, ks, vs, w.n_sink, w.rope_base, es)
    torch.cuda.synchronize()
    evh = ev.cpu().numpy()
    for l in range(w.layers):
        _assert_parity(Ls[l], evh[l], samples[l], 0)
        assert batch.ctrs[l].n_kept == budgets[l]


# ---------------------------------------------------------------------------
# the general entry point: recent window and TOVA-adapted scoring
# ---------------------------------------------------------------------------

def _wl(name, kind, d, prompt, decode, budget, recent, batch=1, heads=8, tau=(0.0, 0.0, 0)):
    return synth.Workload(name, batch, 1, heads, d, prompt, decode, budget, 4, kind, *tau,
                          recent=recent)


POLICY_TRAJECTORIES = [
    _wl("kf-recent4", "keyformer", 64, 64, 64, 32, 4, tau=(1.0, 2.0, 64)),
    _wl("h2o-recent1", "pyramid", 64, 64, 64, 32, 1),
    _wl("tova", "tova", 64, 64, 64, 32, 0),
    _wl("tova-recent8", "tova", 128, 64, 64, 32, 8),
    _wl("llama-kf-recent32", "keyformer", 128, 2048, 1024, 512, 32, tau=(1.0, 2.0, 1024)),
    _wl("llama-tova-recent16", "tova", 128, 600, 400, 512, 16),
]


@pytest.mark.parametrize("w", POLICY_TRAJECTORIES, ids=lambda w: w.name)
def test_policy_full_trajectory_oracle(dev, w):
    """kve_step with a recent window and/or TOVA scoring: every cache of one
    layer through the whole token stream, against the oracle."""
    T = w.tokens
    _say(f"[policy-traj] {w.name} kind={w.kind} recent={w.recent} bh={w.bh} T={T}")
    samples = oracle_samples(w, 1, range(w.bh), w.budget, T, w.budget + 1)
    L, ev, ctr = run_layer(w, 1, w.budget, T, samples, None, 0, dev)
    _assert_parity(L, ev, samples, 0)
    assert (ctr.n_kept, ctr.next_pos) == (w.budget, T)
    late = ev[w.budget:]
    if w.recent > 0:                       # the window makes every eviction interior
        assert bool((late < w.budget - w.recent + 1).all()) and bool((late >= 4).all())
    elif w.kind == "tova":                 # no window: the newest row always goes
        assert bool((late == w.budget).all())


def test_policy_full_size_sampled_late_riser(dev):
    """The 8B late-riser launch (256 caches, budget 1024) under Keyformer with a
    64-row window, from a steady state, four caches checked."""
    base = synth.WORKLOADS[3]
    w = synth.Workload("8b-late-riser-recent64", base.batch, base.layers, base.kv_heads, base.d,
                       base.prompt, base.decode, base.budget, base.n_sink, base.kind,
                       base.tau_init, base.tau_end, base.anneal_steps,
                       late_riser=base.late_riser, recent=64)
    T, next_pos = 40, w.prompt
    hhs = [0, 77, 200, 255]
    _say(f"[policy-full] {w.name} bh={w.bh} sampled={hhs} T={T}")
    samples = oracle_samples(w, 5, hhs, w.budget, T, w.budget + 1, init_n=w.budget,
                             next_pos=next_pos)
    L, ev, _ = run_layer(w, 5, w.budget, T, samples, w.budget, next_pos, dev)
    _assert_parity(L, ev, samples, next_pos)
    assert bool((ev <= w.budget - 64).all())


@pytest.mark.parametrize("kind,recent", [("keyformer", 3), ("tova", 5), ("tova", 0),
                                         ("pyramid", 2)])
@pytest.mark.parametrize("S", [1, 9])
def test_policy_layers_tokens_equals_single(dev, kind, recent, S):
    """kve_step over three layers and S tokens per call gives the same bits as
    kve_step one layer and one token at a time."""
    import kv_cache_eviction_step_amd as kve
    kf = kind == "keyformer"
    shapes = [(6, 24, 25, 0), (3, 12, 20, 9), (10, 40, 41, 50)]   # bh, budget, cap, hh_base
    T, d = 90, 64
    _say(f"[policy layers*tokens==single] kind={kind} recent={recent} S={S} T={T}")
    w = _wl("pol", kind, d, T, 0, 24, recent, tau=(1.0, 2.0, 40) if kf else (0.0, 0.0, 0))
    pol = policy_for(w)
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    nks, nvs, As, Bs, evas, evbs = [], [], [], [], [], []
    for bh, budget, cap, hb in shapes:
        k, v = synth.bulk_kv_torch(w, 0, T, bh, gen, dev)
        nks.append(k)
        nvs.append(v)
        As.append(kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=hb))
        Bs.append(kve.Layer.empty(bh, cap, d, dev, gumbel=kf, hh_base=hb))
        evas.append(torch.empty((T, bh), dtype=torch.int32, device=dev))
        evbs.append(torch.full((T, bh), -9, dtype=torch.int32, device=dev))
    budgets = [x[1] for x in shapes]
    singles = [kve.LayerBatch([As[l]], [budgets[l]]) for l in range(3)]
    for t in range(T):
        for l in range(3):
            kve.step(singles[l], [nks[l][t]], [nvs[l][t]], pol, [evas[l][t]])
    batch = kve.LayerBatch(Bs, budgets)
    for t0 in range(0, T, S):
        t1 = min(T, t0 + S)
        kve.step(batch, [x[t0:t1] for x in nks], [x[t0:t1] for x in nvs], pol,
                 [x[t0:t1] for x in evbs], n_tokens=t1 - t0)
    torch.cuda.synchronize()
    for l in range(3):
        a, b = singles[l].ctrs[0], batch.ctrs[l]
        assert (a.n_kept, a.next_pos, a.pos) == (b.n_kept, b.next_pos, b.pos)
        assert torch.equal(evas[l], evbs[l]), l
        n = a.n_kept
        for name in ("k", "v", "scores", "positions") + (("gumbel",) if kf else ()):
            assert torch.equal(getattr(As[l], name)[:, :n], getattr(Bs[l], name)[:, :n]), \
                (l, name)


@pytest.mark.parametrize("kind,d,n,recent,bh,sampled", [
    ("tova", 128, 1500, 16, 6, None),              # 8 score slots per thread; a long in-place move
    ("pyramid", 64, 5000, 8, 3, None),             # 24 slots: the weights go through LDS
    ("tova", 128, 700, 200, 300, [0, 37, 150, 299]),   # 300 caches: moves handed over (workspace)
])
def test_exact_tie_goes_to_lowest_candidate(dev, kind, d, n, recent, bh, sampled):
    """Every stored key the same vector: every stored row gets the same softmax
    weight, exactly 1/n on both sides, so every candidate row has the same
    eviction key (TOVA: the weight; H2O: equal old scores plus the weight).
    With a window the new row is no candidate, and the lowest candidate row,
    n_sink, must go in every cache, whichever wave and score slot holds it.
    Sampled caches are compared with the oracle in full."""
    import kv_cache_eviction_step_amd as kve
    n_sink, budget, next_pos, cap = 4, n, 10_000, n + 1
    w = _wl(f"tie-{kind}", kind, d, 64, 0, budget, recent, heads=bh)
    hhs = list(range(bh)) if sampled is None else sampled
    _say(f"[exact tie] kind={kind} d={d} n={n} recent={recent} bh={bh} sampled={hhs}")
    L = kve.Layer.empty(bh, cap, d, dev, gumbel=False)
    nk = torch.empty((bh, d), dtype=torch.float16)
    nv = torch.empty((bh, d), dtype=torch.float16)
    samples = []
    for hh in range(bh):
        c = random_state(w, 0, hh, n, cap, next_pos, seed=hh + 3)
        c.k[:n] = c.k[0]
        c.s[:n] = 1.5
        init = c.snapshot()
        load_state_into(L, hh, init)
        if hh in hhs:
            tr = guarded_trajectory(w, 0, hh, budget, 1, cap=cap, t0=next_pos, cache=c,
                                    params=params_for(w, budget, hh), min_margin_rel=-1.0)
            assert tr.evicted[0] == n_sink
            samples.append(Sample(hh, budget, init, tr.ks, tr.vs, tr.evicted,
                                  tr.cache.snapshot(), int(tr.attempts.sum())))
            k1, v1 = tr.ks[0], tr.vs[0]
        else:
            k1, v1 = (x[0] for x in synth.token_kv(w, 0, hh, [next_pos]))
        nk[hh] = torch.from_numpy(k1.view(np.float16))
        nv[hh] = torch.from_numpy(v1.view(np.float16))
    ev = torch.full((bh,), -7, dtype=torch.int32, device=dev)
    batch = kve.LayerBatch([L], [budget], [kve.Counters(n, next_pos, next_pos)])
    kve.step(batch, [nk.to(dev)], [nv.to(dev)], policy_for(w), [ev],
             workspace=kve.workspace(bh, budget, d, dev))
    torch.cuda.synchronize()
    evn = ev.cpu().numpy()[None, :]
    assert bool((evn == n_sink).all()), np.unique(evn)
    _assert_parity(L, evn, samples, next_pos)


def test_policy_plain_equals_named_entry_points(dev):
    """kve_step with recent 0 and the cumulative score is keyformer_step /
    pyramid_step, bit for bit."""
    import kv_cache_eviction_step_amd as kve
    T, bh, d, budget = 70, 7, 128, 30
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    for kind in ("keyformer", "pyramid"):
        kf = kind == "keyformer"
        w = _wl("eq", kind, d, T, 0, budget, 0, tau=(1.0, 2.0, 32) if kf else (0.0, 0.0, 0))
        nk, nv = synth.bulk_kv_torch(w, 0, T, bh, gen, dev)
        A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=kf)
        B = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=kf)
        ca = kve.Counters(0, 0, 0)
        batch = kve.LayerBatch([B], [budget])
        pol = policy_for(w)
        for t in range(T):
            if kf:
                kve.keyformer_step(A, nk[t], nv[t], ca, budget, 4, 1.0, 2.0, 32, 1e4, 0)
            else:
                kve.pyramid_step(A, nk[t], nv[t], ca, budget, 4, 1e4)
            kve.step(batch, [nk[t]], [nv[t]], pol)
        torch.cuda.synchronize()
        for name in ("k", "v", "scores", "positions") + (("gumbel",) if kf else ()):
            assert torch.equal(getattr(A, name)[:, :budget], getattr(B, name)[:, :budget]), name


def _layers_tokens_equal_single_calls(dev, kind, shapes, T, S, seed, d=128, ws=False):
    """Layers (bh, budget, hh_base) from full synthetic states stepped T
    tokens, S per call of the batched form, give the same bits as single-token
    calls per layer.  ws: the batched form is kve_step_ws with a workspace."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    kf = kind == "kf"
    pos0 = 9000
    _say(f"[layers*tokens==single] kind={kind} d={d} shapes={shapes} T={T} S={S}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    As, Bs, nks, nvs, evas, evbs = [], [], [], [], [], []
    for bh, budget, hb in shapes:
        w = synth.Workload("lg", 1, 1, bh, d, pos0, T, budget, 4, "keyformer" if kf else "pyramid",
                           1.0 if kf else 0.0, 2.0 if kf else 0.0, 64 if kf else 0)
        A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=kf, hh_base=hb)
        bulk_state(A, budget, w, gen)
        B = kve.Layer(A.k.clone(), A.v.clone(), A.scores.clone(),
                      A.gumbel.clone() if kf else None, A.positions.clone(), hh_base=hb)
        k, v = synth.bulk_kv_torch(w, pos0, T, bh, gen, dev)
        As.append(A); Bs.append(B); nks.append(k); nvs.append(v)
        evas.append(torch.empty((T, bh), dtype=torch.int32, device=dev))
        evbs.append(torch.full((T, bh), -9, dtype=torch.int32, device=dev))
    budgets = [x[1] for x in shapes]
    cas = [kve.Counters(b, pos0, pos0) for b in budgets]
    args = (4, 1.0, 2.0, 64, 1e4, 3) if kf else (4, 1e4)
    for t in range(T):
        for l in range(len(shapes)):
            if kf:
                kve.keyformer_step(As[l], nks[l][t], nvs[l][t], cas[l], budgets[l], *args,
                                   evas[l][t])
            else:
                kve.pyramid_step(As[l], nks[l][t], nvs[l][t], cas[l], budgets[l], *args, evas[l][t])
    batch = kve.LayerBatch(Bs, budgets, [kve.Counters(b, pos0, pos0) for b in budgets])
    wsb = kve.workspace(sum(x[0] for x in shapes), max(budgets), d, dev) if ws else None
    pol = (kve.policy("keyformer", 4, 0, 1.0, 2.0, 64, 1e4, 3) if kf else
           kve.policy("pyramid", 4, rope_base=1e4))
    for t0 in range(0, T, S):
        t1 = min(T, t0 + S)
        ks = [x[t0:t1] for x in nks]
        vs = [x[t0:t1] for x in nvs]
        es = [x[t0:t1] for x in evbs]
        if ws:
            kve.step(batch, ks, vs, pol, es, n_tokens=t1 - t0, workspace=wsb)
        elif kf:
            kve.keyformer_step_layers_tokens(batch, ks, vs, *args, es)
        else:
            kve.pyramid_step_layers_tokens(batch, ks, vs, *args, es)
    torch.cuda.synchronize()
    if ws:
        assert workspace_ready(wsb)                     # ready for the next call
    for l in range(len(shapes)):
        assert torch.equal(evas[l], evbs[l]), l
        n = budgets[l]
        for name in ("k", "v", "scores", "positions") + (("gumbel",) if kf else ()):
            assert torch.equal(getattr(As[l], name)[:, :n], getattr(Bs[l], name)[:, :n]), \
                (l, name)
    if kf:
        assert any(bool(((e >= 0) & (e < b)).any()) for e, b in zip(evas, budgets))


@pytest.mark.parametrize("kind", ["kf", "pk"])
@pytest.mark.parametrize("S,ws", [(1, False), (1, True), (8, False)])
def test_more_layers_than_one_launch_equal_single_calls(dev, kind, S, ws):
    """40 layers in one call are two launches (descriptors of up to 32 layers
    travel with a launch); with one token per call and a workspace the first
    launch holds 256 caches, so Keyformer hands its long moves over, and the
    second (64 caches) does not: the two launches share one workspace.
    Budgets 40 .. 313, Gumbel streams offset per layer."""
    shapes = [(8, 40 + 7 * l, 8 * l) for l in range(40)]
    _layers_tokens_equal_single_calls(dev, kind, shapes, 24, S, 61 + S, ws=ws)


@pytest.mark.parametrize("kind", ["kf", "pk"])
def test_layers_tokens_large_budgets_equal_single_calls(dev, kind):
    """The token loop with 8 and 24 score slots per thread (budgets 2000 and
    5000); the five caches hold 4 MB of keys, which the launch reads cached."""
    _layers_tokens_equal_single_calls(dev, kind, [(3, 2000, 0), (2, 5000, 11)], 40, 16, 57)


@pytest.mark.parametrize("kind", ["kf", "pk"])
@pytest.mark.parametrize("d", [128, 64])
def test_layers_tokens_wide_workgroups_equal_single_calls(dev, kind, d):
    """600 caches of 600 and 400 rows: at most 79 MB of keys resident at once,
    so the launch keeps them cached between tokens, and with more workgroups
    than the GPU holds at once it runs 1024-thread workgroups."""
    _layers_tokens_equal_single_calls(dev, kind, [(300, 600, 0), (300, 400, 300)], 24, 12, 59,
                                      d=d)


@pytest.mark.parametrize("kind", ["kf", "pk"])
def test_layers_tokens_wide_largest_slots_equal_single_calls(dev, kind):
    """512 caches of 9000 rows in a 4-token call: 1024-thread workgroups with
    their largest score-slot count (12 per thread) against single-token calls
    (512 threads, 24 slots per thread)."""
    _layers_tokens_equal_single_calls(dev, kind, [(256, 9000, 0), (256, 8500, 256)], 8, 4, 60)


@pytest.mark.parametrize("kind", ["kf", "pk"])
def test_layers_tokens_streamed_keys_equal_single_calls(dev, kind):
    """512 caches of 1536 and 2048 rows, all resident at once: 235 MB of
    keys (268 MB by the launch's bound, 512 caches x 2048 rows), more than
    the 192 MB a launch keeps cached between tokens, so the token loop streams
    them non-temporally (and, filling the GPU, runs 1024-thread workgroups)."""
    _layers_tokens_equal_single_calls(dev, kind, [(256, 2048, 0), (256, 1536, 256)], 24, 12, 58)


@pytest.mark.parametrize("kind", ["kf", "pk"])
@pytest.mark.parametrize("budget", [1000, 3000])
@pytest.mark.parametrize("S", [1, 16])
@pytest.mark.parametrize("d", [128, 64])
def test_launch_size_paths_agree(dev, kind, budget, S, d):
    """A launch's grid size picks code paths that must not change any bit:
    320 caches in one launch (more workgroups than compute units: state loads
    after the key pass; single tokens go through kve_step_ws, so Keyformer
    hands moves over 128 rows to the move kernel; at budget 3000 with S = 16,
    keys streamed) against the same caches in two launches of 160 (state
    loads before the key pass; every cache compacted by its own workgroup;
    keys cached between tokens), from a full synthetic state."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    kf = kind == "kf"
    bh, half, T, pos0 = 320, 160, 32, 7000
    _say(f"[grid paths] kind={kind} d={d} budget={budget} S={S} bh={bh} vs 2x{half} T={T}")
    w = synth.Workload("grid", 1, 1, bh, d, pos0, T, budget, 4, "keyformer" if kf else "pyramid",
                       1.0 if kf else 0.0, 2.0 if kf else 0.0, 64 if kf else 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(61 + budget + S)
    A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=kf)
    bulk_state(A, budget, w, gen)
    parts = []
    for i in range(2):
        sl = slice(i * half, (i + 1) * half)
        parts.append(kve.Layer(A.k[sl].clone(), A.v[sl].clone(), A.scores[sl].clone(),
                               A.gumbel[sl].clone() if kf else None, A.positions[sl].clone(),
                               hh_base=i * half))
    nk, nv = synth.bulk_kv_torch(w, pos0, T, bh, gen, dev)
    ev_a = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    ev_p = [torch.full((T, half), -9, dtype=torch.int32, device=dev) for _ in range(2)]
    args = (4, 1.0, 2.0, 64, 1e4, 5) if kf else (4, 1e4)
    pol = (kve.policy("keyformer", 4, 0, 1.0, 2.0, 64, 1e4, 5) if kf else
           kve.policy("pyramid", 4, rope_base=1e4))
    wsa = kve.workspace(bh, budget, d, dev)

    def run(L, ks, vs, ev, c, ws=None):
        b = kve.LayerBatch([L], [budget], [c]) if ws is not None else None
        for t0 in range(0, T, S):
            if S == 1 and ws is not None:
                kve.step(b, [ks[t0]], [vs[t0]], pol, [ev[t0]], workspace=ws)
            elif S == 1 and kf:
                kve.keyformer_step(L, ks[t0], vs[t0], c, budget, *args, ev[t0])
            elif S == 1:
                kve.pyramid_step(L, ks[t0], vs[t0], c, budget, *args, ev[t0])
            elif kf:
                kve.keyformer_step_tokens(L, ks[t0:t0 + S], vs[t0:t0 + S], c, budget, *args,
                                          ev[t0:t0 + S])
            else:
                kve.pyramid_step_tokens(L, ks[t0:t0 + S], vs[t0:t0 + S], c, budget, *args,
                                        ev[t0:t0 + S])

    run(A, nk, nv, ev_a, kve.Counters(budget, pos0, pos0), wsa if S == 1 else None)
    for i in range(2):
        sl = slice(i * half, (i + 1) * half)
        run(parts[i], nk[:, sl].contiguous(), nv[:, sl].contiguous(), ev_p[i],
            kve.Counters(budget, pos0, pos0))
    torch.cuda.synchronize()
    assert workspace_ready(wsa)
    assert torch.equal(ev_a, torch.cat(ev_p, dim=1))
    for name in ("k", "v", "scores", "positions") + (("gumbel",) if kf else ()):
        joined = torch.cat([getattr(p, name) for p in parts])
        assert torch.equal(getattr(A, name)[:, :budget], joined[:, :budget]), name
    if kf:
        assert bool(((ev_a >= 0) & (ev_a < budget)).any())     # interior evictions happened


@pytest.mark.parametrize("recent", [8, 200])
def test_tova_handoff_equals_own_moves(dev, recent):
    """TOVA scoring with a window (without one the incoming row, at score 0,
    is always the one evicted) on 320 caches, one token per kve_step_ws call:
    long moves go to the move kernel; two kve_step calls of 160 caches compact
    every cache in its own workgroup.  Same bits."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    bh, half, d, budget, T, pos0 = 320, 160, 128, 1500, 24, 5000
    _say(f"[tova handoff] recent={recent} bh={bh} vs 2x{half} budget={budget} T={T}")
    w = synth.Workload("tv", 1, 1, bh, d, pos0, T, budget, 4, "tova", recent=recent)
    gen = torch.Generator(device=dev)
    gen.manual_seed(71 + recent)
    A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=False)
    bulk_state(A, budget, w, gen)
    parts = []
    for i in range(2):
        sl = slice(i * half, (i + 1) * half)
        parts.append(kve.Layer(A.k[sl].clone(), A.v[sl].clone(), A.scores[sl].clone(), None,
                               A.positions[sl].clone(), hh_base=i * half))
    nk, nv = synth.bulk_kv_torch(w, pos0, T, bh, gen, dev)
    pol = kve.policy("tova", n_sink=4, recent=recent, rope_base=1e4)
    ev_a = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    ev_p = [torch.full((T, half), -9, dtype=torch.int32, device=dev) for _ in range(2)]
    ba = kve.LayerBatch([A], [budget], [kve.Counters(budget, pos0, pos0)])
    bp = [kve.LayerBatch([parts[i]], [budget], [kve.Counters(budget, pos0, pos0)])
          for i in range(2)]
    ws = kve.workspace(bh, budget, d, dev)
    for t in range(T):
        kve.step(ba, [nk[t]], [nv[t]], pol, [ev_a[t]], workspace=ws)
        for i in range(2):
            sl = slice(i * half, (i + 1) * half)
            kve.step(bp[i], [nk[t, sl].contiguous()], [nv[t, sl].contiguous()], pol, [ev_p[i][t]])
    torch.cuda.synchronize()
    assert workspace_ready(ws)
    assert torch.equal(ev_a, torch.cat(ev_p, dim=1))
    for name in ("k", "v", "scores", "positions"):
        joined = torch.cat([getattr(p, name) for p in parts])
        assert torch.equal(getattr(A, name)[:, :budget], joined[:, :budget]), name
    moved = torch.where((ev_a >= 0) & (ev_a < budget), budget - 1 - ev_a, 0)
    assert int(moved.max()) > 128                      # some move was handed over


def test_handoff_queue_longer_than_grid_equals_own_moves(dev):
    """A queue of handed-over chunks longer than the move kernel's grid (so
    its workgroups take chunks in turn, each loading its next chunk's item
    while the current one moves): TOVA scoring with a 200-row window on 512
    caches of 4096 rows, one token per kve_step_ws call, against the same
    caches compacted in place by kve_step.  Same bits on every cache."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    bh, d, budget, T, pos0, recent = 512, 128, 4096, 4, 9000, 200
    grid = 1024                                        # the move kernel's largest grid
    _say(f"[handoff long queue] bh={bh} budget={budget} T={T} recent={recent}")
    w = synth.Workload("tvq", 1, 1, bh, d, pos0, T, budget, 4, "tova", recent=recent)
    gen = torch.Generator(device=dev)
    gen.manual_seed(131)
    A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=False)
    bulk_state(A, budget, w, gen)
    B = kve.Layer(A.k.clone(), A.v.clone(), A.scores.clone(), None, A.positions.clone())
    nk, nv = synth.bulk_kv_torch(w, pos0, T, bh, gen, dev)
    pol = kve.policy("tova", n_sink=4, recent=recent, rope_base=1e4)
    ev_a = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    ev_b = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    ba = kve.LayerBatch([A], [budget], [kve.Counters(budget, pos0, pos0)])
    bb = kve.LayerBatch([B], [budget], [kve.Counters(budget, pos0, pos0)])
    ws = kve.workspace(bh, budget, d, dev)
    for t in range(T):
        kve.step(ba, [nk[t]], [nv[t]], pol, [ev_a[t]], workspace=ws)
        kve.step(bb, [nk[t]], [nv[t]], pol, [ev_b[t]])
    torch.cuda.synchronize()
    assert workspace_ready(ws)
    assert torch.equal(ev_a, ev_b)
    for name in ("k", "v", "scores", "positions"):
        assert torch.equal(getattr(A, name)[:, :budget], getattr(B, name)[:, :budget]), name
    # every token queued more chunks than the move kernel has workgroups
    e = ev_a.to(torch.int64).cpu()
    rows = budget - 1 - e
    handed = (e >= 0) & (e < budget - 1) & (rows > 128)
    chunks = torch.where(handed, (rows + 63) // 64, 0).sum(dim=1)
    assert int(chunks.min()) > grid, chunks.tolist()


@pytest.mark.parametrize("d", [128, 64])
def test_handoff_edges_against_oracle(dev, d):
    """One single-token Keyformer kve_step_ws launch of 320 caches (moves over
    128 rows go to the move kernel), sampled caches steered to the edges of the handoff
    and checked against the oracle bit for bit: row 0 with no sinks (999 rows
    move: every one of the 16 scratch chunk slots is used), 998 rows, exactly
    129 rows (the shortest move handed over, a last chunk of one row), exactly
    128 rows (kept in place), 193 and 482 rows (ragged last chunks), and the
    newest stored row (nothing moves).  The other caches get random states and
    must evict a valid row."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    bh, budget, n_sink = 320, 1000, 0
    n, cap = budget, budget + 5
    next_pos = 5000 + n
    targets = {0: 0, 37: 1, 101: n - 1 - 129, 150: n - 1 - 128, 203: n - 1 - 193,
               260: n - 1 - 482, 319: n - 1}
    _say(f"[handoff edges] d={d} bh={bh} budget={budget} targets={targets}")
    w = synth.Workload(f"handoff{d}", 40, 1, 8, d, 64, 0, budget, n_sink, "keyformer",
                       1.0, 2.0, 64)
    assert w.bh == bh
    samples = []
    for hh, target in targets.items():
        c = _forced(w, hh, n, cap, next_pos, target)
        init = c.snapshot()
        tr = guarded_trajectory(w, 0, hh, budget, 1, cap=cap, t0=next_pos, cache=c,
                                params=params_for(w, budget, hh))
        assert tr.evicted[0] == target
        samples.append(Sample(hh, budget, init, tr.ks, tr.vs, tr.evicted, tr.cache.snapshot(),
                              int(tr.attempts.sum())))
    gen = torch.Generator(device=dev)
    gen.manual_seed(97 + d)
    L = kve.Layer.empty(bh, cap, d, dev, gumbel=True)
    bulk_state(L, n, w, gen)
    for s in samples:
        load_state_into(L, s.hh, s.init)
    nk, nv = synth.bulk_kv_torch(w, next_pos, 1, bh, gen, dev)
    nk, nv = nk[0].contiguous(), nv[0].contiguous()
    for s in samples:
        nk[s.hh] = torch.from_numpy(s.ks[0].view(np.float16)).to(dev)
        nv[s.hh] = torch.from_numpy(s.vs[0].view(np.float16)).to(dev)
    ev = torch.full((bh,), -7, dtype=torch.int32, device=dev)
    batch = kve.LayerBatch([L], [budget], [kve.Counters(n, next_pos, next_pos)])
    ws = kve.workspace(bh, budget, d, dev)
    kve.step(batch, [nk], [nv], policy_for(w), [ev], workspace=ws)
    torch.cuda.synchronize()
    ctr = batch.ctrs[0]
    assert workspace_ready(ws)
    evn = ev.cpu().numpy()
    _assert_parity(L, evn[None, :], samples, next_pos)
    assert ((evn >= 0) & (evn <= n)).all()
    assert ctr.n_kept == budget

def test_handoff_largest_budget_against_oracle(dev):
    """The largest budget (12288 rows) in a single-token Keyformer kve_step_ws
    launch of 256 caches, which hands long moves over: sampled caches steered to row 0 with
    no sinks (12287 rows move: 192 chunks, every scratch slot of the launch),
    a middle row, and the newest stored row; bit for bit against the oracle."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    bh, budget, n_sink, d = 256, 12288, 0, 128
    n, cap = budget, budget + 1
    next_pos = 20000
    targets = {0: 0, 129: 6001, 255: n - 1}
    _say(f"[handoff max budget] bh={bh} budget={budget} targets={targets}")
    w = synth.Workload("handoffmax", 32, 1, 8, d, 64, 0, budget, n_sink, "keyformer",
                       1.0, 2.0, 64)
    samples = []
    for hh, target in targets.items():
        c = _forced(w, hh, n, cap, next_pos, target)
        init = c.snapshot()
        tr = guarded_trajectory(w, 0, hh, budget, 1, cap=cap, t0=next_pos, cache=c,
                                params=params_for(w, budget, hh))
        assert tr.evicted[0] == target
        samples.append(Sample(hh, budget, init, tr.ks, tr.vs, tr.evicted, tr.cache.snapshot(),
                              int(tr.attempts.sum())))
    gen = torch.Generator(device=dev)
    gen.manual_seed(101)
    L = kve.Layer.empty(bh, cap, d, dev, gumbel=True)
    bulk_state(L, n, w, gen)
    for s in samples:
        load_state_into(L, s.hh, s.init)
    nk, nv = synth.bulk_kv_torch(w, next_pos, 1, bh, gen, dev)
    nk, nv = nk[0].contiguous(), nv[0].contiguous()
    for s in samples:
        nk[s.hh] = torch.from_numpy(s.ks[0].view(np.float16)).to(dev)
        nv[s.hh] = torch.from_numpy(s.vs[0].view(np.float16)).to(dev)
    ev = torch.full((bh,), -7, dtype=torch.int32, device=dev)
    batch = kve.LayerBatch([L], [budget], [kve.Counters(n, next_pos, next_pos)])
    ws = kve.workspace(bh, budget, d, dev)
    kve.step(batch, [nk], [nv], policy_for(w), [ev], workspace=ws)
    torch.cuda.synchronize()
    ctr = batch.ctrs[0]
    assert workspace_ready(ws)
    evn = ev.cpu().numpy()
    _assert_parity(L, evn[None, :], samples, next_pos)
    assert ((evn >= 0) & (evn <= n)).all()

def test_batched_handoff_mixed_budgets_equals_own_moves(dev):
    """TOVA scoring and a 200-row window over two layers of 160 caches with
    budgets 1500 and 700, one token per call: as one kve_step_ws launch (320
    caches: long moves go to the move kernel, the workspace sized by the larger
    budget and shared by both layers) and as one kve_step launch per layer
    (160 caches: every cache compacted by its own workgroup).  Same bits."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    half, d, T, pos0, recent = 160, 128, 16, 6000, 200
    budgets = [1500, 700]
    _say(f"[batched handoff] budgets={budgets} 2x{half} caches T={T}")
    pol = kve.policy("tova", n_sink=4, recent=recent, rope_base=1e4)
    gen = torch.Generator(device=dev)
    gen.manual_seed(113)
    A, B = [], []
    for i, b in enumerate(budgets):
        w = synth.Workload(f"bh{i}", 20, 1, 8, d, pos0, T, b, 4, "tova", recent=recent)
        L = kve.Layer.empty(half, b + 1, d, dev, gumbel=False)
        bulk_state(L, b, w, gen)
        A.append(L)
        B.append(kve.Layer(L.k.clone(), L.v.clone(), L.scores.clone(), None, L.positions.clone()))
    nk = torch.randn(2, T, half, d, generator=gen, device=dev).half()
    nv = torch.randn(2, T, half, d, generator=gen, device=dev).half()
    ev_a = torch.full((2, T, half), -9, dtype=torch.int32, device=dev)
    ev_b = torch.full((2, T, half), -9, dtype=torch.int32, device=dev)
    ba = kve.LayerBatch(A, budgets, [kve.Counters(b, pos0, pos0) for b in budgets])
    bb = [kve.LayerBatch([B[i]], [budgets[i]], [kve.Counters(budgets[i], pos0, pos0)])
          for i in range(2)]
    ws = kve.workspace(2 * half, max(budgets), d, dev)
    for t in range(T):
        kve.step(ba, [nk[0, t], nk[1, t]], [nv[0, t], nv[1, t]], pol, [ev_a[0, t], ev_a[1, t]],
                 workspace=ws)
        for i in range(2):
            kve.step(bb[i], [nk[i, t]], [nv[i, t]], pol, [ev_b[i, t]])
    torch.cuda.synchronize()
    assert workspace_ready(ws)
    assert torch.equal(ev_a, ev_b)
    for i, b in enumerate(budgets):
        for name in ("k", "v", "scores", "positions"):
            assert torch.equal(getattr(A[i], name)[:, :b], getattr(B[i], name)[:, :b]), (i, name)
        moved = torch.where((ev_a[i] >= 0) & (ev_a[i] < b), b - 1 - ev_a[i], 0)
        assert int(moved.max()) > 128                  # some move was handed over

def test_captured_step_replays_match_eager(dev):
    """A Keyformer kve_step_ws call on 320 caches, which hands its long moves
    to the move kernel through the workspace, captured into a graph: the
    captured work itself leaves the workspace ready for the next call (its
    header advances a phase per call), so each replay, from the same restored
    state and with eager work and a synchronisation between replays, gives
    the eager call's bits (and the in-place keyformer_step's)."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    bh, d, budget, pos0 = 320, 128, 1000, 6000
    _say(f"[graph capture] kve_step_ws bh={bh} budget={budget} d={d}")
    w = synth.Workload("graph", 1, 1, bh, d, pos0, 1, budget, 4, "keyformer", 1.0, 2.0, 64)
    gen = torch.Generator(device=dev)
    gen.manual_seed(83)
    S0 = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=True)
    bulk_state(S0, budget, w, gen)
    nk, nv = synth.bulk_kv_torch(w, pos0, 1, bh, gen, dev)
    names = ("k", "v", "scores", "gumbel", "positions")
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 64, 1e4, 5)

    def copy_of(L):
        return kve.Layer(*[getattr(L, x).clone() for x in names])

    def call(L, ev, ws):
        b = kve.LayerBatch([L], [budget], [kve.Counters(budget, pos0, pos0)])
        kve.step(b, [nk[0]], [nv[0]], pol, [ev], workspace=ws)

    P = copy_of(S0)                                   # in place, for reference
    ev_p = torch.full((bh,), -9, dtype=torch.int32, device=dev)
    kve.keyformer_step(P, nk[0], nv[0], kve.Counters(budget, pos0, pos0), budget, 4, 1.0, 2.0,
                       64, 1e4, 5, ev_p)
    E = copy_of(S0)
    ev_e = torch.full((bh,), -9, dtype=torch.int32, device=dev)
    ws = kve.workspace(bh, budget, d, dev)
    call(E, ev_e, ws)
    torch.cuda.synchronize()
    assert int((budget - ev_e)[ev_e >= 0].max()) > 128   # some move was handed over
    assert workspace_ready(ws)                          # ready for the next call
    assert torch.equal(ev_e, ev_p)
    for x in names:
        assert torch.equal(getattr(E, x)[:, :budget], getattr(P, x)[:, :budget]), x

    G = copy_of(S0)
    ev_g = torch.full((bh,), -9, dtype=torch.int32, device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(G, ev_g, ws)
    for replay in range(3):
        for x in names:
            getattr(G, x).copy_(getattr(S0, x))
        ev_g.fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert workspace_ready(ws), replay
        assert torch.equal(ev_g, ev_e), replay
        for x in names:
            assert torch.equal(getattr(G, x)[:, :budget], getattr(E, x)[:, :budget]), (replay, x)


@pytest.mark.parametrize("items", [1, 3, 12])
def test_workspace_too_small_falls_back_in_place(dev, items):
    """kve_step_ws with a workspace of only 1, 3 or 12 items on 320 Keyformer
    caches of 1000 rows: caches whose reservation does not fit compact in
    place, the rest hand their moves over; every call equals the in-place
    keyformer_step bit for bit, and the workspace stays ready for the next."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    bh, d, budget, pos0, T = 320, 128, 1000, 6000, 12
    _say(f"[small workspace] items={items} bh={bh} budget={budget} T={T}")
    w = synth.Workload("small-ws", 1, 1, bh, d, pos0, T, budget, 4, "keyformer", 1.0, 2.0, 64)
    gen = torch.Generator(device=dev)
    gen.manual_seed(131 + items)
    A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=True)
    bulk_state(A, budget, w, gen)
    names = ("k", "v", "scores", "gumbel", "positions")
    B = kve.Layer(*[getattr(A, x).clone() for x in names])
    nk, nv = synth.bulk_kv_torch(w, pos0, T, bh, gen, dev)
    nbytes = 256 + -(-items * 32 // 256) * 256 + items * 4 * d   # kve_workspace_size's layout
    raw = torch.zeros(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + nbytes]
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 64, 1e4, 5)
    ba = kve.LayerBatch([A], [budget], [kve.Counters(budget, pos0, pos0)])
    cb = kve.Counters(budget, pos0, pos0)
    ev_a = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    ev_b = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    for t in range(T):
        kve.step(ba, [nk[t]], [nv[t]], pol, [ev_a[t]], workspace=ws)
        kve.keyformer_step(B, nk[t], nv[t], cb, budget, 4, 1.0, 2.0, 64, 1e4, 5, ev_b[t])
    torch.cuda.synchronize()
    assert workspace_ready(ws)
    assert torch.equal(ev_a, ev_b)
    for x in names:
        assert torch.equal(getattr(A, x)[:, :budget], getattr(B, x)[:, :budget]), x
    long_moves = int(((ev_a >= 0) & (budget - 1 - ev_a > 128)).sum())
    assert long_moves > items                        # some moves could not be handed over


def test_captured_batched_call_replays_match_eager(dev):
    """keyformer_step_layers_tokens over 3 layers and 8 tokens, captured into a
    graph (its descriptors travel by value with the launch) and replayed three
    times from a restored state, with eager work and synchronisations between
    replays: every replay equals the eager call bit for bit."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    d, S, pos0 = 128, 8, 4000
    shapes = [(8, 300, 0), (16, 200, 8), (8, 100, 24)]
    _say(f"[graph capture] keyformer_step_layers_tokens shapes={shapes} S={S}")
    names = ("k", "v", "scores", "gumbel", "positions")
    gen = torch.Generator(device=dev)
    gen.manual_seed(89)
    S0, nks, nvs = [], [], []
    for bh, budget, hb in shapes:
        w = synth.Workload("gc", 1, 1, bh, d, pos0, S, budget, 4, "keyformer", 1.0, 2.0, 64)
        L = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=True, hh_base=hb)
        bulk_state(L, budget, w, gen)
        S0.append(L)
        k, v = synth.bulk_kv_torch(w, pos0, S, bh, gen, dev)
        nks.append(k)
        nvs.append(v)
    budgets = [x[1] for x in shapes]

    def copy_of(L):
        return kve.Layer(*[getattr(L, x).clone() for x in names], hh_base=L.hh_base)

    def batch_of(Ls):
        return kve.LayerBatch(Ls, budgets, [kve.Counters(b, pos0, pos0) for b in budgets])

    args = (4, 1.0, 2.0, 64, 1e4, 3)
    E = [copy_of(L) for L in S0]
    ev_e = [torch.full((S, bh), -9, dtype=torch.int32, device=dev) for bh, _, _ in shapes]
    kve.keyformer_step_layers_tokens(batch_of(E), nks, nvs, *args, ev_e)
    torch.cuda.synchronize()
    G = [copy_of(L) for L in S0]
    ev_g = [torch.full((S, bh), -9, dtype=torch.int32, device=dev) for bh, _, _ in shapes]
    bg = batch_of(G)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kve.keyformer_step_layers_tokens(bg, nks, nvs, *args, ev_g)
    for replay in range(3):
        for Lg, L0 in zip(G, S0):
            for x in names:
                getattr(Lg, x).copy_(getattr(L0, x))
        for e in ev_g:
            e.fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l, (Lg, Le) in enumerate(zip(G, E)):
            assert torch.equal(ev_g[l], ev_e[l]), (replay, l)
            n = budgets[l]
            for x in names:
                assert torch.equal(getattr(Lg, x)[:, :n], getattr(Le, x)[:, :n]), (replay, l, x)

# ---------------------------------------------------------------------------
# the long-context workload's whole run, as the benchmark times it
# ---------------------------------------------------------------------------

def _token_stream(args):
    """The unguarded input stream of one cache (worker process)."""
    w, layer, hh, T = args
    return synth.token_kv(w, layer, hh, np.arange(T))


@pytest.mark.timeout(1200)
def test_whole_run_long_context_every_layer(dev):
    """The long-context PyramidKV workload's whole run: 16384 prompt + 1024
    decode tokens from empty caches through all 32 layers x 512 caches
    (budgets 6144 .. 2048), one pyramid_step launch per layer per token -- the
    benchmark's launch form.  On the way each cache grows through the 2-, 8-
    and 24-slot paths of a launch of more workgroups than compute units, and
    its oldest rows take 17408 score increments.

    One cache per layer, spread over batch and head and so over every budget
    of the taper, runs through the oracle in worker processes while the GPU
    runs; at the end every one of its evicted indices, kept tokens, values,
    keys, positions and scores is compared.  Every other cache is checked by
    what holds at any size at tau 0 ("PyramidKV -- Layer-Adaptive Budget
    Attention-Mass Eviction", How it works; Relationship to H2O): a stored
    row's score is positive by the time the argmin is taken, so each
    over-budget step evicts exactly the incoming row, at index n, and no step
    under the budget evicts; positions stay 0 .. n-1; scores stay finite and
    non-negative.  The margin guard of the sampled caches never redraws here
    (the two smallest keys are the incoming row's 0 and a positive score,
    whose gap passes the relative margin), which the test asserts, since the
    GPU is fed the undrawn stream."""
    import os
    from concurrent.futures import ProcessPoolExecutor
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import _sample_job
    w = synth.WORKLOADS[4]
    budgets = oracle.pyramid_budgets(w.layers, w.budget, w.n_sink, w.beta)
    L, bh, d, T = w.layers, w.bh, w.d, w.tokens
    picks = [(l, (5 + 97 * l) % bh) for l in range(L)]
    _say(f"[whole-run] {w.name} layers={L} bh={bh} T={T} budgets {budgets[0]}..{budgets[-1]}; "
         f"sampled {picks}")
    # worker processes start before any of the run's device memory exists
    workers = max(1, min(16, (os.cpu_count() or 2) - 1))
    ex = ProcessPoolExecutor(workers)
    try:
        streams = [ex.submit(_token_stream, (w, l, hh, T)) for l, hh in picks]
        jobs = sorted(((w, l, hh, budgets[l], T, budgets[l] + 1, None, 0) for l, hh in picks),
                      key=lambda j: -j[3])             # the longest oracle runs first
        futs = {j[1]: ex.submit(_sample_job, j) for j in jobs}

        layers = [kve.Layer.empty(bh, b + 1, d, dev, gumbel=False) for b in budgets]
        cls = [x.c_struct() for x in layers]
        ctrs = [kve.Counters(0, 0, 0) for _ in range(L)]
        sk = torch.empty((L, T, d), dtype=torch.float16, device=dev)
        sv = torch.empty_like(sk)
        for l, f in enumerate(streams):
            k, v = f.result()
            sk[l] = torch.from_numpy(k.view(np.float16)).to(dev)
            sv[l] = torch.from_numpy(v.view(np.float16)).to(dev)
        _say(f"[whole-run] inputs of the sampled caches ready; GPU run")
        chunk = 64
        gen = torch.Generator(device=dev)
        gen.manual_seed(4242)
        ins_k = torch.empty((L, chunk, bh, d), dtype=torch.float16, device=dev)
        ins_v = torch.empty_like(ins_k)
        ev = torch.empty((L, chunk, bh), dtype=torch.int32, device=dev)
        vk = [[ins_k[l, s] for s in range(chunk)] for l in range(L)]
        vv = [[ins_v[l, s] for s in range(chunk)] for l in range(L)]
        ve = [[ev[l, s] for s in range(chunk)] for l in range(L)]
        lidx = torch.arange(L, device=dev)
        hidx = torch.tensor([hh for _, hh in picks], device=dev)
        bud = torch.tensor(budgets, device=dev, dtype=torch.int64)
        n_all = torch.minimum(torch.arange(T, device=dev)[None, :], bud[:, None])  # [L, T]
        expect = torch.where(n_all + 1 > bud[:, None], n_all, -1).to(torch.int32)
        ev_s = torch.empty((L, T), dtype=torch.int32, device=dev)
        bad = torch.zeros((), dtype=torch.int64, device=dev)
        for t0 in range(0, T, chunk):
            cnt = min(chunk, T - t0)
            for l, (_, hh) in enumerate(picks):
                synth.bulk_kv_torch(w, t0, cnt, bh, gen, dev, out_k=ins_k[l, :cnt],
                                    out_v=ins_v[l, :cnt])
                ins_k[l, :cnt, hh] = sk[l, t0:t0 + cnt]
                ins_v[l, :cnt, hh] = sv[l, t0:t0 + cnt]
            for s in range(cnt):
                for l in range(L):
                    kve.pyramid_step(layers[l], vk[l][s], vv[l][s], ctrs[l], budgets[l],
                                     w.n_sink, w.rope_base, ve[l][s], c_layer=cls[l])
            bad += (ev[:, :cnt] != expect[:, t0:t0 + cnt, None]).sum()
            ev_s[:, t0:t0 + cnt] = ev[lidx[:, None], torch.arange(cnt, device=dev)[None, :],
                                      hidx[:, None]]
            if t0 % 4096 == 0:
                _say(f"[whole-run] token {t0} of {T} enqueued")
        torch.cuda.synchronize()
        _say("[whole-run] GPU done; waiting for the oracle")
        assert int(bad) == 0, f"{int(bad)} cache-steps evicted other than the incoming row"
        for l in range(L):
            assert (ctrs[l].n_kept, ctrs[l].next_pos, ctrs[l].pos) == (budgets[l], T, T)
            b = budgets[l]
            assert torch.equal(layers[l].positions[:, :b],
                               torch.arange(b, device=dev, dtype=torch.int32)[None, :].expand(bh, b))
            sc = layers[l].scores[:, :b]
            assert bool(torch.isfinite(sc).all()) and bool((sc >= 0).all())
        evn = ev_s.cpu().numpy()
        errs = []
        for l, hh in picks:
            s = futs[l].result()
            assert s.attempts == 0, f"layer {l} cache {hh}: the guard redrew {s.attempts} tokens"
            k, v = streams[l].result()
            assert np.array_equal(s.ks, k) and np.array_equal(s.vs, v)
            errs += [f"layer {l}: {e}" for e in compare_cache(layers[l], hh, s, evn[l], 0)]
        assert not errs, "\n".join(errs[:20])
    finally:
        ex.shutdown(wait=False, cancel_futures=True)


# ---------------------------------------------------------------------------
# checkpoint / resume
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("form", ["single-token", "48-token"])
def test_save_restore_resumes_bit_exact(dev, tmp_path, form):
    """KeyformerState's `pos` ("veloxquant_mlx.quantizers.keyformer module"):
    the frozen noise and the temperature depend on the running position
    alone, not on how the stream is cut into calls.  A Keyformer layer
    stepped T1 tokens, its tensors and counters written with torch.save, the
    originals freed, the file loaded into fresh device tensors and stepped T2
    more tokens, equals T1 + T2 tokens stepped straight, bit for bit: evicted
    indices, keys, values, scores, Gumbel values, positions and counters.
    The resumed part runs as single-token calls or as calls of 48 tokens
    (the last one ragged); the budget is crossed before the save and the
    annealing ends after it."""
    import kv_cache_eviction_step_amd as kve
    bh, d, budget, T1, T2 = 48, 128, 300, 420, 260
    T = T1 + T2
    _say(f"[save/restore] form={form} bh={bh} budget={budget} T1={T1} T2={T2}")
    w = synth.Workload("resume", 1, 1, bh, d, T, 0, budget, 4, "keyformer", 1.0, 2.0, 500)
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    nk, nv = synth.bulk_kv_torch(w, 0, T, bh, gen, dev)
    args = (budget, 4, 1.0, 2.0, 500, 1e4, 11)
    names = ("k", "v", "scores", "gumbel", "positions")

    A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=True)
    ca = kve.Counters(0, 0, 0)
    ev_a = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    for t in range(T):
        kve.keyformer_step(A, nk[t], nv[t], ca, *args, ev_a[t])

    B = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=True)
    cb = kve.Counters(0, 0, 0)
    ev_b = torch.full((T, bh), -9, dtype=torch.int32, device=dev)
    for t in range(T1):
        kve.keyformer_step(B, nk[t], nv[t], cb, *args, ev_b[t])
    torch.cuda.synchronize()
    path = tmp_path / "layer_state.pt"
    torch.save({**{x: getattr(B, x) for x in names},
                "counters": [cb.n_kept, cb.next_pos, cb.pos]}, path)
    del B
    torch.cuda.empty_cache()
    st = torch.load(path, weights_only=True, map_location=dev)
    C = kve.Layer(*[st[x] for x in names])
    cc = kve.Counters(*st["counters"])
    assert (cc.n_kept, cc.next_pos, cc.pos) == (budget, T1, T1)
    if form == "single-token":
        for t in range(T1, T):
            kve.keyformer_step(C, nk[t], nv[t], cc, *args, ev_b[t])
    else:
        for t0 in range(T1, T, 48):
            t1 = min(T, t0 + 48)
            kve.keyformer_step_tokens(C, nk[t0:t1], nv[t0:t1], cc, *args, ev_b[t0:t1])
    torch.cuda.synchronize()
    assert (cc.n_kept, cc.next_pos, cc.pos) == (ca.n_kept, ca.next_pos, ca.pos)
    assert torch.equal(ev_a, ev_b)
    for x in names:
        assert torch.equal(getattr(A, x)[:, :budget], getattr(C, x)[:, :budget]), x
    assert bool(((ev_a[T1:] >= 0) & (ev_a[T1:] < budget)).any())   # interior evictions resumed
