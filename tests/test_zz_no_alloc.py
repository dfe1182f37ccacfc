"""kve_step_noalloc on the GPU against kve_step_ws, the entry point whose
kernels use the same scratch protocol with a caller-owned workspace.

kve_step_noalloc keeps its scratch in a fixed device array of the library,
shared by every call on the GPU and holding whatever the last call left.
Each case below runs the same Keyformer launch through both entry points on
copies of one state and requires the same bits: evicted indices, keys,
values, scores, Gumbel values and positions.
"""
from __future__ import annotations

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

NAMES = ("k", "v", "scores", "gumbel", "positions")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _state(dev, bh, budget, d, seed):
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    w = synth.Workload("noalloc", 1, 1, bh, d, 7000, 8, budget, 4, "keyformer", 1.0, 2.0, 64)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=True)
    bulk_state(A, budget, w, gen)
    B = kve.Layer(*[getattr(A, x).clone() for x in NAMES])
    nk, nv = synth.bulk_kv_torch(w, 7000, 8, bh, gen, dev)
    return A, B, nk, nv


def _compare(A, B, ev_a, ev_b, budget):
    assert torch.equal(ev_a, ev_b)
    for x in NAMES:
        assert torch.equal(getattr(A, x)[:, :budget], getattr(B, x)[:, :budget]), x


def test_noalloc_two_calls_match_workspace_form(dev):
    """Two calls in a row, the second on a smaller input: 320 caches of 1000
    rows, then 260 caches of 600 rows (fewer items in the shared array than
    the first call left there).  Both calls hand long moves over."""
    import kv_cache_eviction_step_amd as kve
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 64, 1e4, 9)
    for bh, budget, seed in ((320, 1000, 201), (260, 600, 202)):
        print(f"[noalloc] bh={bh} budget={budget}", flush=True)
        A, B, nk, nv = _state(dev, bh, budget, 128, seed)
        ba = kve.LayerBatch([A], [budget], [kve.Counters(budget, 7000, 7000)])
        bb = kve.LayerBatch([B], [budget], [kve.Counters(budget, 7000, 7000)])
        ev_a = torch.full((bh,), -9, dtype=torch.int32, device=dev)
        ev_b = torch.full((bh,), -9, dtype=torch.int32, device=dev)
        kve.step_noalloc(ba, [nk[0]], [nv[0]], pol, [ev_a])
        kve.step(bb, [nk[0]], [nv[0]], pol, [ev_b], workspace=kve.workspace(bh, budget, 128, dev))
        torch.cuda.synchronize()
        _compare(A, B, ev_a, ev_b, budget)
        assert int((budget - 1 - ev_a)[(ev_a >= 0) & (ev_a < budget)].max()) > 128


def test_noalloc_token_sequence_and_layers_match_workspace_form(dev):
    """Eight tokens through two layers (200 + 120 caches, budgets 900 and
    500, d = 64) per call, then the same layers alone: every call equals
    kve_step_ws on copies, and the counters advance alike."""
    import kv_cache_eviction_step_amd as kve
    from gpu_harness import bulk_state
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 64, 1e4, 13)
    shapes = [(200, 900, 0), (120, 500, 200)]
    d, T = 64, 8
    gen = torch.Generator(device=dev)
    gen.manual_seed(211)
    As, Bs, ks, vs = [], [], [], []
    for bh, budget, hb in shapes:
        w = synth.Workload("noalloc2", 1, 1, bh, d, 7000, T, budget, 4, "keyformer", 1.0, 2.0, 64)
        A = kve.Layer.empty(bh, budget + 1, d, dev, gumbel=True, hh_base=hb)
        bulk_state(A, budget, w, gen)
        As.append(A)
        Bs.append(kve.Layer(*[getattr(A, x).clone() for x in NAMES], hh_base=hb))
        k, v = synth.bulk_kv_torch(w, 7000, T, bh, gen, dev)
        ks.append(k)
        vs.append(v)
    budgets = [b for _, b, _ in shapes]
    ba = kve.LayerBatch(As, budgets, [kve.Counters(b, 7000, 7000) for b in budgets])
    bb = kve.LayerBatch(Bs, budgets, [kve.Counters(b, 7000, 7000) for b in budgets])
    ws = kve.workspace(sum(bh for bh, _, _ in shapes), max(budgets), d, dev)
    ev_a = [torch.full((T, bh), -9, dtype=torch.int32, device=dev) for bh, _, _ in shapes]
    ev_b = [torch.full((T, bh), -9, dtype=torch.int32, device=dev) for bh, _, _ in shapes]
    for t in range(T):
        kve.step_noalloc(ba, [k[t] for k in ks], [v[t] for v in vs], pol, [e[t] for e in ev_a])
        kve.step(bb, [k[t] for k in ks], [v[t] for v in vs], pol, [e[t] for e in ev_b],
                 workspace=ws)
    torch.cuda.synchronize()
    for l, (_, budget, _) in enumerate(shapes):
        _compare(As[l], Bs[l], ev_a[l], ev_b[l], budget)
        assert (ba.ctrs[l].n_kept, ba.ctrs[l].pos) == (bb.ctrs[l].n_kept, bb.ctrs[l].pos)


def test_noalloc_captured_replays_match_eager(dev):
    """kve_step_noalloc captured into a graph (its header-clearing kernel,
    step and move kernels are all captured work) and replayed three times
    from a restored state, with eager work and synchronisations between
    replays: every replay equals the eager call."""
    import kv_cache_eviction_step_amd as kve
    bh, budget = 300, 1000
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 64, 1e4, 17)
    S0, E, nk, nv = _state(dev, bh, budget, 128, 221)
    ev_e = torch.full((bh,), -9, dtype=torch.int32, device=dev)
    kve.step_noalloc(kve.LayerBatch([E], [budget], [kve.Counters(budget, 7000, 7000)]),
                     [nk[0]], [nv[0]], pol, [ev_e])
    torch.cuda.synchronize()
    # E now holds the eager result; S0 the start state (E was its copy)
    G = kve.Layer(*[getattr(S0, x).clone() for x in NAMES])
    ev_g = torch.full((bh,), -9, dtype=torch.int32, device=dev)
    bg = kve.LayerBatch([G], [budget], [kve.Counters(budget, 7000, 7000)])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kve.step_noalloc(bg, [nk[0]], [nv[0]], pol, [ev_g])
    for replay in range(3):
        for x in NAMES:
            getattr(G, x).copy_(getattr(S0, x))
        ev_g.fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _compare(G, E, ev_g, ev_e, budget)
