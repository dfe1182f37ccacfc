"""The C-ABI library on the host: it loads, exports what include/kve.h
declares, rejects bad arguments before touching any device, and computes the
pyramid schedule of the PyramidKV page ("The budget schedule")."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_step_amd as kve
from kv_cache_eviction_step_amd import Counters, KveLayer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kve.h")


def _declared() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|int32_t|int64_t|const char \*)\s*(\w+)\s*\(", text,
                      flags=re.M)


def test_header_declares_the_abi():
    assert set(_declared()) == {"keyformer_step", "pyramid_step", "keyformer_step_layers",
                                "pyramid_step_layers", "keyformer_step_tokens",
                                "pyramid_step_tokens", "keyformer_step_layers_tokens",
                                "pyramid_step_layers_tokens", "kve_step", "kve_step_ws",
                                "kve_workspace_size", "kve_step_noalloc", "pyramid_budgets",
                                "kve_kept_indices", "kve_fp16_bytes", "kve_full_fp16_bytes",
                                "kve_strerror"}


# HIP runtime calls the library may import: kernel and device-variable
# registration and launch, the LDS-size attribute of a launch, the
# launch-error query, and -- for kve_step_noalloc's fixed buffer -- the
# current device and the device address of that buffer.  No allocation
# (hipMalloc, hipHostMalloc, hipMallocAsync, ...), free, memset, copy, event or
# synchronisation call is imported, so no path of any entry point can
# allocate device memory or stall the caller's streams.
ALLOWED_HIP_IMPORTS = {"__hipPopCallConfiguration", "__hipPushCallConfiguration",
                       "__hipRegisterFatBinary", "__hipRegisterFunction", "__hipRegisterVar",
                       "__hipUnregisterFatBinary", "hipFuncSetAttribute", "hipGetLastError",
                       "hipLaunchKernel", "hipGetDevice", "hipGetSymbolAddress"}


def test_library_imports_no_allocation_or_synchronisation():
    out = subprocess.run(["nm", "-D", "--undefined-only", kve.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    hip = {line.split()[-1].split("@")[0] for line in out.splitlines()
           if "hip" in line.lower()}
    assert hip, "no HIP import found: the check would prove nothing"
    assert hip <= ALLOWED_HIP_IMPORTS, sorted(hip - ALLOWED_HIP_IMPORTS)
    for banned in ("hipMalloc", "hipFree", "hipDeviceSynchronize", "hipStreamSynchronize",
                   "hipMemset", "hipEventCreate", "hipHostMalloc", "hipMallocAsync"):
        assert not any(h.startswith(banned) for h in hip), banned


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", kve.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in syms, f"{name} not exported"
        assert hasattr(kve.lib(), name)


def test_single_hip_runtime_mapped():
    rts = kve.hip_runtimes_mapped()
    assert len(rts) <= 1, rts


def test_strerror():
    assert kve.strerror(0) == "ok"
    assert "invalid" in kve.strerror(-1)
    assert kve.strerror(12345) == "unknown error"


# ---------------------------------------------------------------------------
# pyramid_budgets: "The budget schedule" (PyramidKV page)
# ---------------------------------------------------------------------------

def test_pyramid_budgets_page_example():
    assert kve.pyramid_budgets(12, 512, 4, 2.0) == \
        [1019, 927, 835, 742, 650, 558, 466, 374, 282, 189, 97, 5]


@pytest.mark.parametrize("args", [(28, 512, 4, 2.0), (28, 512, 4, 1.0), (32, 4096, 4, 1.5),
                                  (12, 512, 4, 1.5), (0, 512, 4, 2.0), (1, 77, 4, 3.0),
                                  (64, 1000, 7, 1.77), (9, 6, 5, 2.5), (3, 8, 2, 1.0)])
def test_pyramid_budgets_matches_oracle(args):
    assert kve.pyramid_budgets(*args) == oracle.pyramid_budgets(*args)


@pytest.mark.parametrize("args", [(12, 512, 4, 0.5), (12, 512, 4, float("nan")),
                                  (-1, 512, 4, 2.0), (12, 4, 4, 2.0), (12, 512, -1, 2.0)])
def test_pyramid_budgets_rejects(args):
    with pytest.raises(ValueError):
        kve.pyramid_budgets(*args)


def test_pyramid_budgets_null_out():
    assert kve.lib().pyramid_budgets(3, 512, 4, 2.0, None) == kve.KVE_EINVAL
    assert kve.lib().pyramid_budgets(0, 512, 4, 2.0, None) == kve.KVE_OK


# ---------------------------------------------------------------------------
# host-side argument checks: no device is touched, counters stay unchanged
# ---------------------------------------------------------------------------

FAKE = 0x10000          # aligned, never dereferenced: every case fails a host check first


def _layer(**kw) -> KveLayer:
    base = dict(k=FAKE, v=FAKE, scores=FAKE, gumbel=FAKE, positions=FAKE, bh=8, cap=33, d=64,
                hh_base=0)
    base.update(kw)
    return KveLayer(**base)


def _kf(layer, ctr, budget=32, n_sink=4, tau_init=1.0, tau_end=2.0, anneal=64, base=1e4,
        new_k=FAKE, new_v=FAKE):
    return kve.lib().keyformer_step(ctypes.byref(layer) if layer is not None else None,
                                    new_k, new_v, ctypes.byref(ctr) if ctr is not None else None,
                                    budget, n_sink, tau_init, tau_end, anneal, base, 0, None,
                                    None)


BAD_CASES = {
    "null_layer": dict(layer=None),
    "null_k": dict(layer_kw=dict(k=None)),
    "null_scores": dict(layer_kw=dict(scores=None)),
    "null_positions": dict(layer_kw=dict(positions=None)),
    "null_gumbel_keyformer": dict(layer_kw=dict(gumbel=None)),
    "null_new_k": dict(call_kw=dict(new_k=None)),
    "misaligned_k": dict(layer_kw=dict(k=FAKE + 2)),
    "misaligned_new_v": dict(call_kw=dict(new_v=FAKE + 8)),
    "d_96": dict(layer_kw=dict(d=96)),
    "bh_0": dict(layer_kw=dict(bh=0)),
    "cap_too_small": dict(layer_kw=dict(cap=32)),
    "budget_le_sink": dict(call_kw=dict(budget=4, n_sink=4)),
    "negative_sink": dict(call_kw=dict(n_sink=-1)),
    "budget_over_max": dict(call_kw=dict(budget=12289), layer_kw=dict(cap=12290)),
    "negative_tau": dict(call_kw=dict(tau_init=-0.1)),
    "nan_tau": dict(call_kw=dict(tau_end=float("nan"))),
    "negative_anneal": dict(call_kw=dict(anneal=-1)),
    "bad_rope_base": dict(call_kw=dict(base=0.0)),
    "n_kept_over_budget": dict(ctr=(33, 40, 40)),
    "n_kept_negative": dict(ctr=(-1, 0, 0)),
    "gap_without_eviction": dict(ctr=(10, 50, 50)),   # next_pos != n_kept, no eviction
    "next_pos_below_n_kept": dict(ctr=(32, 10, 10)),
}


@pytest.mark.parametrize("name", sorted(BAD_CASES))
def test_keyformer_step_rejects_before_any_launch(name):
    case = BAD_CASES[name]
    layer = None if case.get("layer", 1) is None else _layer(**case.get("layer_kw", {}))
    ctr = Counters(*case.get("ctr", (32, 100, 100)))
    rc = _kf(layer, ctr, **case.get("call_kw", {}))
    assert rc == kve.KVE_EINVAL
    assert (ctr.n_kept, ctr.next_pos, ctr.pos) == case.get("ctr", (32, 100, 100))


def test_null_counters_rejected():
    assert _kf(_layer(), None) == kve.KVE_EINVAL


def test_pyramid_step_accepts_null_gumbel_then_needs_a_device():
    layer = _layer(gumbel=None)
    ctr = Counters(32, 100, 100)
    rc = kve.lib().pyramid_step(ctypes.byref(layer), FAKE, FAKE, ctypes.byref(ctr), 32, 4, 1e4,
                                None, None)
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the no-device path is not reachable")
    assert rc == kve.KVE_ENODEV                    # passed every host check
    assert (ctr.n_kept, ctr.next_pos, ctr.pos) == (32, 100, 100)


def test_python_binding_validates_tensors():
    L = kve.Layer.empty(2, 9, 64, "cpu", gumbel=True)
    with pytest.raises(ValueError):
        kve.keyformer_step(L, torch.zeros(2, 32, dtype=torch.float16),
                           torch.zeros(2, 64, dtype=torch.float16), Counters(0, 0, 0), 8, 2,
                           1.0, 2.0, 8, 1e4, 0)
    with pytest.raises(ValueError):
        kve.Layer(torch.zeros(2, 9, 64, dtype=torch.float32), L.v, L.scores, L.gumbel,
                  L.positions)
    _ = np


# ---------------------------------------------------------------------------
# batched calls: every layer is checked before anything is enqueued
# ---------------------------------------------------------------------------

def _batch_call(layers, ctrs, budgets, n=None, kf=True):
    n = len(layers) if n is None else n
    arr = (KveLayer * max(len(layers), 1))(*layers)
    cs = (Counters * max(len(ctrs), 1))(*ctrs)
    bs = (ctypes.c_int32 * max(len(budgets), 1))(*budgets)
    ptrs = (ctypes.c_void_p * max(len(layers), 1))(*([FAKE] * len(layers)))
    if kf:
        rc = kve.lib().keyformer_step_layers(n, arr, ptrs, ptrs, cs, bs, 4, 1.0, 2.0, 64, 1e4, 0,
                                             None, None)
    else:
        rc = kve.lib().pyramid_step_layers(n, arr, ptrs, ptrs, cs, bs, 4, 1e4, None, None)
    return rc, [(c.n_kept, c.next_pos, c.pos) for c in cs]


@pytest.mark.parametrize("case", ["zero_layers", "too_many", "mixed_d", "one_bad_budget",
                                  "one_bad_counter", "one_null_gumbel", "same_layer_twice",
                                  "overlapping_keys"])
def test_batched_rejects_before_any_launch(case):
    layer_bytes = 8 * 33 * 64 * 2
    layers = [_layer(k=FAKE + i * layer_bytes) for i in range(3)]
    ctrs = [Counters(32, 100, 100) for _ in range(3)]
    budgets = [32, 32, 32]
    n = None
    if case == "zero_layers":
        n = 0
    elif case == "too_many":
        layers = [_layer(k=FAKE + i * layer_bytes) for i in range(129)]
        ctrs, budgets = [Counters(32, 100, 100)] * 129, [32] * 129
    elif case == "mixed_d":
        layers[1] = _layer(d=128)
    elif case == "one_bad_budget":
        budgets[2] = 40                                   # cap 33 < budget + 1
    elif case == "one_bad_counter":
        ctrs[1] = Counters(10, 50, 50)
    elif case == "one_null_gumbel":
        layers[0] = _layer(gumbel=None)
    elif case == "same_layer_twice":
        layers[2] = layers[0]
    elif case == "overlapping_keys":
        layers[1] = _layer(k=FAKE + layer_bytes - 256)      # last row of layer 0
    before = [(c.n_kept, c.next_pos, c.pos) for c in ctrs]
    rc, after = _batch_call(layers, ctrs, budgets, n)
    assert rc == kve.KVE_EINVAL
    assert after == before


def test_batched_pyramid_null_gumbel_passes_host_checks():
    layers = [_layer(gumbel=None, k=FAKE + i * 8 * 33 * 64 * 2) for i in range(2)]
    rc, after = _batch_call(layers, [Counters(32, 100, 100)] * 2, [32, 32], kf=False)
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the no-device path is not reachable")
    assert rc == kve.KVE_ENODEV
    assert after == [(32, 100, 100)] * 2


@pytest.mark.parametrize("n_tokens,ctr", [(0, (32, 100, 100)), (129, (32, 100, 100)),
                                          (4, (10, 50, 50)), (4, (40, 100, 100))])
def test_multi_token_rejects_before_any_launch(n_tokens, ctr):
    layer = _layer()
    c = Counters(*ctr)
    rc = kve.lib().keyformer_step_tokens(ctypes.byref(layer), n_tokens, FAKE, FAKE, ctypes.byref(c),
                                         32, 4, 1.0, 2.0, 64, 1e4, 0, None, None)
    assert rc == kve.KVE_EINVAL
    assert (c.n_kept, c.next_pos, c.pos) == ctr
    assert kve.lib().pyramid_step_tokens(None, 4, FAKE, FAKE, ctypes.byref(c), 32, 4, 1e4, None,
                                         None) == kve.KVE_EINVAL


def _policy_call(layers, ctrs, budgets, pol, n_tokens=1):
    n = len(layers)
    arr = (KveLayer * n)(*layers)
    cs = (Counters * n)(*ctrs)
    bs = (ctypes.c_int32 * n)(*budgets)
    ptrs = (ctypes.c_void_p * n)(*([FAKE] * n))
    rc = kve.lib().kve_step(n, n_tokens, arr, ptrs, ptrs, cs, bs,
                            ctypes.byref(pol) if pol is not None else None, None, None)
    return rc, [(c.n_kept, c.next_pos, c.pos) for c in cs]


@pytest.mark.parametrize("case", ["null_policy", "bad_score", "bad_gumbel_flag", "negative_recent",
                                  "window_fills_budget", "window_fills_budget_batched",
                                  "negative_tau_with_gumbel", "null_gumbel_with_noise",
                                  "tokens_129"])
def test_kve_step_rejects_before_any_launch(case):
    """kve_step checks its policy as init_keyformer_state does: sinks plus the
    recent window must leave room to evict within every layer's budget."""
    layers = [_layer(), _layer(k=FAKE + (1 << 20))]
    budgets = [32, 32]
    pol = kve.policy("keyformer", 4, recent=3, tau_init=1.0, tau_end=2.0, anneal_steps=64)
    n_layers, n_tokens = 1, 1
    if case == "null_policy":
        pol = None
    elif case == "bad_score":
        pol.score = 2
    elif case == "bad_gumbel_flag":
        pol.gumbel = 2
    elif case == "negative_recent":
        pol.recent = -1
    elif case == "window_fills_budget":
        pol.recent = 28                                   # 4 + 28 == 32: no room
    elif case == "window_fills_budget_batched":
        n_layers, budgets, pol.recent = 2, [40, 20], 16   # layer 1: 4 + 16 >= 20
    elif case == "negative_tau_with_gumbel":
        pol.tau_init = -1.0
    elif case == "null_gumbel_with_noise":
        layers = [_layer(gumbel=None), _layer(k=FAKE + (1 << 20))]
    elif case == "tokens_129":
        n_tokens = 129
    ctrs = [Counters(32, 100, 100), Counters(32, 100, 100)]
    if case == "window_fills_budget_batched":
        ctrs = [Counters(40, 100, 100), Counters(20, 100, 100)]
        layers = [_layer(cap=41), _layer(cap=41, k=FAKE + (1 << 20))]
    before = [(c.n_kept, c.next_pos, c.pos) for c in ctrs[:n_layers]]
    rc, after = _policy_call(layers[:n_layers], ctrs[:n_layers], budgets[:n_layers], pol, n_tokens)
    assert rc == kve.KVE_EINVAL
    assert after == before


def test_kve_step_policy_passes_host_checks():
    """The largest window that leaves one evictable row, with TOVA scoring and
    no noise (NULL gumbel allowed), reaches the device check."""
    pol = kve.policy("tova", 4, recent=27)
    rc, after = _policy_call([_layer(gumbel=None)], [Counters(32, 100, 100)], [32], pol)
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the no-device path is not reachable")
    assert rc == kve.KVE_ENODEV
    assert after == [(32, 100, 100)]


def test_policy_helper():
    p = kve.policy("keyformer", 4, 2, 1.0, 2.0, 64, 5e5, seed=-1)
    assert (p.n_sink, p.recent, p.score, p.gumbel, p.anneal_steps) == (4, 2, 0, 1, 64)
    assert p.seed == 2**64 - 1 and p.rope_base == 5e5
    t = kve.policy("tova", 4, 1, 1.0, 2.0, 64)
    assert (t.score, t.gumbel, t.tau_init, t.anneal_steps) == (kve.SCORE_CURRENT, 0, 0.0, 0)
    with pytest.raises(ValueError):
        kve.policy("snapkv", 4)


# ---------------------------------------------------------------------------
# inspection helpers: return_indices, get_kv, byte accounting (Keyformer page:
# keyformer_update_batched return_indices, keyformer_get_kv,
# keyformer_fp16_bytes, full_keyformer_fp16_bytes)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,recent", [("keyformer", 0), ("h2o", 3), ("tova", 2)])
def test_kept_indices_match_oracle_token_ids(kind, recent):
    """The composed evicted log names the same surviving rows as the oracle's
    own token-id bookkeeping, from an empty cache and from a mid-run state."""
    import numpy as np
    import synth
    w = synth.TINY_ANNEALED
    prm = oracle.Params(20, 4, kind == "keyformer", 1.0, 2.0, 64, seed=0, hh=1, recent=recent,
                        current_score=kind == "tova")
    ks, vs = synth.token_kv(w, 0, 1, np.arange(160))
    c = oracle.OracleCache(64, 21)
    ev0 = c.run(ks[:100], vs[:100], prm)
    assert kve.kept_indices(0, ev0) == list(c.tid[:c.n])
    prior = list(c.tid[:c.n])
    n_prev, t0 = c.n, c.next_pos
    ev1 = c.run(ks[100:], vs[100:], prm)
    idx = kve.kept_indices(n_prev, ev1)
    assert [prior[i] if i < n_prev else t0 + i - n_prev for i in idx] == list(c.tid[:c.n])


def test_kept_indices_edges_and_rejects():
    assert kve.kept_indices(0, []) == []
    assert kve.kept_indices(3, []) == [0, 1, 2]
    assert kve.kept_indices(3, [-1, 4, 0]) == [1, 2, 3, 5]
    assert kve.kept_indices(2, [2]) == [0, 1]                  # the new row itself
    for n_prev, ev in ((2, [3]), (2, [-2]), (-1, [])):
        with pytest.raises(ValueError):
            kve.kept_indices(n_prev, ev)
    assert kve.lib().kve_kept_indices(0, 1, None, None) == kve.KVE_EINVAL


def test_byte_accounting_and_get_kv_views():
    L = kve.Layer.empty(3, 17, 64, "cpu", gumbel=False)
    k, v = L.get_kv(9)
    assert tuple(k.shape) == (3, 9, 64) and k.data_ptr() == L.k.data_ptr()
    assert v.data_ptr() == L.v.data_ptr()
    per_cache = (k[0].numel() + v[0].numel()) * k.element_size()
    assert kve.fp16_bytes(9, 64) == per_cache == 4 * 9 * 64
    assert kve.full_fp16_bytes(3072, 128) == 4 * 3072 * 128
    assert kve.full_fp16_bytes(3072, 128) / kve.fp16_bytes(512, 128) == 6.0
    k0, v0 = L.get_kv(0)
    assert tuple(k0.shape) == (3, 0, 64) and v0.numel() == 0
    with pytest.raises(ValueError):
        L.get_kv(18)
    with pytest.raises(ValueError):
        kve.fp16_bytes(-1, 64)
    assert kve.lib().kve_full_fp16_bytes(10, 0) == -1


def test_binding_refuses_tensors_off_the_current_gpu():
    """The library launches on the current device; the binding refuses a layer
    whose tensors live elsewhere (here: host memory) before calling it."""
    L = kve.Layer.empty(2, 9, 64, "cpu", gumbel=True)
    k = torch.zeros(2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="current"):
        kve.keyformer_step(L, k, k, Counters(0, 0, 0), 8, 2, 1.0, 2.0, 8, 1e4, 0)
    with pytest.raises(ValueError, match="current"):
        kve.pyramid_step_tokens(L, k[None], k[None], Counters(0, 0, 0), 8, 2, 1e4)


def test_layer_batch_pointer_arrays():
    """The batched calls' per-layer pointers from one whole-batch tensor:
    block l of a [n_layers, ...] tensor starts at data_ptr + l * stride(0)
    elements, contiguous or a slice of a longer axis; a pointer list of
    per-layer tensors works too; bad tensors are refused before any call."""
    layers = [kve.Layer.empty(4, 17, 64, "cpu", gumbel=True) for _ in range(3)]
    batch = kve.LayerBatch(layers, [16] * 3)
    for tok in (None, 5):
        t_axis = () if tok is None else (tok,)
        big = torch.zeros((3, *((9,) if tok else ()), 4, 64), dtype=torch.float16)
        src = big if tok is None else big[:, 2:2 + tok]      # strided along the layer axis
        ev_big = torch.zeros((3, *((9,) if tok else ()), 4), dtype=torch.int32)
        ev = ev_big if tok is None else ev_big[:, 1:1 + tok]
        pe = batch._fill(src, src, ev, tok)
        for l in range(3):
            assert batch._pk[l] == src.data_ptr() + l * src.stride(0) * 2
            assert batch._pv[l] == src.data_ptr() + l * src.stride(0) * 2
            assert pe[l] == ev.data_ptr() + l * ev.stride(0) * 4
        per = [src[l].contiguous() for l in range(3)]
        batch._fill(per, per, None, tok)
        assert [batch._pk[l] for l in range(3)] == [p.data_ptr() for p in per]
        with pytest.raises(ValueError):                     # wrong dtype
            batch._fill(src.float(), src, None, tok)
        with pytest.raises(ValueError):                     # wrong row shape
            batch._fill(torch.zeros((3, *t_axis, 4, 32), dtype=torch.float16), src, None, tok)
    for s in range(20):                                     # the offsets cache stays small
        batch._layer_offsets(128 * (s + 1))
    assert len(batch._offsets) <= 16
    assert (batch._layer_offsets(256) == np.arange(3, dtype=np.uint64) * np.uint64(256)).all()


# ---------------------------------------------------------------------------
# the workspace form (kve_step_ws, kve_workspace_size)
# ---------------------------------------------------------------------------

def _ws_bytes(caches, budget, d):
    """The layout kve_workspace_size documents: 256 bytes of counters, one
    32-byte item per 64-row chunk of each cache's longest move (budget - 1
    rows, at least one chunk), rounded up to 256 bytes, and one parked row of
    4*d bytes per item."""
    items = caches * max(1, -(-(budget - 1) // 64))
    return 256 + -(-items * 32 // 256) * 256 + items * 4 * d


@pytest.mark.parametrize("args", [(256, 1024, 128), (8192, 1024, 128), (512, 6144, 128),
                                  (1, 1, 64), (1, 2, 64), (3, 65, 64), (3, 66, 64),
                                  (300, 12288, 128), (7, 129, 64)])
def test_workspace_size(args):
    assert kve.workspace_size(*args) == _ws_bytes(*args)


@pytest.mark.parametrize("args", [(0, 1024, 128), (256, 0, 128), (256, 12289, 128),
                                  (256, 1024, 96), (2**31, 1024, 128), (2**24, 12288, 128)])
def test_workspace_size_rejects(args):
    assert kve.lib().kve_workspace_size(*args) == -1


def _ws_call(ws, nbytes, layers=None, ctrs=None, budgets=(32,)):
    layers = layers or [_layer()]
    n = len(layers)
    arr = (KveLayer * n)(*layers)
    cs = (Counters * n)(*(ctrs or [Counters(32, 100, 100)] * n))
    bs = (ctypes.c_int32 * n)(*budgets)
    ptrs = (ctypes.c_void_p * n)(*([FAKE] * n))
    pol = kve.policy("keyformer", 4, tau_init=1.0, tau_end=2.0, anneal_steps=64)
    rc = kve.lib().kve_step_ws(n, 1, arr, ptrs, ptrs, cs, bs, ctypes.byref(pol), None, ws,
                               nbytes, None)
    return rc, [(c.n_kept, c.next_pos, c.pos) for c in cs]


@pytest.mark.parametrize("case", ["misaligned", "one_byte_short", "header_only", "null_with_size",
                                  "negative", "null_layers"])
def test_kve_step_ws_rejects_bad_workspace(case):
    """A workspace must be 256-byte aligned and hold at least one item (one
    32-byte item and one parked 4*d-byte row, after 256 bytes of counters);
    NULL means none and then its size must be 0."""
    one_item = _ws_bytes(1, 2, 64)                  # 256 + 256 + 256 at d = 64
    ws, nbytes = {"misaligned": (FAKE + 16, 1 << 20), "one_byte_short": (FAKE, one_item - 1),
                  "header_only": (FAKE, 256), "null_with_size": (None, 4096),
                  "negative": (FAKE, -1), "null_layers": (FAKE, 1 << 20)}[case]
    if case == "null_layers":
        pol = kve.policy("keyformer", 4)
        assert kve.lib().kve_step_ws(1, 1, None, None, None, None, None, ctypes.byref(pol), None,
                                     ws, nbytes, None) == kve.KVE_EINVAL
        return
    rc, after = _ws_call(ws, nbytes)
    assert rc == kve.KVE_EINVAL
    assert after == [(32, 100, 100)]


@pytest.mark.parametrize("ws,nbytes", [(None, 0), (FAKE, _ws_bytes(1, 2, 64)),
                                       (FAKE, 1 << 20)])
def test_kve_step_ws_passes_host_checks(ws, nbytes):
    """No workspace, the smallest one, and a large one all pass the host checks
    and reach the launch (no device here)."""
    rc, after = _ws_call(ws, nbytes)
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the no-device path is not reachable")
    assert rc == kve.KVE_ENODEV
    assert after == [(32, 100, 100)]


def test_kve_step_ws_checks_layers_like_kve_step():
    layers = [_layer(), _layer(k=FAKE + (1 << 20))]
    rc, after = _ws_call(FAKE, 1 << 20, layers, [Counters(32, 100, 100), Counters(10, 50, 50)],
                         budgets=(32, 32))
    assert rc == kve.KVE_EINVAL
    assert after == [(32, 100, 100), (10, 50, 50)]


def test_binding_workspace_is_aligned_zeroed_and_sized():
    ws = kve.workspace(300, 1000, 128, "cpu")
    assert ws.dtype == torch.uint8 and ws.numel() == kve.workspace_size(300, 1000, 128)
    assert ws.data_ptr() % 256 == 0 and not bool(ws.any())
    with pytest.raises(ValueError):
        kve.workspace_size(0, 1000, 128)


# ---------------------------------------------------------------------------
# kve_step_noalloc: the size check happens before anything touches a device
# ---------------------------------------------------------------------------

def _noalloc_call(layers, budgets, pol, n_tokens=1):
    n = len(layers)
    arr = (KveLayer * n)(*layers)
    cs = (Counters * n)(*[Counters(b, 5000, 5000) for b in budgets])
    bs = (ctypes.c_int32 * n)(*budgets)
    ptrs = (ctypes.c_void_p * n)(*([FAKE] * n))
    rc = kve.lib().kve_step_noalloc(n, n_tokens, arr, ptrs, ptrs, cs, bs, ctypes.byref(pol), None,
                                    None)
    return rc, [(c.n_kept, c.next_pos, c.pos) for c in cs]


def test_noalloc_rejects_calls_beyond_its_buffer():
    """32 layers of 256 caches at budget 1024 (the 8B-shaped decode in one
    launch) would need 68 MiB of scratch to hand every move over: more than
    the fixed 16 MiB buffer, so the call is refused before any launch."""
    gib = 1 << 30
    layers = [_layer(bh=256, cap=1025, d=128, k=FAKE + l * gib, v=FAKE + l * gib)
              for l in range(32)]
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 512, 1e4, 0)
    assert kve.workspace_size(32 * 256, 1024, 128) > kve.NOALLOC_SCRATCH_BYTES
    rc, after = _noalloc_call(layers, [1024] * 32, pol)
    assert rc == kve.KVE_ENOSPACE
    assert after == [(1024, 5000, 5000)] * 32
    assert "fixed device buffer" in kve.strerror(kve.KVE_ENOSPACE)


@pytest.mark.parametrize("case", ["fits", "no_handover_tokens", "no_handover_policy"])
def test_noalloc_accepts_what_fits_or_needs_no_scratch(case):
    """Within the buffer (one 256-cache layer at budget 1024: 2.1 MiB), or a
    call that hands nothing over (several tokens; H2O without a window): the
    host checks pass and the call reaches the device (none here)."""
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 512, 1e4, 0)
    layers, n_tokens = [_layer(bh=256, cap=1025, d=128)], 1
    if case == "no_handover_tokens":
        layers = [_layer(bh=256 * 32, cap=1025, d=128)]
        n_tokens = 4
    elif case == "no_handover_policy":
        layers = [_layer(bh=256 * 32, cap=1025, d=128, gumbel=None)]
        pol = kve.policy("h2o", 4)
    assert kve.workspace_size(256, 1024, 128) <= kve.NOALLOC_SCRATCH_BYTES
    rc, after = _noalloc_call(layers, [1024], pol, n_tokens)
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the no-device path is not reachable")
    assert rc == kve.KVE_ENODEV
    assert after == [(1024, 5000, 5000)]


def test_noalloc_checks_arguments_like_kve_step():
    pol = kve.policy("keyformer", 4, 0, 1.0, 2.0, 512, 1e4, 0)
    rc, _ = _noalloc_call([_layer(bh=256, cap=1025, d=96)], [1024], pol)
    assert rc == kve.KVE_EINVAL
    rc, _ = _noalloc_call([_layer(bh=256, cap=1000, d=128)], [1024], pol)
    assert rc == kve.KVE_EINVAL
    assert kve.lib().kve_step_noalloc(1, 1, None, None, None, None, None, ctypes.byref(pol), None,
                                      None) == kve.KVE_EINVAL
