#!/usr/bin/env python3
"""Throughput of the KV-cache eviction step on one MI355X.

A step is one decode token through every layer.  By default that is L
launches (one per layer), each stepping all B*H caches of that layer through
keyformer_step or pyramid_step; --batched puts all layers in one launch and
--tokens-per-call S steps S tokens per launch.  Inputs are resident in HBM
before the timed region.  Timing is bracketed by HIP events on the stream the
kernels run on.

Prints ONE JSON line: cache-row updates/s (B*L*H*tokens per second) as
`value`, the achieved algorithmic HBM bandwidth of the step kernel against
MI355X's 8 TB/s in `roofline`, and the CPU oracle timed on the host cores in
`cpu_baseline`.

Algorithmic bytes per cache-step (n = rows stored before the step, D = head
dim, m = rows whose slot changes: n - e for an evicted stored row e, 0 when
nothing or the incoming row is evicted):
  Keyformer: 2nD + 12n + 8D + 12 + m(8D + 24)
  PyramidKV: 2nD +  8n + 8D +  8 + m(8D + 16)
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", type=int, default=4, help="workload index 0..4")
    ap.add_argument("--fill", choices=["synthetic", "real"], default="synthetic",
                    help="reach the steady state by synthesising it (default) or by "
                         "stepping the prompt through the real step")
    ap.add_argument("--batched", action="store_true",
                    help="one launch per token for all layers (keyformer_step_layers / "
                         "pyramid_step_layers) instead of one launch per layer")
    ap.add_argument("--tokens-per-call", type=int, default=1,
                    help="S > 1: each launch steps S tokens (*_step_tokens per layer, or "
                         "*_step_layers_tokens with --batched); S must divide --steps and "
                         "--warmup")
    ap.add_argument("--recent", type=int, default=0,
                    help="protect the last R rows from eviction (kve_step)")
    ap.add_argument("--tova", action="store_true",
                    help="TOVA-adapted scoring (current-step weight; kve_step)")
    ap.add_argument("--whole-run", action="store_true",
                    help="time the whole trajectory instead (prompt + decode from empty "
                         "caches, token by token; --steps / --warmup / --fill unused)")
    ap.add_argument("--skip-whole-run", action="store_true",
                    help="after the K timed steps, do not also time the whole trajectory "
                         "(reported as the line's 'whole_run' object)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU oracle baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of known size (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


KERNEL_SOURCES = ["kv_cache_eviction_step_amd/csrc/kve_step.hip",
                  "kv_cache_eviction_step_amd/csrc/kve_step.h"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that
    an edit of a comment does not invalidate a measurement."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def launch_mode(batched: bool, tokens_per_call: int) -> str:
    return ("all-layers" if batched else "per-layer") + f"_x{tokens_per_call}tok"


def measured_traffic(workload: str, kernel: str, mode: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload and launch mode, or None when it is missing or the kernel changed
    since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_{mode}_pmc_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain elementwise copy: reads and writes exactly 1 GiB per dispatch."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "elementwise mul by 1.0",
                                           "read_bytes_per_dispatch": n * 4,
                                           "write_bytes_per_dispatch": n * 4,
                                           "dispatches": 5}}), flush=True)


def bandwidth_context(dev) -> dict:
    """What a plain torch kernel reaches on this GPU in the same run: a 1 GiB
    elementwise copy (reads and writes 1 GiB each), HIP events around 5
    repetitions after one untimed."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    b.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * n * 4 / (a.elapsed_time(b) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_kernel_GBs": copy_gbs,
            "copy_kernel": "torch elementwise copy, 1 GiB read + 1 GiB written"}


def step_bytes(kind: str, n: int, d: int, m, over: bool = True):
    """Algorithmic bytes of one cache-step (m may be an array).  TOVA-adapted
    ("tova") moves the PyramidKV bytes minus the 4n-byte read of the old
    scores; the caller subtracts that.  A Keyformer step under its budget
    (`over` false: nothing is evicted) reads no Gumbel values."""
    if kind == "keyformer":
        return 2 * n * d + (12 if over else 8) * n + 8 * d + 12 + m * (8 * d + 24)
    return 2 * n * d + 8 * n + 8 * d + 8 + m * (8 * d + 16)


def cpu_baseline(w, budgets, seconds: float):
    """The CPU oracle stepping caches of the same workload at their steady state."""
    from concurrent.futures import ProcessPoolExecutor
    procs = max(1, min(16, os.cpu_count() or 1))
    layers = [l % w.layers for l in range(procs)]
    with ProcessPoolExecutor(procs) as ex:
        res = list(ex.map(_cpu_worker, [(w, l, budgets[l], seconds / 2) for l in layers]))
    one = _cpu_worker((w, layers[0], budgets[layers[0]], seconds / 2))
    steps_all = sum(r[0] for r in res)
    wall_all = max(r[1] for r in res)
    return {
        "value": steps_all / wall_all, "unit": "cache-row updates/s", "cores": procs,
        "kind": "oracle", "single_core": one[0] / one[1],
        "sample": (f"{procs} caches (one per process, layers {layers[0]}..{layers[-1]}), each "
                   f"from a synthetic steady state at its layer budget, stepped token by token "
                   f"for ~{seconds / 2:.0f} s; single_core = one such cache alone"),
        "cpu": cpu_model(),
    }


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _cpu_worker(args):
    w, layer, budget, seconds = args
    import numpy as np
    import synth
    from oracle.guard import params_for
    from oracle.states import random_state
    c = random_state(w, layer, 0, budget, budget + 1, w.prompt)
    prm = params_for(w, budget, 0)
    ks, vs = synth.token_kv(w, layer, 0, np.arange(w.prompt, w.prompt + 4096))
    t0 = time.perf_counter()
    steps = 0
    while time.perf_counter() - t0 < seconds and steps < len(ks):
        c.step(ks[steps], vs[steps], prm)
        steps += 1
    return steps, time.perf_counter() - t0


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the eviction step shards with no exchange; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)
    import dataclasses
    import numpy as np
    import torch
    import synth
    import kv_cache_eviction_step_amd as kve

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.config]
    if args.tova or args.recent:
        w = dataclasses.replace(w, kind="tova" if args.tova else w.kind, recent=args.recent,
                                name=w.name + ("-tova" if args.tova else "") +
                                (f"-recent{args.recent}" if args.recent else ""))
    kf = w.kind == "keyformer"
    budgets = w.budgets(kve.pyramid_budgets)
    L, bh, d = w.layers, w.bh, w.d
    layers = [kve.Layer.empty(bh, b + 1, d, dev, gumbel=kf) for b in budgets]
    cls = [x.c_struct() for x in layers]
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    pos0 = w.prompt
    TPC = args.tokens_per_call
    if w.recent > 0 and args.fill == "synthetic" and args.warmup < w.recent:
        # The synthetic state's scores are random: until `recent` tokens have
        # passed, the rows leaving the window are synthetic rows at random
        # depths (a transient that moves half the cache per step).  Warm up
        # past it; the JSON reports the warmup used.
        args.warmup = -(-w.recent // TPC) * TPC
    if TPC < 1 or TPC > 128 or (not args.whole_run and (args.steps % TPC or args.warmup % TPC)):
        print("--tokens-per-call must be 1..128 and divide --steps and --warmup",
              file=sys.stderr)
        sys.exit(2)

    # ---- the calls: named entry points, or kve_step for the extensions --------
    use_policy = w.kind == "tova" or w.recent > 0
    pol = (kve.policy(w.kind, w.n_sink, w.recent, w.tau_init, w.tau_end, w.anneal_steps,
                      w.rope_base, w.gumbel_seed) if use_policy else None)
    name = "keyformer" if kf else "pyramid"
    if args.batched:
        batch = kve.LayerBatch(layers, budgets)
        singles = None
        entry = ("kve_step" if use_policy else
                 f"{name}_step_layers" + ("_tokens" if TPC > 1 else ""))
    else:
        batch = None
        singles = [kve.LayerBatch([layers[l]], [budgets[l]]) for l in range(L)]
        entry = "kve_step" if use_policy else f"{name}_step" + ("_tokens" if TPC > 1 else "")

    def ctr(l):
        return batch.ctrs[l] if batch is not None else singles[l].ctrs[0]

    def call(nk, nv, s0, S, ev_out=None):
        """Tokens s0 .. s0+S-1 of nk/nv ([L, tokens, bh, d]) through every layer;
        ev_out: None or [L, S, bh]."""
        if batch is not None:
            ks, vs = nk[:, s0:s0 + S], nv[:, s0:s0 + S]
            if use_policy:
                kve.step(batch, ks, vs, pol, ev_out, n_tokens=S)
            elif S > 1 and kf:
                kve.keyformer_step_layers_tokens(batch, ks, vs, w.n_sink, w.tau_init,
                                                 w.tau_end, w.anneal_steps, w.rope_base,
                                                 w.gumbel_seed, ev_out, n_tokens=S)
            elif S > 1:
                kve.pyramid_step_layers_tokens(batch, ks, vs, w.n_sink, w.rope_base, ev_out,
                                               n_tokens=S)
            elif kf:
                kve.keyformer_step_layers(batch, ks[:, 0], vs[:, 0], w.n_sink, w.tau_init,
                                          w.tau_end, w.anneal_steps, w.rope_base, w.gumbel_seed,
                                          ev_out[:, 0] if ev_out is not None else None)
            else:
                kve.pyramid_step_layers(batch, ks[:, 0], vs[:, 0], w.n_sink, w.rope_base,
                                        ev_out[:, 0] if ev_out is not None else None)
            return
        for l in range(L):
            ks, vs = nk[l, s0:s0 + S], nv[l, s0:s0 + S]
            e_l = ev_out[l] if ev_out is not None else None
            c = singles[l].ctrs[0]
            if use_policy:
                kve.step(singles[l], ks[None], vs[None], pol,
                         e_l[None] if e_l is not None else None, n_tokens=S)
            elif S > 1 and kf:
                kve.keyformer_step_tokens(layers[l], ks, vs, c, budgets[l], w.n_sink,
                                          w.tau_init, w.tau_end, w.anneal_steps, w.rope_base,
                                          w.gumbel_seed, e_l, c_layer=cls[l])
            elif S > 1:
                kve.pyramid_step_tokens(layers[l], ks, vs, c, budgets[l], w.n_sink, w.rope_base,
                                        e_l, c_layer=cls[l])
            elif kf:
                kve.keyformer_step(layers[l], ks[0], vs[0], c, budgets[l], w.n_sink, w.tau_init,
                                   w.tau_end, w.anneal_steps, w.rope_base, w.gumbel_seed,
                                   e_l[0] if e_l is not None else None, c_layer=cls[l])
            else:
                kve.pyramid_step(layers[l], ks[0], vs[0], c, budgets[l], w.n_sink, w.rope_base,
                                 e_l[0] if e_l is not None else None, c_layer=cls[l])

    def set_counters(l, c):
        if batch is not None:
            batch.ctrs[l] = c
        else:
            singles[l].ctrs[0] = c

    stream = torch.cuda.current_stream(dev)
    if args.whole_run:
        whole_run(args, w, budgets, bh, L, d, TPC, call, ctr, batch, entry, stream, gen, dev)
        return

    # ---- reach the steady state (untimed) ------------------------------------
    t_fill = time.time()
    if args.fill == "synthetic":
        for l in range(L):
            x = layers[l]
            synth.bulk_state_torch(x.k, x.v, x.scores, x.gumbel, x.positions, budgets[l], w, gen)
            set_counters(l, kve.Counters(budgets[l], pos0, pos0))
    else:
        # the prompt through the same calls as the timed steps
        chunk = 64 * TPC if TPC > 1 else 64
        for t0 in range(0, w.prompt, chunk):
            cnt = min(chunk, w.prompt - t0)
            ins_k = torch.empty((L, cnt, bh, d), dtype=torch.float16, device=dev)
            ins_v = torch.empty_like(ins_k)
            for l in range(L):
                ins_k[l], ins_v[l] = synth.bulk_kv_torch(w, t0, cnt, bh, gen, dev)
            for s0 in range(0, cnt, TPC):
                call(ins_k, ins_v, s0, min(TPC, cnt - s0))
    torch.cuda.synchronize()
    t_fill = time.time() - t_fill

    # ---- inputs for warmup + timed steps, resident in HBM ----------------------
    S = args.warmup + args.steps
    # [L, S, bh, d]: each layer's tokens contiguous, so that any run of TPC
    # tokens of a layer is one contiguous [TPC, bh, d] block
    nk = torch.empty((L, S, bh, d), dtype=torch.float16, device=dev)
    nv = torch.empty_like(nk)
    for l in range(L):
        nk[l], nv[l] = synth.bulk_kv_torch(w, pos0, S, bh, gen, dev)
    ev = torch.full((L, args.steps, bh), -9, dtype=torch.int32, device=dev)
    n_prev = np.zeros((args.steps, L), dtype=np.int64)
    torch.cuda.synchronize()

    for s0 in range(0, args.warmup, TPC):
        call(nk, nv, s0, TPC)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # rows stored before each timed step (byte model), from the counters now:
    # every step adds one row up to the layer's budget
    bud = np.asarray(budgets, dtype=np.int64)
    nk0 = np.fromiter((ctr(l).n_kept for l in range(L)), dtype=np.int64, count=L)
    n_prev[:] = np.minimum(nk0[None, :] + np.arange(args.steps, dtype=np.int64)[:, None],
                           bud[None, :])
    torch.cuda.synchronize()
    e0.record(stream)
    for s0 in range(0, args.steps, TPC):
        call(nk, nv, args.warmup + s0, TPC, ev[:, s0:s0 + TPC])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)

    # ---- algorithmic bytes from the eviction log --------------------------------
    evn = ev.cpu().numpy().transpose(1, 0, 2)              # [steps, L, bh]
    total_bytes = 0
    for s in range(args.steps):
        for l in range(L):
            n = int(n_prev[s, l])
            e = evn[s, l]
            m = np.where((e >= 0) & (e < n), n - e, 0).astype(np.int64)
            total_bytes += int(step_bytes(w.kind, n, d, m).sum())
            if w.kind == "tova":                # the old scores are not read
                total_bytes -= 4 * n * bh
    launches = (args.steps // TPC) * (1 if batch is not None else L)
    mean_m = float(np.where(evn >= 0, np.maximum(0, n_prev[:, :, None] - evn), 0).mean())

    kernel = "step_layers_kernel" if batch is not None or TPC > 1 else "step_kernel"
    traffic = measured_traffic(w.name, kernel, launch_mode(args.batched, TPC))
    out = result_line(args, w, budgets, bh, L, d, TPC, batch, entry, args.steps, args.warmup,
                      ms, launches, total_bytes, mean_m, traffic, kernel)
    out["config"]["steady_state_fill"] = args.fill
    out["config"]["fill_seconds"] = round(t_fill, 1)
    out["context"] = bandwidth_context(dev)
    if not args.skip_whole_run:
        # the same calls again from empty caches (the tensors are reused: a
        # cache reads only its first n_kept rows), CPU baseline not repeated
        del nk, nv, ev
        for l in range(L):
            set_counters(l, kve.Counters(0, 0, 0))
        wr_args = argparse.Namespace(**{**vars(args), "cpu_seconds": 0})
        wr = whole_run(wr_args, w, budgets, bh, L, d, TPC, call, ctr, batch, entry, stream, gen,
                       dev, print_line=False)
        out["whole_run"] = {
            "value": wr["value"], "unit": wr["unit"], "tokens": w.tokens,
            "seconds": wr["steps"] * wr["ms_per_step"] / 1e3,
            "achieved_GBs": wr["roofline"]["achieved"], "frac": wr["roofline"]["frac"],
            "avg_launch_us": wr["roofline"]["avg_launch_us"],
            "mean_rows_moved_per_cache_step": wr["config"]["mean_rows_moved_per_cache_step"],
            "timing": wr["config"]["timing"],
        }
    print(json.dumps(out), flush=True)


def result_line(args, w, budgets, bh, L, d, TPC, batch, entry, steps, warmup, ms, launches,
                total_bytes, mean_m, traffic, kernel):
    """The JSON result (without the fill fields), CPU baseline included."""
    kf = w.kind == "keyformer"
    sec = ms / 1e3
    avg_launch_s = sec / launches
    bytes_per_launch = total_bytes / launches
    achieved = bytes_per_launch / avg_launch_s / 1e9
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, budgets, args.cpu_seconds)
    return {
        "metric": "cache-row updates/sec (B·L·H·tokens) and achieved HBM GB/s vs peak, 1 GPU",
        "value": bh * L * steps / sec,
        "unit": "cache-row updates/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.batch} layers={L} "
                        f"kv_heads={w.kv_heads} D={d} {w.kind} budget="
                        f"{'pyramid avg ' if w.kind == 'pyramid' else ''}{w.budget} "
                        f"n_sink={w.n_sink}",
            "policy": {"score": "current (TOVA)" if w.kind == "tova" else "cumulative",
                       "gumbel": kf, "recent": w.recent, "n_sink": w.n_sink},
            "kv_storage": "f16", "bh_per_launch": bh, "layers": L,
            "budgets": [budgets[0], budgets[-1]],
            "mean_rows_moved_per_cache_step": mean_m,
            "launch": (f"one launch per {TPC} token(s) "
                       f"{'over all layers' if batch is not None else 'per layer'} ({entry})"),
            "tokens_per_launch": TPC, "layers_per_launch": L if batch is not None else 1,
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
            "kernel": "kve::" + kernel,
            "avg_launch_us": avg_launch_s * 1e6,
            "algorithmic_bytes_per_launch": bytes_per_launch,
        },
        "cpu_baseline": cpu,
    }


def whole_run(args, w, budgets, bh, L, d, TPC, call, ctr, batch, entry, stream, gen, dev,
              print_line: bool = True):
    """The whole trajectory -- every prompt token appended one by one, then the
    decode tokens -- from empty caches.  Inputs are generated on the device 64
    tokens (all layers) at a time, between the timed parts: HIP events bracket
    each chunk's launches and the chunks' times are summed."""
    import numpy as np
    import torch
    import synth
    T = w.tokens
    chunk = -(-64 // TPC) * TPC
    ins_k = torch.empty((L, chunk, bh, d), dtype=torch.float16, device=dev)
    ins_v = torch.empty_like(ins_k)
    ev = torch.empty((L, chunk, bh), dtype=torch.int32, device=dev)
    bud = np.asarray(budgets, dtype=np.int64)
    marks, m_sums, n_all = [], [], []
    launches = 0
    for t0 in range(0, T, chunk):
        cnt = min(chunk, T - t0)
        for l in range(L):
            synth.bulk_kv_torch(w, t0, cnt, bh, gen, dev, out_k=ins_k[l, :cnt],
                                out_v=ins_v[l, :cnt])
        # rows stored before each step of the chunk (byte model), outside the
        # timed part: every step adds one row up to the layer's budget
        nk0 = np.fromiter((ctr(l).n_kept for l in range(L)), dtype=np.int64, count=L)
        n_prev = np.minimum(nk0[None, :] + np.arange(cnt, dtype=np.int64)[:, None], bud[None, :])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for s0 in range(0, cnt, TPC):
            call(ins_k, ins_v, s0, min(TPC, cnt - s0), ev[:, s0:s0 + min(TPC, cnt - s0)])
        b.record(stream)
        launches += -(-cnt // TPC) * (1 if batch is not None else L)
        marks.append((a, b))
        # rows moved per (layer, token), summed over the caches (outside the events)
        npt = torch.from_numpy(np.ascontiguousarray(n_prev.T)).to(dev)[:, :, None]
        e = ev[:, :cnt].to(torch.int64)
        m_sums.append(torch.where((e >= 0) & (e < npt), npt - e, 0).sum(dim=2).cpu().numpy())
        n_all.append(n_prev.T.copy())
    torch.cuda.synchronize()
    ms = sum(x.elapsed_time(y) for x, y in marks)
    n_prev = np.concatenate(n_all, axis=1)                 # [L, T]
    m_sum = np.concatenate(m_sums, axis=1)                 # [L, T]
    over = n_prev + 1 > bud[:, None]
    base = step_bytes(w.kind, n_prev, d, 0, over=True)
    if w.kind == "keyformer":
        base = np.where(over, base, step_bytes(w.kind, n_prev, d, 0, over=False))
    total_bytes = int((base * bh).sum()) + int((m_sum * (8 * d + (24 if w.kind == "keyformer"
                                                                    else 16))).sum())
    if w.kind == "tova":
        total_bytes -= int((4 * n_prev * bh).sum())
    mean_m = float(m_sum.sum() / (L * T * bh))
    kernel = "step_layers_kernel" if batch is not None or TPC > 1 else "step_kernel"
    out = result_line(args, w, budgets, bh, L, d, TPC, batch, entry, T, 0, ms, launches,
                      total_bytes, mean_m, None, kernel)
    out["config"]["timing"] = (f"whole run: {w.prompt} prompt + {w.decode} decode tokens from "
                               f"empty caches, HIP events around the launches of each "
                               f"{chunk}-token chunk, summed")
    if print_line:
        print(json.dumps(out), flush=True)
    return out


if __name__ == "__main__":
    main()
