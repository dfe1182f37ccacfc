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
    ap.add_argument("--fill-tokens-per-call", type=int, default=0,
                    help="with --fill real: tokens per launch of the prompt (default: "
                         "--tokens-per-call), e.g. 32 to ingest the prompt as a model would")
    ap.add_argument("--workspace", action="store_true",
                    help="single-token launches through kve_step_ws with a workspace sized for "
                         "every move (long compactions handed to the move kernel)")
    ap.add_argument("--skip-late-riser", action="store_true",
                    help="leave out the 8B-shaped late-riser decode object of the default line")
    ap.add_argument("--late-riser-only", action="store_true",
                    help="run only the 8B-shaped late-riser object (prompt, then the three "
                         "decode forms) and print it")
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
                  "kv_cache_eviction_step_amd/csrc/kve_step.h",
                  "kv_cache_eviction_step_amd/csrc/kve_move_plan.h"]


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


def launch_mode(batched: bool, tokens_per_call: int, workspace: bool = False) -> str:
    return (("all-layers" if batched else "per-layer") + f"_x{tokens_per_call}tok" +
            ("_ws" if workspace and tokens_per_call == 1 else ""))


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
    del dst
    # a read stream: row sums of 4 GiB of fp32 in rows of 1024 (4 GiB read, 4
    # MiB written; the eviction step reads far more than it writes)
    big = torch.ones(((1 << 32) // 4 // 1024, 1024), dtype=torch.float32, device=dev)
    acc = torch.empty(big.shape[0], dtype=torch.float32, device=dev)
    torch.sum(big, dim=1, out=acc)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        torch.sum(big, dim=1, out=acc)
    b.record()
    torch.cuda.synchronize()
    read_gbs = 5 * big.numel() * 4 / (a.elapsed_time(b) / 1e3) / 1e9
    del src, big, acc
    torch.cuda.empty_cache()
    return {"copy_kernel_GBs": copy_gbs,
            "copy_kernel": "torch elementwise copy, 1 GiB read + 1 GiB written",
            "read_kernel_GBs": read_gbs,
            "read_kernel": "torch row sums of 4 GiB of fp32, rows of 1024 (4 GiB read)"}


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
        "host_cores": os.cpu_count(), "kind": "oracle", "single_core": one[0] / one[1],
        "sample": (f"{procs} caches (one per process, layers {layers[0]}..{layers[-1]}), each "
                   f"from a synthetic steady state at its layer budget, stepped token by token "
                   f"for ~{seconds / 2:.0f} s; single_core = one such cache alone; "
                   f"{procs} of the host's {os.cpu_count()} cores used, one oracle "
                   f"process each"),
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
    if args.late_riser_only:
        print(json.dumps({"late_riser_8b": late_riser_decode(dev)}), flush=True)
        return
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
    use_policy = w.kind == "tova" or w.recent > 0 or args.workspace
    pol = (kve.policy(w.kind, w.n_sink, w.recent, w.tau_init, w.tau_end, w.anneal_steps,
                      w.rope_base, w.gumbel_seed) if use_policy else None)
    name = "keyformer" if kf else "pyramid"
    general = "kve_step_ws" if args.workspace else "kve_step"
    if args.batched:
        batch = kve.LayerBatch(layers, budgets)
        singles = None
        entry = (general if use_policy else
                 f"{name}_step_layers" + ("_tokens" if TPC > 1 else ""))
    else:
        batch = None
        singles = [kve.LayerBatch([layers[l]], [budgets[l]]) for l in range(L)]
        entry = general if use_policy else f"{name}_step" + ("_tokens" if TPC > 1 else "")
    # one workspace serves every launch (calls on one stream are ordered)
    ws = (kve.workspace(bh * (L if args.batched else 1), max(budgets), d, dev)
          if args.workspace else None)

    def ctr(l):
        return batch.ctrs[l] if batch is not None else singles[l].ctrs[0]

    def call(nk, nv, s0, S, ev_out=None):
        """Tokens s0 .. s0+S-1 of nk/nv ([L, tokens, bh, d]) through every layer;
        ev_out: None or [L, S, bh]."""
        if batch is not None:
            ks, vs = nk[:, s0:s0 + S], nv[:, s0:s0 + S]
            if use_policy:
                kve.step(batch, ks, vs, pol, ev_out, n_tokens=S, workspace=ws)
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
                         e_l[None] if e_l is not None else None, n_tokens=S, workspace=ws)
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
        # the prompt through the same calls as the timed steps (or as many
        # tokens per launch as --fill-tokens-per-call asks)
        FT = args.fill_tokens_per_call or TPC
        chunk = 64 * FT if FT > 1 else 64
        for t0 in range(0, w.prompt, chunk):
            cnt = min(chunk, w.prompt - t0)
            ins_k = torch.empty((L, cnt, bh, d), dtype=torch.float16, device=dev)
            ins_v = torch.empty_like(ins_k)
            for l in range(L):
                ins_k[l], ins_v[l] = synth.bulk_kv_torch(w, t0, cnt, bh, gen, dev)
            for s0 in range(0, cnt, FT):
                call(ins_k, ins_v, s0, min(FT, cnt - s0))
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
    traffic = measured_traffic(w.name, kernel, launch_mode(args.batched, TPC, args.workspace))
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
    if not args.skip_late_riser and not (args.config == 3 or args.tova or args.recent or
                                         args.workspace or args.batched or TPC > 1):
        # the default line also carries the 8B-shaped workload, decoded
        del layers, cls
        batch = singles = None
        torch.cuda.empty_cache()
        out["late_riser_8b"] = late_riser_decode(dev)
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


def late_riser_decode(dev) -> dict:
    """The 8B-shaped late-riser Keyformer workload (B=32, 32 layers, 8 kv-heads,
    D=128, budget 1024, tau 1 -> 2 over 512) as a model serves it: its 4096-token
    prompt ingested 32 tokens per launch over all layers (every prompt key is
    known at once), then its 512 decode tokens one launch per token.  The
    decode is timed in three forms from the same state after the prompt (the
    state is saved and restored between them): all 32 layers per launch
    through kve_step_ws (8192 caches; long moves handed to the move kernel;
    the eviction step run once per token after the forward pass has made every
    layer's new key), one kve_step_ws launch per layer, and one in-place
    keyformer_step launch per layer.  All three must evict the same rows.
    Decode inputs are resident in HBM before each timed region; HIP events on
    the launch stream bracket it.  Bytes follow the Keyformer byte model with
    each cache-step's moved rows taken from the kernel's evicted output."""
    import numpy as np
    import torch
    import synth
    import kv_cache_eviction_step_amd as kve
    w = synth.WORKLOADS[3]
    L, bh, d, B, T = w.layers, w.bh, w.d, w.budget, w.decode
    S = 32
    names = ("k", "v", "scores", "gumbel", "positions")
    layers = [kve.Layer.empty(bh, B + 1, d, dev, gumbel=True) for _ in range(L)]
    batch = kve.LayerBatch(layers, [B] * L)
    gen = torch.Generator(device=dev)
    gen.manual_seed(3031)
    stream = torch.cuda.current_stream(dev)
    kargs = (w.n_sink, w.tau_init, w.tau_end, w.anneal_steps, w.rope_base, w.gumbel_seed)

    # ---- prompt: S tokens per launch over all layers ----------------------------
    G = 512                                            # tokens generated at a time
    pk = torch.empty((L, G, bh, d), dtype=torch.float16, device=dev)
    pv = torch.empty_like(pk)
    pev = torch.empty((L, S, bh), dtype=torch.int32, device=dev)
    marks, m_sum, p_bytes = [], torch.zeros((), dtype=torch.int64, device=dev), 0
    for g0 in range(0, w.prompt, G):
        for l in range(L):
            synth.bulk_kv_torch(w, g0, G, bh, gen, dev, out_k=pk[l], out_v=pv[l])
        for s0 in range(0, G, S):
            t0 = g0 + s0
            n_prev = torch.minimum(torch.arange(t0, t0 + S, device=dev), torch.tensor(B, device=dev))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            kve.keyformer_step_layers_tokens(batch, pk[:, s0:s0 + S], pv[:, s0:s0 + S], *kargs,
                                             pev, n_tokens=S)
            b.record(stream)
            marks.append((a, b))
            e = pev.to(torch.int64)
            npr = n_prev[None, :, None]
            m_sum += torch.where((e >= 0) & (e < npr), npr - e, 0).sum()
            for t in range(t0, t0 + S):
                n = min(t, B)
                p_bytes += L * bh * int(step_bytes("keyformer", n, d, 0, over=n + 1 > B))
    torch.cuda.synchronize()
    p_ms = sum(x.elapsed_time(y) for x, y in marks)
    p_bytes += int(m_sum) * (8 * d + 24)
    del pk, pv, pev
    prompt = {
        "tokens": w.prompt, "tokens_per_launch": S,
        "launch": "keyformer_step_layers_tokens, all 32 layers x 32 tokens per launch",
        "seconds": p_ms / 1e3, "value": bh * L * w.prompt / (p_ms / 1e3),
        "achieved_GBs": p_bytes / (p_ms / 1e3) / 1e9,
        "frac": p_bytes / (p_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "note": "prompt ingestion: each launch re-reads its caches' keys for 32 tokens, "
                "mostly from the last-level cache, so this rate is not an HBM rate",
    }

    # ---- decode: three launch forms from one saved state -------------------------
    dk = torch.empty((L, T, bh, d), dtype=torch.float16, device=dev)
    dv = torch.empty_like(dk)
    for l in range(L):
        synth.bulk_kv_torch(w, w.prompt, T, bh, gen, dev, out_k=dk[l], out_v=dv[l])
    snap = [[getattr(x, nm).clone() for nm in names] for x in layers]
    ctr0 = [batch.ctrs[l].copy() for l in range(L)]
    pol = kve.policy("keyformer", w.n_sink, 0, w.tau_init, w.tau_end, w.anneal_steps,
                     w.rope_base, w.gumbel_seed)
    ws_all = kve.workspace(L * bh, B, d, dev)
    ws_one = kve.workspace(bh, B, d, dev)
    singles = [kve.LayerBatch([layers[l]], [B]) for l in range(L)]
    cls = [x.c_struct() for x in layers]
    views = [[(dk[l, t], dv[l, t]) for t in range(T)] for l in range(L)]

    def restore():
        for x, sn in zip(layers, snap):
            for nm, t in zip(names, sn):
                getattr(x, nm).copy_(t)
        for l in range(L):
            batch.ctrs[l] = ctr0[l].copy()
            singles[l].ctrs[0] = ctr0[l].copy()
        torch.cuda.synchronize()

    # Host time per call: the enqueueing of tokens 1 .. HOST_TOKENS only (token
    # 0 also pays one-time costs such as a kernel's first load).  Over the
    # whole loop the launch queue fills and the host then waits for the GPU,
    # so a longer span would report the GPU's rate, not the host's.
    HOST_TOKENS = 2
    host = {}

    def timed(run_token, key):
        ev = torch.full((T, L, bh), -9, dtype=torch.int32, device=dev)
        evl = [[ev[t, l] for l in range(L)] for t in range(T)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for t in range(T):
            if t == 1:
                h0 = time.perf_counter()
            run_token(t, ev[t], evl[t])
            if t == HOST_TOKENS:
                host[key] = (time.perf_counter() - h0) / HOST_TOKENS   # per token
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), ev

    def all_layers(t, e, _el):
        kve.step(batch, dk[:, t], dv[:, t], pol, e, workspace=ws_all)

    def per_layer_ws(t, _e, el):
        for l in range(L):
            k, v = views[l][t]
            kve.step(singles[l], [k], [v], pol, [el[l]], workspace=ws_one)

    def per_layer_in_place(t, _e, el):
        for l in range(L):
            k, v = views[l][t]
            kve.keyformer_step(layers[l], k, v, singles[l].ctrs[0], B, *kargs, el[l],
                               c_layer=cls[l])

    ms_all, ev_all = timed(all_layers, "all")
    restore()
    ms_ws, ev_ws = timed(per_layer_ws, "ws")
    restore()
    ms_ip, ev_ip = timed(per_layer_in_place, "ip")
    same = bool(torch.equal(ev_all, ev_ws)) and bool(torch.equal(ev_all, ev_ip))
    e = ev_all.to(torch.int64)
    m = torch.where((e >= 0) & (e < B), B - e, 0)
    d_bytes = T * L * bh * int(step_bytes("keyformer", B, d, 0)) + int(m.sum()) * (8 * d + 24)
    mean_m = float(m.double().mean())

    def form(ms, launches, launch, key):
        sec = ms / 1e3
        ach = d_bytes / sec / 1e9
        return {"launch": launch, "value": bh * L * T / sec, "unit": "cache-row updates/s",
                "ms_per_token": ms / T, "avg_launch_us": ms * 1e3 / launches,
                "host_us_per_call": host[key] * 1e6 / (launches / T),
                "achieved_GBs": ach, "frac": ach / PEAK_HBM_GBS}

    dec = form(ms_all, T, "one kve_step_ws launch per token over all 32 layers (8192 caches)",
               "all")
    traffic = measured_traffic(w.name, "step_layers_kernel", "all-layers_x1tok_ws")
    dec["roofline"] = {
        "bound": "hbm", "achieved": dec["achieved_GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": dec["frac"], "traffic": traffic,
        "kernel": "kve::step_layers_kernel + kve::move_kernel",
        "avg_launch_us": dec["avg_launch_us"], "algorithmic_bytes_per_launch": d_bytes / T,
    }
    return {
        "workload": (f"{w.name}: B={w.batch} layers={L} kv_heads={w.kv_heads} D={d} keyformer "
                     f"budget={B} n_sink={w.n_sink} tau {w.tau_init}->{w.tau_end} over "
                     f"{w.anneal_steps}"),
        "prompt": prompt,
        "decode": {"tokens": T, "mean_rows_moved_per_cache_step": mean_m, **dec},
        "decode_per_layer": form(ms_ws, T * L, "one kve_step_ws launch per layer per token "
                                 "(256 caches; long moves handed to the move kernel)", "ws"),
        "decode_per_layer_in_place": form(ms_ip, T * L, "one keyformer_step launch per layer "
                                          "per token (every cache compacts in place)", "ip"),
        "evictions_identical_across_forms": same,
        "timing": "HIP events around the 512 decode tokens of each form, inputs resident; "
                  f"host_us_per_call: the host's enqueueing of tokens 1..{HOST_TOKENS}, per call, "
                  "before the launch queue fills",
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
