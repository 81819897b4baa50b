"""Benchmark of the MoE-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_q4_0] [--no-graph]

A step is one pass of the whole layer (route, permute, grouped SwiGLU FFN, combine) over one batch:
for the default decode workload (T=8, d=2048, E=128, k=8, I=768, Q4_0 banks) a step is 48 independent
layers run back to back on one stream, captured once into a HIP graph and replayed.  Inputs are seeded
synthetic tensors already resident in HBM.  Prints one JSON line.

The dominant unit is the layer call; its average duration is timed with HIP events on the stream
it runs on, over timed eager replays of the same steps, and compared with the HBM and MFMA
rooflines of its algorithmic bytes and flops (the bound is the one with the longer roofline time).
A single-layer decode workload rotates over copies of its bank (at least 4, and at least 1 GB
touched per pass) so that the 256 MB MALL cannot serve it.  The run exits with status 3, printing
nothing, if the one-kernel decode layer reports a dependency wait that gave up.
Beside a decode workload the same run also measures the prefill workload (default: 4096 tokens,
bf16 banks, Zipf routing) and adds it to the line as "prefill" (tokens/s, its own roofline).
The CPU baseline times the scalar oracle on a bounded sample of the same workload on the host
cores (all usable cores up to 16, and one core), with the CPU model.

Other modes print their own line instead: --route-proj (router projection + top-k), --cache SLOTS
(layer steps with the expert cache streaming cold experts from pinned host memory), --residual
(the cold pairs computed on the host cores), --coexec Q (the cold experts of each step split
between the host link and the host cores by load fraction Q).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import routed_expert_ffn_wave_amd as ft  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "routed_expert_ffn_wave_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def build_layers(w: synth.Workload, T: int, n_layers: int, copies: int = 1, flags: int = 0):
    """The step's layers.  copies > 1 (single-layer workloads): the layer is repeated over that many
    copies of its bank and buffers at distinct addresses, run back to back, so that one pass touches
    more bytes than the caches hold (the MALL is 256 MB)."""
    layers = []
    for l in range(n_layers):
        canon = synth.make_bank(w, layer=l, device="cuda")
        bank = ft.ft_moe_pack_bank(canon.fmt, canon.n_slots, canon.d, canon.I, canon.w13, canon.w2, canon.s13,
                                   canon.s2)
        del canon
        slot = synth.slot_table(w, l).cuda()
        logits = synth.logits(w, l, T, device="cuda")
        x = synth.activations(w, l, T, device="cuda")
        for c in range(copies):
            b = bank if c == 0 else ft.DeviceBank(bank.fmt, bank.n_slots, bank.d, bank.I,
                                                  *[None if t is None else t.clone()
                                                    for t in (bank.w13, bank.w2, bank.s13, bank.s2)])
            layer = ft.MoELayer(b, slot.clone(), w.k, T, shared_slot=w.shared_slot, flags=flags)
            layers.append((layer, logits.clone(), x.clone()))
        if (l + 1) % 8 == 0 or l + 1 == n_layers:
            log(f"generated {l + 1}/{n_layers} layers" + (f" ({copies} copies each)" if copies > 1 else ""))
    torch.cuda.synchronize()
    return layers


def run_step(layers):
    for layer, logits, x in layers:
        layer.forward(logits, x)


def check_status(layers, what: str):
    """Exit non-zero if the one-kernel decode path of any layer reports a dependency wait that gave up
    (its results would be invalid, so no figure of the run may be printed)."""
    bad = [i for i, (layer, _, _) in enumerate(layers) if layer.status_word() != 0]
    if bad:
        log(f"{what}: status word set in layer(s) {bad[:8]}: a dependency wait of the fused kernel gave up")
        sys.exit(3)


def algorithmic_work(w: synth.Workload, layers, T: int):
    """Per layer call, averaged over the layers, from the actual routing of each layer:
    bytes = touched resident experts (+ shared) x stored bytes per expert + x + logits + out,
    flops = 2 * 3 * d * I per computed (token, expert) pair."""
    per_expert = synth.expert_bytes(w.fmt, w.d, w.I)
    tot_b, tot_f, tot_pairs, tot_touched = 0.0, 0.0, 0, 0
    for layer, _, _ in layers:
        counts = layer.counts.cpu()
        slot = layer.slot_of.cpu()
        resident = slot >= 0
        touched = int(((counts > 0) & resident).sum()) + (1 if w.shared else 0)
        pairs = int(counts[resident].sum()) + (T if w.shared else 0)
        tot_touched += touched
        tot_pairs += pairs
        tot_b += touched * per_expert + T * w.d * 2 + T * w.E * 4 + T * w.d * layer.out.element_size()
        tot_f += 2.0 * 3.0 * w.d * w.I * pairs
    n = len(layers)
    return tot_b / n, tot_f / n, tot_pairs / n, tot_touched / n


def time_layer_calls(layers, reps: int):
    """Average duration of one layer call (ft_moe_layer: its kernels back to back), with HIP events
    recorded on the stream the kernels run on, over eager passes through the layers."""
    s = torch.cuda.current_stream()
    evs = []
    for _ in range(reps):
        for layer, logits, x in layers:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            layer.forward(logits, x, stream=s)
            e1.record(s)
            evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return sum(ms) / len(ms) * 1e3  # us


def host_cpu():
    """Model name of the host CPU, the cores the OS reports and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return model, os.cpu_count() or 1, usable


def cpu_baseline(w: synth.Workload, T: int, budget_s: float, workers: int = 1, max_layers: int | None = None):
    """Time the scalar oracle on host cores over whole layers of the same workload until the budget
    is used (at least one layer); workers > 1 runs its expert groups on that many threads."""
    import oracle
    t_total, n = 0.0, 0
    limit = w.layers if max_layers is None else min(w.layers, max_layers)
    while t_total < budget_s and n < limit:
        li = synth.layer_inputs(w, layer=n, T=T, device="cuda")
        bank_cpu = li.bank.to("cpu")
        L, x, so = li.logits.cpu(), li.x.cpu(), li.slot_of_expert.cpu()
        del li
        t0 = time.perf_counter()
        oracle.layer(L, x, bank_cpu, so, w.k, shared_slot=w.shared_slot, workers=workers)
        t_total += time.perf_counter() - t0
        n += 1
    return t_total, n


def cpu_baseline_record(w: synth.Workload, T: int, budget_s: float, decode: bool):
    """The oracle on the host cores (all the cores this process may use, at most the 16 of a one-GPU
    share), and on one core, each over whole layers within its share of the budget."""
    model, nproc, usable = host_cpu()
    workers = max(1, min(16, usable))

    def rate(t, n):
        return round(t / n * 1e6, 1) if decode else round(T * n / t, 3)
    t_all, n_all = cpu_baseline(w, T, budget_s / 2, workers=workers)
    t_one, n_one = cpu_baseline(w, T, budget_s / 2, workers=1)
    rec = {"value": rate(t_all, n_all), "unit": "us/layer" if decode else "tokens/s", "cores": workers,
           "kind": "oracle",
           "sample": f"{n_all} whole layer(s) of {w.name} (T={T}), scalar C oracle, expert groups on {workers} threads",
           "single_core": {"value": rate(t_one, n_one), "cores": 1,
                           "sample": f"{n_one} whole layer(s), one thread"},
           "cpu_model": model, "nproc": nproc, "usable_cores": usable}
    log(f"cpu baseline {rec}")
    return rec


def copy_probe(nbytes: int, reps: int = 5):
    """A plain elementwise copy of known size (fp32 negation: reads and writes `nbytes` each),
    the calibration kernel for the HBM byte counters."""
    src = torch.randn(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} x neg over {nbytes} bytes")


def _pmc_per_kernel(path: str, counter: str):
    """Average value of one counter per dispatch, by kernel name, from a rocprofv3 counter CSV."""
    import csv
    acc = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            a = acc.setdefault(row["Kernel_Name"], [0.0, 0])
            a[0] += float(row["Counter_Value"])
            a[1] += 1
    return {k: (v[0] / v[1], v[1]) for k, v in acc.items()}


def traffic_key(workload: str, T: int) -> str:
    return f"{workload}@T{T}"


def pmc_summary(workload: str, T: int, fetch_csv: str, write_csv: str, copy_bytes: int, out_json: str):
    """HBM bytes per layer call from two counter runs (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by what the counter reads for the copy probe of known size: the bytes of
    every dispatch of the layer's kernels divided by the number of layer calls."""
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    copy_f = [v for k, v in fetch.items() if "neg_kernel" in k]
    copy_w = [v for k, v in write.items() if "neg_kernel" in k]
    assert copy_f and copy_w, "the copy probe was not profiled"
    kib = copy_bytes / 1024.0
    f_fetch, f_write = kib / copy_f[0][0], kib / copy_w[0][0]
    kernels = {}
    for name, (v, n) in fetch.items():
        if "ftk::" not in name or "pack" in name or "dequant" in name or "interleave" in name:
            continue
        wv = write.get(name, (0.0, 0))[0]
        kernels[name] = {"dispatches": n, "fetch_kib": round(v, 1), "write_kib": round(wv, 1),
                         "fetch_bytes": round(v * 1024 * f_fetch), "write_bytes": round(wv * 1024 * f_write)}
    # every layer call launches exactly one routing kernel or one fused decode-layer kernel
    calls = sum(k["dispatches"] for name, k in kernels.items() if "route_kernel" in name or "layer_decode" in name)
    assert calls > 0, "no routing kernel in the counter run"
    per_call = lambda key: round(sum(k[key] * k["dispatches"] for k in kernels.values()) / calls)
    rec = {"T": T, "source_hash": kernel_source_hash(), "copy_probe_bytes": copy_bytes,
           "copy_factor_fetch": round(f_fetch, 5), "copy_factor_write": round(f_write, 5), "kernels": kernels,
           "layer_calls": calls, "fetch_bytes_per_call": per_call("fetch_bytes"),
           "write_bytes_per_call": per_call("write_bytes")}
    rec["bytes_per_call"] = rec["fetch_bytes_per_call"] + rec["write_bytes_per_call"]
    db = json.load(open(out_json)) if os.path.exists(out_json) else {}
    db[traffic_key(workload, T)] = rec
    with open(out_json, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def calibrate():
    """The device's achievable rates against the published peaks: a 4 GiB streaming read over every
    CU (HBM), a 1 GiB read of pinned host memory by the cache fill's 8 blocks (host link), and
    register-only MFMA loops (bf16, e4m3 x e4m3, e2m3 x e2m1).  Own JSON line."""
    r = ft.ft_moe_measure_rates(dev_bytes=4 << 30, host_bytes=1 << 30, reps=5)
    peaks = {"hbm_read_gbs": HBM_PEAK_GBS, "host_read_gbs": PCIE_PEAK_GBS, "mfma_bf16_tflops": MFMA_PEAK_TFLOPS["bf16"],
             "mfma_fp8_tflops": MFMA_PEAK_TFLOPS["fp8"], "mfma_fp6_fp4_tflops": MFMA_PEAK_TFLOPS["fp4"]}
    rates = {k: {"achieved": round(r[k], 1), "peak": p, "frac": round(r[k] / p, 4)} for k, p in peaks.items()}
    log(f"rates: {rates}; MFMA clock implied by the bf16 rate {r['mfma_clock_ghz']:.3f} GHz")
    print(json.dumps({"metric": "achievable device rates (ft_moe_measure_rates)", "value": round(r["hbm_read_gbs"], 1),
                      "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "vs_baseline": None,
                      "data": "synthetic", "rates": rates, "mfma_clock_ghz": round(r["mfma_clock_ghz"], 3),
                      "compute_units": r["compute_units"], "stream_blocks": r["stream_blocks"]}), flush=True)


def bench_layer_proj(w: synth.Workload, T: int, n_layers: int, steps: int, warmup: int):
    """The decode layer from its activations (router projection + layer) over the workload's layers,
    each way captured into a HIP graph and replayed: ft_moe_route_proj then ft_moe_layer (two
    launches per layer), and ft_moe_layer_proj (the projection inside the one launch).  Own JSON
    line: value = us per layer of the one-launch form."""
    layers = build_layers(w, T, n_layers)
    wrs = [synth.router_rows(w, l, device="cuda") for l in range(n_layers)]
    xs = [x for _, _, x in layers]
    lgs = [torch.empty(T, w.E, dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    rws = [torch.zeros(max(ft.ft_moe_route_proj_workspace(T), 16), dtype=torch.uint8, device="cuda")
           for _ in range(n_layers)]
    ids = torch.empty(T, w.k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, w.k, dtype=torch.float32, device="cuda")

    def two():
        for (layer, _, x), wr, lg, rw in zip(layers, wrs, lgs, rws):
            ft.ft_moe_route_proj(x, wr, w.k, logits=lg, ids=ids, w=wt, ws=rw)
            layer.forward(lg, x)

    def one():
        for (layer, _, x), wr in zip(layers, wrs):
            layer.forward_proj(x, wr)

    res = {}
    for name, fn in (("route_proj_then_layer", two), ("layer_proj", one)):
        for _ in range(max(warmup, 1)):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s):
                fn()
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / steps / n_layers * 1e6
        check_status(layers, name)
        del graph
    log(f"layer from x: {res}")
    print(json.dumps({"metric": "MoE-layer decode latency from the activations (router projection + layer)",
                      "value": round(res["layer_proj"], 3), "unit": "us/layer", "n_gpus": 1, "steps": steps,
                      "warmup": warmup, "higher_is_better": False, "vs_baseline": None, "data": "synthetic (seeded)",
                      "config": {"workload": w.name, "T": T, "d": w.d, "E": w.E, "k": w.k, "I": w.I,
                                 "bank_format": synth.FMT_NAMES[w.fmt], "layers_per_step": n_layers, "graph": True},
                      "us_per_layer": {k: round(v, 3) for k, v in res.items()}}), flush=True)


def bench_route_proj(w: synth.Workload, T: int, steps: int, warmup: int):
    """Router projection + route (ft_moe_route_proj) on the workload's shape: one call is one step;
    printed as its own JSON line (the step before the layer, not part of the layer's metric)."""
    x = synth.activations(w, 0, T, device="cuda")
    wr = synth.router_rows(w, 0, device="cuda")
    ws = torch.zeros(max(ft.ft_moe_route_proj_workspace(T), 16), dtype=torch.uint8, device="cuda")
    logits = torch.empty(T, w.E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, w.k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, w.k, dtype=torch.float32, device="cuda")
    call = lambda: ft.ft_moe_route_proj(x, wr, w.k, logits=logits, ids=ids, w=wt, ws=ws)  # noqa: E731
    for _ in range(max(warmup, 1)):
        call()
    torch.cuda.synchronize()
    reps = max(steps, 1) * 10
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        call()
    b.record(s)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    nbytes = T * w.d * 2 + w.E * w.d * 2 + T * w.E * 4 + T * w.k * 8
    flops = 2.0 * T * w.E * w.d
    hbm = nbytes / (us * 1e-6) / 1e9
    tf = flops / (us * 1e-6) / 1e12
    decode = T <= 64
    roof = ({"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(hbm / HBM_PEAK_GBS, 4)}
            if decode else
            {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
             "frac": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4)})
    roof.update({"traffic": None, "kernel": "route_proj_kernel (router projection on MFMA + top-k, one launch)",
                 "per_call_us": round(us, 3), "algorithmic_bytes_per_call": nbytes, "algorithmic_flops_per_call": int(flops)})
    print(json.dumps({"metric": "router projection + top-k latency", "value": round(us, 3), "unit": "us/call",
                      "n_gpus": 1, "steps": reps, "warmup": warmup, "ms_per_step": round(us / 1e3, 5),
                      "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                      "data": "synthetic (seeded)",
                      "config": {"workload": f"route_proj/{w.name}", "T": T, "d": w.d, "E": w.E, "k": w.k},
                      "roofline": roof, "cpu_baseline": None}), flush=True)


PCIE_PEAK_GBS = 63.0   # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8


def bench_cache(w: synth.Workload, T: int, steps: int, warmup: int, n_slots: int, max_loads: int):
    """Layer steps with the global LRU expert cache: route, permute and the cache update on the main
    stream; the fill of the chosen experts from pinned host memory on a second stream beside the
    grouped FFN and combine (which use the step's compute_slot); the streams join at the end of the
    step.  Logits change every step over one Zipf popularity order.  Printed as its own JSON line:
    value = bytes the fill kernel moved per second of its own duration (the dominant kernel here,
    bound by the host link)."""
    full_w = w.replace(n_resident=None, shared=False)
    log(f"cache: {w.name} T={T} E={w.E} slots={n_slots} max_loads={max_loads}; packing {w.E} experts")
    c = synth.make_bank(full_w, 0, device="cuda")
    full = ft.ft_moe_pack_bank(c.fmt, w.E, c.d, c.I, c.w13, c.w2, c.s13, c.s2)
    del c
    src = full.to_pinned_host()
    del full
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    dst = ft.DeviceBank.empty(w.fmt, n_slots, w.d, w.I)
    cache = ft.ExpertCache(w.E, n_slots, max_loads)
    n_seq = warmup + steps
    logits = [synth.step_logits(w, i, T, device="cuda") for i in range(n_seq)]
    x = synth.activations(w, 0, T, device="cuda")
    k, E = w.k, w.E
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    gather = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pws = torch.empty(max(ft.ft_moe_permute_workspace(T, E, k), 16), dtype=torch.uint8, device="cuda")
    y = torch.empty(T * k, w.d, dtype=torch.bfloat16, device="cuda")
    fws = torch.empty(max(ft.ft_moe_grouped_ffn_workspace(dst, T, E, k), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, w.d, dtype=torch.float32, device="cuda")
    mask = torch.empty(T, dtype=torch.int32, device="cuda")
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    nl_hist = torch.zeros(n_seq, dtype=torch.int32, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    marks = [(ev(), ev(), ev(), ev(), ev()) for _ in range(n_seq)]

    def step(i, fill=True):
        t0, f0, f1, g0, g1 = marks[i]
        t0.record(main)
        ft.ft_moe_route(logits[i], k, ids=ids, w=wt)
        ft.ft_moe_permute(ids, E, counts=counts, offsets=offsets, gather=gather, inv=inv, ws=pws)
        cs, _, nl = cache.update(counts)
        if fill:
            side.wait_stream(main)
            f0.record(side)
            cache.fill(src, dst, stream=side)
            f1.record(side)
        g0.record(main)
        ft.ft_moe_grouped_ffn(dst, cs, x, k, offsets, gather, y_sorted=y, ws=fws)
        ft.ft_moe_combine(y, None, ids, wt, inv, cs, w.d, out=out, residual_mask=mask)
        g1.record(main)
        if fill:
            main.wait_stream(side)
        nl_hist[i:i + 1].copy_(nl)

    def run(fill):
        for i in range(warmup):
            step(i, fill)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(main)
        for i in range(warmup, n_seq):
            step(i, fill)
        b.record(main)
        torch.cuda.synchronize()
        ffn = sum(marks[i][3].elapsed_time(marks[i][4]) for i in range(warmup, n_seq)) * 1e3 / steps
        return a.elapsed_time(b) * 1e3 / steps, ffn

    step_us, ffn_us = run(True)
    fill_us = sum(marks[i][1].elapsed_time(marks[i][2]) for i in range(warmup, n_seq)) * 1e3 / steps
    nls = nl_hist[warmup:].cpu().numpy()
    # the same steps again without the fill (the cache tables still advance; the slots keep what
    # they hold): the grouped FFN and combine alone on the device, for the slowdown beside the fill
    _, ffn_alone_us = run(False)
    per_expert = sum(ft.ft_moe_bank_bytes(w.fmt, 1, w.d, w.I, which) for which in range(4))
    moved = float(nls.sum()) * per_expert
    gbs = moved / (fill_us * steps * 1e-6) / 1e9 if fill_us > 0 else 0.0
    log(f"cache: {nls.sum()} loads over {steps} steps ({moved / 1e6:.1f} MB); fill {fill_us:.1f} us/step, "
        f"FFN+combine {ffn_us:.1f} us/step beside it ({ffn_alone_us:.1f} alone), whole step {step_us:.1f} us")
    roof = {"bound": "pcie", "achieved": round(gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / PCIE_PEAK_GBS, 4), "traffic": None,
            "kernel": "cache_fill_kernel (pinned host bank -> device slots, 8 blocks)",
            "bytes_per_expert": per_expert, "loads": int(nls.sum()), "fill_us_per_step": round(fill_us, 2),
            "ffn_combine_us_per_step": round(ffn_us, 2), "ffn_combine_us_alone": round(ffn_alone_us, 2),
            "ffn_slowdown_beside_fill": round(ffn_us / ffn_alone_us, 3) if ffn_alone_us > 0 else None,
            "step_us": round(step_us, 2)}
    print(json.dumps({"metric": "expert streaming bandwidth (fill kernel)", "value": round(gbs, 2), "unit": "GB/s",
                      "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(step_us / 1e3, 5),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                      "dtype": synth.FMT_NAMES[w.fmt], "data": "synthetic (seeded)",
                      "config": {"workload": f"cache/{w.name}", "T": T, "E": E, "k": k, "d": w.d, "I": w.I,
                                 "slots": n_slots, "max_loads": max_loads},
                      "roofline": roof, "cpu_baseline": None}), flush=True)


def bench_residual(w: synth.Workload, T: int, steps: int, warmup: int, threads: int):
    """The layer with its cold experts: the device layer on the workload's resident bank, then the
    masked pairs on the host cores from the bank of every expert in host memory, merged into the
    device output.  Own JSON line: value = host residual time per layer call; roofline = bytes of
    the cold experts' weights the host decoded per second against the host's read bandwidth measured
    in the same process (a multi-threaded sum over 2 GiB)."""
    import time as _time
    li = synth.layer_inputs(w, 0, T, device="cuda")
    bank = ft.ft_moe_pack_bank(li.bank.fmt, li.bank.n_slots, w.d, w.I, li.bank.w13, li.bank.w2, li.bank.s13,
                               li.bank.s2)
    log(f"residual: {w.name} T={T}; packing the {w.E} experts for the host bank")
    c = synth.make_bank(w.replace(n_resident=None, shared=False), 0, device="cuda")
    host = ft.ft_moe_pack_bank(c.fmt, w.E, w.d, w.I, c.w13, c.w2, c.s13, c.s2).to_pinned_host()
    del c
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    layer = ft.MoELayer(bank, li.slot_of_expert, w.k, T, shared_slot=w.shared_slot)
    x_host = li.x.cpu()
    res_dev = torch.empty(T, w.d, dtype=torch.float32, device="cuda")
    torch.set_num_threads(threads)
    probe = torch.ones(1 << 29, dtype=torch.float32)
    probe.sum()
    t0 = _time.perf_counter()
    for _ in range(3):
        probe.sum()
    host_gbs = 3 * probe.numel() * 4 / (_time.perf_counter() - t0) / 1e9
    del probe
    per_expert = sum(ft.ft_moe_bank_bytes(w.fmt, 1, w.d, w.I, which) for which in range(4))

    def step():
        t_a = _time.perf_counter()
        out, mask = layer.forward(li.logits, li.x)
        ids, wt, m = layer.ids[:T].cpu(), layer.w[:T].cpu(), mask.cpu()
        t_b = _time.perf_counter()
        res = ft.ft_moe_residual_host(host, x_host, ids, wt, m, n_threads=threads)
        t_c = _time.perf_counter()
        res_dev.copy_(res, non_blocking=False)
        ft.ft_moe_residual_add(out, res_dev)
        torch.cuda.synchronize()
        t_d = _time.perf_counter()
        mk = m.numpy().view(np.uint32)
        cold = {int(ids[t, j]) for t in range(T) for j in range(w.k) if (mk[t] >> j) & 1}
        pairs = sum(bin(int(v)).count("1") for v in mk)
        return t_b - t_a, t_c - t_b, t_d - t_c, len(cold), pairs

    for _ in range(max(warmup, 1)):
        step()
    r = [step() for _ in range(max(steps, 1))]
    dev_ms = 1e3 * sum(v[0] for v in r) / len(r)
    host_ms = 1e3 * sum(v[1] for v in r) / len(r)
    merge_ms = 1e3 * sum(v[2] for v in r) / len(r)
    cold, pairs = r[-1][3], r[-1][4]
    gbs = cold * per_expert / (host_ms * 1e-3) / 1e9
    log(f"residual: {pairs} cold pairs on {cold} experts; device layer + copies {dev_ms:.2f} ms, host residual "
        f"{host_ms:.2f} ms ({gbs:.1f} GB/s of weights; host read bandwidth {host_gbs:.1f} GB/s), merge {merge_ms:.2f} ms")
    roof = {"bound": "host", "achieved": round(gbs, 2), "peak": round(host_gbs, 1), "unit": "GB/s",
            "frac": round(gbs / host_gbs, 4), "traffic": None,
            "kernel": f"ft_moe_residual_host ({threads} host threads)", "cold_pairs": pairs, "cold_experts": cold,
            "bytes_per_expert": per_expert, "device_layer_and_copies_ms": round(dev_ms, 3),
            "merge_ms": round(merge_ms, 3)}
    print(json.dumps({"metric": "cold-expert residual on the host", "value": round(host_ms, 3), "unit": "ms/layer",
                      "n_gpus": 1, "steps": len(r), "warmup": warmup, "ms_per_step": round(dev_ms + host_ms + merge_ms, 3),
                      "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
                      "dtype": synth.FMT_NAMES[w.fmt], "data": "synthetic (seeded)",
                      "config": {"workload": f"residual/{w.name}", "T": T, "E": w.E, "k": w.k, "d": w.d, "I": w.I,
                                 "resident": w.n_resident, "threads": threads},
                      "roofline": roof, "cpu_baseline": None}), flush=True)


def bench_coexec(w: synth.Workload, T: int, steps: int, warmup: int, threads: int, fraction, max_loads: int):
    """Co-executed steps: the cold experts of each step are split between the host link (a fraction
    q of them copied to the GPU and computed there after the copy) and the host cores (the rest),
    both at once, beside the device FFN of the resident experts.  The device bank starts with the
    workload's resident set.  The same steps run with q = 0 (every cold pair on the host) for
    comparison.  With fraction "auto" the split is chosen the way the pages' engine does at start-up:
    the host link rate P (one fill of 8 experts) and the host residual rate H (every pair of the first
    step on the host) are measured, and q = P / (P + H) makes both paths finish together.  Own JSON
    line: value = ms per co-executed step (host thread joined, result merged)."""
    import threading
    import time as _time
    S = w.n_resident or w.E
    log(f"coexec: {w.name} T={T} slots={S} q={fraction} max_loads={max_loads}; packing {w.E} experts")
    c = synth.make_bank(w.replace(n_resident=None, shared=False), 0, device="cuda")
    host = ft.ft_moe_pack_bank(c.fmt, w.E, w.d, w.I, c.w13, c.w2, c.s13, c.s2).to_pinned_host()
    del c
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    table = synth.slot_table(w, 0)
    eos = torch.full((S,), -1, dtype=torch.int32)
    for e in torch.nonzero(table >= 0).flatten().tolist():
        eos[int(table[e])] = e
    dst = ft.DeviceBank.empty(w.fmt, S, w.d, w.I)
    x_host = synth.activations(w, 0, T)
    per_expert = sum(ft.ft_moe_bank_bytes(w.fmt, 1, w.d, w.I, which) for which in range(4))
    auto = None
    if fraction == "auto":
        nprobe = min(8, S)
        probe = ft.ExpertCache(w.E, S, nprobe)
        probe.loads.copy_(torch.stack([torch.arange(nprobe, dtype=torch.int32)] * 2, dim=1))
        probe.n_loads.fill_(nprobe)
        probe.fill(host, dst)                         # first touch of the pages
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        probe.fill(host, dst)
        b.record()
        torch.cuda.synchronize()
        P = nprobe * per_expert / (a.elapsed_time(b) * 1e-3) / 1e9
        ids0, w0 = ft.ft_moe_route(synth.step_logits(w, 0, T, device="cuda"), w.k)
        ids0, w0 = ids0.cpu(), w0.cpu()
        nocache = torch.full((w.E,), -1, dtype=torch.int32)
        ft.ft_moe_residual_host(host, x_host, ids0, w0, None, n_threads=threads, slot_of_expert=nocache)
        t0 = _time.perf_counter()
        ft.ft_moe_residual_host(host, x_host, ids0, w0, None, n_threads=threads, slot_of_expert=nocache)
        H = len(set(ids0.flatten().tolist())) * per_expert / (_time.perf_counter() - t0) / 1e9
        fraction = round(P / (P + H), 3)
        auto = {"link_gbs": round(P, 2), "host_gbs": round(H, 2), "q": fraction}
        log(f"coexec: measured host link {P:.1f} GB/s, host residual {H:.1f} GB/s of weights -> q = {fraction}")
    else:
        fraction = float(fraction)
    pre = ft.ExpertCache(w.E, S, S)
    pre.loads.copy_(torch.stack([eos, torch.arange(S, dtype=torch.int32)], dim=1))
    pre.n_loads.fill_(S)
    pre.fill(host, dst)
    x = x_host.cuda()
    k, E = w.k, w.E
    n_seq = warmup + steps
    logits = [synth.step_logits(w, i, T, device="cuda") for i in range(n_seq)]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()

    def run(q, ml):
        cache = ft.ExpertCache(E, S, ml, load_fraction=q)
        cache.slot_of_expert.copy_(table)
        cache.expert_of_slot.copy_(eos)
        torch.cuda.synchronize()
        rows = []
        for i in range(n_seq):
            t0 = _time.perf_counter()
            ids, wt = ft.ft_moe_route(logits[i], k)
            counts, offsets, gather, inv = ft.ft_moe_permute(ids, E)
            cs, _, nl = cache.update(counts)
            ids_h, w_h, slots_h = ids.cpu(), wt.cpu(), cache.slot_of_expert.cpu()
            res, ht = {}, {}

            def host_part():
                a = _time.perf_counter()
                res["r"] = ft.ft_moe_residual_host(host, x_host, ids_h, w_h, None, n_threads=threads,
                                                   slot_of_expert=slots_h)
                ht["s"] = _time.perf_counter() - a

            th = threading.Thread(target=host_part)
            th.start()
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            side.wait_stream(main)
            f0.record(side)
            cache.fill(host, dst, stream=side)
            f1.record(side)
            y, _ = ft.ft_moe_grouped_ffn(dst, cs, x, k, offsets, gather)
            main.wait_stream(side)
            ft.ft_moe_grouped_ffn(dst, cache.load_slot, x, k, offsets, gather, y_sorted=y)
            out, mask = ft.ft_moe_combine(y, None, ids, wt, inv, cache.slot_of_expert, w.d)
            torch.cuda.synchronize()
            t_gpu = _time.perf_counter() - t0
            th.join()
            ft.ft_moe_residual_add(out, res["r"].cuda())
            torch.cuda.synchronize()
            t_all = _time.perf_counter() - t0
            cold = int((slots_h.numpy()[ids_h.numpy()] < 0).sum())
            rows.append((t_all, t_gpu, ht["s"], f0.elapsed_time(f1) * 1e-3, int(nl.item()), cold))
        return rows[warmup:]

    base = run(0.0, 0)
    co = run(fraction, max_loads)
    mean = lambda rows, i: sum(r[i] for r in rows) / len(rows)  # noqa: E731
    base_ms, co_ms = 1e3 * mean(base, 0), 1e3 * mean(co, 0)
    host_ms, fill_ms, gpu_ms = 1e3 * mean(co, 2), 1e3 * mean(co, 3), 1e3 * mean(co, 1)
    loads, cold = mean(co, 4), mean(co, 5)
    log(f"coexec: host only {base_ms:.2f} ms/step (host {1e3 * mean(base, 2):.2f} ms, {mean(base, 5):.1f} cold pairs); "
        f"q={fraction}: {co_ms:.2f} ms/step (host {host_ms:.2f} ms for {cold:.1f} pairs, fill {fill_ms:.2f} ms for "
        f"{loads:.1f} experts, device part {gpu_ms:.2f} ms)")
    fill_gbs = loads * per_expert / (fill_ms * 1e-3) / 1e9 if fill_ms > 0 else 0.0
    if fill_ms >= host_ms:
        roof = {"bound": "pcie", "achieved": round(fill_gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                "frac": round(fill_gbs / PCIE_PEAK_GBS, 4)}
    else:
        roof = {"bound": "host", "achieved": round(host_ms, 3), "peak": None, "unit": "ms", "frac": None}
    roof.update({"traffic": None, "kernel": "cache_fill_kernel (host link) beside ft_moe_residual_host (host cores)",
                 "host_only_ms_per_step": round(base_ms, 3), "host_ms": round(host_ms, 3), "fill_ms": round(fill_ms, 3),
                 "device_part_ms": round(gpu_ms, 3), "loads_per_step": round(loads, 2),
                 "host_pairs_per_step": round(cold, 2), "fill_gbs": round(fill_gbs, 2), "measured_split": auto})
    print(json.dumps({"metric": "co-executed layer step (cold experts split between host link and host cores)",
                      "value": round(co_ms, 3), "unit": "ms/step", "n_gpus": 1, "steps": steps, "warmup": warmup,
                      "ms_per_step": round(co_ms, 3), "higher_is_better": False, "scaling": "weak",
                      "vs_baseline": None, "dtype": synth.FMT_NAMES[w.fmt], "data": "synthetic (seeded)",
                      "config": {"workload": f"coexec/{w.name}", "T": T, "E": E, "k": k, "d": w.d, "I": w.I,
                                 "slots": S, "load_fraction": fraction, "max_loads": max_loads, "threads": threads},
                      "roofline": roof, "cpu_baseline": None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_q4_0", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--T", type=int, default=None, help="tokens (default: the workload's)")
    ap.add_argument("--layers", type=int, default=None, help="layers per step (default: the workload's)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle time for the CPU baseline (half all-core, half one core)")
    ap.add_argument("--ffn-reps", type=int, default=3)
    ap.add_argument("--copies", type=int, default=None,
                    help="bank copies a single-layer workload rotates over (default: >= 4 and >= 1 GB per pass at decode)")
    ap.add_argument("--prefill", default="prefill_bf16_zipf", metavar="WORKLOAD",
                    help="prefill workload measured beside a decode workload in the same run ('' for none)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--widen", action="store_true",
                    help="MXFP4 / FP8 GEMM groups on the bf16 MFMA with widened weights (FT_GEMM_WIDEN)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="first run the counter-calibration copy kernel over BYTES")
    ap.add_argument("--route-proj", action="store_true",
                    help="time ft_moe_route_proj (router projection + top-k) on the workload's shape instead")
    ap.add_argument("--cache", type=int, default=0, metavar="SLOTS",
                    help="time layer steps with the LRU expert cache over SLOTS device slots instead")
    ap.add_argument("--max-loads", type=int, default=4, help="experts the cache may load per step")
    ap.add_argument("--residual", action="store_true",
                    help="time the layer with its cold experts on the host (ft_moe_residual_host) instead")
    ap.add_argument("--threads", type=int, default=16, help="host threads of the residual path")
    ap.add_argument("--coexec", default=None, metavar="Q",
                    help="time co-executed steps: a fraction Q of each step's cold experts copied to the GPU, the rest "
                         "on the host ('auto': Q from the host link and host residual rates measured first)")
    ap.add_argument("--layer-proj", action="store_true",
                    help="time the decode layer from its activations: router projection + layer, in two launches "
                         "and in one (ft_moe_layer_proj)")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure the device's achievable rates (ft_moe_measure_rates) and print them as one JSON line")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 counter CSVs into profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        w = synth.WORKLOADS[args.workload]
        pmc_summary(w.name, args.T or w.T, args.pmc_summary[0], args.pmc_summary[1], args.copy_probe,
                    os.path.join(ROOT, "profiles", "traffic.json"))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this layer is not sharded across GPUs here "
              "(see the sharding design); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS[args.workload]
    T = args.T or w.T
    n_layers = args.layers or w.layers
    decode = T <= 64
    if args.calibrate:
        calibrate()
        return
    if args.layer_proj:
        bench_layer_proj(w, T, n_layers, args.steps, args.warmup)
        return
    if args.route_proj:
        bench_route_proj(w, T, args.steps, args.warmup)
        return
    if args.coexec is not None:
        bench_coexec(w, T, args.steps, args.warmup, args.threads, args.coexec, args.max_loads)
        return
    if args.residual:
        bench_residual(w, T, args.steps, args.warmup, args.threads)
        return
    if args.cache:
        bench_cache(w, T, args.steps, args.warmup, args.cache, args.max_loads)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
    copies = args.copies
    if copies is None:  # single-layer decode workloads: at least 4 copies and 1 GB touched per pass
        copies = 1
        if n_layers == 1 and decode:
            per_layer = expected_touched_bytes(w, T)
            copies = int(min(16, max(4, -(-1e9 // per_layer))))
    m = measure(w, T, n_layers, args.steps, args.warmup, not args.no_graph, args.ffn_reps, copies,
                ft.FT_GEMM_WIDEN if args.widen else 0)

    # ---- the prefill half of the metric, measured in the same run beside the default decode workload
    prefill = None
    if args.prefill and decode:
        wp = synth.WORKLOADS[args.prefill]
        mp = measure(wp, wp.T, 1, args.prefill_steps, args.warmup, not args.no_graph, args.ffn_reps, 1)
        prefill = {"metric": "MoE-layer prefill throughput", "value": round(mp["tokens_per_s"], 1),
                   "unit": "tokens/s", "ms_per_layer": round(mp["ms_per_step"], 4), "steps": args.prefill_steps,
                   "config": mp["config"], "roofline": mp["roofline"], "step_ms": mp["spread"]}

    # ---- CPU baseline: the oracle on host cores, bounded sample
    cpu = cpu_baseline_record(w, T, args.cpu_budget, decode) if args.cpu_budget > 0 else None

    if decode:
        metric, value, unit, hib = "MoE-layer decode latency", m["us_per_layer"], "us/layer", False
    else:
        metric, value, unit, hib = "MoE-layer prefill throughput", m["tokens_per_s"], "tokens/s", True
    line = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(m["ms_per_step"], 4), "higher_is_better": hib, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": m["config"],
        "roofline": m["roofline"],
        "cpu_baseline": cpu,
        "step_ms": m["spread"],
    }
    if prefill is not None:
        line["prefill"] = prefill
    print(json.dumps(line), flush=True)


def expected_touched_bytes(w: synth.Workload, T: int) -> float:
    """Bytes a layer call is expected to touch before its routing is known: the resident experts a
    batch of T tokens reaches at most (T * k, E or the resident count), plus the shared expert."""
    resident = w.n_resident or w.E
    experts = min(T * w.k, resident) + (1 if w.shared else 0)
    return max(experts * synth.expert_bytes(w.fmt, w.d, w.I), 1.0)


def measure(w: synth.Workload, T: int, n_layers: int, steps: int, warmup: int, use_graph: bool, ffn_reps: int,
            copies: int = 1, flags: int = 0):
    """One workload: warm-up, a HIP graph of one step (every layer call of it) replayed `steps`
    times in the timed region, then the layer call timed on its stream against the rooflines."""
    log(f"workload {w.name}: T={T} d={w.d} E={w.E} k={w.k} I={w.I} fmt={synth.FMT_NAMES[w.fmt]} layers={n_layers}"
        + (f" x {copies} bank copies" if copies > 1 else ""))
    layers = build_layers(w, T, n_layers, copies, flags)
    calls = n_layers * copies  # layer calls per step

    for _ in range(max(warmup, 1)):
        run_step(layers)
    torch.cuda.synchronize()
    check_status(layers, "warm-up")
    graph = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run_step(layers)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s):
                run_step(layers)
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        check_status(layers, "graph warm-up")

    # ---- timed region (events between steps give the spread; the value is the whole region's time)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(steps):
        if graph is not None:
            graph.replay()
        else:
            run_step(layers)
        marks[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    check_status(layers, "timed steps")
    ms_per_step = elapsed / steps * 1e3
    us_per_layer = ms_per_step * 1e3 / calls
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
    spread = {q: round(float(np.percentile(per_step, p)), 4) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}
    log(f"{ms_per_step:.3f} ms/step, {us_per_layer:.2f} us/layer; per-step ms {spread}")

    # ---- dominant unit: the layer call, event-timed on its stream
    ffn_us = time_layer_calls(layers, ffn_reps)
    check_status(layers, "event-timed layer calls")
    bytes_call, flops_call, pairs, touched = algorithmic_work(w, layers, T)
    # the bound is the resource whose roofline time (algorithmic bytes at the HBM peak, or algorithmic
    # flops at the bf16 MFMA peak) is the longer, i.e. the one with the larger fraction; the other is
    # reported beside it
    gbs = bytes_call / (ffn_us * 1e-6) / 1e9
    tfs = flops_call / (ffn_us * 1e-6) / 1e12
    # the MFMA type the GEMM groups run on: MXFP4 (e2m3 activation terms x e2m1 weights) and FP8-B128
    # (e4m3 x e4m3) on the scaled low-precision MFMA above the one-launch decode sizes, unless widened
    # to bf16; two activation terms per element issue twice the algorithmic MFMA flops
    mx = T > 16 and not (flags & ft.FT_GEMM_WIDEN) and w.fmt in (synth.FMT_MXFP4, synth.FMT_FP8_B128)
    mfma_dtype = ("fp4" if w.fmt == synth.FMT_MXFP4 else "fp8") if mx else "bf16"
    peak = MFMA_PEAK_TFLOPS[mfma_dtype]
    hbm = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    mfma = {"bound": "mfma", "achieved": round(tfs, 1), "peak": peak, "unit": "TFLOP/s", "frac": round(tfs / peak, 4),
            "mfma_dtype": mfma_dtype}
    if mx:
        mfma["two_term_issued_flops_per_call"] = round(2 * flops_call)
    roof, other = (hbm, mfma) if gbs / HBM_PEAK_GBS >= tfs / peak else (mfma, hbm)
    roof = dict(roof)
    roof["traffic"] = None
    prof = os.path.join(ROOT, "profiles", "traffic.json")
    src_hash = kernel_source_hash()
    if os.path.exists(prof):
        rec = json.load(open(prof)).get(traffic_key(w.name, T))
        if rec and rec.get("source_hash") == src_hash and rec.get("T") == T:
            roof["traffic"] = rec["bytes_per_call"]
    roof["kernel"] = ("ft_moe_layer: layer_decode_kernel (one launch: routing, permutation, streaming GEMV, "
                      "combine)" if T <= 16 else
                      "ft_moe_layer: route, permute, grouped FFN (MFMA GEMM + GEMV), combine kernels")
    roof["per_call_us"] = round(ffn_us, 3)
    roof["algorithmic_bytes_per_call"] = round(bytes_call)
    roof["algorithmic_flops_per_call"] = round(flops_call)
    roof["other_bound"] = other
    # intermediate rows that cross kernel (or, in the one-launch layer, block) boundaries through
    # memory: h written by gate/up and read by down, y written by down and read by combine
    roof["boundary_bytes_per_call"] = round(2 * pairs * (w.d + w.I) * 2)
    log(f"layer call {ffn_us:.2f} us; {touched:.1f} experts touched, {pairs:.1f} pairs; {roof}")
    config = {"workload": w.name, "T": T, "d": w.d, "E": w.E, "k": w.k, "I": w.I,
              "bank_format": synth.FMT_NAMES[w.fmt], "layers_per_step": n_layers,
              "shared_expert": w.shared, "resident_experts": w.n_resident or w.E, "graph": graph is not None}
    if copies > 1:
        config["bank_copies"] = copies
    if flags & ft.FT_GEMM_WIDEN:
        config["gemm"] = "bf16 MFMA, weights widened"
    out = dict(ms_per_step=ms_per_step, us_per_layer=us_per_layer, tokens_per_s=T / (ms_per_step * 1e-3 / calls),
               spread=spread, roofline=roof, config=config)
    del graph, layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
